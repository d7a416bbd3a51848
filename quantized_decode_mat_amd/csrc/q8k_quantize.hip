// q8k_quantize.hip — f32 activations -> q8_K blocks on gfx950.
//
// "25 — Writing XPU Kernels", section 25.2 (integer-route bullet): the
// activation is quantized once to q8_K, 256 int8 codes, eight sums of 32 codes
// and one f32 scale in 320 bytes; section 25.2.1 gives the offsets (+0 codes,
// +256 sums, +288 scale).
//
// One wave per 256-block, four blocks per 256-thread workgroup. Lane l holds
// elements 4l..4l+3 (one 16-byte load), so the block's 1 KiB is read by one
// coalesced wave load. The scale is amax/127 and each code x/d, both as IEEE
// f32 divisions (HIP's default division is correctly rounded; nothing here is
// built with fast-math), rounded to nearest-even by v_rndne_f32.
#include "xq_device.h"
#include "xq_launch.h"

namespace xq {
namespace {

__device__ __forceinline__ int code_of(float x, float d) {
  float r = rintf(x / d);
  r = fminf(fmaxf(r, -127.0f), 127.0f);  // never active: |x/d| <= 127*(1+2^-23)
  return static_cast<int>(r);
}

__global__ __launch_bounds__(256) void q8k_quantize_kernel(uint8_t* __restrict__ xq,
                                                           const float* __restrict__ x,
                                                           int64_t nblocks) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (blk >= nblocks) return;  // wave-uniform: no cross-wave sync follows

  const float4 v = *reinterpret_cast<const float4*>(x + blk * 256 + lane * 4);
  const float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  const float amax = wave_max(a);
  const float d = amax / 127.0f;

  int q0 = 0, q1 = 0, q2 = 0, q3 = 0;
  if (d != 0.0f) {
    q0 = code_of(v.x, d);
    q1 = code_of(v.y, d);
    q2 = code_of(v.z, d);
    q3 = code_of(v.w, d);
  }
  const uint32_t packed = (static_cast<uint32_t>(q0) & 0xFFu) |
                          ((static_cast<uint32_t>(q1) & 0xFFu) << 8) |
                          ((static_cast<uint32_t>(q2) & 0xFFu) << 16) |
                          ((static_cast<uint32_t>(q3) & 0xFFu) << 24);
  const int s = lane8_sum(q0 + q1 + q2 + q3);  // lanes 8j..8j+7 hold codes 32j..32j+31

  uint8_t* out = xq + blk * kQ8KBytes;
  reinterpret_cast<uint32_t*>(out)[lane] = packed;
  if ((lane & 7) == 0) reinterpret_cast<int32_t*>(out + 256)[lane >> 3] = s;
  if (lane == 0) *reinterpret_cast<float*>(out + 288) = d;
  if (lane >= 1 && lane < 8) reinterpret_cast<uint32_t*>(out + 288)[lane] = 0u;  // 292..319
}

}  // namespace

hipError_t launch_quantize_q8k(void* xq, const float* x, int64_t rows, int64_t K,
                               hipStream_t stream) {
  const int64_t nblocks = rows * (K / 256);
  const int64_t grid = (nblocks + 3) / 4;
  hipLaunchKernelGGL(q8k_quantize_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream,
                     static_cast<uint8_t*>(xq), x, nblocks);
  return hipGetLastError();
}

}  // namespace xq
