// q8k_quantize.hip — f32 activations -> q8_K blocks on gfx950.
//
// "25 — Writing XPU Kernels", section 25.2 (integer-route bullet): the
// activation is quantized once to q8_K, 256 int8 codes, eight sums of 32 codes
// and one f32 scale in 320 bytes; section 25.2.1 gives the offsets (+0 codes,
// +256 sums, +288 scale).
//
// One wave per 256-block, four blocks per 256-thread workgroup. Lane l holds
// elements 4l..4l+3 (one 16-byte load when the rows start 16-byte aligned,
// else four 4-byte loads of the same elements), so the block's 1 KiB is read
// by coalesced wave loads; the block arithmetic is q8k_block_wave.
#include "q8k_block.h"
#include "xq_launch.h"

namespace xq {
namespace {

template <bool VEC>
__global__ __launch_bounds__(256) void q8k_quantize_kernel(uint8_t* __restrict__ xq,
                                                           const float* __restrict__ x,
                                                           int64_t nblocks) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (blk >= nblocks) return;  // wave-uniform: no cross-wave sync follows

  const float* p = x + blk * 256 + lane * 4;
  float4 v;
  if constexpr (VEC) {
    v = *reinterpret_cast<const float4*>(p);
  } else {
    v = make_float4(p[0], p[1], p[2], p[3]);
  }
  q8k_block_wave(v, xq + blk * kQ8KBytes, lane);
}

}  // namespace

hipError_t launch_quantize_q8k(void* xq, const float* x, int64_t rows, int64_t K,
                               hipStream_t stream) {
  const int64_t nblocks = rows * (K / 256);
  const int64_t grid = (nblocks + 3) / 4;
  // K is a multiple of 256, so every row starts as aligned as x.
  if (reinterpret_cast<uintptr_t>(x) % 16 == 0)
    hipLaunchKernelGGL(q8k_quantize_kernel<true>, dim3(static_cast<uint32_t>(grid)), dim3(256), 0,
                       stream, static_cast<uint8_t*>(xq), x, nblocks);
  else
    hipLaunchKernelGGL(q8k_quantize_kernel<false>, dim3(static_cast<uint32_t>(grid)), dim3(256), 0,
                       stream, static_cast<uint8_t*>(xq), x, nblocks);
  return hipGetLastError();
}

}  // namespace xq
