// stream_read.hip — streaming-read probe: the bandwidth ceiling the mat-vecs
// are held against ("25 — Writing XPU Kernels", section 25.1: measure the
// bandwidth once per device with a streaming pass well past L2).
//
// Every 16-byte chunk of the buffer is read exactly once with a 16-byte
// non-temporal load (the data is used once); a workgroup's chunks are folded
// into one word so no load is dead. Four loads per lane are in flight per
// loop trip, two workgroups per CU: the fastest of the grid sizes, unroll
// depths and load kinds measured on MI355X for a 2 GiB read.
#include "xq_device.h"
#include "xq_launch.h"

namespace xq {
namespace {

constexpr int kThreads = 256;
constexpr int kGrid = 256 * 2;  // two workgroups per CU

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ldnt(const uint4* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ buf,
                                                               int64_t n16,
                                                               uint32_t* __restrict__ sink) {
  __shared__ uint32_t part[kThreads / kWave];
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = ldnt(buf + i), b = ldnt(buf + i + stride), c = ldnt(buf + i + 2 * stride),
                d = ldnt(buf + i + 3 * stride);
    acc ^= (a.x ^ a.y ^ a.z ^ a.w) + (b.x ^ b.y ^ b.z ^ b.w) + (c.x ^ c.y ^ c.z ^ c.w) +
           (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < n16; i += stride) {
    const u32x4 a = ldnt(buf + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  const float f = wave_sum(static_cast<float>(acc & 0xFFFF));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = __builtin_bit_cast(uint32_t, f);
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

int64_t stream_read_sink_words(int64_t bytes) {
  const int64_t n16 = bytes / 16;
  const int64_t need = (n16 + kThreads - 1) / kThreads;
  return need < kGrid ? (need < 1 ? 1 : need) : kGrid;
}

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink,
                              hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  const int grid = static_cast<int>(stream_read_sink_words(bytes));
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kThreads), 0, stream,
                     static_cast<const uint4*>(buf), n16, sink);
  return hipGetLastError();
}

}  // namespace xq
