// stream_read.hip — streaming-read probe: the bandwidth ceiling the mat-vecs
// are held against ("25 — Writing XPU Kernels", section 25.1: measure the
// bandwidth once per device with a streaming pass well past L2).
//
// Every 16-byte chunk of the buffer is read exactly once with a 16-byte
// non-temporal load (the data is used once), all of them issued at once: one
// workgroup of 512 lanes per 16 KiB, two loads per lane, no loop. This was the
// fastest shape measured on MI355X at 33 MB and at 295 MB (against looping
// grids of 512 workgroups, more or fewer loads per lane, 256 or 1024 lanes,
// and plain loads), so the ceiling it reports holds at the mat-vecs' own
// sizes. A workgroup's chunks are folded into one word so no load is dead.
#include "xq_device.h"
#include "xq_launch.h"

namespace xq {
namespace {

constexpr int kThreads = 512;
constexpr int kLoads = 2;  // 16-byte loads per lane
constexpr int64_t kChunksPerGroup = static_cast<int64_t>(kThreads) * kLoads;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ldnt(const uint4* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ buf,
                                                               int64_t n16,
                                                               uint32_t* __restrict__ sink) {
  __shared__ uint32_t part[kThreads / kWave];
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * kChunksPerGroup + threadIdx.x;
  const int64_t i1 = i0 + kThreads;
  // The last workgroup may pass the end: its extra lanes re-read the last
  // chunk and drop it.
  const u32x4 a = ldnt(buf + (i0 < n16 ? i0 : n16 - 1));
  const u32x4 b = ldnt(buf + (i1 < n16 ? i1 : n16 - 1));
  uint32_t acc = (i0 < n16 ? (a.x ^ a.y ^ a.z ^ a.w) : 0u) + (i1 < n16 ? (b.x ^ b.y ^ b.z ^ b.w) : 0u);
  const float f = wave_sum(static_cast<float>(acc & 0xFFFF));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = __builtin_bit_cast(uint32_t, f);
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
#pragma unroll
    for (int k = 0; k < kThreads / kWave; ++k) r ^= part[k];
    sink[blockIdx.x] = r;
  }
}

}  // namespace

int64_t stream_read_sink_words(int64_t bytes) {
  const int64_t n16 = bytes / 16;
  const int64_t groups = (n16 + kChunksPerGroup - 1) / kChunksPerGroup;
  return groups < 1 ? 1 : groups;
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
