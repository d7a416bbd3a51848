// route_experts.hip — the expert map of a grouped product, built on the GPU.
//
// "25 — Writing XPU Kernels", section 25.3: a mixture-of-experts prefill is
// one launch over an expert map (mul_mat_id), never one GEMM per expert, and
// a ragged expert batch is padded only to the finest tile. This kernel turns
// the router's selections ids[t][k] (expert of token t's slot k) into that
// map: the pairs p = t * n_used + k grouped by expert, and two lists of
// tiles of one expert each: whole tiles of up to tile_m pairs, and the
// expert's remainder, when it is at most two small tiles' worth, in tiles of
// up to tile_s pairs (a larger remainder takes one more tile_m tile), so an
// expert's few leftover pairs are not padded to tile_m. Selections outside
// 0..n_experts-1 form one more bucket, whose tiles the product fills with NaN.
//
// One workgroup of 1024 threads. The first kWindow pairs are read in one batch
// of independent loads per thread, and the LDS atomic that counts a pair also
// hands it its rank in its bucket, kept in registers for the scatter; pairs
// past the window (up to 2^20) are counted after them and ranked by a second
// atomic at the scatter, from where the window's counts end. One wave scans the
// buckets (pair offsets and both lists' tile offsets at once), then the pairs
// are scattered and the tile descriptors written. The order of the pairs inside
// a bucket follows LDS atomics and may differ from run to run; the product
// computes every output from its own token row and expert alone, so the result
// does not depend on it.
#include <algorithm>

#include "xq_device.h"
#include "xq_launch.h"

namespace xq {
namespace {

constexpr int kRouteThreads = 1024;
constexpr int kRouteBuckets = 2048;
constexpr int kWindowPerThread = 8;
constexpr int kWindow = kRouteThreads * kWindowPerThread;

// A bucket of c pairs: c / tile_m whole tiles; its remainder r in small
// tiles when r <= 2 * tile_s, else in one more whole tile.
struct BucketTiles {
  int big, small;
};
__device__ __forceinline__ BucketTiles bucket_tiles(int c, int tile_m, int tile_s) {
  const int full = c / tile_m;
  const int r = c - full * tile_m;
  if (r > 2 * tile_s) return BucketTiles{full + 1, 0};
  return BucketTiles{full, (r + tile_s - 1) / tile_s};
}

__device__ __forceinline__ int bucket_of(int e, int n_experts) {
  return (e >= 0 && e < n_experts) ? e : n_experts;
}

// Inclusive scan of v over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int u = __shfl_up(v, d, kWave);
    if (lane >= d) v += u;
  }
  return v;
}

__global__ __launch_bounds__(kRouteThreads) void route_experts_kernel(
    const int32_t* __restrict__ ids, int n_pairs, int n_experts, int tile_m, int tile_s,
    int32_t* __restrict__ sorted, int4* __restrict__ desc, int32_t* __restrict__ n_tiles,
    int4* __restrict__ desc_s, int32_t* __restrict__ n_small) {
  __shared__ int cnt[kRouteBuckets];
  __shared__ int fill[kRouteBuckets];  // next rank for pairs past the window
  __shared__ int off[kRouteBuckets];
  __shared__ int toff[kRouteBuckets];
  __shared__ int soff[kRouteBuckets];
  const int tid = threadIdx.x;
  const int B = n_experts + 1;  // the last bucket holds out-of-range selections

  for (int b = tid; b < B; b += kRouteThreads) cnt[b] = 0;
  __syncthreads();

  // The window: pair j * kRouteThreads + tid for j < kWindowPerThread.
  int bk[kWindowPerThread], rk[kWindowPerThread];
#pragma unroll
  for (int j = 0; j < kWindowPerThread; ++j) {
    const int p = j * kRouteThreads + tid;
    bk[j] = (p < n_pairs) ? bucket_of(ids[p], n_experts) : -1;
  }
#pragma unroll
  for (int j = 0; j < kWindowPerThread; ++j)
    if (bk[j] >= 0) rk[j] = atomicAdd(&cnt[bk[j]], 1);
  __syncthreads();
  if (n_pairs > kWindow) {
    for (int b = tid; b < B; b += kRouteThreads) fill[b] = cnt[b];
    __syncthreads();  // the snapshot is taken before the rest is counted
    for (int p = kWindow + tid; p < n_pairs; p += kRouteThreads)
      atomicAdd(&cnt[bucket_of(ids[p], n_experts)], 1);
    __syncthreads();
  }

  // One wave scans the buckets, lane l taking a run of q consecutive ones.
  if (tid < kWave) {
    const int lane = tid;
    const int q = (B + kWave - 1) / kWave;
    const int lo = min(B, lane * q), hi = min(B, lo + q);
    int sc = 0, sb = 0, ss = 0;
    for (int b = lo; b < hi; ++b) {
      const int c = cnt[b];
      const BucketTiles t = bucket_tiles(c, tile_m, tile_s);
      sc += c;
      sb += t.big;
      ss += t.small;
    }
    const int ic = wave_inclusive_scan(sc, lane);
    const int ib = wave_inclusive_scan(sb, lane);
    const int is = wave_inclusive_scan(ss, lane);
    int oc = ic - sc, ob = ib - sb, os = is - ss;
    for (int b = lo; b < hi; ++b) {
      const int c = cnt[b];
      const BucketTiles t = bucket_tiles(c, tile_m, tile_s);
      off[b] = oc;
      toff[b] = ob;
      soff[b] = os;
      oc += c;
      ob += t.big;
      os += t.small;
    }
    if (lane == kWave - 1) {
      *n_tiles = ib;
      *n_small = is;
    }
  }
  __syncthreads();

#pragma unroll
  for (int j = 0; j < kWindowPerThread; ++j)
    if (bk[j] >= 0) sorted[off[bk[j]] + rk[j]] = j * kRouteThreads + tid;
  for (int p = kWindow + tid; p < n_pairs; p += kRouteThreads) {
    const int b = bucket_of(ids[p], n_experts);
    sorted[off[b] + atomicAdd(&fill[b], 1)] = p;
  }
  for (int b = tid; b < B; b += kRouteThreads) {
    const int c = cnt[b];
    const BucketTiles t = bucket_tiles(c, tile_m, tile_s);
    for (int j = 0; j < t.big; ++j)
      desc[toff[b] + j] = make_int4(b, off[b] + j * tile_m, min(tile_m, c - j * tile_m), 0);
    const int first = off[b] + t.big * tile_m;  // the small tiles' pairs follow the whole tiles'
    const int r = c - t.big * tile_m;
    for (int k = 0; k < t.small; ++k)
      desc_s[soff[b] + k] = make_int4(b, first + k * tile_s, min(tile_s, r - k * tile_s), 0);
  }
}

}  // namespace

int64_t route_max_tiles(int64_t n_pairs, int64_t n_experts, int tile_m) {
  // Each bucket b holds c_b pairs in at most ceil(c_b / tile_m) whole tiles,
  // and no tile is empty.
  return std::min<int64_t>(n_pairs, (n_pairs + (tile_m - 1) * (n_experts + 1)) / tile_m);
}

int64_t route_max_small_tiles(int64_t n_pairs, int64_t n_experts) {
  // At most two small tiles per bucket, and no tile is empty.
  return std::min<int64_t>(n_pairs, 2 * (n_experts + 1));
}

hipError_t launch_route_experts(const int32_t* ids, int64_t n_pairs, int64_t n_experts,
                                int tile_m, int tile_s, int32_t* sorted, void* desc,
                                int32_t* n_tiles, void* desc_s, int32_t* n_small,
                                hipStream_t stream) {
  if (n_experts + 1 > kRouteBuckets || tile_s < 1 || 2 * tile_s >= tile_m)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(route_experts_kernel, dim3(1), dim3(kRouteThreads), 0, stream, ids,
                     static_cast<int>(n_pairs), static_cast<int>(n_experts), tile_m, tile_s,
                     sorted, static_cast<int4*>(desc), n_tiles, static_cast<int4*>(desc_s),
                     n_small);
  return hipGetLastError();
}

}  // namespace xq
