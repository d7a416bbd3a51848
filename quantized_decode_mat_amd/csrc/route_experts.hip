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
// One workgroup of 1024 threads: a histogram of the buckets in LDS, three
// block-wide exclusive scans (pair offsets and the two lists' tile offsets),
// a scatter of the pairs, then the tile descriptors. The order of the pairs inside a
// bucket follows LDS atomics and may differ from run to run; the product
// computes every output from its own token row and expert alone, so the
// result does not depend on it.
#include <algorithm>

#include "xq_device.h"
#include "xq_launch.h"

namespace xq {
namespace {

constexpr int kRouteThreads = 1024;
constexpr int kRouteBuckets = 2 * kRouteThreads;  // each thread owns two buckets

// Exclusive scan over the workgroup of one value per thread; *total gets the
// sum. Every thread must call it.
__device__ int block_exclusive_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int u = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += u;
  }
  if (lane == kWave - 1) wsum[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const int n = kRouteThreads / kWave;
    int w = (lane < n) ? wsum[lane] : 0;
#pragma unroll
    for (int d = 1; d < n; d <<= 1) {
      const int u = __shfl_up(w, d, kWave);
      if (lane >= d) w += u;
    }
    if (lane < n) wsum[lane] = w;  // inclusive over waves
  }
  __syncthreads();
  const int before = (wave > 0) ? wsum[wave - 1] : 0;
  *total = wsum[kRouteThreads / kWave - 1];
  __syncthreads();  // wsum is reused by the next scan
  return before + inc - v;
}

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

__global__ __launch_bounds__(kRouteThreads) void route_experts_kernel(
    const int32_t* __restrict__ ids, int n_pairs, int n_experts, int tile_m, int tile_s,
    int32_t* __restrict__ sorted, int4* __restrict__ desc, int32_t* __restrict__ n_tiles,
    int4* __restrict__ desc_s, int32_t* __restrict__ n_small) {
  __shared__ int cnt[kRouteBuckets];
  __shared__ int fill[kRouteBuckets];
  __shared__ int off[kRouteBuckets];
  __shared__ int toff[kRouteBuckets];
  __shared__ int soff[kRouteBuckets];
  __shared__ int wsum[kRouteThreads / kWave];
  const int tid = threadIdx.x;
  const int B = n_experts + 1;  // the last bucket holds out-of-range selections

  for (int b = tid; b < kRouteBuckets; b += kRouteThreads) {
    cnt[b] = 0;
    fill[b] = 0;
  }
  __syncthreads();
  for (int p = tid; p < n_pairs; p += kRouteThreads) {
    const int e = ids[p];
    atomicAdd(&cnt[(e >= 0 && e < n_experts) ? e : n_experts], 1);
  }
  __syncthreads();

  const int b0 = 2 * tid, b1 = 2 * tid + 1;
  const int c0 = (b0 < B) ? cnt[b0] : 0;
  const int c1 = (b1 < B) ? cnt[b1] : 0;
  const BucketTiles t0 = bucket_tiles(c0, tile_m, tile_s);
  const BucketTiles t1 = bucket_tiles(c1, tile_m, tile_s);
  int pairs_total = 0, tiles_total = 0, small_total = 0;
  const int oc = block_exclusive_scan(c0 + c1, wsum, &pairs_total);
  const int ot = block_exclusive_scan(t0.big + t1.big, wsum, &tiles_total);
  const int os = block_exclusive_scan(t0.small + t1.small, wsum, &small_total);
  off[b0] = oc;
  off[b1] = oc + c0;
  toff[b0] = ot;
  toff[b1] = ot + t0.big;
  soff[b0] = os;
  soff[b1] = os + t0.small;
  if (tid == 0) {
    *n_tiles = tiles_total;
    *n_small = small_total;
  }
  __syncthreads();

  for (int p = tid; p < n_pairs; p += kRouteThreads) {
    const int e = ids[p];
    const int b = (e >= 0 && e < n_experts) ? e : n_experts;
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
