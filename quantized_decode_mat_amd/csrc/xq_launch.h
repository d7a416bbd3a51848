// xq_launch.h — internal launchers called by the C ABI (xq_api.cpp) after it
// has validated every argument. Each returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xq {

// The longest row whose q8_K activation the mat-vecs stage whole in a
// workgroup's LDS (192 blocks = 60 KiB); longer rows (up to XQ_MAX_K) read it
// from global memory instead.
constexpr int64_t kMaxStagedK = 49152;

// Three launchers take a caller-owned device workspace (`ws`, `ws_bytes`):
// the split-K partials and arrival counters of the small-M product, the
// arrival counters of the fused quantizing mat-vec, and the grouped
// product's expert map. The *_workspace_bytes functions give the bytes a
// call needs (0: none). Arrival counters must be zero before a workspace's
// first use; every completed call leaves them at zero again.
hipError_t launch_quantize_q8k(void* xq, const float* x, int64_t rows, int64_t K,
                               hipStream_t stream);
hipError_t launch_gemv_q4k(float* y, const void* w, const void* xq, int64_t N, int64_t K,
                           hipStream_t stream);
hipError_t launch_gemv_iq4nl(float* y, const void* w, const void* xq, int64_t N, int64_t K,
                             hipStream_t stream);
// Expert-grouped mat-vecs: `used` slots, slot kk reads expert sel[kk] (rows
// rows of the slab) and the activation x_stride_blocks q8_K blocks per slot
// into xq; output slot-major.
// y = W x as launch_gemv_q4k, and yq = q8_K(y) as launch_quantize_q8k(yq, y,
// 1, N) would give, in the same launch (N a multiple of 256, N <= 2^22).
size_t gemv_q4k_q8k_workspace_bytes(int64_t N);
hipError_t launch_gemv_q4k_q8k(float* y, void* yq, const void* w, const void* xq, int64_t N,
                               int64_t K, void* ws, size_t ws_bytes, hipStream_t stream);
hipError_t launch_gemv_q4k_id(float* y, const void* slab, const void* xq, const int32_t* sel,
                              int64_t n_experts, int64_t used, int64_t rows, int64_t K,
                              int64_t x_stride_blocks, hipStream_t stream);
hipError_t launch_gemv_iq4nl_id(float* y, const void* slab, const void* xq, const int32_t* sel,
                                int64_t n_experts, int64_t used, int64_t rows, int64_t K,
                                int64_t x_stride_blocks, hipStream_t stream);
// IQ4_NL file blocks (18 B) -> resident rows; the count of launches that
// took the row-aligned (dword prefix) route.
hipError_t launch_repack_iq4nl(void* resident, const void* file_blocks, int64_t n,
                               int64_t block_base, int64_t bpr, hipStream_t stream);
int64_t repack_dword_prefix_launches();
hipError_t launch_gemv_q4_0(float* y, const void* w, const void* xq, int64_t N, int64_t K,
                            hipStream_t stream);
// M tokens (M <= gemv_q4k_multi_max_tokens(K)) against one pass over the Q4_K
// weights: y [M][N], each row the bits of the mat-vec on that token.
int64_t gemv_q4k_multi_max_tokens(int64_t K);
hipError_t launch_gemv_q4k_multi(float* y, const void* w, const void* xq, int64_t M, int64_t N,
                                 int64_t K, hipStream_t stream);
size_t gemm_q4k_workspace_bytes(int64_t M, int64_t N, int64_t K);
// The same product with its split-K scratch in the library's per-device
// static array (gemm_q4k_noalloc_scratch_bytes of it): no allocation and no
// workspace argument; shapes needing more scratch are refused.
size_t gemm_q4k_noalloc_scratch_bytes();
hipError_t launch_gemm_q4k_noalloc(float* y, const void* w, const void* xq, int64_t M, int64_t N,
                                   int64_t K, hipStream_t stream);
hipError_t launch_gemm_q4k(float* y, const void* w, const void* xq, int64_t M, int64_t N,
                           int64_t K, void* ws, size_t ws_bytes, hipStream_t stream);
// Whether launch_gemm_q4k serves this shape with the mat-vec kernels.
bool gemm_q4k_uses_matvec(int64_t M, int64_t N, int64_t K);
// Whether it serves it with the wave-split short-batch tile (no workspace).
bool gemm_q4k_uses_wave_split(int64_t M, int64_t N, int64_t K);
// The small-M product's launch plan: tiles 0..n_full-1 (of bm tokens x 128
// rows, token tile fastest) run whole, the rest split K ks ways (ks = 1:
// every tile whole). Needs, when ks > 1: 1 <= tiles - n_full <= 768,
// (tiles - n_full) * ks <= 768 and ks <= K/256.
struct GemmPlan {
  int n_full;
  int ks;
};
// The token tile for a shape (16 or 64 tokens), the plan launch_gemm_q4k
// uses, and the product with an explicit tile and plan.
int gemm_q4k_token_tile(int64_t M, int64_t N, int64_t K);
GemmPlan gemm_q4k_plan(int64_t M, int64_t N, int64_t K, int bm);
hipError_t launch_gemm_q4k_split(float* y, const void* w, const void* xq, int64_t M, int64_t N,
                                 int64_t K, const GemmPlan& plan, int bm, void* ws,
                                 size_t ws_bytes, hipStream_t stream);
// Grouped small-M product: route the (token, slot) pairs of ids by expert,
// then one product launch over the tile list (at most 2^20 pairs and 1024
// experts).
size_t gemm_q4k_id_workspace_bytes(int64_t n_pairs, int64_t n_experts);
hipError_t launch_gemm_q4k_id(float* y, const void* slab, const void* xq, const int32_t* ids,
                              int64_t n_tokens, int64_t n_used, int64_t n_experts, int64_t rows,
                              int64_t K, int per_slot_x, void* ws, size_t ws_bytes,
                              hipStream_t stream);
// The expert map: pairs grouped by expert into `sorted`; tiles of at most
// tile_m pairs of one bucket into `desc` (int4: bucket, first, count, 0) and
// their count into *n_tiles; a bucket's remainder of at most 2 * tile_s
// pairs in tiles of at most tile_s pairs into `desc_s`, their count into
// *n_small. route_max_tiles and route_max_small_tiles bound the counts.
hipError_t launch_route_experts(const int32_t* ids, int64_t n_pairs, int64_t n_experts,
                                int tile_m, int tile_s, int32_t* sorted, void* desc,
                                int32_t* n_tiles, void* desc_s, int32_t* n_small,
                                hipStream_t stream);
int64_t route_max_tiles(int64_t n_pairs, int64_t n_experts, int tile_m);
int64_t route_max_small_tiles(int64_t n_pairs, int64_t n_experts);
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink,
                              hipStream_t stream);
int64_t stream_read_sink_words(int64_t bytes);

}  // namespace xq
