// gemv_q4k.hip — Q4_K x q8_K decode mat-vec on gfx950 (wave64).
//
// The integer route of "25 — Writing XPU Kernels", section 25.2: the
// activation arrives quantized to q8_K; every weight nibble meets an int8 code
// in a signed 4 x int8 dot (v_dot4_i32_i8; the 4-bit codes 0..15 are valid
// signed bytes); the sub-block scales multiply the integer sub-block dots in
// 24-bit integer multiplies; the min term is paid from the q8_K's stored
// sub-block sums; the f16/f32 scales are applied once per block after the
// integer work: the sums are reduced in integers and the float scales are
// applied once per block afterwards (section 25.2.1).
//
// Mapping (MI355X-first, not the pages' wave32 one-lane-per-block design):
//  * One wave owns R rows. A "unit" is 16 consecutive super-blocks of one
//    row; lane l takes block 16u + l/4 and its whole 32-byte nibble group
//    g = l%4 in two 16-byte loads, so a lane's header decode and float pass
//    cover 64 weights. The two nibble loads of a wave cover 16 x 128 B of the
//    16 x 144 B span and the header load the other 16 x 16 B: every line the
//    wave touches is one it needs (section 25.2: the cache lines a wave
//    touches are what costs, not its load count).
//  * Each lane also loads its block's 16-byte header; the four lanes of a
//    block load the same 16 bytes, which the cache serves once per line.
//  * All of a lane's loads for a batch of PF units are issued before any is
//    used, and the first batch before the activation's LDS stores (whose
//    loads come first), so each wave keeps R*PF*32 bytes per lane in flight.
//  * The row's q8_K activation is staged once per workgroup in LDS (the only
//    LDS use); every wave of the workgroup reads its codes, sums and scales
//    from there.
//  * The per-block float work is one pass: xs * (d*S - dmin*M).
//  * Lane partials are f32; the wave reduces them with DPP row sums and four
//    v_readlane, and lane 0 stores y.
#include <algorithm>
#include <atomic>

#include "q4k_row.h"
#include "q8k_block.h"
#include "xq_launch.h"

namespace xq {
namespace {

constexpr int kWaitVm0 = 0x0F70;             // s_waitcnt vmcnt(0), other counters not waited on
constexpr int64_t kQuantTailBlocks = 16384;  // arrival counters: N <= 2^22 rows
constexpr int kCounterStride = 32;           // ints: one 128-byte line per counter

// Loads of the activation row into registers, issued before the weight
// loads; the LDS stores follow them.
template <int NA, int THREADS>
__device__ __forceinline__ void act_load(uint4 (&a)[NA], const uint8_t* xq, int n16) {
#pragma unroll
  for (int k = 0; k < NA; ++k) {
    const int i = threadIdx.x + k * THREADS;
    a[k] = (i < n16) ? reinterpret_cast<const uint4*>(xq)[i] : make_uint4(0, 0, 0, 0);
  }
}

template <int NA, int THREADS>
__device__ __forceinline__ void act_store(const uint4 (&a)[NA], uint8_t* lds, const uint8_t* xq,
                                          int n16) {
#pragma unroll
  for (int k = 0; k < NA; ++k) {
    const int i = threadIdx.x + k * THREADS;
    if (i < n16) reinterpret_cast<uint4*>(lds)[i] = a[k];
  }
  // Rows longer than NA*THREADS chunks stage the rest directly.
  for (int i = threadIdx.x + NA * THREADS; i < n16; i += THREADS)
    reinterpret_cast<uint4*>(lds)[i] = reinterpret_cast<const uint4*>(xq)[i];
}

// R rows per wave, PF units per load batch, W waves per workgroup, NA
// activation chunks per thread held in registers. CLAMP: every load is
// issued (block index clamped into the row, the contribution of a clamped
// block masked), which keeps the loads unconditional so the wait counts
// stay static; without CLAMP, loads and compute of blocks past the row end
// are skipped (cheaper when PF does not divide the row's units).
// ID: the expert-grouped form. blockIdx.y is the selection slot kk; the
// workgroup reads sel[kk] once and works on expert sel[kk]'s N rows of the
// slab `w`, the activation kk * x_stride bytes into `xq`, and the output rows
// kk * N .. kk * N + N - 1. A selection outside 0..n_experts-1 writes NaN to
// the slot's rows and reads nothing. Every row then runs the dense code
// below unchanged, so the result is bit-identical to a dense launch on the
// expert's rows.
// QOUT: the output is also quantized to q8_K ("25 — Writing XPU Kernels",
// section 25.5: the FFN pair's fused tail, the up product handing the down
// product its q8_K activation). N is a multiple of 256 and the R*W rows of a
// workgroup divide 256, so 256/(R*W) workgroups make each q8_K block of y.
// Each stores its rows with agent-scope atomic stores (coherent across XCDs),
// waits for them, and counts its arrival on the block's counter; the last to
// arrive resets the counter, reads the block's 256 values back with
// agent-scope atomic loads and quantizes it with one wave, the quantize
// kernel's own arithmetic (q8k_block_wave), so yq holds the bytes
// xq_quantize_q8k gives for y.
// GACT: rows longer than the LDS can stage (K > kMaxStagedK): no staging,
// every lane reads its slices of the q8_K row from global memory (the row is
// shared by every workgroup, so it is served from L2), with the same
// arithmetic, so the bits are those of the staged form.
template <int R, int PF, int W, int NA, bool CLAMP, bool ID, bool QOUT, bool GACT = false>
__global__ __launch_bounds__(W * kWave) void gemv_q4k_kernel(float* __restrict__ y,
                                                             const uint8_t* __restrict__ w,
                                                             const uint8_t* __restrict__ xq,
                                                             int N, int nb,
                                                             const int32_t* __restrict__ sel,
                                                             int n_experts, int64_t x_stride,
                                                             uint8_t* __restrict__ yq,
                                                             int* __restrict__ qcnt) {
  extern __shared__ __align__(16) uint8_t act_lds[];
  constexpr int kThreads = W * kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int row0 = (blockIdx.x * W + wave) * R;
  const int units = (nb + kUnitBlocks - 1) / kUnitBlocks;
  const LaneGeom L = lane_geom(lane);
  const int64_t row_bytes = static_cast<int64_t>(nb) * kQ4KBytes;
  const int n16 = nb * (kQ8KBytes / 16);

  if constexpr (ID) {
    const int kk = blockIdx.y;
    const int e = sel[kk];
    y += static_cast<int64_t>(kk) * N;
    if (e < 0 || e >= n_experts) {  // workgroup-uniform: no barrier is skipped
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (lane == 0 && row0 + r < N) y[row0 + r] = __builtin_nanf("");
      return;
    }
    w += static_cast<int64_t>(e) * N * row_bytes;
    xq += static_cast<int64_t>(kk) * x_stride;
  }

  Nib nib[R][PF];
  uint4 hdr[R][PF];
  auto load_batch = [&](int u0) {
#pragma unroll
    for (int p = 0; p < PF; ++p)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = min(row0 + r, N - 1);
        const int bb = (u0 + p) * kUnitBlocks + L.bsub;
        const uint8_t* wr = w + static_cast<int64_t>(row) * row_bytes;
        if (CLAMP || bb < nb) {
          const uint8_t* blk = wr + static_cast<int64_t>(min(bb, nb - 1)) * kQ4KBytes;
          nib[r][p] = load_group(blk, L);
          hdr[r][p] = *reinterpret_cast<const uint4*>(blk);
        } else {
          nib[r][p] = zero_group();
          hdr[r][p] = make_uint4(0, 0, 0, 0);
        }
      }
  };

  const uint8_t* act = GACT ? xq : act_lds;
  if constexpr (GACT) {
    load_batch(0);
  } else {
    uint4 areg[NA];
    act_load<NA, kThreads>(areg, xq, n16);
    load_batch(0);
    act_store<NA, kThreads>(areg, act_lds, xq, n16);
    __syncthreads();
  }

  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;

  for (int u0 = 0; u0 < units; u0 += PF) {
    if (u0 > 0) load_batch(u0);
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int bb = (u0 + p) * kUnitBlocks + L.bsub;
      if (CLAMP) {
        const int b = min(bb, nb - 1);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float v = unit_partial(nib[r][p], hdr[r][p], act, b, L);
          acc[r] += (bb < nb) ? v : 0.0f;
        }
      } else if (bb < nb) {
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] += unit_partial(nib[r][p], hdr[r][p], act, bb, L);
      }
    }
  }

  if constexpr (QOUT) {
    __shared__ int q_last;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float tot = wave_sum(acc[r]);
      if (lane == 0)
        __hip_atomic_store(y + row0 + r, tot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // As the split-K handoff of the product: agent-scope (device-coherent)
    // atomic stores, loads and counter; each wave waits for its stores to be
    // acknowledged before the barrier, whose workgroup fences keep the
    // compiler from moving them. (A release/acquire pair at agent scope
    // writes back and invalidates the whole L2 per workgroup on gfx950:
    // 9.2 -> 58.8 us for this launch.)
    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wave's row stores have completed
    __syncthreads();
    const int blk = (blockIdx.x * W * R) >> 8;
    if (threadIdx.x == 0)
      q_last = __hip_atomic_fetch_add(qcnt + blk * kCounterStride, 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) == 256 / (R * W) - 1;
    __syncthreads();
    if (!q_last) return;  // workgroup-uniform
    if (threadIdx.x == 0)
      __hip_atomic_store(qcnt + blk * kCounterStride, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (wave == 0) {
      const float* hb = y + 256 * blk + 4 * lane;
      float4 v;
      v.x = __hip_atomic_load(hb + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      v.y = __hip_atomic_load(hb + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      v.z = __hip_atomic_load(hb + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      v.w = __hip_atomic_load(hb + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      q8k_block_wave(v, yq + static_cast<int64_t>(blk) * kQ8KBytes, lane);
    }
    return;
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float tot = wave_sum(acc[r]);
    if (lane == 0 && row0 + r < N) y[row0 + r] = tot;
  }
}

// A short batch against one pass over the weights: up to TM tokens
// (`tokens` of them live, a workgroup-uniform count), their q8_K rows staged
// back to back in LDS. The weight chunk's header is decoded once per chunk
// and every token then runs the mat-vec's integer dots and float pass in the
// mat-vec's order, so token t's outputs are the bits xq_gemv_q4k gives for
// its row alone (same launch table, same clamping).
template <int TM, int R, int PF, int W, int NA, bool CLAMP>
__global__ __launch_bounds__(W * kWave) void gemv_q4k_multi_kernel(float* __restrict__ y,
                                                                   const uint8_t* __restrict__ w,
                                                                   const uint8_t* __restrict__ xq,
                                                                   int N, int nb, int tokens) {
  extern __shared__ __align__(16) uint8_t act[];
  constexpr int kThreads = W * kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int row0 = (blockIdx.x * W + wave) * R;
  const int units = (nb + kUnitBlocks - 1) / kUnitBlocks;
  const LaneGeom L = lane_geom(lane);
  const int64_t row_bytes = static_cast<int64_t>(nb) * kQ4KBytes;
  const int xrow = nb * kQ8KBytes;
  const int n16 = tokens * nb * (kQ8KBytes / 16);

  Nib nib[R][PF];
  uint4 hdr[R][PF];
  auto load_batch = [&](int u0) {
#pragma unroll
    for (int p = 0; p < PF; ++p)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = min(row0 + r, N - 1);
        const int bb = (u0 + p) * kUnitBlocks + L.bsub;
        const uint8_t* wr = w + static_cast<int64_t>(row) * row_bytes;
        if (CLAMP || bb < nb) {
          const uint8_t* blk = wr + static_cast<int64_t>(min(bb, nb - 1)) * kQ4KBytes;
          nib[r][p] = load_group(blk, L);
          hdr[r][p] = *reinterpret_cast<const uint4*>(blk);
        } else {
          nib[r][p] = zero_group();
          hdr[r][p] = make_uint4(0, 0, 0, 0);
        }
      }
  };

  uint4 areg[NA];
  act_load<NA, kThreads>(areg, xq, n16);
  load_batch(0);
  act_store<NA, kThreads>(areg, act, xq, n16);
  __syncthreads();

  float acc[R][TM];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < TM; ++t) acc[r][t] = 0.0f;

  for (int u0 = 0; u0 < units; u0 += PF) {
    if (u0 > 0) load_batch(u0);
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int bb = (u0 + p) * kUnitBlocks + L.bsub;
      if (CLAMP) {
        const int b = min(bb, nb - 1);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const ChunkDecode c = chunk_decode(nib[r][p], hdr[r][p], L);
#pragma unroll
          for (int t = 0; t < TM; ++t) {
            if (t < tokens) {
              const float v = chunk_token(c, act + t * xrow, b, L);
              acc[r][t] += (bb < nb) ? v : 0.0f;
            }
          }
        }
      } else if (bb < nb) {
        // Long rows hold at most three tokens in 64 KB, so the header is
        // decoded per token here, through the mat-vec's own unit_partial.
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int t = 0; t < TM; ++t)
            if (t < tokens) acc[r][t] += unit_partial(nib[r][p], hdr[r][p], act + t * xrow, bb, L);
      }
    }
  }

#pragma unroll
  for (int t = 0; t < TM; ++t) {
    if (t >= tokens) break;  // workgroup-uniform
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float tot = wave_sum(acc[r][t]);
      if (lane == 0 && row0 + r < N) y[static_cast<int64_t>(t) * N + row0 + r] = tot;
    }
  }
}

// A short batch of up to eight tokens on rows of one unit, as a
// persistent grid: each lane copies its slice of every token's q8_K row
// (codes, sub-block sums and scale of its block in each unit) from the
// workgroup's LDS copy into registers once, then the wave walks rows with a
// stride of the grid's waves, each row's weight loads issued one row ahead
// (two register sets). Every token's row is computed with the multi-token
// kernel's arithmetic (chunk_decode, then chunk_token_slice per token, the
// same clamped accumulation and wave_sum), so it carries the mat-vec's bits;
// only the activation's reads move from LDS per row to registers per wave.
constexpr int kMresWaves = 8;
constexpr int kMresThreads = kMresWaves * kWave;

template <int TM, int U>
__global__ __launch_bounds__(kMresThreads) void gemv_q4k_multi_res_kernel(
    float* __restrict__ y, const uint8_t* __restrict__ w, const uint8_t* __restrict__ xq, int N,
    int nb, int tokens) {
  extern __shared__ __align__(16) uint8_t act[];
  const int lane = threadIdx.x & (kWave - 1);
  const int xrow = nb * kQ8KBytes;
  {
    const uint4* src = reinterpret_cast<const uint4*>(xq);
    uint4* dst = reinterpret_cast<uint4*>(act);
    const int n16 = tokens * xrow / 16;
    for (int i = threadIdx.x; i < n16; i += kMresThreads) dst[i] = src[i];
  }
  __syncthreads();
  const int row_first = blockIdx.x * kMresWaves + (threadIdx.x >> 6);
  const int row_step = gridDim.x * kMresWaves;
  if (row_first >= N) return;  // no barrier follows

  const LaneGeom L = lane_geom(lane);
  const int64_t row_bytes = static_cast<int64_t>(nb) * kQ4KBytes;
  int bb[U], bc[U];
  TokenSlice ts[U][TM];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    bb[u] = u * kUnitBlocks + L.bsub;
    bc[u] = min(bb[u], nb - 1);
#pragma unroll
    for (int t = 0; t < TM; ++t)
      ts[u][t] = token_slice(act + min(t, tokens - 1) * xrow, bc[u], L);
  }

  Nib na[U], nq[U];
  uint4 ha[U], hq[U];
  auto load_row = [&](Nib (&n)[U], uint4 (&h)[U], int row) {
    const uint8_t* wr = w + static_cast<int64_t>(row) * row_bytes;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint8_t* blk = wr + static_cast<int64_t>(bc[u]) * kQ4KBytes;
      n[u] = load_group(blk, L);
      h[u] = *reinterpret_cast<const uint4*>(blk);
    }
  };
  auto reduce_row = [&](const Nib (&n)[U], const uint4 (&h)[U], int row) {
    float acc[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) acc[t] = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const ChunkDecode c = chunk_decode(n[u], h[u], L);
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        if (t < tokens) {
          const float v = chunk_token_slice(c, ts[u][t]);
          acc[t] += (bb[u] < nb) ? v : 0.0f;
        }
      }
    }
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      if (t >= tokens) break;  // wave-uniform
      const float tot = wave_sum(acc[t]);
      if (lane == 0) y[static_cast<int64_t>(t) * N + row] = tot;
    }
  };

  // The row after the last is replaced by a reload of the last (a cache hit)
  // so every load is unconditional.
  int r0 = row_first;
  load_row(na, ha, r0);
  while (true) {
    const int r1 = r0 + row_step;
    const bool more1 = r1 < N;
    load_row(nq, hq, more1 ? r1 : r0);
    reduce_row(na, ha, r0);
    if (!more1) break;
    const int r2 = r1 + row_step;
    const bool more2 = r2 < N;
    load_row(na, ha, more2 ? r2 : r1);
    reduce_row(nq, hq, r1);
    if (!more2) break;
    r0 = r2;
  }
}

// Three tokens on rows of four units (K in 12544..14336), a row's
// units split across the waves of a workgroup: wave u takes unit u of R
// consecutive rows. Each lane reads its slice of every token's q8_K block of
// that unit from global memory into registers once (no LDS staging of the
// activation row), then the R rows' weight chunks of its unit in one batch.
// The per-lane partial of each (row, token, unit) goes to LDS; after one
// barrier each (row, token) is summed over the units in unit order from 0.0f
// and reduced across the wave, so the sequence of float additions, and so the
// bits, are those of the clamped mat-vec (masked blocks add 0.0f there too).
constexpr int kSplitMaxUnits = 4;

template <int TM, int R>
__global__ __launch_bounds__(kSplitMaxUnits * kWave) void gemv_q4k_unit_split_kernel(
    float* __restrict__ y, const uint8_t* __restrict__ w, const uint8_t* __restrict__ xq, int N,
    int nb, int tokens) {
  __shared__ float part[R * TM][kSplitMaxUnits][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int u = threadIdx.x >> 6;          // this wave's unit
  const int units = blockDim.x >> 6;       // the row's units of 16 blocks
  const int row0 = blockIdx.x * R;
  const LaneGeom L = lane_geom(lane);
  const int64_t row_bytes = static_cast<int64_t>(nb) * kQ4KBytes;
  const int64_t xrow = static_cast<int64_t>(nb) * kQ8KBytes;
  const int bb = u * kUnitBlocks + L.bsub;
  const int bc = min(bb, nb - 1);

  TokenSlice ts[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) ts[t] = token_slice(xq + min(t, tokens - 1) * xrow, bc, L);
  Nib nib[R];
  uint4 hdr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = min(row0 + r, N - 1);  // rows past N reload the last (not stored)
    const uint8_t* blk =
        w + static_cast<int64_t>(row) * row_bytes + static_cast<int64_t>(bc) * kQ4KBytes;
    nib[r] = load_group(blk, L);
    hdr[r] = *reinterpret_cast<const uint4*>(blk);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const ChunkDecode c = chunk_decode(nib[r], hdr[r], L);
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      if (t < tokens) {
        const float v = chunk_token_slice(c, ts[t]);
        part[r * TM + t][u][lane] = (bb < nb) ? v : 0.0f;
      }
    }
  }
  __syncthreads();
  for (int k = u; k < R * TM; k += units) {
    const int r = k / TM, t = k - r * TM;
    if (t >= tokens || row0 + r >= N) continue;  // wave-uniform
    float acc = 0.0f;
    for (int v = 0; v < units; ++v) acc += part[k][v][lane];
    const float tot = wave_sum(acc);
    if (lane == 0) y[static_cast<int64_t>(t) * N + row0 + r] = tot;
  }
}

struct IdArgs {
  const int32_t* sel;  // device selection buffer (null: dense launch)
  int used;            // selection slots (grid.y)
  int n_experts;       // experts in the slab
  int64_t x_stride;    // bytes between the slots' activations (0: shared)
  uint8_t* yq;         // fused q8_K output (null: none); excludes sel
  int* qcnt;           // its per-block arrival counters
};

template <int R, int PF, int W, int NA, bool CLAMP, bool GACT = false>
hipError_t launch_cfg(float* y, const uint8_t* w, const uint8_t* xq, int N, int nb,
                      const IdArgs& id, hipStream_t stream) {
  const int waves = (N + R - 1) / R;
  const int grid = (waves + W - 1) / W;
  const size_t lds = GACT ? 0 : static_cast<size_t>(nb) * kQ8KBytes;
  if (id.sel)
    hipLaunchKernelGGL((gemv_q4k_kernel<R, PF, W, NA, CLAMP, true, false, GACT>),
                       dim3(grid, id.used), dim3(W * kWave), lds, stream, y, w, xq, N, nb, id.sel,
                       id.n_experts, id.x_stride, nullptr, nullptr);
  else if (id.yq)
    hipLaunchKernelGGL((gemv_q4k_kernel<R, PF, W, NA, CLAMP, false, true, GACT>), dim3(grid),
                       dim3(W * kWave), lds, stream, y, w, xq, N, nb, nullptr, 0, int64_t{0}, id.yq,
                       id.qcnt);
  else
    hipLaunchKernelGGL((gemv_q4k_kernel<R, PF, W, NA, CLAMP, false, false, GACT>), dim3(grid),
                       dim3(W * kWave), lds, stream, y, w, xq, N, nb, nullptr, 0, int64_t{0},
                       nullptr, nullptr);
  return hipGetLastError();
}

// Dense (id.sel null) or expert-grouped launch of N rows per slot.
hipError_t launch_rows(float* y, const void* w, const void* xq, int64_t N, int64_t K,
                       const IdArgs& id, hipStream_t stream) {
  const int nb = static_cast<int>(K / 256);
  const int units = (nb + kUnitBlocks - 1) / kUnitBlocks;
  const uint8_t* wb = static_cast<const uint8_t*>(w);
  const uint8_t* xb = static_cast<const uint8_t*>(xq);
  const int n = static_cast<int>(N);
  // Launch shapes chosen by measurement on MI355X (cold weights):
  //  * rows of one unit: one row per wave, four waves per workgroup, the
  //    whole row in flight (14336x4096: 6.75-6.96 us against 7.03 with two
  //    rows per wave and 7.40-7.77 with two waves per workgroup; 4096x4096:
  //    3.41 us against 3.52 with eight waves per workgroup). The fused
  //    q8_K tail keeps two rows per wave: half as many workgroups count
  //    their arrival on each 256-row block (14336x4096 with its tail 8.87
  //    us against 9.38 with one row per wave);
  //  * rows of two to four units: the whole row in flight at once (clamped
  //    loads, static wait counts), eight waves per workgroup (the activation
  //    row is staged half as often) (4096x14336: 7.66-7.70 us against
  //    8.00 in two batches and 8.6-9.9 with four, twelve or sixteen waves or
  //    two rows per wave);
  //  * longer rows: batches of two units, eight waves per workgroup, loads
  //    past the row skipped.
  // A grouped launch takes the dense shape for its rows; a row's arithmetic
  // is the same for every shape.
  if (units == 1) {
    if (id.yq) return launch_cfg<2, 1, 4, 2, true>(y, wb, xb, n, nb, id, stream);
    return launch_cfg<1, 1, 4, 2, true>(y, wb, xb, n, nb, id, stream);
  }
  if (units == 2) return launch_cfg<1, 2, 8, 2, true>(y, wb, xb, n, nb, id, stream);
  if (units == 3) return launch_cfg<1, 3, 8, 3, true>(y, wb, xb, n, nb, id, stream);
  if (units == 4) return launch_cfg<1, 4, 8, 3, true>(y, wb, xb, n, nb, id, stream);
  if (K <= kMaxStagedK) return launch_cfg<1, 2, 8, 3, false>(y, wb, xb, n, nb, id, stream);
  // Rows too long to stage: the activation from global memory.
  return launch_cfg<1, 2, 8, 3, false, true>(y, wb, xb, n, nb, id, stream);
}

template <int TM, int R, int PF, int W, int NA, bool CLAMP>
hipError_t launch_multi_cfg(float* y, const uint8_t* w, const uint8_t* xq, int N, int nb,
                            int tokens, hipStream_t stream) {
  const int waves = (N + R - 1) / R;
  const int grid = (waves + W - 1) / W;
  const size_t lds = static_cast<size_t>(tokens) * nb * kQ8KBytes;
  hipLaunchKernelGGL((gemv_q4k_multi_kernel<TM, R, PF, W, NA, CLAMP>), dim3(grid),
                     dim3(W * kWave), lds, stream, y, w, xq, N, nb, tokens);
  return hipGetLastError();
}

// The mat-vec's launch table with a token cap TM.
template <int TM>
hipError_t launch_multi_rows(float* y, const void* w, const void* xq, int64_t N, int64_t K,
                             int tokens, hipStream_t stream) {
  const int nb = static_cast<int>(K / 256);
  const int units = (nb + kUnitBlocks - 1) / kUnitBlocks;
  const uint8_t* wb = static_cast<const uint8_t*>(w);
  const uint8_t* xb = static_cast<const uint8_t*>(xq);
  const int n = static_cast<int>(N);
  if (units == 1) return launch_multi_cfg<TM, 1, 1, 4, 2, true>(y, wb, xb, n, nb, tokens, stream);
  if (units == 2) return launch_multi_cfg<TM, 1, 2, 8, 2, true>(y, wb, xb, n, nb, tokens, stream);
  if (units == 3) return launch_multi_cfg<TM, 1, 3, 8, 3, true>(y, wb, xb, n, nb, tokens, stream);
  if (units == 4) return launch_multi_cfg<TM, 1, 4, 8, 3, true>(y, wb, xb, n, nb, tokens, stream);
  return launch_multi_cfg<TM, 1, 2, 8, 3, false>(y, wb, xb, n, nb, tokens, stream);
}

template <int TM, int R>
hipError_t launch_unit_split(float* y, const uint8_t* w, const uint8_t* xq, int N, int nb,
                             int tokens, hipStream_t stream) {
  const int units = (nb + kUnitBlocks - 1) / kUnitBlocks;
  if (units < 1 || units > kSplitMaxUnits || tokens < 1 || tokens > TM)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemv_q4k_unit_split_kernel<TM, R>), dim3((N + R - 1) / R),
                     dim3(units * kWave), 0, stream, y, w, xq, N, nb, tokens);
  return hipGetLastError();
}

// The persistent grid is the device's resident capacity for the kernel
// (queried once per kernel and device), so each wave visits N / (grid's
// waves) rows and the copy of the activation is paid once per wave.
template <int TM, int U>
hipError_t launch_multi_res(float* y, const uint8_t* w, const uint8_t* xq, int N, int nb,
                            int tokens, hipStream_t stream) {
  constexpr int kMaxDev = 64;
  static std::atomic<int> resident[kMaxDev];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  const size_t lds = static_cast<size_t>(tokens) * nb * kQ8KBytes;
  int cap = resident[dev].load(std::memory_order_relaxed);
  if (cap == 0) {
    int per_cu = 0, cus = 0;
    // The largest staging a call can ask for: TM tokens of 16 blocks.
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per_cu, reinterpret_cast<const void*>(&gemv_q4k_multi_res_kernel<TM, U>), kMresThreads,
        static_cast<size_t>(TM) * 16 * kQ8KBytes);
    if (e != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
      return e;
    cap = std::max(1, per_cu) * std::max(1, cus);
    resident[dev].store(cap, std::memory_order_relaxed);
  }
  const int grid = std::min((N + kMresWaves - 1) / kMresWaves, cap);
  hipLaunchKernelGGL((gemv_q4k_multi_res_kernel<TM, U>), dim3(grid), dim3(kMresThreads), lds,
                     stream, y, w, xq, N, nb, tokens);
  return hipGetLastError();
}

}  // namespace

int64_t gemv_q4k_multi_max_tokens(int64_t K) {
  // The tokens' q8_K rows share 64 KB of LDS (two workgroups per CU).
  return std::min<int64_t>(8, 65536 / ((K / 256) * kQ8KBytes));
}

hipError_t launch_gemv_q4k_multi(float* y, const void* w, const void* xq, int64_t M, int64_t N,
                                 int64_t K, hipStream_t stream) {
  if (M < 1 || M > gemv_q4k_multi_max_tokens(K)) return hipErrorInvalidValue;
  const int t = static_cast<int>(M);
  const int nb = static_cast<int>(K / 256);
  const uint8_t* wb = static_cast<const uint8_t*>(w);
  const uint8_t* xb = static_cast<const uint8_t*>(xq);
  if (nb <= kUnitBlocks) {
    // Rows of one unit: the persistent grid with the activation in
    // registers, one instantiation per token count (registers, and so
    // resident waves, grow with it). Measured on MI355X (cold weights),
    // against the kernel below: 14336x4096 at 2 and 3 tokens 8.7 and 10.2 us
    // against 9.9 and 12.2; 4096x4096 at 2, 3, 4 tokens 4.2, 4.6, 5.3 us
    // against 4.4, 5.5, 6.1 (first layout); 4096x4096 at 6 tokens 6.5 us
    // against 7.6.
    const int n = static_cast<int>(N);
    if (M <= 2) return launch_multi_res<2, 1>(y, wb, xb, n, nb, t, stream);
    if (M == 3) return launch_multi_res<3, 1>(y, wb, xb, n, nb, t, stream);
    if (M == 4) return launch_multi_res<4, 1>(y, wb, xb, n, nb, t, stream);
    if (M <= 6) return launch_multi_res<6, 1>(y, wb, xb, n, nb, t, stream);
    return launch_multi_res<8, 1>(y, wb, xb, n, nb, t, stream);
  }
  if (nb > 48 && nb <= 56 && M == 3) {
    // Three tokens on rows of 49 to 56 blocks (four units): the units split
    // across a workgroup's waves, eight rows per workgroup (4096x14336: 12.3
    // us against 12.6-15.2 with 4, 6, 12 or 16 rows and 14.1 for the kernel
    // below). Two tokens run below (9.8-9.9 us against 10.3 split).
    return launch_unit_split<3, 8>(y, wb, xb, static_cast<int>(N), nb, t, stream);
  }
  if (M <= 2) return launch_multi_rows<2>(y, w, xq, N, K, t, stream);
  if (M <= 4) return launch_multi_rows<4>(y, w, xq, N, K, t, stream);
  return launch_multi_rows<8>(y, w, xq, N, K, t, stream);
}

hipError_t launch_gemv_q4k(float* y, const void* w, const void* xq, int64_t N, int64_t K,
                           hipStream_t stream) {
  return launch_rows(y, w, xq, N, K, IdArgs{nullptr, 1, 0, 0, nullptr, nullptr}, stream);
}

size_t gemv_q4k_q8k_workspace_bytes(int64_t N) {
  if (N < 256 || N % 256 != 0 || N / 256 > kQuantTailBlocks) return 0;
  return static_cast<size_t>(N / 256) * kCounterStride * sizeof(int);
}

hipError_t launch_gemv_q4k_q8k(float* y, void* yq, const void* w, const void* xq, int64_t N,
                               int64_t K, void* ws, size_t ws_bytes, hipStream_t stream) {
  // Every launch shape of the table puts 4 or 8 rows in a workgroup, so the
  // workgroups of a 256-row block never straddle two blocks.
  if (N % 256 != 0 || N / 256 > kQuantTailBlocks) return hipErrorInvalidValue;
  if (!ws || ws_bytes < gemv_q4k_q8k_workspace_bytes(N)) return hipErrorInvalidValue;
  return launch_rows(y, w, xq, N, K,
                     IdArgs{nullptr, 1, 0, 0, static_cast<uint8_t*>(yq), static_cast<int*>(ws)},
                     stream);
}

hipError_t launch_gemv_q4k_id(float* y, const void* slab, const void* xq, const int32_t* sel,
                              int64_t n_experts, int64_t used, int64_t rows, int64_t K,
                              int64_t x_stride_blocks, hipStream_t stream) {
  const IdArgs id{sel, static_cast<int>(used), static_cast<int>(n_experts),
                  x_stride_blocks * kQ8KBytes, nullptr, nullptr};
  return launch_rows(y, slab, xq, rows, K, id, stream);
}

}  // namespace xq
