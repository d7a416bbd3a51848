// gemv_iq4nl.hip — IQ4_NL x q8_K decode mat-vec on gfx950 (wave64).
//
// "25 — Writing XPU Kernels", section 25.2.1: resident rows (the row's f16
// block scales padded to a dword, then 16-byte payloads), each nibble mapped
// through the 16-entry codebook to an int8 (never to f16), a signed int8 dot
// against the q8_K codes, one float multiply per 32-block after the integer
// dot, one wave reduction, one store.
//
// MI355X mapping: a wave's 64 lanes take 64 consecutive 32-blocks of a row (one
// "unit", 1 KiB of payload and the 128 bytes of their scales, both coalesced
// loads). The codebook lookup is done in registers with v_perm_b32: one perm
// over table bytes 0..7 and one over bytes 8..15, both indexed by the low three
// bits of the nibble, and a third perm that takes each byte from the first or
// the second result by the nibble's bit 3. (A single v_perm_b32 addresses
// only eight table bytes, so a 16-entry table needs the pair plus the select.)
//
// Two kernels:
//  * rows of up to kResidentUnits units (K <= 8192): a persistent grid. The
//    workgroup stages the q8_K row in LDS once; every lane then copies the
//    slice it will need for every row (its block of each unit: 32 codes and
//    the block's f32 scale) into registers, and the wave walks rows with a
//    grid stride, the next row's payload (non-temporal: it is read once) and
//    scales loaded before the current row is reduced. No LDS traffic and no
//    barrier per row; the activation leaves L2 once per workgroup.
//  * longer rows: one row per wave, up to eight units of loads in flight,
//    the activation read from the LDS copy per row.
#include <algorithm>
#include <atomic>

#include "xq_device.h"
#include "xq_launch.h"

namespace xq {
namespace {

constexpr int kWavesPerGroup = 4;
constexpr int kThreads = kWavesPerGroup * kWave;

// The IQ4_NL codebook, nibble 0..15, packed four signed bytes per word.
constexpr int8_t kCodebook[16] = {-127, -104, -83, -65, -49, -35, -22, -10,
                                  1,    13,   25,  38,  53,  69,  89,  113};
constexpr uint32_t pack4(int i) {
  return (static_cast<uint32_t>(static_cast<uint8_t>(kCodebook[i]))) |
         (static_cast<uint32_t>(static_cast<uint8_t>(kCodebook[i + 1])) << 8) |
         (static_cast<uint32_t>(static_cast<uint8_t>(kCodebook[i + 2])) << 16) |
         (static_cast<uint32_t>(static_cast<uint8_t>(kCodebook[i + 3])) << 24);
}
constexpr uint32_t kT0 = pack4(0), kT1 = pack4(4), kT2 = pack4(8), kT3 = pack4(12);

// Four nibbles (one per byte, values 0..15 in bits 0-3 of each byte; bits 4-7
// ignored) -> four codebook int8 values.
__device__ __forceinline__ uint32_t lut4(uint32_t nib) {
  const uint32_t idx = nib & 0x07070707u;
  const uint32_t lo = __builtin_amdgcn_perm(kT1, kT0, idx);
  const uint32_t hi = __builtin_amdgcn_perm(kT3, kT2, idx);
  // byte i of the result: byte i of `lo` (selector i) or of `hi` (selector
  // i+4) as bit 3 of nibble i is clear or set.
  const uint32_t sel = ((nib >> 1) & 0x04040404u) | 0x03020100u;
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// The two formats on this row shape. IQ4_NL: weight = d * kv[nibble].
// Q4_0: weight = d * (nibble - 8), the -8 paid once per 32-block from the
// activation's stored sum of those 32 codes ("25 — Writing XPU Kernels",
// section 25.2: the Q4_0 twin, whose offset rides on the activation sum).
constexpr int kFmtIQ4NL = 0;
constexpr int kFmtQ4_0 = 1;

// Integer dot of one 32-block: payload byte t gives weight t (low nibble,
// against a0) and weight t+16 (high nibble, against a1); s is the block's
// activation code sum (read only by Q4_0).
template <int FMT>
__device__ __forceinline__ int block_dot(const uint4 pay, const uint4 a0, const uint4 a1, int s) {
  if constexpr (FMT == kFmtIQ4NL) {
    int dot = sdot4(lut4(pay.x), a0.x, 0);
    dot = sdot4(lut4(pay.y), a0.y, dot);
    dot = sdot4(lut4(pay.z), a0.z, dot);
    dot = sdot4(lut4(pay.w), a0.w, dot);
    dot = sdot4(lut4(pay.x >> 4), a1.x, dot);
    dot = sdot4(lut4(pay.y >> 4), a1.y, dot);
    dot = sdot4(lut4(pay.z >> 4), a1.z, dot);
    return sdot4(lut4(pay.w >> 4), a1.w, dot);
  } else {
    // The 4-bit codes 0..15 are valid signed bytes.
    int dot = sdot4(pay.x & 0x0F0F0F0Fu, a0.x, -8 * s);
    dot = sdot4(pay.y & 0x0F0F0F0Fu, a0.y, dot);
    dot = sdot4(pay.z & 0x0F0F0F0Fu, a0.z, dot);
    dot = sdot4(pay.w & 0x0F0F0F0Fu, a0.w, dot);
    dot = sdot4((pay.x >> 4) & 0x0F0F0F0Fu, a1.x, dot);
    dot = sdot4((pay.y >> 4) & 0x0F0F0F0Fu, a1.y, dot);
    dot = sdot4((pay.z >> 4) & 0x0F0F0F0Fu, a1.z, dot);
    return sdot4((pay.w >> 4) & 0x0F0F0F0Fu, a1.w, dot);
  }
}

template <int FMT>
__device__ __forceinline__ float block_partial(const uint4 pay, uint32_t dbits,
                                               const uint8_t* act, int c) {
  const uint8_t* xb = act + (c >> 3) * kQ8KBytes;
  const uint4 a0 = *reinterpret_cast<const uint4*>(xb + (c & 7) * 32);
  const uint4 a1 = *reinterpret_cast<const uint4*>(xb + (c & 7) * 32 + 16);
  const float xs = *reinterpret_cast<const float*>(xb + 288);
  const int s = (FMT == kFmtQ4_0) ? *reinterpret_cast<const int*>(xb + 256 + 4 * (c & 7)) : 0;
  const int dot = block_dot<FMT>(pay, a0, a1, s);
  const float d = half_bits_to_float(dbits);
  return (d * xs) * static_cast<float>(dot);
}

// Expert-grouped launches (ID): blockIdx.y is the selection slot kk; the
// workgroup reads sel[kk] once and works on expert sel[kk]'s N rows of the
// slab, the activation kk * x_stride bytes into xq, and output rows kk * N ..
// kk * N + N - 1. A selection outside 0..n_experts-1 writes NaN to the slot's
// rows and reads nothing. The rows then run the dense code unchanged, so the
// result is bit-identical to a dense launch on the expert's rows.
struct IdArgs {
  const int32_t* sel;  // device selection buffer (null: dense launch)
  int used;            // selection slots (grid.y)
  int n_experts;       // experts in the slab
  int64_t x_stride;    // bytes between the slots' activations (0: shared)
};

// Applies the slot's offsets; false when the selection is out of range
// (the slot's rows row0 .. row0 + nrows - 1 have been set to NaN).
template <bool ID, typename YPtr, typename BPtr>
__device__ __forceinline__ bool select_slot(YPtr& y, BPtr& w, BPtr& xq, int N, int64_t row_bytes,
                                            const IdArgs& id, int lane, int row0, int nrows,
                                            int row_step) {
  if constexpr (ID) {
    const int kk = blockIdx.y;
    const int e = id.sel[kk];
    y += static_cast<int64_t>(kk) * N;
    if (e < 0 || e >= id.n_experts) {
      for (int r = row0; r < N && nrows > 0; r += row_step, --nrows)
        if (lane == 0) y[r] = __builtin_nanf("");
      return false;
    }
    w += static_cast<int64_t>(e) * N * row_bytes;
    xq += static_cast<int64_t>(kk) * id.x_stride;
  }
  return true;
}

// GACT: rows too long to stage (K > kMaxStagedK) read the q8_K row from
// global memory (served from L2: every workgroup reads the same row), with
// the same arithmetic.
template <int R, int PF, bool ID, int FMT, bool GACT = false>
__global__ __launch_bounds__(kThreads) void gemv_iq4nl_kernel(float* __restrict__ y,
                                                              const uint8_t* __restrict__ w,
                                                              const uint8_t* __restrict__ xq,
                                                              int N, int bpr, int prefix,
                                                              int64_t row_bytes, int nq8,
                                                              IdArgs id) {
  extern __shared__ __align__(16) uint8_t act_lds[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int row0 = (blockIdx.x * kWavesPerGroup + wave) * R;
  const int units = (bpr + kWave - 1) / kWave;
  // Workgroup-uniform: no barrier is skipped.
  if (!select_slot<ID>(y, w, xq, N, row_bytes, id, lane, row0, R, 1)) return;

  uint4 pay[R][PF];
  uint32_t dsc[R][PF];
  auto load_batch = [&](int u0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = min(row0 + r, N - 1);
      const uint8_t* wr = w + static_cast<int64_t>(row) * row_bytes;
#pragma unroll
      for (int p = 0; p < PF; ++p) {
        const int c = (u0 + p) * kWave + lane;
        if (c < bpr) {
          pay[r][p] = *reinterpret_cast<const uint4*>(wr + prefix + 16 * c);
          dsc[r][p] = *reinterpret_cast<const uint16_t*>(wr + 2 * c);
        } else {
          pay[r][p] = make_uint4(0, 0, 0, 0);
          dsc[r][p] = 0;
        }
      }
    }
  };

  load_batch(0);
  const uint8_t* act = GACT ? xq : act_lds;
  if constexpr (!GACT) {
    const uint4* src = reinterpret_cast<const uint4*>(xq);
    uint4* dst = reinterpret_cast<uint4*>(act_lds);
    const int n16 = nq8 * (kQ8KBytes / 16);
    for (int i = threadIdx.x; i < n16; i += kThreads) dst[i] = src[i];
    __syncthreads();
  }

  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;

  for (int u0 = 0; u0 < units; u0 += PF) {
    if (u0 > 0) load_batch(u0);
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int c = (u0 + p) * kWave + lane;
      if (c < bpr) {
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] += block_partial<FMT>(pay[r][p], dsc[r][p], act, c);
      }
    }
  }

#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float tot = wave_sum(acc[r]);
    if (lane == 0 && row0 + r < N) y[row0 + r] = tot;
  }
}

constexpr int kResidentUnits = 4;
constexpr int kResWaves = 8;
constexpr int kResThreads = kResWaves * kWave;
constexpr int kResMaxGroups = 2048;  // grouped launches: workgroups per slot

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_nt16(const uint8_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// U: units per row (1..kResidentUnits). One row per wave per step.
template <int U, bool ID, int FMT>
__global__ __launch_bounds__(kResThreads) void gemv_iq4nl_resident_kernel(
    float* __restrict__ y, const uint8_t* __restrict__ w, const uint8_t* __restrict__ xq, int N,
    int bpr, int prefix, int64_t row_bytes, int nq8, IdArgs id) {
  extern __shared__ __align__(16) uint8_t act[];
  // Workgroup-uniform: no barrier is skipped.
  if (!select_slot<ID>(y, w, xq, N, row_bytes, id, threadIdx.x & (kWave - 1),
                       blockIdx.x * kResWaves + (threadIdx.x >> 6), 1 << 30,
                       gridDim.x * kResWaves))
    return;
  {
    const uint4* src = reinterpret_cast<const uint4*>(xq);
    uint4* dst = reinterpret_cast<uint4*>(act);
    const int n16 = nq8 * (kQ8KBytes / 16);
    for (int i = threadIdx.x; i < n16; i += kResThreads) dst[i] = src[i];
  }
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int row_first = blockIdx.x * kResWaves + (threadIdx.x >> 6);
  const int row_step = gridDim.x * kResWaves;
  if (row_first >= N) return;  // no barrier follows

  // This lane's block of every unit: its codes and q8_K scale stay in
  // registers for all rows. Lanes past the row's last block repeat the last
  // block's loads and drop their contribution.
  uint4 a0[U], a1[U];
  float xs[U];
  int sums[U];
  int cc[U];
  bool live[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = u * kWave + lane;
    live[u] = c < bpr;
    cc[u] = min(c, bpr - 1);
    const uint8_t* xb = act + (cc[u] >> 3) * kQ8KBytes;
    a0[u] = *reinterpret_cast<const uint4*>(xb + (cc[u] & 7) * 32);
    a1[u] = *reinterpret_cast<const uint4*>(xb + (cc[u] & 7) * 32 + 16);
    xs[u] = *reinterpret_cast<const float*>(xb + 288);
    sums[u] = (FMT == kFmtQ4_0) ? *reinterpret_cast<const int*>(xb + 256 + 4 * (cc[u] & 7)) : 0;
  }

  uint4 pa[U], pb[U];
  uint32_t da[U], db[U];
  auto load_row = [&](uint4 (&p)[U], uint32_t (&d)[U], int row) {
    const uint8_t* wr = w + static_cast<int64_t>(row) * row_bytes;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      p[u] = load_nt16(wr + prefix + 16 * cc[u]);
      d[u] = *reinterpret_cast<const uint16_t*>(wr + 2 * cc[u]);
    }
  };
  auto reduce_row = [&](const uint4 (&p)[U], const uint32_t (&d)[U], int row) {
    float acc = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int dot = block_dot<FMT>(p[u], a0[u], a1[u], sums[u]);
      const float v = (half_bits_to_float(d[u]) * xs[u]) * static_cast<float>(dot);
      acc += live[u] ? v : 0.0f;
    }
    const float tot = wave_sum(acc);
    if (lane == 0) y[row] = tot;
  };

  // Two register sets, the loop unrolled by two so that no copy stands
  // between a row's loads and its use. The row after the last is replaced
  // by a reload of the last (an L2 hit) so every load is unconditional.
  int r0 = row_first;
  load_row(pa, da, r0);
  while (true) {
    const int r1 = r0 + row_step;
    const bool more1 = r1 < N;
    load_row(pb, db, more1 ? r1 : r0);
    reduce_row(pa, da, r0);
    if (!more1) break;
    const int r2 = r1 + row_step;
    const bool more2 = r2 < N;
    load_row(pa, da, more2 ? r2 : r1);
    reduce_row(pb, db, r1);
    if (!more2) break;
    r0 = r2;
  }
}

// The device's CU count and the workgroups of gemv_iq4nl_resident_kernel<U,
// false, FMT> resident at once on it (queried once per instance and device).
template <int U, int FMT>
hipError_t resident_shape(int* cus_out, int* cap_out) {
  constexpr int kMaxDev = 64;
  static std::atomic<int> resident[kMaxDev];
  static std::atomic<int> cu_count[kMaxDev];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  int cap = resident[dev].load(std::memory_order_relaxed);
  int cus = cu_count[dev].load(std::memory_order_relaxed);
  if (cap == 0 || cus == 0) {
    int per_cu = 0;
    // The largest staging a row of U units asks for: 8*U q8_K blocks.
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per_cu, reinterpret_cast<const void*>(&gemv_iq4nl_resident_kernel<U, false, FMT>),
        kResThreads, static_cast<size_t>(8 * U) * kQ8KBytes);
    if (e != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
      return e;
    cus = std::max(1, cus);
    cap = std::max(1, per_cu) * cus;
    cu_count[dev].store(cus, std::memory_order_relaxed);
    resident[dev].store(cap, std::memory_order_relaxed);
  }
  *cus_out = cus;
  *cap_out = cap;
  return hipSuccess;
}

template <int U, int FMT>
hipError_t launch_resident(float* y, const uint8_t* w, const uint8_t* xq, int N, int bpr,
                           int prefix, int64_t row_bytes, int nq8, const IdArgs& id,
                           hipStream_t stream) {
  int grid = (N + kResWaves - 1) / kResWaves;
  if (!id.sel) {
    // Dense launches, by rows (measured on MI355X, cold weights, K = 4096 and
    // 8192): up to 16384 rows one workgroup per CU, each wave walking two to
    // eight rows (4096x4096 4.09 -> 3.99 us, 8192x4096 6.53 -> 5.51,
    // 14336x4096 8.15 -> 7.72, 16384x8192 16.5 -> 14.0); up to 65536 rows two
    // per CU (24576x4096 13.2 -> 11.2, 49152x4096 21.3 -> 19.7); longer, two
    // rounds of resident workgroups (the 128256x4096 head: 47.1 us against
    // 47.4 at two per CU and 49.1 at one). Grids that are not whole multiples
    // of the CUs measured slower (384 workgroups: 4.5 us on 4096x4096).
    int cus = 0, cap = 0;
    const hipError_t e = resident_shape<U, FMT>(&cus, &cap);
    if (e != hipSuccess) return e;
    const int target = (N <= 16384) ? cus : (N <= 65536) ? 2 * cus : 2 * cap;
    grid = std::min(grid, target);
  } else if (grid > kResMaxGroups) {
    grid = kResMaxGroups;
  }
  const size_t lds = static_cast<size_t>(nq8) * kQ8KBytes;
  if (id.sel)
    hipLaunchKernelGGL((gemv_iq4nl_resident_kernel<U, true, FMT>), dim3(grid, id.used),
                       dim3(kResThreads), lds, stream, y, w, xq, N, bpr, prefix, row_bytes, nq8,
                       id);
  else
    hipLaunchKernelGGL((gemv_iq4nl_resident_kernel<U, false, FMT>), dim3(grid), dim3(kResThreads),
                       lds, stream, y, w, xq, N, bpr, prefix, row_bytes, nq8, id);
  return hipGetLastError();
}

template <int PF, int FMT, bool GACT = false>
hipError_t launch_staged(float* y, const uint8_t* w, const uint8_t* xq, int N, int bpr, int prefix,
                         int64_t row_bytes, int nq8, const IdArgs& id, hipStream_t stream) {
  const int grid = (N + kWavesPerGroup - 1) / kWavesPerGroup;
  const size_t lds = GACT ? 0 : static_cast<size_t>(nq8) * kQ8KBytes;
  if (id.sel)
    hipLaunchKernelGGL((gemv_iq4nl_kernel<1, PF, true, FMT, GACT>), dim3(grid, id.used),
                       dim3(kThreads), lds, stream, y, w, xq, N, bpr, prefix, row_bytes, nq8, id);
  else
    hipLaunchKernelGGL((gemv_iq4nl_kernel<1, PF, false, FMT, GACT>), dim3(grid), dim3(kThreads),
                       lds, stream, y, w, xq, N, bpr, prefix, row_bytes, nq8, id);
  return hipGetLastError();
}

// Dense (id.sel null) or expert-grouped launch of N rows per slot.
template <int FMT>
hipError_t launch_rows(float* y, const void* w, const void* xq, int64_t N, int64_t K,
                       const IdArgs& id, hipStream_t stream) {
  const int bpr = static_cast<int>(K / 32);
  const int prefix = ((bpr * 2 + 3) / 4) * 4;
  const int64_t row_bytes = prefix + 16 * static_cast<int64_t>(bpr);
  const int nq8 = static_cast<int>(K / 256);
  const int units = (bpr + kWave - 1) / kWave;
  const uint8_t* wb = static_cast<const uint8_t*>(w);
  const uint8_t* xb = static_cast<const uint8_t*>(xq);
  const int n = static_cast<int>(N);
  // Launch shapes chosen by measurement on MI355X (cold weights; 128256 x
  // 4096: 76.4 us with one row-pair per wave and the activation read from LDS
  // per row, 47.5 us resident). Grouped launches of single-unit rows over a
  // few thousand rows per expert leave the resident kernel one row per wave
  // and nothing to reuse its register copy of the activation for: 8 of 64
  // experts of 1408 x 2048, 5.6 us staged against 6.2 resident (dense
  // single-unit shapes: equal up to 8192 rows, resident ahead beyond). Both
  // kernels give the same bits on single-unit rows.
  if (units == 1 && id.sel && N <= 4096)
    return launch_staged<1, FMT>(y, wb, xb, n, bpr, prefix, row_bytes, nq8, id, stream);
  switch (units) {
    case 1: return launch_resident<1, FMT>(y, wb, xb, n, bpr, prefix, row_bytes, nq8, id, stream);
    case 2: return launch_resident<2, FMT>(y, wb, xb, n, bpr, prefix, row_bytes, nq8, id, stream);
    case 3: return launch_resident<3, FMT>(y, wb, xb, n, bpr, prefix, row_bytes, nq8, id, stream);
    case 4: return launch_resident<4, FMT>(y, wb, xb, n, bpr, prefix, row_bytes, nq8, id, stream);
    case 5: return launch_staged<5, FMT>(y, wb, xb, n, bpr, prefix, row_bytes, nq8, id, stream);
    case 6: return launch_staged<6, FMT>(y, wb, xb, n, bpr, prefix, row_bytes, nq8, id, stream);
    case 7: return launch_staged<7, FMT>(y, wb, xb, n, bpr, prefix, row_bytes, nq8, id, stream);
    default:
      if (K <= kMaxStagedK)
        return launch_staged<8, FMT>(y, wb, xb, n, bpr, prefix, row_bytes, nq8, id, stream);
      // Rows too long to stage: the activation from global memory.
      return launch_staged<8, FMT, true>(y, wb, xb, n, bpr, prefix, row_bytes, nq8, id, stream);
  }
}

}  // namespace

hipError_t launch_gemv_iq4nl(float* y, const void* w, const void* xq, int64_t N, int64_t K,
                             hipStream_t stream) {
  return launch_rows<kFmtIQ4NL>(y, w, xq, N, K, IdArgs{nullptr, 1, 0, 0}, stream);
}

hipError_t launch_gemv_q4_0(float* y, const void* w, const void* xq, int64_t N, int64_t K,
                            hipStream_t stream) {
  return launch_rows<kFmtQ4_0>(y, w, xq, N, K, IdArgs{nullptr, 1, 0, 0}, stream);
}

hipError_t launch_gemv_iq4nl_id(float* y, const void* slab, const void* xq, const int32_t* sel,
                                int64_t n_experts, int64_t used, int64_t rows, int64_t K,
                                int64_t x_stride_blocks, hipStream_t stream) {
  const IdArgs id{sel, static_cast<int>(used), static_cast<int>(n_experts),
                  x_stride_blocks * kQ8KBytes};
  return launch_rows<kFmtIQ4NL>(y, slab, xq, rows, K, id, stream);
}

}  // namespace xq
