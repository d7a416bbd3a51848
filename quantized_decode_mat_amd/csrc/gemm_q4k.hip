// gemm_q4k.hip — Q4_K x q8_K small-M product (multi-token prefill) on gfx950.
//
// Y[m][n] = sum_b xs_mb * (d_nb * S_mnb - dmin_nb * M_mnb), with the exact
// int32 block partials S_mnb = sum_k sc_j(k) * q_nk * code_mk and
// M_mnb = sum_k m_j(k) * code_mk over the 256 k of super-block b.
//
// "25 — Writing XPU Kernels", section 25.3: fill the device first, then feed
// the tile; a GEMM that reuses the weight tile across the token block is the
// point of the prefill path. Here the integer products are a dense
// contraction, so they run on int8 MFMA (v_mfma_i32_16x16x64_i8, K = 64: two
// sub-blocks' worth of weights per MFMA).
//
// One MFMA's K spans two sub-blocks with different 6-bit scales, so the
// scale cannot be applied after the MFMA without splitting K. Instead the
// scale goes into the weight operand, exactly: sc = 8a + b with a, b in 0..7,
// and the two int8 planes a*q and b*q (each <= 105) give S = 8*S_a + S_b.
// S is exact int32 (|S| <= 30.7M per block); f32 appears only in the
// per-block epilogue xs * d * S.
//
// The min term's integer M_mnb = sum_j m_nbj * s_mbj, with s_mbj the q8_K's
// stored sub-block sums, is a contraction over the block's 8 sub-blocks. It
// runs on one f16 MFMA per tile and block (v_mfma_f32_16x16x16_f16, K = 16)
// with the integers split so every operand is exact in f16: s = 128*sh + sl
// with sl in 0..127 and sh in -32..31, A = [sl_0..7, sh_0..7] for the token,
// B = [m_0..7, 128*m_0..7] for the row. Every product (at most 127*63 or
// 32*8064) and partial sum (|M| <= 2.05M < 2^24) is an exact f32 integer, so
// M comes out exact whatever the order. The block's float pass then applies
// both scales at once, xs * (d * S - dmin * M), like the mat-vec: the
// per-block terms are exact integers scaled once, so the f32 error stays a
// few units of 2^-24 of |d*xs*S| + |dmin*xs*M| per block.
//
// Tile: 64 tokens x 128 weight rows per 256-thread workgroup, four waves side
// by side along the rows, each wave 64 x 32 = 4 x 2 MFMA tiles of 16 x 16, so
// every weight fragment is decoded by exactly one wave. Super-blocks stream
// through a two-stage LDS ring filled by direct global-to-LDS loads (no
// registers): super-block b+1 is in flight while b is computed. Two
// workgroups share a CU and run out of phase, so one's VALU work (decode,
// epilogue) overlaps the other's MFMAs. Workgroups are laid out so that the
// token tiles sharing one weight tile land on one XCD (one L2).
//
// Split-K (section 25.3: a launch that cannot fill the device cannot be
// fast). With few tiles (a short token batch, or few weight rows) every tile
// splits: the grid is tiles x ks, split s of a tile takes super-blocks
// [s*nb/ks, (s+1)*nb/ks), writes its f32 partial to a workspace slot and
// counts its arrival; the split that arrives last sums the ks partials in
// the fixed order 0..ks-1 and writes Y, so the result does not depend on
// arrival order. With more tiles than whole rounds of resident workgroups,
// the same launch runs the whole rounds of whole tiles and may split the
// short remainder the same way (gemm_q4k_plan). Partials
// and counters live in the caller's workspace and cross XCDs through
// agent-scope atomic loads and stores (coherent without an L2 write-back);
// the last arrival resets the counter, so counters are zero again between
// launches (the caller zeroes a workspace once, before its first use).
//
// Short batches (M = 1, or up to the LDS token cap while M <= 3, M = 4 on
// rows of at most 16 super-blocks or matrices of at most 2^25 weights, M <= 6
// on at most 2^24, M <= 8 on at most 2^23 or on rows of at most 16
// super-blocks of at most 2^24 weights; see gemm_q4k_uses_matvec) skip
// the MFMA tile: they are a weight stream, and the dot4 mat-vec reads the
// weights once for all M tokens (launch_gemv_q4k_multi; each token's row is
// the mat-vec's bits). 5 to 16 tokens on tall matrices of 8 to 16
// super-blocks per row use the
// wave-split tile (gemm_q4k_wave_split_kernel); other batches of up to 32
// tokens (up to 128 on matrices with few weight tiles; see
// gemm_q4k_token_tile) use the 16-token tile.
//
// Grouped form (mul_mat_id, section 25.3: one launch over an expert map,
// never one per expert, padded only to the finest tile): the same tile code
// over device tile lists built by route_experts. A tile holds up to 64
// (token, slot) pairs routed to one expert, or up to 16 of an expert's
// remainder (gemm_q4k_id_mixed_kernel runs both lists in one grid); the
// workgroup gathers their q8_K rows, multiplies them by that expert's weight
// tile and scatters the outputs to the pairs' rows. Each region of the grid
// is sized by an upper bound on its list's length; workgroups past the end
// return at once. Tiles of out-of-range selections write NaN.
#include <algorithm>
#include <mutex>

#include "lds_dma.h"
#include "xq_device.h"
#include "xq_launch.h"

namespace xq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int BN = 128;          // weight rows per workgroup tile
constexpr int kWaves = BN / 32;  // waves side by side along the weight rows
constexpr int kThreads = 64 * kWaves;
constexpr int kStages = 2;       // LDS ring: compute b while b+1 lands
constexpr int kWInstr = BN * kQ4KBytes / 1024;     // 18 (BN * 9 chunks, 64 per load)
static_assert(BN * 9 % 64 == 0, "weight chunks fill whole 64-lane loads");

// The token tile: 64 tokens (4 MFMA tiles of 16 per wave), or 16 for short
// batches (one MFMA tile per wave: the finest tile the MFMA has, section
// 25.3's padding rule). One LDS stage holds one super-block of the tile:
//  act  BM rows x 256 codes; row m's 16-byte chunk c sits in slot c ^ (m & 15)
//       (the XOR spreads the 16 rows of an MFMA operand read over all banks);
//  xs   BM f32 token scales;
//  sums BM x 8 int32 sub-block sums of the token rows;
//  w    BN raw 144-byte Q4_K blocks, back to back.
template <int BMv>
struct Tile {
  static constexpr int BM = BMv;                   // tokens per workgroup tile
  static constexpr int MT = BMv / 16;              // 16-token MFMA tiles per wave
  static constexpr int kActBytes = BMv * 256;
  static constexpr int kXsOff = kActBytes;
  static constexpr int kSumOff = kXsOff + BMv * 4;
  static constexpr int kWOff = kSumOff + BMv * 32;
  static constexpr int kStageBytes = kWOff + BN * kQ4KBytes;
  static constexpr int kActPerWave = BMv / 16;     // 64-lane act loads per wave
  static constexpr int kPartFloats = kThreads * 8 * MT;  // split-K partial slot
  static_assert(BMv == 16 || BMv == 64, "token tiles of 16 or 64");
  static_assert(2 * kStages * kStageBytes <= 160 * 1024, "two workgroups' rings exceed 160 KiB");
};

__device__ __forceinline__ uint32_t mul_bytes(uint32_t nib, uint32_t f) {
  // Each byte of `nib` is 0..15 and f <= 7, so no product crosses its byte.
  const u16x2 v = __builtin_bit_cast(u16x2, nib);
  const u16x2 r = v * (u16x2){static_cast<unsigned short>(f), static_cast<unsigned short>(f)};
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ v4i mfma(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Stage loads per wave: wave w takes act rows 4j..4j+3 for j = w, w+4, ...
// (BM/16 loads); weight chunks 64j.. for j = w, w+4, w+8, w+12 (and w+16 <
// 18); wave 2 the sums of tokens 0..31 (lanes 0..31 when BM = 16), wave 3
// those of tokens 32..63 (BM = 64) and the BM token scales. A step waits for
// all of its wave's loads (vmcnt(0)) before the barrier that publishes the
// stage.
static_assert(kWaves == 4 && kWInstr == 18, "the load split below is written for this tile");

// Per-lane byte offsets of this wave's stage loads relative to super-block
// 0 (xq or w base); super-block b adds b*320 (codes, scales) or b*144
// (weights). Offsets stay below 2^31 (the entry point refuses larger
// inputs), so the loads use a scalar base plus a 32-bit lane offset.
template <int BMv>
struct StageOffsets {
  uint32_t act[Tile<BMv>::kActPerWave];
  uint32_t wt[4];
  uint32_t extra;   // fifth weight load, sums (tokens 0..31), or token scales
  uint32_t sums;    // wave 3 when BM = 64: sums of tokens 32..63
};

// ID: token rows come from xrow[m] (the gathered pairs' q8_K rows).
template <int BMv, bool ID>
__device__ __forceinline__ StageOffsets<BMv> stage_offsets(int M, int N, int nb, int m0, int n0,
                                                           int wave, int lane, const int* xrow) {
  StageOffsets<BMv> o;
  auto act_off = [&](int j) {
    const int m = 4 * j + (lane >> 4);
    const int c = (lane & 15) ^ (m & 15);      // source chunk of this lane's slot
    const int gm = ID ? xrow[m] : min(m0 + m, M - 1);
    return static_cast<uint32_t>(gm) * static_cast<uint32_t>(nb) * kQ8KBytes + 16u * c;
  };
  auto w_off = [&](int j) {
    const int i = 64 * j + lane;
    const int n = i / 9, c = i - 9 * (i / 9);
    const int gn = min(n0 + n, N - 1);
    return static_cast<uint32_t>(gn) * static_cast<uint32_t>(nb) * kQ4KBytes + 16u * c;
  };
#pragma unroll
  for (int k = 0; k < Tile<BMv>::kActPerWave; ++k) o.act[k] = act_off(wave + 4 * k);
#pragma unroll
  for (int k = 0; k < 4; ++k) o.wt[k] = w_off(wave + 4 * k);
  if (wave < 2) {
    o.extra = w_off(wave + 16);
  }
  auto sum_off = [&](int h) {
    const int m = min(32 * h + (lane >> 1), BMv - 1);  // lanes past the tile: loads masked
    const int gm = ID ? xrow[m] : min(m0 + m, M - 1);
    return static_cast<uint32_t>(gm) * static_cast<uint32_t>(nb) * kQ8KBytes + 256u +
           16u * (lane & 1);
  };
  if (wave == 2) {
    o.extra = sum_off(0);
  } else if (wave == 3) {
    const int m = min(lane, BMv - 1);
    const int gm = ID ? xrow[m] : min(m0 + m, M - 1);
    o.extra = static_cast<uint32_t>(gm) * static_cast<uint32_t>(nb) * kQ8KBytes + 288u;
    o.sums = (BMv == 64) ? sum_off(1) : 0u;
  }
  return o;
}

// The grouped form's tile list (see route_experts.hip).
struct IdGemm {
  const int32_t* sorted;  // pairs p = t * n_used + k, grouped by expert
  const int4* desc;       // tile: (bucket, first index into sorted, pairs)
  const int32_t* n_tiles; // tiles in the list
  int n_experts;          // bucket n_experts: out-of-range selections
  int n_used;
  int per_slot_x;         // 1: pair p reads q8_K row p; 0: row p / n_used
  int64_t expert_bytes;   // one expert's weights in the slab
};

template <int BMv>
__device__ __forceinline__ void issue_stage(uint8_t* base, const uint8_t* xq_in,
                                            const uint8_t* w_in, const StageOffsets<BMv>& o, int b,
                                            int wave, int lane) {
  using T = Tile<BMv>;
  // Super-block b's offset rides on the scalar base, so the per-lane
  // offsets are the same every step (no vector address arithmetic per load).
  const uint8_t* xq = uniform_ptr(xq_in + static_cast<size_t>(b) * kQ8KBytes);
  const uint8_t* w = uniform_ptr(w_in + static_cast<size_t>(b) * kQ4KBytes);
  // The LDS destination of each load is wave-uniform.
  const uint32_t lb = __builtin_amdgcn_readfirstlane(lds_u32(base));
  const int wv = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
  for (int k = 0; k < T::kActPerWave; ++k) lds_dma16(xq, o.act[k], lb + 1024 * (wv + 4 * k));
#pragma unroll
  for (int k = 0; k < 4; ++k) lds_dma16(w, o.wt[k], lb + T::kWOff + 1024 * (wv + 4 * k));
  if (wv < 2) {
    lds_dma16(w, o.extra, lb + T::kWOff + 1024 * (wv + 16));
  } else if (wv == 2) {
    // BM = 16: 32 chunks of sums, lanes 0..31 (an inactive lane writes no LDS)
    if (BMv == 64 || lane < 2 * BMv) lds_dma16(xq, o.extra, lb + T::kSumOff);
  } else {
    if (BMv == 64 || lane < BMv) lds_dma4(xq, o.extra, lb + T::kXsOff);
    if (BMv == 64) lds_dma16(xq, o.sums, lb + T::kSumOff + 1024);
  }
}

// s_waitcnt immediates (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt
// [6:4] and lgkmcnt [11:8] left at their maxima, i.e. not waited on).
constexpr int kWaitVm0 = 0x0F70;

// Waits until at most one stage's loads of this wave are in flight (the
// three-stage ring, whose next stage is issued before this one is needed):
// issue_stage makes 4 + BM/16 loads per wave (codes and weights), plus a
// fifth weight load on waves 0 and 1, the sums on wave 2, and the token
// scales (and, when BM = 64, the second half of the sums) on wave 3.
template <int BMv>
__device__ __forceinline__ void wait_stage_behind_one(int wave) {
  constexpr int base = 4 + BMv / 16;
  static_assert(base + 2 <= 15, "the wait count below is a 4-bit vmcnt");
  if (BMv == 64 && wave == 3)
    __builtin_amdgcn_s_waitcnt(0x0F70 | (base + 2));
  else
    __builtin_amdgcn_s_waitcnt(0x0F70 | (base + 1));
}

// A partial slot: the 8*MT f32 accumulators of each of the 256 threads,
// element r of thread i at r * kThreads + i (one wave store covers 256
// consecutive bytes); Tile<BM>::kPartFloats floats.
// Arrival counters sit one 128-byte line apart: counters sharing a line
// serialize every workgroup's atomic on that line.
constexpr int kCounterStride = 32;

// LDS of one workgroup: the two stages of the ring, the last-arrival flag of
// split-K, and the grouped form's pair and q8_K row of each token row.
struct TileLds {
  uint8_t* stage0;
  uint8_t* stage1;
  uint8_t* stage2;  // the third stage of a three-stage ring (else unused)
  int* last_arrival;
  int* pair_s;
  int* xrow_s;
};

// One super-block of a wave's 32 weight rows (two 16-row MFMA tiles) against
// the tile's 16*MT tokens, accumulated into acc. The weight operands come in
// registers: each row tile's 16-byte block header and the lane's two 16-byte
// nibble chunks (chunk q and chunk q + 4 of the row's 128 nibble bytes). The
// tokens' codes, scales and sub-block sums come from LDS, in a stage's layout
// (`stg`: codes with the XOR-swizzled chunks, the scales at xs_off, the sums at
// sum_off). The caller has raised the wave's priority; it is lowered here for
// the float pass.
template <int MT>
__device__ __forceinline__ void block_product(const uint8_t* stg, int xs_off, int sum_off,
                                              const uint4 (&hdrs)[2], const uint4 (&rw)[2][2],
                                              int lane, float4 (&acc)[MT][2]) {
  const int l16 = lane & 15;
  const int q = lane >> 4;  // k-quarter of an MFMA operand
  const v4i zero = {0, 0, 0, 0};
  const v4f zerof = {0.f, 0.f, 0.f, 0.f};
  // The min term's operand split by lane quarter: q < 2 carry the low 7 bits
  // of each sum (and m_j), q >= 2 the sum shifted down by 7 (and 128*m_j).
  const int a_shift = (q >> 1) ? 7 : 0;
  const int a_mask = (q >> 1) ? -1 : 127;
  const _Float16 b_scale = static_cast<_Float16>((q >> 1) ? 128.0f : 1.0f);
  v4i sa[MT][2], sb[MT][2];
  const uint8_t* act = stg;
  const float* xs_s = reinterpret_cast<const float*>(stg + xs_off);
  const int* sum_s = reinterpret_cast<const int*>(stg + sum_off);

  // ---- this lane's weight rows: the sub-block scale of each (row, MFMA t)
  // for this lane (sub-block 2*(q>>1) + (t&1) + 4*(t>>1), below), the
  // block's d and dmin, and the min term's B operand (m_j or 128*m_j for
  // k = 4q..4q+3) ----
  uint32_t scj[2][4];
  float dn[2], dmn[2];
  h4 mbh[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const uint4 hdr = hdrs[nt];
    const uint32_t h1 = hdr.y, h2 = hdr.z, h3 = hdr.w;
    const uint32_t sc_lo = h1 & 0x3F3F3F3Fu;
    const uint32_t m_lo = h2 & 0x3F3F3F3Fu;
    const uint32_t sc_hi = (h3 & 0x0F0F0F0Fu) | ((h1 >> 2) & 0x30303030u);
    const uint32_t m_hi = ((h3 >> 4) & 0x0F0F0F0Fu) | ((h2 >> 2) & 0x30303030u);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int shift = 8 * (2 * (q >> 1) + (t & 1));
      scj[nt][t] = (((t < 2) ? sc_lo : sc_hi) >> shift) & 0xFFu;
    }
    dn[nt] = half_bits_to_float(hdr.x & 0xFFFFu);
    dmn[nt] = half_bits_to_float(hdr.x >> 16);
    const uint32_t mw4 = (q & 1) ? m_hi : m_lo;  // mins 4(q&1) .. 4(q&1)+3
#pragma unroll
    for (int i = 0; i < 4; ++i)
      mbh[nt][i] =
          static_cast<_Float16>(static_cast<unsigned short>((mw4 >> (8 * i)) & 0xFFu)) * b_scale;
  }
  // ---- this block's M = sum_j m_j * s_j, exact: A = sl_j (lanes q < 2)
  // or sh_j (q >= 2) of token m = 16mt + l16 for j = 4(q&1) .. +3 ----
  v4f cm[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = 16 * mt + l16;
    const int4 s4 = *reinterpret_cast<const int4*>(sum_s + 8 * r + 4 * (q & 1));
    h4 ah;
    ah[0] = static_cast<_Float16>(static_cast<short>((s4.x >> a_shift) & a_mask));
    ah[1] = static_cast<_Float16>(static_cast<short>((s4.y >> a_shift) & a_mask));
    ah[2] = static_cast<_Float16>(static_cast<short>((s4.z >> a_shift) & a_mask));
    ah[3] = static_cast<_Float16>(static_cast<short>((s4.w >> a_shift) & a_mask));
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
      cm[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x16f16(ah, mbh[nt], zerof, 0, 0, 0);
  }

  // ---- the four MFMAs of a tile: MFMA t takes, in lane q, one nibble half
  // of a 16-byte chunk of the row's nibbles: chunk q (bytes 16q..16q+15)
  // for t = 0, 1 and chunk q + 4 for t = 2, 3, low nibbles for even t and
  // high nibbles for odd t. Chunk c holds the low (sub-block 2*(c/2)) and
  // high (sub-block 2*(c/2)+1) nibbles of weights 64*(c/2) + 16*(c%2) + i,
  // so every loaded byte feeds two MFMAs, and lane q's sub-block in MFMA t
  // is j = 2*(q>>1) + (t&1) + 4*(t>>1). The A operand reads the codes of
  // the same weights: 16-byte code chunk 4*(q>>1) + (q&1) + 2*(t&1) +
  // 8*(t>>1). (Any assignment of the 64 k of an MFMA to lanes is the same
  // contraction as long as A and B agree on it.) ----
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int ct = 4 * (q >> 1) + (q & 1) + 2 * (t & 1) + 8 * (t >> 1);
    v4i a[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int r = 16 * mt + l16;
      a[mt] = *reinterpret_cast<const v4i*>(act + 256 * r + 16 * (ct ^ (r & 15)));
    }
    v4i ba[2], bb[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const uint4 raw = rw[nt][t >> 1];
      const uint32_t hs = (t & 1) ? 4u : 0u;
      const uint32_t c0 = (raw.x >> hs) & 0x0F0F0F0Fu, c1 = (raw.y >> hs) & 0x0F0F0F0Fu;
      const uint32_t c2 = (raw.z >> hs) & 0x0F0F0F0Fu, c3 = (raw.w >> hs) & 0x0F0F0F0Fu;
      const uint32_t fa = scj[nt][t] >> 3, fb = scj[nt][t] & 7u;
      ba[nt] = (v4i){(int)mul_bytes(c0, fa), (int)mul_bytes(c1, fa), (int)mul_bytes(c2, fa),
                     (int)mul_bytes(c3, fa)};
      bb[nt] = (v4i){(int)mul_bytes(c0, fb), (int)mul_bytes(c1, fb), (int)mul_bytes(c2, fb),
                     (int)mul_bytes(c3, fb)};
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        sa[mt][nt] = mfma(a[mt], ba[nt], t == 0 ? zero : sa[mt][nt]);
        sb[mt][nt] = mfma(a[mt], bb[nt], t == 0 ? zero : sb[mt][nt]);
      }
  }

  __builtin_amdgcn_s_setprio(0);
  // ---- per-block epilogue: one float pass per output,
  // xs * (d * S - dmin * M) ----
  // C layout of a 16x16 tile: lane holds column l16, rows 4q..4q+3.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int mr = 16 * mt + 4 * q;
    const float x0 = xs_s[mr], x1 = xs_s[mr + 1], x2 = xs_s[mr + 2], x3 = xs_s[mr + 3];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const v4i sv = (sa[mt][nt] << 3) + sb[mt][nt];
      const float d = dn[nt], dm = -dmn[nt];
      const v4f mv = cm[mt][nt];
      acc[mt][nt].x += x0 * __builtin_fmaf(dm, mv[0], d * static_cast<float>(sv.x));
      acc[mt][nt].y += x1 * __builtin_fmaf(dm, mv[1], d * static_cast<float>(sv.y));
      acc[mt][nt].z += x2 * __builtin_fmaf(dm, mv[2], d * static_cast<float>(sv.z));
      acc[mt][nt].w += x3 * __builtin_fmaf(dm, mv[3], d * static_cast<float>(sv.w));
    }
  }
}

// The end of a tile: a split's partial handed over through the workspace (the
// last arriving split sums all of them in the fixed order 0..kst-1), then the
// store of the tile's outputs (rows m0.., or the pairs' rows in the grouped
// form). Workgroup-uniform: returns early on every split but the last.
template <int BMv, bool ID>
__device__ __forceinline__ void finish_tile(float4 (&acc)[BMv / 16][2], float* __restrict__ y,
                                            int M, int N, int m0, int n0, int kst, int split,
                                            int wt, float* __restrict__ part,
                                            int* __restrict__ cnt, int& last_arrival,
                                            const int* pair_s) {
  using TL = Tile<BMv>;
  constexpr int MT = TL::MT;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int q = lane >> 4;
  if (kst > 1) {
    // ---- split-K: publish this split's partial, count the arrival ----
    float* mine = part + static_cast<int64_t>(wt * kst + split) * TL::kPartFloats + tid;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int r = 4 * (2 * mt + nt);
        __hip_atomic_store(mine + (r + 0) * kThreads, acc[mt][nt].x, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(mine + (r + 1) * kThreads, acc[mt][nt].y, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(mine + (r + 2) * kThreads, acc[mt][nt].z, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(mine + (r + 3) * kThreads, acc[mt][nt].w, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    // Every store of this wave has completed before the workgroup counts its
    // arrival, so the split that sees the count reach ks - 1 reads whole
    // partials. The order rests on three things: the partials and the counter
    // are agent-scope atomics (device-coherent: they bypass the per-XCD L2's
    // non-coherent state, so no write-back or invalidate is needed); each
    // wave waits for the acknowledgement of its stores (vmcnt 0) before the
    // barrier; and the barrier's workgroup fences keep the compiler from
    // moving any of these accesses across it. A C++ release/acquire pair on
    // the counter at agent scope adds a write-back and an invalidate of the
    // whole L2 per workgroup on gfx950, measured 1.2-1.75x slower here.
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    if (tid == 0)
      last_arrival = __hip_atomic_fetch_add(cnt + wt * kCounterStride, 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT) == kst - 1;
    __syncthreads();
    if (!last_arrival) return;  // workgroup-uniform
    if (tid == 0)
      __hip_atomic_store(cnt + wt * kCounterStride, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // The sum over splits in the fixed order 0..ks-1 (this split's own
    // values from registers).
    float4 sum[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) sum[mt][nt] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < kst; ++j) {
      const float* pj = part + static_cast<int64_t>(wt * kst + j) * TL::kPartFloats + tid;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          float4 v;
          if (j == split) {
            v = acc[mt][nt];
          } else {
            const int r = 4 * (2 * mt + nt);
            v.x = __hip_atomic_load(pj + (r + 0) * kThreads, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            v.y = __hip_atomic_load(pj + (r + 1) * kThreads, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            v.z = __hip_atomic_load(pj + (r + 2) * kThreads, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            v.w = __hip_atomic_load(pj + (r + 3) * kThreads, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          sum[mt][nt].x += v.x;
          sum[mt][nt].y += v.y;
          sum[mt][nt].z += v.z;
          sum[mt][nt].w += v.w;
        }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = sum[mt][nt];
  }

  // ---- store ----
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int n = n0 + 32 * wave + 16 * nt + l16;
      const int mr = m0 + 16 * mt + 4 * q;
      if (n < N) {
        const float v[4] = {acc[mt][nt].x, acc[mt][nt].y, acc[mt][nt].z, acc[mt][nt].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (mr + i >= M) continue;
          const int64_t row = ID ? pair_s[mr + i] : mr + i;
          y[row * N + n] = v[i];
        }
      }
    }
}

// One workgroup's tile: `wg` is its index in the launch's grid (or in its
// region of a grid that runs two tile sizes).
template <int BMv, bool ID, int NST = 2>
__device__ __forceinline__ void gemm_tile(const TileLds& lds, int wg, float* __restrict__ y,
                                          const uint8_t* __restrict__ w,
                                          const uint8_t* __restrict__ xq, int M, int N, int nb,
                                          int mtiles, int ntiles, int n_full, int ks,
                                          float* __restrict__ part, int* __restrict__ cnt,
                                          const IdGemm& id) {
  using TL = Tile<BMv>;
  constexpr int BM = BMv;
  constexpr int MT = TL::MT;
  static_assert(NST == 2 || NST == 3, "two- or three-stage ring");
  uint8_t* const stage0 = lds.stage0;
  uint8_t* const stage1 = lds.stage1;
  uint8_t* const stage2 = lds.stage2;
  int& last_arrival = *lds.last_arrival;
  int* const pair_s = lds.pair_s;
  int* const xrow_s = lds.xrow_s;

  // Workgroup -> (tile, split). The first n_full workgroups take tiles
  // 0..n_full-1 whole; the others split each remaining tile's K ks ways
  // (split-major). When a region's workgroup count is a multiple of the 8
  // XCDs, XCD x (= id % 8) takes a contiguous run of it, in which the token
  // tiles of one weight tile (same split) are adjacent.
  const int tiles = mtiles * ntiles;
  int tile, split = 0, kst = 1;
  if (wg < n_full) {
    const int t = (n_full % 8 == 0) ? (wg % 8) * (n_full / 8) + wg / 8 : wg;
    tile = t;
  } else {
    const int rest = tiles - n_full;
    const int G = rest * ks;
    const int v = wg - n_full;
    const int u = (G % 8 == 0) ? (v % 8) * (G / 8) + v / 8 : v;
    split = u / rest;
    tile = n_full + (u - split * rest);
    kst = ks;
  }
  const int wt = tile - n_full;  // workspace slot of a split tile
  const int ntile = tile / mtiles;
  const int mtile = tile % mtiles;
  int m0 = mtile * BM;
  const int n0 = ntile * BN;
  const int b_lo = static_cast<int>(static_cast<int64_t>(split) * nb / kst);
  const int b_hi = static_cast<int>(static_cast<int64_t>(split + 1) * nb / kst);

  const int tid = threadIdx.x;
  if constexpr (ID) {
    // mtile indexes the tile list; its pairs become the tile's token rows.
    // Every lane reads the same words; readfirstlane makes that explicit, so
    // the expert's weight base is a scalar (the direct-to-LDS loads take a
    // scalar base).
    if (mtile >= __builtin_amdgcn_readfirstlane(*id.n_tiles)) return;  // workgroup-uniform
    const int4 dv = id.desc[mtile];
    const int4 d = make_int4(__builtin_amdgcn_readfirstlane(dv.x),
                             __builtin_amdgcn_readfirstlane(dv.y),
                             __builtin_amdgcn_readfirstlane(dv.z), 0);
    if (tid < BM) {
      const int p = id.sorted[d.y + min(tid, d.z - 1)];
      pair_s[tid] = p;
      xrow_s[tid] = id.per_slot_x ? p : p / id.n_used;
    }
    __syncthreads();
    if (d.x == id.n_experts) {  // out-of-range selections: NaN rows
      for (int i = tid; i < d.z * BN; i += kThreads) {
        const int n = n0 + i % BN;
        if (n < N) y[static_cast<int64_t>(pair_s[i / BN]) * N + n] = __builtin_nanf("");
      }
      return;
    }
    w += static_cast<int64_t>(d.x) * id.expert_bytes;
    M = d.z;
    m0 = 0;
  }
  const int lane = tid & 63;
  const int wave = tid >> 6;       // 32-row slice of the weight tile
  const int l16 = lane & 15;
  const int q = lane >> 4;         // k-quarter of an MFMA operand: k = 16q..16q+15

  float4 acc[MT][2];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = make_float4(0.f, 0.f, 0.f, 0.f);

  const StageOffsets<BMv> so = stage_offsets<BMv, ID>(M, N, nb, m0, n0, wave, lane, xrow_s);
  issue_stage<BMv>(stage0, xq, w, so, b_lo, wave, lane);
  if (NST == 3 && b_lo + 1 < b_hi) issue_stage<BMv>(stage1, xq, w, so, b_lo + 1, wave, lane);

  // One super-block: wait for its stage, refill the stage computed in the
  // previous step (every wave finished reading it: it passed the barrier
  // below, which follows the compute of b-1) with super-block b+1 (two
  // stages) or b+2 (three stages, so b+1 stays in flight while b is
  // computed), then compute from `stg`.
  auto step = [&](int b, const uint8_t* stg, uint8_t* refill) {
    if constexpr (NST == 2) {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
      if (b + 1 < b_hi) issue_stage<BMv>(refill, xq, w, so, b + 1, wave, lane);
    } else {
      if (b + 1 < b_hi)
        wait_stage_behind_one<BMv>(wave);
      else
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
      if (b + 2 < b_hi) issue_stage<BMv>(refill, xq, w, so, b + 2, wave, lane);
    }
    // Wave priority: raised from here through the MFMA loop, lowered for the
    // epilogue, so that of the two waves sharing a SIMD the one feeding the
    // matrix core issues first and the other's VALU epilogue fills the gaps
    // (measured: 7-11% faster at 512 tokens).
    __builtin_amdgcn_s_setprio(1);

    // This lane's weight operands from the stage.
    const uint8_t* wblk = stg + TL::kWOff;
    uint4 hdr[2], rw[2][2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const uint8_t* blk = wblk + (32 * wave + 16 * nt + l16) * kQ4KBytes;
      hdr[nt] = *reinterpret_cast<const uint4*>(blk);
      rw[nt][0] = *reinterpret_cast<const uint4*>(blk + 16 + 16 * q);
      rw[nt][1] = *reinterpret_cast<const uint4*>(blk + 16 + 64 + 16 * q);
    }
    block_product<MT>(stg, TL::kXsOff, TL::kSumOff, hdr, rw, lane, acc);
  };

  // The ring unrolled by its depth so each stage is a distinct LDS object;
  // super-block b uses stage (b - b_lo) % NST.
  if constexpr (NST == 2) {
    for (int b = b_lo; b < b_hi; b += 2) {
      step(b, stage0, stage1);
      if (b + 1 < b_hi) step(b + 1, stage1, stage0);
    }
  } else {
    for (int b = b_lo; b < b_hi; b += 3) {
      step(b, stage0, stage2);
      if (b + 1 < b_hi) step(b + 1, stage1, stage0);
      if (b + 2 < b_hi) step(b + 2, stage2, stage1);
    }
  }
  finish_tile<BMv, ID>(acc, y, M, N, m0, n0, kst, split, wt, part, cnt, last_arrival, pair_s);
}

template <int BMv, bool ID>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void gemm_q4k_kernel(float* __restrict__ y, const uint8_t* __restrict__ w,
                     const uint8_t* __restrict__ xq, int M, int N, int nb, int mtiles,
                     int ntiles, int n_full, int ks, float* __restrict__ part,
                     int* __restrict__ cnt, IdGemm id) {
  __shared__ __align__(16) uint8_t stage0[Tile<BMv>::kStageBytes];
  __shared__ __align__(16) uint8_t stage1[Tile<BMv>::kStageBytes];
  __shared__ int last_arrival;
  __shared__ int pair_s[ID ? BMv : 1];
  __shared__ int xrow_s[ID ? BMv : 1];
  gemm_tile<BMv, ID>(TileLds{stage0, stage1, nullptr, &last_arrival, pair_s, xrow_s},
                     static_cast<int>(blockIdx.x), y, w, xq, M, N, nb, mtiles, ntiles, n_full, ks,
                     part, cnt, id);
}

// The 16-token tile with a three-stage ring: two super-blocks in flight
// while one is computed (69 KB of LDS), for grids of at most one workgroup
// per CU. (The 64-token tile's three-stage ring, 111 KB, measured slower on
// such grids: 64 x 4096x14336 25.9 us against 25.0, 96 x 4096x4096 20.1
// against 19.2; its compute per super-block covers the refill.)
template <int BMv>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void gemm_q4k_deep_ring_kernel(float* __restrict__ y, const uint8_t* __restrict__ w,
                               const uint8_t* __restrict__ xq, int M, int N, int nb, int mtiles,
                               int ntiles, int n_full, int ks, float* __restrict__ part,
                               int* __restrict__ cnt) {
  static_assert(3 * Tile<BMv>::kStageBytes <= 160 * 1024, "the ring exceeds 160 KiB");
  __shared__ __align__(16) uint8_t stage0[Tile<BMv>::kStageBytes];
  __shared__ __align__(16) uint8_t stage1[Tile<BMv>::kStageBytes];
  __shared__ __align__(16) uint8_t stage2[Tile<BMv>::kStageBytes];
  __shared__ int last_arrival;
  __shared__ int pair_s[1];
  __shared__ int xrow_s[1];
  gemm_tile<BMv, false, 3>(TileLds{stage0, stage1, stage2, &last_arrival, pair_s, xrow_s},
                           static_cast<int>(blockIdx.x), y, w, xq, M, N, nb, mtiles, ntiles,
                           n_full, ks, part, cnt, IdGemm{});
}

// ---- short batches on tall matrices: K split across a workgroup's waves ----
// Tile: up to 16 tokens x 32 weight rows per 256-thread workgroup. Wave g
// takes super-blocks [g*nb/4, (g+1)*nb/4) of all 32 rows through a two-stage
// LDS ring of its own (its own loads, its own waits: no barrier between the
// waves until the end), with the 16-token tile's arithmetic per super-block.
// The four partial tiles are summed in LDS in the fixed order 0..3, so a
// grid of one workgroup per 32 rows fills the device without the split-K
// workspace and its cross-workgroup hand-off (section 25.3: fill the device;
// a timing probe put the hand-off at about 2 us of the 16-token tile's 13 us
// at 16 x 14336 x 4096). The price is four copies of the tokens' q8_K rows
// per workgroup, read from L2, and one stage in flight per wave.
struct WsStage {
  static constexpr int kRows = 32;
  static constexpr int kActBytes = 16 * 256;              // codes, chunks XOR-swizzled
  static constexpr int kXsOff = kActBytes;                 // 16 f32 token scales
  static constexpr int kSumOff = kXsOff + 16 * 4;          // 16 x 8 int32 sub-block sums
  static constexpr int kWOff = kSumOff + 16 * 32;          // 32 raw Q4_K blocks
  static constexpr int kBytes = kWOff + kRows * kQ4KBytes;  // 9280
  static constexpr int kLoads = 4 + 5 + 1 + 1;              // DMA instructions per stage
};
static_assert(WsStage::kBytes % 16 == 0 && WsStage::kWOff % 16 == 0, "16-byte LDS slots");
static_assert(8 * WsStage::kBytes * 2 <= 160 * 1024, "two workgroups' rings exceed 160 KiB");
static_assert(WsStage::kLoads == 11, "the wait count below assumes 11 loads per stage");

// This lane's byte offsets of one stage's loads relative to super-block 0.
struct WsOffsets {
  uint32_t act[4];
  uint32_t wt[5];
  uint32_t sums, xs;
};

__device__ __forceinline__ WsOffsets ws_offsets(int M, int N, int nb, int m0, int n0, int lane) {
  WsOffsets o;
  const uint32_t xrow = static_cast<uint32_t>(nb) * kQ8KBytes;
  const uint32_t wrow = static_cast<uint32_t>(nb) * kQ4KBytes;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = 4 * j + (lane >> 4);
    const int c = (lane & 15) ^ (m & 15);  // source chunk of this lane's slot
    o.act[j] = static_cast<uint32_t>(min(m0 + m, M - 1)) * xrow + 16u * c;
  }
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    const int i = min(64 * j + lane, WsStage::kRows * 9 - 1);  // lanes past 288: masked
    const int n = i / 9, c = i - 9 * (i / 9);
    o.wt[j] = static_cast<uint32_t>(min(n0 + n, N - 1)) * wrow + 16u * c;
  }
  const int ms = min(lane >> 1, 15);  // lanes 0..31: the sums, two chunks per token
  o.sums = static_cast<uint32_t>(min(m0 + ms, M - 1)) * xrow + 256u + 16u * (lane & 1);
  o.xs = static_cast<uint32_t>(min(m0 + min(lane, 15), M - 1)) * xrow + 288u;
  return o;
}

// Eleven loads, every one issued with at least one active lane (so each
// counts once in vmcnt): codes 4, weights 5 (the fifth on lanes 0..31),
// sums (lanes 0..31) and token scales (lanes 0..15). Token rows past the
// batch (m0 + m >= M) are not loaded, except lane 0 of a code load that
// would have none (it keeps the count): their LDS rows hold stale bytes,
// which reach only the MFMA rows of outputs that are never stored (an
// output row reads its own token row of each operand and nothing else).
__device__ __forceinline__ void ws_issue(uint8_t* stage, const uint8_t* xq_in,
                                         const uint8_t* w_in, const WsOffsets& o, int b,
                                         int lane, int rows) {
  const uint8_t* xq = uniform_ptr(xq_in + static_cast<size_t>(b) * kQ8KBytes);
  const uint8_t* w = uniform_ptr(w_in + static_cast<size_t>(b) * kQ4KBytes);
  const uint32_t lb = __builtin_amdgcn_readfirstlane(lds_u32(stage));
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (4 * j + (lane >> 4) < rows || lane == 0) lds_dma16(xq, o.act[j], lb + 1024 * j);
#pragma unroll
  for (int j = 0; j < 4; ++j) lds_dma16(w, o.wt[j], lb + WsStage::kWOff + 1024 * j);
  if (lane < 32) lds_dma16(w, o.wt[4], lb + WsStage::kWOff + 4096);
  if (lane < 32 && (lane >> 1) < rows) lds_dma16(xq, o.sums, lb + WsStage::kSumOff);
  if (lane < 16 && lane < rows) lds_dma4(xq, o.xs, lb + WsStage::kXsOff);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void gemm_q4k_wave_split_kernel(float* __restrict__ y, const uint8_t* __restrict__ w,
                                const uint8_t* __restrict__ xq, int M, int N, int nb,
                                int mtiles) {
  static_assert(kThreads == 256, "four waves, one K quarter each");
  __shared__ __align__(16) uint8_t ring[4][2][WsStage::kBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int q = lane >> 4;
  const int wg = static_cast<int>(blockIdx.x);
  const int m0 = 16 * (wg % mtiles);
  const int n0 = WsStage::kRows * (wg / mtiles);
  const int b_lo = static_cast<int>(static_cast<int64_t>(wave) * nb / 4);
  const int b_hi = static_cast<int>(static_cast<int64_t>(wave + 1) * nb / 4);
  uint8_t* const st0 = ring[wave][0];
  uint8_t* const st1 = ring[wave][1];

  float4 acc[1][2];
  acc[0][0] = make_float4(0.f, 0.f, 0.f, 0.f);
  acc[0][1] = acc[0][0];
  const WsOffsets so = ws_offsets(M, N, nb, m0, n0, lane);
  const int rows = min(M - m0, 16);  // token rows of this tile, >= 1
  if (b_lo < b_hi) ws_issue(st0, xq, w, so, b_lo, lane, rows);
  if (b_lo + 1 < b_hi) ws_issue(st1, xq, w, so, b_lo + 1, lane, rows);

  // Super-block b from `stg`: wait until its eleven loads have landed (the
  // next stage's eleven may still be in flight; loads complete in order),
  // compute, then refill `stg` with b + 2 once every read of it is done.
  auto step = [&](int b, uint8_t* stg) {
    if (b + 1 < b_hi)
      __builtin_amdgcn_s_waitcnt(kWaitVm0 | WsStage::kLoads);
    else
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __builtin_amdgcn_s_setprio(1);
    uint4 hdr[2], rw[2][2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const uint8_t* blk = stg + WsStage::kWOff + (16 * nt + l16) * kQ4KBytes;
      hdr[nt] = *reinterpret_cast<const uint4*>(blk);
      rw[nt][0] = *reinterpret_cast<const uint4*>(blk + 16 + 16 * q);
      rw[nt][1] = *reinterpret_cast<const uint4*>(blk + 16 + 64 + 16 * q);
    }
    block_product<1>(stg, WsStage::kXsOff, WsStage::kSumOff, hdr, rw, lane, acc);
    if (b + 2 < b_hi) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of stg are done
      ws_issue(stg, xq, w, so, b + 2, lane, rows);
    }
  };
  for (int b = b_lo; b < b_hi; b += 2) {
    step(b, st0);
    if (b + 1 < b_hi) step(b + 1, st1);
  }

  // ---- the four partial tiles, summed in the order 0, 1, 2, 3 ----
  // Waves 1..3 leave theirs in their own first stage (all their loads have
  // landed and their reads are done); wave 0 adds them to its own.
  float4* red = reinterpret_cast<float4*>(st0) + 2 * lane;
  if (wave > 0) {
    red[0] = acc[0][0];
    red[1] = acc[0][1];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int g = 1; g < 4; ++g) {
    const float4* pg = reinterpret_cast<const float4*>(ring[g][0]) + 2 * lane;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const float4 v = pg[nt];
      acc[0][nt].x += v.x;
      acc[0][nt].y += v.y;
      acc[0][nt].z += v.z;
      acc[0][nt].w += v.w;
    }
  }
  // C layout of a 16x16 tile: lane holds row column l16, tokens 4q..4q+3.
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int n = n0 + 16 * nt + l16;
    const int mr = m0 + 4 * q;
    if (n >= N) continue;
    const float v[4] = {acc[0][nt].x, acc[0][nt].y, acc[0][nt].z, acc[0][nt].w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (mr + i < M) y[static_cast<int64_t>(mr + i) * N + n] = v[i];
  }
}

// The grouped form over two tile lists in one grid: the experts' whole tiles
// of up to 64 pairs on the 64-token tile (workgroups 0 .. big_wgs-1), then
// their remainders of at most 32 pairs in tiles of up to 16 on the 16-token
// tile (workgroups from small_base on, a multiple of 8 so that each region
// keeps its XCD layout). The small tiles run in the slots the whole tiles'
// last round leaves free. Every output's arithmetic is the same on both
// tiles.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void gemm_q4k_id_mixed_kernel(float* __restrict__ y, const uint8_t* __restrict__ w,
                              const uint8_t* __restrict__ xq, int M, int N, int nb,
                              int ntiles, int big_tiles, int small_tiles, int small_base,
                              IdGemm big, IdGemm small) {
  __shared__ __align__(16) uint8_t stage0[Tile<64>::kStageBytes];
  __shared__ __align__(16) uint8_t stage1[Tile<64>::kStageBytes];
  __shared__ int last_arrival;
  __shared__ int pair_s[64];
  __shared__ int xrow_s[64];
  const TileLds lds{stage0, stage1, nullptr, &last_arrival, pair_s, xrow_s};
  const int b = static_cast<int>(blockIdx.x);
  const int big_wgs = big_tiles * ntiles;
  if (b < big_wgs) {
    gemm_tile<64, true>(lds, b, y, w, xq, M, N, nb, big_tiles, ntiles, big_wgs, 1, nullptr,
                        nullptr, big);
  } else if (b >= small_base) {
    gemm_tile<16, true>(lds, b - small_base, y, w, xq, M, N, nb, small_tiles, ntiles,
                        small_tiles * ntiles, 1, nullptr, nullptr, small);
  }
}

// Split-K: the planner keeps the split workgroups of a launch within one
// round of resident workgroups (512 for the all-split rule, at most 768 for
// a remainder); the caller's workspace holds one arrival counter per split
// tile (one 128-byte line each) and one partial slot per split workgroup.
constexpr int kSplitSlots = 768;     // split workgroups of a launch
constexpr int kSplitCounters = 768;  // split tiles of a launch
constexpr int kSplitTiles = 256;     // up to this many tiles, every tile splits
constexpr int kRound = 512;          // the all-split rule's one round of workgroups

// Workgroups resident at once over the 256 CUs: two 64-token tiles or three
// 16-token tiles per CU (their two-stage LDS rings, 73 KB and 46 KB of the
// 160 KB).
constexpr int64_t resident_tiles(int bm) { return bm == 16 ? 768 : 512; }

// The grouped form's tile list: up to kIdMaxPairs pairs.
constexpr int64_t kIdMaxPairs = int64_t{1} << 20;
constexpr int kIdMaxExperts = 1024;
constexpr int kIdBM = 64;  // the grouped form's whole tile
constexpr int kIdBS = 16;  // its small tiles: an expert's remainder of at most 32 pairs

constexpr size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Split-K workspace of a plan: a fixed region of kSplitCounters arrival
// counters (96 KiB; a plan uses the first `rest`), then the partial slots of
// its split workgroups. The counters' region is the same for every plan, so
// a workspace that served one shape serves the next: partials never land on
// bytes another plan reads as counters.
constexpr size_t kSplitCounterBytes = static_cast<size_t>(kSplitCounters) * kCounterStride * 4;
size_t split_workspace_bytes(int rest, int ks, int bm) {
  const size_t slot = (bm == 16 ? Tile<16>::kPartFloats : Tile<64>::kPartFloats) * sizeof(float);
  return kSplitCounterBytes + static_cast<size_t>(rest) * ks * slot;
}

// The grouped product's workspace: whole-tile descriptors, small-tile
// descriptors, the pairs grouped by expert, then the two tile counts.
struct IdLayout {
  size_t desc, desc_s, sorted, counts, bytes;
};
IdLayout id_layout(int64_t n_pairs, int64_t n_experts) {
  IdLayout L;
  L.desc = 0;
  L.desc_s = L.desc + static_cast<size_t>(route_max_tiles(n_pairs, n_experts, kIdBM)) * 16;
  L.sorted = L.desc_s + static_cast<size_t>(route_max_small_tiles(n_pairs, n_experts)) * 16;
  L.counts = align_up(L.sorted + static_cast<size_t>(n_pairs) * sizeof(int32_t), 16);
  L.bytes = L.counts + 16;
  return L;
}

template <int BMv>
hipError_t launch_split(float* y, const void* w, const void* xq, int64_t M, int64_t N, int64_t K,
                        const GemmPlan& plan, void* ws, size_t ws_bytes, hipStream_t stream) {
  const int nb = static_cast<int>(K / 256);
  const int mtiles = static_cast<int>((M + BMv - 1) / BMv);
  const int ntiles = static_cast<int>((N + BN - 1) / BN);
  const int tiles = mtiles * ntiles;
  int n_full = tiles, ks = 1;
  float* part = nullptr;
  int* cnt = nullptr;
  if (plan.ks > 1) {
    n_full = plan.n_full;
    ks = plan.ks;
    const int rest = tiles - n_full;
    if (n_full < 0 || rest < 1 || rest > kSplitCounters || rest * ks > kSplitSlots || ks > nb)
      return hipErrorInvalidValue;
    if (!ws || ws_bytes < split_workspace_bytes(rest, ks, BMv)) return hipErrorInvalidValue;
    cnt = static_cast<int*>(ws);
    part = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kSplitCounterBytes);
  }
  const int grid = n_full + (tiles - n_full) * ks;
  // The 16-token tile computes little per super-block. On a grid of at most
  // one workgroup per CU (256), nothing else on the CU hides a super-block's
  // load, so its ring goes three deep: 4096x14336 at 7 and 16 tokens 14.3
  // us against 15.7. With more workgroups than CUs the second workgroup on a
  // CU does that better (14336x4096 at 4-32 tokens: 12.5-16.9 us with two
  // stages against 13.9-18.4 with three), and the two-stage ring keeps three
  // per CU.
  if (BMv == 16 && grid <= 256)
    hipLaunchKernelGGL((gemm_q4k_deep_ring_kernel<16>), dim3(grid), dim3(kThreads), 0, stream, y,
                       static_cast<const uint8_t*>(w), static_cast<const uint8_t*>(xq),
                       static_cast<int>(M), static_cast<int>(N), nb, mtiles, ntiles, n_full, ks,
                       part, cnt);
  else
    hipLaunchKernelGGL((gemm_q4k_kernel<BMv, false>), dim3(grid), dim3(kThreads), 0, stream, y,
                       static_cast<const uint8_t*>(w), static_cast<const uint8_t*>(xq),
                       static_cast<int>(M), static_cast<int>(N), nb, mtiles, ntiles, n_full, ks,
                       part, cnt, IdGemm{});
  return hipGetLastError();
}

}  // namespace

GemmPlan gemm_q4k_plan(int64_t M, int64_t N, int64_t K, int bm) {
  const int64_t tiles = ((M + bm - 1) / bm) * ((N + BN - 1) / BN);
  const int64_t nb = K / 256;
  if (tiles <= kSplitTiles) {
    // Measured on MI355X (cold weights; 14336x4096, 4096x14336 and 4096x4096
    // at 7..512 tokens, both token tiles, ks = 1..8): the best launches stay
    // within about one round of resident workgroups (512), give each split
    // at least four super-blocks, and gain nothing past eight splits.
    const int64_t ks = std::max<int64_t>(
        1, std::min<int64_t>(std::min<int64_t>(kRound / tiles, nb / 4), 8));
    return GemmPlan{0, static_cast<int>(ks)};
  }
  // More tiles than that: whole rounds of whole tiles, then the remainder,
  // which leaves the device part-idle for a last round of nb super-blocks
  // (section 25.3: fill the device). The remainder splits over K when the
  // split workgroups fit one round and that round is shorter. Cost in tenths
  // of a super-block step of a CU running two tiles, measured on MI355X
  // (cold weights, 14336x4096 and 8192x4096): a CU with one tile runs a step
  // in 0.7 of that, and a round of split workgroups pays about 2.5 steps
  // more (the ring's first load, the partials and their sum). 320 x 14336 x
  // 4096 (560 tiles = 512 whole + 48 in four splits): 59 us against 75;
  // 576 x 8192 x 4096: 60 against 74. Remainders that would need several
  // rounds of splits lose: 896 tiles with 384 in four splits, 100 us
  // against 89.
  const int64_t S = resident_tiles(bm);
  const int64_t rest = tiles % S;
  GemmPlan plan{static_cast<int>(tiles), 1};
  if (rest == 0) return plan;
  auto step_cost = [&](int64_t wgs) { return wgs <= S / 2 ? 7 : 10; };
  int64_t best = nb * step_cost(rest);
  for (int64_t ks = 2; ks <= 8 && nb / ks >= 4 && rest * ks <= S; ks *= 2) {
    const int64_t cost = ((nb + ks - 1) / ks) * step_cost(rest * ks) + 25;
    if (cost < best) {
      best = cost;
      plan = GemmPlan{static_cast<int>(tiles - rest), static_cast<int>(ks)};
    }
  }
  return plan;
}

hipError_t launch_gemm_q4k_split(float* y, const void* w, const void* xq, int64_t M, int64_t N,
                                 int64_t K, const GemmPlan& plan, int bm, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
  if (bm == 16) return launch_split<16>(y, w, xq, M, N, K, plan, ws, ws_bytes, stream);
  if (bm == 64) return launch_split<64>(y, w, xq, M, N, K, plan, ws, ws_bytes, stream);
  return hipErrorInvalidValue;
}

size_t gemm_q4k_id_workspace_bytes(int64_t n_pairs, int64_t n_experts) {
  if (n_pairs < 1 || n_pairs > kIdMaxPairs || n_experts < 1 || n_experts > kIdMaxExperts) return 0;
  return id_layout(n_pairs, n_experts).bytes;
}

hipError_t launch_gemm_q4k_id(float* y, const void* slab, const void* xq, const int32_t* ids,
                              int64_t n_tokens, int64_t n_used, int64_t n_experts, int64_t rows,
                              int64_t K, int per_slot_x, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  const int64_t n_pairs = n_tokens * n_used;
  if (n_pairs > kIdMaxPairs || n_experts > kIdMaxExperts) return hipErrorInvalidValue;
  const IdLayout lay = id_layout(n_pairs, n_experts);
  if (!ws || ws_bytes < lay.bytes) return hipErrorInvalidValue;
  uint8_t* base = static_cast<uint8_t*>(ws);
  int4* desc = reinterpret_cast<int4*>(base + lay.desc);
  int4* desc_s = reinterpret_cast<int4*>(base + lay.desc_s);
  int32_t* sorted = reinterpret_cast<int32_t*>(base + lay.sorted);
  int32_t* n_tiles = reinterpret_cast<int32_t*>(base + lay.counts);
  int32_t* n_small = n_tiles + 1;
  hipError_t e;
  if ((e = launch_route_experts(ids, n_pairs, n_experts, kIdBM, kIdBS, sorted, desc, n_tiles,
                                desc_s, n_small, stream)) != hipSuccess)
    return e;
  const int nb = static_cast<int>(K / 256);
  const int ntiles = static_cast<int>((rows + BN - 1) / BN);
  const int64_t expert_bytes = rows * nb * static_cast<int64_t>(kQ4KBytes);
  // One grid over both lists: whole tiles first, the small tiles from the
  // next multiple of 8 workgroups on. Each region is sized by its list's
  // bound; workgroups past a list's end return at once.
  const int big = static_cast<int>(route_max_tiles(n_pairs, n_experts, kIdBM));
  const int small = static_cast<int>(route_max_small_tiles(n_pairs, n_experts));
  const int small_base = (big * ntiles + 7) / 8 * 8;
  const IdGemm id_big{sorted, desc, n_tiles, static_cast<int>(n_experts),
                      static_cast<int>(n_used), per_slot_x, expert_bytes};
  const IdGemm id_small{sorted, desc_s, n_small, static_cast<int>(n_experts),
                        static_cast<int>(n_used), per_slot_x, expert_bytes};
  hipLaunchKernelGGL(gemm_q4k_id_mixed_kernel, dim3(small_base + small * ntiles), dim3(kThreads),
                     0, stream, y, static_cast<const uint8_t*>(slab),
                     static_cast<const uint8_t*>(xq), static_cast<int>(n_pairs),
                     static_cast<int>(rows), nb, ntiles, big, small, small_base, id_big, id_small);
  return hipGetLastError();
}

int gemm_q4k_token_tile(int64_t M, int64_t N, int64_t K) {
  // The 16-token tile (one MFMA tile per wave, a quarter of the accumulators,
  // three workgroups per CU) against the 64-token one, measured: 14336x4096
  // at 7..16 tokens 12.4-12.8 us against 19.3-21.2, at 48 tokens 24.4 against
  // 21.0; 4096x4096 at 64 tokens 12.0 against 16.5. Where the weight tiles
  // are few (short matrices) the finer token tile fills the device at more
  // tokens: 4096x4096 at 96 and 128 tokens 14.4 and 15.0 us against 17.7 and
  // 17.6, 2048x2048 8.7 and 9.1 against 12.7 and 12.8; 5120x5120 and
  // 8192x4096 at 96 tokens 17.1 and 20.5 against 19.9 and 22.3 (at 128 the
  // 64-token tile is ahead again: 20.3 and 22.7 against 22.8 and 23.1);
  // 4096 rows of 11008 and 14336 at 48 tokens 17.2 and 21.2 against 20.8 and
  // 22.5.
  const int64_t nk = N * K;
  if (M <= 32) return 16;
  if (M <= 64 && (nk <= (int64_t{1} << 25) || N <= 4096)) return 16;
  if (M <= 96 && nk <= (int64_t{1} << 25)) return 16;
  if (M <= 128 && nk <= (int64_t{1} << 24)) return 16;
  return 64;
}

namespace {
// The wave-split tile's shapes: 256 to 512 row tiles of 32 (one round of two
// workgroups per CU) and 8 to 16 super-blocks (two to four per wave).
bool wave_split_shape(int64_t N, int64_t K) {
  const int64_t rt = (N + WsStage::kRows - 1) / WsStage::kRows, nb = K / 256;
  return rt >= 256 && rt <= 512 && nb >= 8 && nb <= 16;
}
}  // namespace

bool gemm_q4k_uses_wave_split(int64_t M, int64_t N, int64_t K) {
  // Measured on MI355X (cold weights), against the 16-token tile split four
  // ways over K through the workspace: 14336x4096 at 4, 8, 12, 16 tokens
  // 11.0, 11.7, 12.1, 12.5 us against 11.8, 12.0, 12.2, 12.4; 16 x 8192x4096
  // 7.8 against 9.6; 16 x 14336x3072 10.0 against 11.7; 16384x4096 at 4 and
  // 16 tokens 11.4 and 12.8 against 12.3 and 13.0. Rows of 32 super-blocks
  // lose (8 x 14336x8192: 19.1 against 18.5): each wave reads its own copy of
  // the tokens' rows, and that grows with K while the hand-off it saves does
  // not.
  return M >= 4 && M <= 16 && !gemm_q4k_uses_matvec(M, N, K) && wave_split_shape(N, K);
}

hipError_t launch_gemm_q4k_wave_split(float* y, const void* w, const void* xq, int64_t M,
                                      int64_t N, int64_t K, hipStream_t stream) {
  const int mtiles = static_cast<int>((M + 15) / 16);
  const int64_t grid = (N + WsStage::kRows - 1) / WsStage::kRows * mtiles;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_q4k_wave_split_kernel, dim3(static_cast<unsigned>(grid)),
                     dim3(kThreads), 0, stream, y, static_cast<const uint8_t*>(w),
                     static_cast<const uint8_t*>(xq), static_cast<int>(M), static_cast<int>(N),
                     static_cast<int>(K / 256), mtiles);
  return hipGetLastError();
}

bool gemm_q4k_uses_matvec(int64_t M, int64_t N, int64_t K) {
  // A very short batch is a weight stream, not a dense contraction: one pass
  // of the dot4 mat-vec over the weights for all M tokens costs less than
  // an MFMA tile while M is small, and its cost grows with M. Measured on
  // MI355X (cold weights), batched mat-vec against the MFMA tiles:
  // 14336x4096 at 3 tokens 9.6-10.2 us on the persistent grid against 12.4;
  // 4096x14336 at 3 tokens 11.8-12.0 with a row's units split across waves
  // against 15.4; 4 tokens on 4096x4096, 6144x4096, 4096x8192 and 11008x2048
  // 5.2, 6.8, 9.6, 6.0 against 8.5, 9.0, 11.2, 6.5, but on 8192x4096 (the
  // wave-split tile) 8.2 against 7.1; 6 tokens on 4096x4096 7.8 against 8.5,
  // on 8192x4096 and 14336x2048 12.8 and 11.5 against 7.2 and 7.0; 5 tokens
  // on 5120x5120 10.4 against 9.4; 8 tokens on 4096x4096, 6144x4096 and
  // 5120x6144 9.3, 13.7, 15.7 against 8.5, 9.0, 10.1; but on 2048x2048
  // (launch-bound on both paths) 8 tokens 4.4 against 7.5.
  if (M == 1) return true;
  if (M > gemv_q4k_multi_max_tokens(K)) return false;
  const int64_t nk = N * K;
  if (M <= 3 || nk <= (int64_t{1} << 23)) return true;
  // Up to eight tokens on rows of one unit of at most 2^24 weights: the
  // batched mat-vec's persistent grid (4096x4096 at 6 and 8 tokens: 6.5 and
  // 7.4 us against 7.6 and 8.6; on 8192x4096 and 14336x4096 it loses from
  // five tokens on: 8.9 against 7.3 us, 13.4 against 11.2).
  if (M <= 8 && K <= 4096 && nk <= (int64_t{1} << 24)) return true;
  // Four tokens on rows of one unit (K <= 4096) run on the batched mat-vec's
  // persistent grid (14336x4096: 9.6 us against 11.0 on the wave-split
  // tile; 12288x4096 8.9 against 10.7; 16384x4096 10.9 against 11.4;
  // 8192x4096 6.8 against 7.1); five or more lose there (5, 6, 8 x
  // 14336x4096: 17.0, 19.7, 25.7 us against 11.1, 11.4, 11.6).
  if (M == 4) return K <= 4096 || nk <= (int64_t{1} << 25);
  return M <= 6 && nk <= (int64_t{1} << 24);
}

// ---- the product for callers that cannot allocate ----
// Split-K scratch of xq_gemm_q4k_small_m_noalloc: every GPU the library runs
// on holds one copy until the process ends, and every call on that GPU shares
// it. In host code `scratch` names a host-side stand-in, not the device
// array: host code uses only the address hipGetSymbolAddress returns for the
// current device (noalloc_scratch below).
constexpr size_t kNoAllocScratchBytes = size_t{8} << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

__global__ void clear_words_kernel(int* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// The device address of `scratch` on the current device, looked up once per
// device. The first call on a device also clears the arrival counters (on
// the caller's stream, ahead of the product); every completed call leaves
// them at zero again.
hipError_t noalloc_scratch(hipStream_t stream, void** out) {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDev];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    constexpr int words = static_cast<int>(kSplitCounterBytes / 4);
    hipLaunchKernelGGL(clear_words_kernel, dim3((words + 255) / 256), dim3(256), 0, stream,
                       static_cast<int*>(p), words);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return hipSuccess;
}

}  // namespace

size_t gemm_q4k_noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

size_t gemm_q4k_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  // Shapes the entry point refuses need nothing (and this keeps every
  // product below in range: M, N <= 2^30, N*K/256*144 < 2^31).
  constexpr int64_t kRows = int64_t{1} << 30, kInt = 2147483647;
  if (M < 1 || N < 1 || M > kRows || N > kRows || K < 256 || K % 256 || K / 256 > kInt) return 0;
  if (M > (kInt / 320) / (K / 256) || N > (kInt / 144) / (K / 256)) return 0;
  if (M == 1 || gemm_q4k_uses_matvec(M, N, K) || gemm_q4k_uses_wave_split(M, N, K)) return 0;
  const int bm = gemm_q4k_token_tile(M, N, K);
  const GemmPlan plan = gemm_q4k_plan(M, N, K, bm);
  if (plan.ks <= 1) return 0;
  const int64_t tiles = ((M + bm - 1) / bm) * ((N + BN - 1) / BN);
  return split_workspace_bytes(static_cast<int>(tiles - plan.n_full), plan.ks, bm);
}

hipError_t launch_gemm_q4k(float* y, const void* w, const void* xq, int64_t M, int64_t N,
                           int64_t K, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (M == 1) return launch_gemv_q4k(y, w, xq, N, K, stream);
  if (gemm_q4k_uses_matvec(M, N, K)) return launch_gemv_q4k_multi(y, w, xq, M, N, K, stream);
  if (gemm_q4k_uses_wave_split(M, N, K))
    return launch_gemm_q4k_wave_split(y, w, xq, M, N, K, stream);
  const int bm = gemm_q4k_token_tile(M, N, K);
  return launch_gemm_q4k_split(y, w, xq, M, N, K, gemm_q4k_plan(M, N, K, bm), bm, ws, ws_bytes,
                               stream);
}

hipError_t launch_gemm_q4k_noalloc(float* y, const void* w, const void* xq, int64_t M, int64_t N,
                                   int64_t K, hipStream_t stream) {
  const size_t need = gemm_q4k_workspace_bytes(M, N, K);
  if (need > kNoAllocScratchBytes) return hipErrorInvalidValue;
  void* p = nullptr;
  if (need > 0) {
    const hipError_t e = noalloc_scratch(stream, &p);
    if (e != hipSuccess) return e;
  }
  return launch_gemm_q4k(y, w, xq, M, N, K, p, kNoAllocScratchBytes, stream);
}

}  // namespace xq
