// q4k_row.h — one lane's share of a Q4_K x q8_K row dot, for wave64 row kernels.
//
// "25 — Writing XPU Kernels", section 25.2: every weight nibble meets an int8
// code in a signed 4 x int8 dot (v_dot4_i32_i8; the 4-bit codes 0..15 are
// valid signed bytes); the sub-block scales multiply the integer sub-block dots
// in 24-bit integer multiplies; the min term is paid from the q8_K's stored
// sub-block sums; the f16/f32 scales are applied once per block after the
// integer work: the sums are reduced in integers and the float scales are
// applied once per block afterwards (section 25.2.1).
//
// Lane layout: a "unit" is 16 consecutive super-blocks of a row; lane l takes
// block 16u + l/4 and its whole 32-byte nibble group g = l%4 (byte i of the
// group holds weight 64g + i in its low nibble and weight 64g + 32 + i in its
// high one, so the low nibbles are sub-block 2g and the high ones sub-block
// 2g + 1), plus the block's 16-byte header. A lane's header decode and float
// pass thus cover 64 weights, and each lane pays the min term of its own two
// sub-blocks. Shared by the single-token and the batched mat-vec kernels, so a
// token's row comes out with the same bits from either.
#pragma once

#include "xq_device.h"

namespace xq {

constexpr int kUnitBlocks = 16;  // super-blocks per unit (four lanes each)

struct LaneGeom {
  int bsub;        // block slot within a unit (0..15)
  int g;           // nibble group (0..3)
  uint32_t selhi;  // all-ones when the group's scales sit in the 6+2-bit form
  int shift;       // bit offset of sub-block 2g's byte in the scale word
};

__device__ __forceinline__ LaneGeom lane_geom(int lane) {
  LaneGeom L;
  L.bsub = lane >> 2;
  L.g = lane & 3;
  L.selhi = (L.g >= 2) ? 0xFFFFFFFFu : 0u;
  L.shift = 16 * (L.g & 1);
  return L;
}

// A lane's 32 bytes of nibbles: group bytes 0..15 and 16..31.
struct Nib {
  uint4 a, b;
};

__device__ __forceinline__ Nib load_group(const uint8_t* blk, const LaneGeom& L) {
  Nib n;
  n.a = *reinterpret_cast<const uint4*>(blk + 16 + 32 * L.g);
  n.b = *reinterpret_cast<const uint4*>(blk + 32 + 32 * L.g);
  return n;
}

__device__ __forceinline__ Nib zero_group() {
  Nib n;
  n.a = make_uint4(0, 0, 0, 0);
  n.b = n.a;
  return n;
}

// The lane's slice of one token's q8_K block: the codes of its two
// sub-blocks (lo: weights 64g..64g+31, hi: 64g+32..64g+63), their two sums
// and the block scale.
struct TokenSlice {
  uint4 lo0, lo1, hi0, hi1;
  int2 sums;
  float xs;
};

__device__ __forceinline__ TokenSlice token_slice(const uint8_t* act, int b, const LaneGeom& L) {
  const uint8_t* xb = act + b * kQ8KBytes;
  const uint8_t* xg = xb + 64 * L.g;
  TokenSlice t;
  t.lo0 = *reinterpret_cast<const uint4*>(xg);
  t.lo1 = *reinterpret_cast<const uint4*>(xg + 16);
  t.hi0 = *reinterpret_cast<const uint4*>(xg + 32);
  t.hi1 = *reinterpret_cast<const uint4*>(xg + 48);
  t.sums = *reinterpret_cast<const int2*>(xb + 256 + 8 * L.g);
  t.xs = *reinterpret_cast<const float*>(xb + 288);
  return t;
}

// The weight side of a lane's group, decoded once: its nibbles, the two
// sub-blocks' scales and mins, and the block's d and dmin.
struct ChunkDecode {
  Nib nib;
  int sc0, sc1, m0, m1;
  float d, dmin;
};

__device__ __forceinline__ ChunkDecode chunk_decode(const Nib nib, const uint4 hdr,
                                                    const LaneGeom& L) {
  // Header: bytes 4..7 (h1) hold sc0..3 in bits 0-5 and the top bits of
  // sc4..7 in bits 6-7; bytes 8..11 (h2) the same for the mins; bytes 12..15
  // (h3) the low nibbles of sc4..7 and m4..7.
  ChunkDecode c;
  c.nib = nib;
  const uint32_t h1 = hdr.y, h2 = hdr.z, h3 = hdr.w;
  const uint32_t sc_lo = h1 & 0x3F3F3F3Fu;
  const uint32_t m_lo = h2 & 0x3F3F3F3Fu;
  const uint32_t sc_hi = (h3 & 0x0F0F0F0Fu) | ((h1 >> 2) & 0x30303030u);
  const uint32_t m_hi = ((h3 >> 4) & 0x0F0F0F0Fu) | ((h2 >> 2) & 0x30303030u);
  const uint32_t scw = (sc_hi & L.selhi) | (sc_lo & ~L.selhi);
  const uint32_t mw = (m_hi & L.selhi) | (m_lo & ~L.selhi);
  c.sc0 = (scw >> L.shift) & 0xFF;
  c.sc1 = (scw >> (L.shift + 8)) & 0xFF;
  c.m0 = (mw >> L.shift) & 0xFF;
  c.m1 = (mw >> (L.shift + 8)) & 0xFF;
  c.d = half_bits_to_float(hdr.x & 0xFFFFu);
  c.dmin = half_bits_to_float(hdr.x >> 16);
  return c;
}

// One token's contribution of a decoded group: the integer dots of the two
// sub-blocks, S = sc0*dlo + sc1*dhi and M = m0*s0 + m1*s1 in integers, then
// one float pass xs * (d*S - dmin*M). The float pass is written out (the
// fused multiply-add explicit, the last product kept from fusing with the
// caller's add), so every kernel that uses it rounds it the same way.
__device__ __forceinline__ float chunk_token_slice(const ChunkDecode& c, const TokenSlice& t) {
  const Nib n = c.nib;
  int dlo = sdot4(n.a.x & 0x0F0F0F0Fu, t.lo0.x, 0);
  dlo = sdot4(n.a.y & 0x0F0F0F0Fu, t.lo0.y, dlo);
  dlo = sdot4(n.a.z & 0x0F0F0F0Fu, t.lo0.z, dlo);
  dlo = sdot4(n.a.w & 0x0F0F0F0Fu, t.lo0.w, dlo);
  dlo = sdot4(n.b.x & 0x0F0F0F0Fu, t.lo1.x, dlo);
  dlo = sdot4(n.b.y & 0x0F0F0F0Fu, t.lo1.y, dlo);
  dlo = sdot4(n.b.z & 0x0F0F0F0Fu, t.lo1.z, dlo);
  dlo = sdot4(n.b.w & 0x0F0F0F0Fu, t.lo1.w, dlo);
  int dhi = sdot4((n.a.x >> 4) & 0x0F0F0F0Fu, t.hi0.x, 0);
  dhi = sdot4((n.a.y >> 4) & 0x0F0F0F0Fu, t.hi0.y, dhi);
  dhi = sdot4((n.a.z >> 4) & 0x0F0F0F0Fu, t.hi0.z, dhi);
  dhi = sdot4((n.a.w >> 4) & 0x0F0F0F0Fu, t.hi0.w, dhi);
  dhi = sdot4((n.b.x >> 4) & 0x0F0F0F0Fu, t.hi1.x, dhi);
  dhi = sdot4((n.b.y >> 4) & 0x0F0F0F0Fu, t.hi1.y, dhi);
  dhi = sdot4((n.b.z >> 4) & 0x0F0F0F0Fu, t.hi1.z, dhi);
  dhi = sdot4((n.b.w >> 4) & 0x0F0F0F0Fu, t.hi1.w, dhi);
  const int S = __mul24(c.sc0, dlo) + __mul24(c.sc1, dhi);
  const int M = __mul24(c.m0, t.sums.x) + __mul24(c.m1, t.sums.y);
  const float u = __builtin_fmaf(-c.dmin, static_cast<float>(M), c.d * static_cast<float>(S));
  float v = t.xs * u;
  __asm__("" : "+v"(v));
  return v;
}

__device__ __forceinline__ float chunk_token(const ChunkDecode& c, const uint8_t* act, int b,
                                             const LaneGeom& L) {
  return chunk_token_slice(c, token_slice(act, b, L));
}

// Contribution of one lane's nibble group of block b against one token's
// q8_K row `act`.
__device__ __forceinline__ float unit_partial(const Nib nib, const uint4 hdr, const uint8_t* act,
                                              int b, const LaneGeom& L) {
  return chunk_token(chunk_decode(nib, hdr, L), act, b, L);
}

}  // namespace xq
