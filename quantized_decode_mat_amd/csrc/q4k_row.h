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
// Lane layout: a "unit" is 8 consecutive super-blocks of a row; lane l takes
// block 8u + l/8 and its 16-byte nibble chunk c = l%8, which is half of nibble
// group g = c/2 (h = c%2), plus the block's 16-byte header. Shared by the
// single-token and the batched mat-vec kernels, so a token's row comes out
// with the same bits from either.
#pragma once

#include "xq_device.h"

namespace xq {

struct LaneGeom {
  int bsub;        // block slot within a unit (0..7)
  int g;           // nibble group (0..3)
  int h;           // half of the group (0..1)
  uint32_t selhi;  // all-ones when the group's scales sit in the 6+2-bit form
  uint32_t mmask;  // all-ones on the lane that pays the block's min term
  int shift;       // bit offset of sub-block 2g's byte in the scale word
};

__device__ __forceinline__ LaneGeom lane_geom(int lane) {
  LaneGeom L;
  L.bsub = lane >> 3;
  const int c = lane & 7;
  L.g = c >> 1;
  L.h = c & 1;
  L.selhi = (L.g >= 2) ? 0xFFFFFFFFu : 0u;
  L.mmask = (L.h == 0) ? 0xFFFFFFFFu : 0u;
  L.shift = 16 * (L.g & 1);
  return L;
}

// Contribution of one lane's 16-byte nibble chunk of block b.
__device__ __forceinline__ float unit_partial(const uint4 nib, const uint4 hdr, const uint8_t* act,
                                              int b, const LaneGeom& L) {
  const uint8_t* xb = act + b * kQ8KBytes;
  // Activation codes of the two half sub-blocks this chunk feeds.
  const uint4 alo = *reinterpret_cast<const uint4*>(xb + 64 * L.g + 16 * L.h);
  const uint4 ahi = *reinterpret_cast<const uint4*>(xb + 64 * L.g + 32 + 16 * L.h);
  const int2 sums = *reinterpret_cast<const int2*>(xb + 256 + 8 * L.g);
  const float xs = *reinterpret_cast<const float*>(xb + 288);

  int dlo = sdot4(nib.x & 0x0F0F0F0Fu, alo.x, 0);
  dlo = sdot4(nib.y & 0x0F0F0F0Fu, alo.y, dlo);
  dlo = sdot4(nib.z & 0x0F0F0F0Fu, alo.z, dlo);
  dlo = sdot4(nib.w & 0x0F0F0F0Fu, alo.w, dlo);
  int dhi = sdot4((nib.x >> 4) & 0x0F0F0F0Fu, ahi.x, 0);
  dhi = sdot4((nib.y >> 4) & 0x0F0F0F0Fu, ahi.y, dhi);
  dhi = sdot4((nib.z >> 4) & 0x0F0F0F0Fu, ahi.z, dhi);
  dhi = sdot4((nib.w >> 4) & 0x0F0F0F0Fu, ahi.w, dhi);

  // Header: bytes 4..7 (h1) hold sc0..3 in bits 0-5 and the top bits of
  // sc4..7 in bits 6-7; bytes 8..11 (h2) the same for the mins; bytes 12..15
  // (h3) the low nibbles of sc4..7 and m4..7.
  const uint32_t h1 = hdr.y, h2 = hdr.z, h3 = hdr.w;
  const uint32_t sc_lo = h1 & 0x3F3F3F3Fu;
  const uint32_t m_lo = h2 & 0x3F3F3F3Fu;
  const uint32_t sc_hi = (h3 & 0x0F0F0F0Fu) | ((h1 >> 2) & 0x30303030u);
  const uint32_t m_hi = ((h3 >> 4) & 0x0F0F0F0Fu) | ((h2 >> 2) & 0x30303030u);
  const uint32_t scw = (sc_hi & L.selhi) | (sc_lo & ~L.selhi);
  const uint32_t mw = ((m_hi & L.selhi) | (m_lo & ~L.selhi)) & L.mmask;
  const int sc0 = (scw >> L.shift) & 0xFF;
  const int sc1 = (scw >> (L.shift + 8)) & 0xFF;
  const int m0 = (mw >> L.shift) & 0xFF;
  const int m1 = (mw >> (L.shift + 8)) & 0xFF;

  const int S = __mul24(sc0, dlo) + __mul24(sc1, dhi);
  const int M = __mul24(m0, sums.x) + __mul24(m1, sums.y);
  const float d = half_bits_to_float(hdr.x & 0xFFFFu);
  const float dmin = half_bits_to_float(hdr.x >> 16);
  return xs * (d * static_cast<float>(S) - dmin * static_cast<float>(M));
}

// The same contribution split in two for several tokens against one weight
// chunk: the weight side (nibbles and header decode) once, then per token the
// integer dots and the one float pass, in the same order and form as
// unit_partial, so each token gets the bits unit_partial gives it.
struct ChunkDecode {
  uint4 nib;
  int sc0, sc1, m0, m1;
  float d, dmin;
};

__device__ __forceinline__ ChunkDecode chunk_decode(const uint4 nib, const uint4 hdr,
                                                    const LaneGeom& L) {
  ChunkDecode c;
  c.nib = nib;
  const uint32_t h1 = hdr.y, h2 = hdr.z, h3 = hdr.w;
  const uint32_t sc_lo = h1 & 0x3F3F3F3Fu;
  const uint32_t m_lo = h2 & 0x3F3F3F3Fu;
  const uint32_t sc_hi = (h3 & 0x0F0F0F0Fu) | ((h1 >> 2) & 0x30303030u);
  const uint32_t m_hi = ((h3 >> 4) & 0x0F0F0F0Fu) | ((h2 >> 2) & 0x30303030u);
  const uint32_t scw = (sc_hi & L.selhi) | (sc_lo & ~L.selhi);
  const uint32_t mw = ((m_hi & L.selhi) | (m_lo & ~L.selhi)) & L.mmask;
  c.sc0 = (scw >> L.shift) & 0xFF;
  c.sc1 = (scw >> (L.shift + 8)) & 0xFF;
  c.m0 = (mw >> L.shift) & 0xFF;
  c.m1 = (mw >> (L.shift + 8)) & 0xFF;
  c.d = half_bits_to_float(hdr.x & 0xFFFFu);
  c.dmin = half_bits_to_float(hdr.x >> 16);
  return c;
}

// One token's share of a decoded chunk, from the lane's slice of that token's
// q8_K block: its two 16-byte code pieces, the two sub-block sums and the
// block scale.
struct TokenSlice {
  uint4 alo, ahi;
  int2 sums;
  float xs;
};

__device__ __forceinline__ TokenSlice token_slice(const uint8_t* act, int b, const LaneGeom& L) {
  const uint8_t* xb = act + b * kQ8KBytes;
  TokenSlice t;
  t.alo = *reinterpret_cast<const uint4*>(xb + 64 * L.g + 16 * L.h);
  t.ahi = *reinterpret_cast<const uint4*>(xb + 64 * L.g + 32 + 16 * L.h);
  t.sums = *reinterpret_cast<const int2*>(xb + 256 + 8 * L.g);
  t.xs = *reinterpret_cast<const float*>(xb + 288);
  return t;
}

__device__ __forceinline__ float chunk_token_slice(const ChunkDecode& c, const TokenSlice& t) {
  const uint4 alo = t.alo, ahi = t.ahi;
  const int2 sums = t.sums;
  const float xs = t.xs;
  const uint4 nib = c.nib;
  int dlo = sdot4(nib.x & 0x0F0F0F0Fu, alo.x, 0);
  dlo = sdot4(nib.y & 0x0F0F0F0Fu, alo.y, dlo);
  dlo = sdot4(nib.z & 0x0F0F0F0Fu, alo.z, dlo);
  dlo = sdot4(nib.w & 0x0F0F0F0Fu, alo.w, dlo);
  int dhi = sdot4((nib.x >> 4) & 0x0F0F0F0Fu, ahi.x, 0);
  dhi = sdot4((nib.y >> 4) & 0x0F0F0F0Fu, ahi.y, dhi);
  dhi = sdot4((nib.z >> 4) & 0x0F0F0F0Fu, ahi.z, dhi);
  dhi = sdot4((nib.w >> 4) & 0x0F0F0F0Fu, ahi.w, dhi);
  const int S = __mul24(c.sc0, dlo) + __mul24(c.sc1, dhi);
  const int M = __mul24(c.m0, sums.x) + __mul24(c.m1, sums.y);
  return xs * (c.d * static_cast<float>(S) - c.dmin * static_cast<float>(M));
}

__device__ __forceinline__ float chunk_token(const ChunkDecode& c, const uint8_t* act, int b,
                                             const LaneGeom& L) {
  return chunk_token_slice(c, token_slice(act, b, L));
}

}  // namespace xq
