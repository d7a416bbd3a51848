// gemm_q4k.hip — Q4_K x q8_K small-M product (multi-token prefill) on gfx950.
//
// Y[m][n] = sum_b xs_mb * (d_nb * S_mnb - dmin_nb * M_mnb), with the exact
// int32 block partials S_mnb = sum_k sc_j(k) * q_nk * code_mk and
// M_mnb = sum_k m_j(k) * code_mk over the 256 k of super-block b.
//
// "25 — Writing XPU Kernels", section 25.3: fill the device first, then feed
// the tile; a GEMM that reuses the weight tile across the token block is the
// point of the prefill path. Here the integer products are a dense
// contraction, so they run on int8 MFMA (v_mfma_i32_16x16x64_i8, K = 64 = one
// nibble group = sub-blocks 2g and 2g+1).
//
// One MFMA's K spans two sub-blocks with different 6-bit scales, so the
// scale cannot be applied after the MFMA without splitting K. Instead the
// scale goes into the weight operand, exactly: sc = 8a + b with a, b in 0..7,
// and the two int8 planes a*q and b*q (each <= 105) give S = 8*S_a + S_b.
// The min term is a third plane whose bytes are m_j (<= 63) over sub-block j,
// contracted with the same codes. All three accumulate exactly in int32
// (|S| <= 30.7M, |M| <= 2.1M per block); f32 appears only in the per-block
// epilogue.
//
// Tile: 128 tokens x 128 weight rows per 512-thread workgroup, eight waves as
// 2 (tokens) x 4 (rows), each wave 64 x 32 = 4 x 2 MFMA tiles of 16 x 16. Per
// super-block the workgroup stages the 128 tokens' codes and scales and the
// 128 rows' raw Q4_K blocks in LDS; waves decode their weight fragments from
// LDS into the three planes in registers. Workgroups are laid out so that the
// token tiles sharing one weight tile land on one XCD (one L2).
#include "xq_device.h"
#include "xq_launch.h"

namespace xq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 128;          // tokens per workgroup tile
constexpr int BN = 128;          // weight rows per workgroup tile
constexpr int kThreads = 512;    // 8 waves
constexpr int kActStride = 272;  // 256 codes + 16 B pad: conflict-free 16-B reads
constexpr int kActBytes = BM * kActStride;
constexpr int kXsBytes = BM * 4;
constexpr int kWBytes = BN * kQ4KBytes;
constexpr int kLdsBytes = kActBytes + kXsBytes + kWBytes;

__device__ __forceinline__ uint32_t mul_bytes(uint32_t nib, uint32_t f) {
  // Each byte of `nib` is 0..15 and f <= 7, so no product crosses its byte.
  const u16x2 v = __builtin_bit_cast(u16x2, nib);
  const u16x2 r = v * (u16x2){static_cast<unsigned short>(f), static_cast<unsigned short>(f)};
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ v4i mfma(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(kThreads) void gemm_q4k_kernel(float* __restrict__ y,
                                                            const uint8_t* __restrict__ w,
                                                            const uint8_t* __restrict__ xq,
                                                            int M, int N, int nb, int mtiles,
                                                            int ntiles) {
  __shared__ __align__(16) uint8_t lds[kLdsBytes];
  uint8_t* act = lds;
  float* xs_s = reinterpret_cast<float*>(lds + kActBytes);
  uint8_t* wblk = lds + kActBytes + kXsBytes;

  // Workgroup -> tile. When the tile count is a multiple of the 8 XCDs,
  // XCD x (= id % 8) takes a contiguous run of tiles in which the token tiles
  // of one weight tile are adjacent.
  const int T = mtiles * ntiles;
  int t = blockIdx.x;
  if (T % 8 == 0) t = (blockIdx.x % 8) * (T / 8) + blockIdx.x / 8;
  const int ntile = t / mtiles;
  const int mtile = t % mtiles;
  const int m0 = mtile * BM;
  const int n0 = ntile * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 2;        // 0..1: 64-token half
  const int wn = wave & 3;         // 0..3: 32-row quarter
  const int l16 = lane & 15;
  const int q = lane >> 4;         // k-quarter of an MFMA operand: k = 16q..16q+15

  v4i sa[4][2], sb[4][2], sm[4][2];
  float4 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = make_float4(0.f, 0.f, 0.f, 0.f);

  const v4i zero = {0, 0, 0, 0};

  for (int b = 0; b < nb; ++b) {
    // ---- stage super-block b ----
    for (int i = tid; i < BM * 16; i += kThreads) {
      const int m = i >> 4, c = i & 15;
      const int gm = min(m0 + m, M - 1);
      const uint8_t* src = xq + (static_cast<int64_t>(gm) * nb + b) * kQ8KBytes;
      *reinterpret_cast<uint4*>(act + m * kActStride + 16 * c) =
          *reinterpret_cast<const uint4*>(src + 16 * c);
    }
    for (int i = tid; i < BM; i += kThreads) {
      const int gm = min(m0 + i, M - 1);
      xs_s[i] = *reinterpret_cast<const float*>(xq + (static_cast<int64_t>(gm) * nb + b) *
                                                         kQ8KBytes + 288);
    }
    for (int i = tid; i < BN * 9; i += kThreads) {
      const int n = i / 9, c = i % 9;
      const int gn = min(n0 + n, N - 1);
      const uint8_t* src = w + (static_cast<int64_t>(gn) * nb + b) * kQ4KBytes;
      *reinterpret_cast<uint4*>(wblk + n * kQ4KBytes + 16 * c) =
          *reinterpret_cast<const uint4*>(src + 16 * c);
    }
    __syncthreads();

    // ---- this lane's weight rows: header words ----
    uint32_t sc_lo[2], sc_hi[2], m_lo[2], m_hi[2];
    float dn[2], dminn[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const uint8_t* blk = wblk + (32 * wn + 16 * nt + l16) * kQ4KBytes;
      const uint4 hdr = *reinterpret_cast<const uint4*>(blk);
      const uint32_t h1 = hdr.y, h2 = hdr.z, h3 = hdr.w;
      sc_lo[nt] = h1 & 0x3F3F3F3Fu;
      m_lo[nt] = h2 & 0x3F3F3F3Fu;
      sc_hi[nt] = (h3 & 0x0F0F0F0Fu) | ((h1 >> 2) & 0x30303030u);
      m_hi[nt] = ((h3 >> 4) & 0x0F0F0F0Fu) | ((h2 >> 2) & 0x30303030u);
      dn[nt] = half_bits_to_float(hdr.x & 0xFFFFu);
      dminn[nt] = half_bits_to_float(hdr.x >> 16);
    }

#pragma unroll
    for (int g = 0; g < 4; ++g) {
      // A operands: token rows, codes k = 64g + 16q .. +15.
      v4i a[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        a[mt] = *reinterpret_cast<const v4i*>(act + (64 * wm + 16 * mt + l16) * kActStride +
                                              64 * g + 16 * q);
      // B operands: weight row n, k = 16q..16q+15 of group g. q = 0, 1: low
      // nibbles of group bytes 0..15 / 16..31 (sub-block 2g); q = 2, 3: high
      // nibbles of the same bytes (sub-block 2g+1).
      const int shift = 8 * (2 * (g & 1) + (q >> 1));
      v4i ba[2], bb[2], bm[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const uint8_t* blk = wblk + (32 * wn + 16 * nt + l16) * kQ4KBytes;
        const uint4 raw = *reinterpret_cast<const uint4*>(blk + 16 + 32 * g + 16 * (q & 1));
        const uint32_t hs = (q >> 1) ? 4u : 0u;
        const uint32_t n0w = (raw.x >> hs) & 0x0F0F0F0Fu, n1w = (raw.y >> hs) & 0x0F0F0F0Fu;
        const uint32_t n2w = (raw.z >> hs) & 0x0F0F0F0Fu, n3w = (raw.w >> hs) & 0x0F0F0F0Fu;
        const uint32_t scw = (g < 2) ? sc_lo[nt] : sc_hi[nt];
        const uint32_t mw = (g < 2) ? m_lo[nt] : m_hi[nt];
        const uint32_t sc = (scw >> shift) & 0xFFu;
        const uint32_t mj = (mw >> shift) & 0xFFu;
        const uint32_t fa = sc >> 3, fb = sc & 7u;
        ba[nt] = (v4i){(int)mul_bytes(n0w, fa), (int)mul_bytes(n1w, fa), (int)mul_bytes(n2w, fa),
                       (int)mul_bytes(n3w, fa)};
        bb[nt] = (v4i){(int)mul_bytes(n0w, fb), (int)mul_bytes(n1w, fb), (int)mul_bytes(n2w, fb),
                       (int)mul_bytes(n3w, fb)};
        const int mb = static_cast<int>(__builtin_amdgcn_perm(0u, mj, 0u));
        bm[nt] = (v4i){mb, mb, mb, mb};
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          sa[mt][nt] = mfma(a[mt], ba[nt], g == 0 ? zero : sa[mt][nt]);
          sb[mt][nt] = mfma(a[mt], bb[nt], g == 0 ? zero : sb[mt][nt]);
          sm[mt][nt] = mfma(a[mt], bm[nt], g == 0 ? zero : sm[mt][nt]);
        }
    }

    // ---- per-block epilogue: one float pass per output ----
    // C layout of a 16x16 tile: lane holds column l16, rows 4q..4q+3.
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int mr = 64 * wm + 16 * mt + 4 * q;
      const float x0 = xs_s[mr], x1 = xs_s[mr + 1], x2 = xs_s[mr + 2], x3 = xs_s[mr + 3];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const v4i s = (sa[mt][nt] << 3) + sb[mt][nt];
        const v4i mm = sm[mt][nt];
        const float d = dn[nt], dm = dminn[nt];
        acc[mt][nt].x += x0 * (d * static_cast<float>(s.x) - dm * static_cast<float>(mm.x));
        acc[mt][nt].y += x1 * (d * static_cast<float>(s.y) - dm * static_cast<float>(mm.y));
        acc[mt][nt].z += x2 * (d * static_cast<float>(s.z) - dm * static_cast<float>(mm.z));
        acc[mt][nt].w += x3 * (d * static_cast<float>(s.w) - dm * static_cast<float>(mm.w));
      }
    }
    __syncthreads();
  }

  // ---- store ----
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int n = n0 + 32 * wn + 16 * nt + l16;
      const int mr = m0 + 64 * wm + 16 * mt + 4 * q;
      if (n < N) {
        const float v[4] = {acc[mt][nt].x, acc[mt][nt].y, acc[mt][nt].z, acc[mt][nt].w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (mr + i < M) y[static_cast<int64_t>(mr + i) * N + n] = v[i];
      }
    }
}

}  // namespace

hipError_t launch_gemm_q4k(float* y, const void* w, const void* xq, int64_t M, int64_t N,
                           int64_t K, hipStream_t stream) {
  const int nb = static_cast<int>(K / 256);
  const int mtiles = static_cast<int>((M + BM - 1) / BM);
  const int ntiles = static_cast<int>((N + BN - 1) / BN);
  const int grid = mtiles * ntiles;
  hipLaunchKernelGGL(gemm_q4k_kernel, dim3(grid), dim3(kThreads), 0, stream, y,
                     static_cast<const uint8_t*>(w), static_cast<const uint8_t*>(xq),
                     static_cast<int>(M), static_cast<int>(N), nb, mtiles, ntiles);
  return hipGetLastError();
}

}  // namespace xq
