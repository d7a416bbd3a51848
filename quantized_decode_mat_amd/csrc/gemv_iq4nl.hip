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
// The q8_K activation is staged once per workgroup in LDS.
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

__device__ __forceinline__ float block_partial(const uint4 pay, uint32_t dbits,
                                               const uint8_t* act, int c) {
  const uint8_t* xb = act + (c >> 3) * kQ8KBytes;
  const uint4 a0 = *reinterpret_cast<const uint4*>(xb + (c & 7) * 32);
  const uint4 a1 = *reinterpret_cast<const uint4*>(xb + (c & 7) * 32 + 16);
  const float xs = *reinterpret_cast<const float*>(xb + 288);
  // Byte t of the payload: low nibble = weight t, high nibble = weight t+16.
  int dot = sdot4(lut4(pay.x), a0.x, 0);
  dot = sdot4(lut4(pay.y), a0.y, dot);
  dot = sdot4(lut4(pay.z), a0.z, dot);
  dot = sdot4(lut4(pay.w), a0.w, dot);
  dot = sdot4(lut4(pay.x >> 4), a1.x, dot);
  dot = sdot4(lut4(pay.y >> 4), a1.y, dot);
  dot = sdot4(lut4(pay.z >> 4), a1.z, dot);
  dot = sdot4(lut4(pay.w >> 4), a1.w, dot);
  const float d = half_bits_to_float(dbits);
  return (d * xs) * static_cast<float>(dot);
}

template <int R, int PF>
__global__ __launch_bounds__(kThreads) void gemv_iq4nl_kernel(float* __restrict__ y,
                                                              const uint8_t* __restrict__ w,
                                                              const uint8_t* __restrict__ xq,
                                                              int N, int bpr, int prefix,
                                                              int64_t row_bytes, int nq8) {
  extern __shared__ __align__(16) uint8_t act[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int row0 = (blockIdx.x * kWavesPerGroup + wave) * R;
  const int units = (bpr + kWave - 1) / kWave;

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
  {
    const uint4* src = reinterpret_cast<const uint4*>(xq);
    uint4* dst = reinterpret_cast<uint4*>(act);
    const int n16 = nq8 * (kQ8KBytes / 16);
    for (int i = threadIdx.x; i < n16; i += kThreads) dst[i] = src[i];
  }
  __syncthreads();

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
        for (int r = 0; r < R; ++r) acc[r] += block_partial(pay[r][p], dsc[r][p], act, c);
      }
    }
  }

#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float tot = wave_sum(acc[r]);
    if (lane == 0 && row0 + r < N) y[row0 + r] = tot;
  }
}

template <int R, int PF>
hipError_t launch_rpf(float* y, const uint8_t* w, const uint8_t* xq, int N, int bpr, int prefix,
                      int64_t row_bytes, int nq8, hipStream_t stream) {
  const int waves = (N + R - 1) / R;
  const int grid = (waves + kWavesPerGroup - 1) / kWavesPerGroup;
  const size_t lds = static_cast<size_t>(nq8) * kQ8KBytes;
  hipLaunchKernelGGL((gemv_iq4nl_kernel<R, PF>), dim3(grid), dim3(kThreads), lds, stream, y, w,
                     xq, N, bpr, prefix, row_bytes, nq8);
  return hipGetLastError();
}

template <int R>
hipError_t launch_r(float* y, const uint8_t* w, const uint8_t* xq, int N, int bpr, int prefix,
                    int64_t row_bytes, int nq8, int pf, hipStream_t stream) {
  switch (pf) {
    case 1: return launch_rpf<R, 1>(y, w, xq, N, bpr, prefix, row_bytes, nq8, stream);
    case 2: return launch_rpf<R, 2>(y, w, xq, N, bpr, prefix, row_bytes, nq8, stream);
    case 3: return launch_rpf<R, 3>(y, w, xq, N, bpr, prefix, row_bytes, nq8, stream);
    case 4: return launch_rpf<R, 4>(y, w, xq, N, bpr, prefix, row_bytes, nq8, stream);
    case 5: return launch_rpf<R, 5>(y, w, xq, N, bpr, prefix, row_bytes, nq8, stream);
    case 6: return launch_rpf<R, 6>(y, w, xq, N, bpr, prefix, row_bytes, nq8, stream);
    case 7: return launch_rpf<R, 7>(y, w, xq, N, bpr, prefix, row_bytes, nq8, stream);
    default: return launch_rpf<R, 8>(y, w, xq, N, bpr, prefix, row_bytes, nq8, stream);
  }
}

}  // namespace

hipError_t launch_gemv_iq4nl(float* y, const void* w, const void* xq, int64_t N, int64_t K,
                             hipStream_t stream) {
  const int bpr = static_cast<int>(K / 32);
  const int prefix = ((bpr * 2 + 3) / 4) * 4;
  const int64_t row_bytes = prefix + 16 * static_cast<int64_t>(bpr);
  const int nq8 = static_cast<int>(K / 256);
  const int units = (bpr + kWave - 1) / kWave;
  const int pf = units < 8 ? units : 8;
  const uint8_t* wb = static_cast<const uint8_t*>(w);
  const uint8_t* xb = static_cast<const uint8_t*>(xq);
  const int n = static_cast<int>(N);
  if (units <= 2 && N >= 8192)
    return launch_r<2>(y, wb, xb, n, bpr, prefix, row_bytes, nq8, pf, stream);
  return launch_r<1>(y, wb, xb, n, bpr, prefix, row_bytes, nq8, pf, stream);
}

}  // namespace xq
