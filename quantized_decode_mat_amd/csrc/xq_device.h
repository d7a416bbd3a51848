// xq_device.h — device helpers shared by the gfx950 kernels of libxq.
//
// Everything here assumes a 64-lane wavefront (CDNA4). Cross-lane sums use
// DPP moves inside each 16-lane row and then read the four row results with
// v_readlane; no LDS tree is used ("25 — Writing XPU Kernels", section 25.2.1:
// the wave's own reduction, then one lane stores).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace xq {

constexpr int kWave = 64;
constexpr int kQ8KBytes = 320;   // q8_K block: 256 codes, 8 int32 sums, f32 scale, pad
constexpr int kQ4KBytes = 144;   // Q4_K block: f16 d, f16 dmin, 12 B scales, 128 B nibbles

// DPP control words (GCN/CDNA encoding).
constexpr int kDppQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i of each 8-lane half reads lane 7-i
constexpr int kDppRowMirror = 0x140;     // lane i of each 16-lane row reads lane 15-i

template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __builtin_bit_cast(float, dpp<CTRL>(__builtin_bit_cast(int, v)));
}

// Sum over the 16 lanes of each row; every lane of the row receives it.
__device__ __forceinline__ float row16_sum(float v) {
  v += dppf<kDppQuadSwap1>(v);
  v += dppf<kDppQuadSwap2>(v);
  v += dppf<kDppRowHalfMirror>(v);
  v += dppf<kDppRowMirror>(v);
  return v;
}

__device__ __forceinline__ float readlane(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over the whole wave; the result is wave-uniform.
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (readlane(v, 0) + readlane(v, 16)) + (readlane(v, 32) + readlane(v, 48));
}

// Max over the whole wave; the result is wave-uniform.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dppf<kDppQuadSwap1>(v));
  v = fmaxf(v, dppf<kDppQuadSwap2>(v));
  v = fmaxf(v, dppf<kDppRowHalfMirror>(v));
  v = fmaxf(v, dppf<kDppRowMirror>(v));
  return fmaxf(fmaxf(readlane(v, 0), readlane(v, 16)), fmaxf(readlane(v, 32), readlane(v, 48)));
}

// Integer sum over each aligned group of 8 lanes; every lane of the group
// receives it.
__device__ __forceinline__ int lane8_sum(int v) {
  v += dpp<kDppQuadSwap1>(v);
  v += dpp<kDppQuadSwap2>(v);
  v += dpp<kDppRowHalfMirror>(v);
  return v;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
  return __half2float(__ushort_as_half(static_cast<unsigned short>(bits16)));
}

// Signed 4 x int8 dot with int32 accumulate (v_dot4_i32_i8).
__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot4(static_cast<int>(a), static_cast<int>(b), c, false);
}

}  // namespace xq
