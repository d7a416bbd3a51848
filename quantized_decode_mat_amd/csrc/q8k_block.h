// q8k_block.h — one wave quantizes one 256-value block to q8_K.
//
// "25 — Writing XPU Kernels", section 25.2 (integer-route bullet) and section
// 25.2.1: 256 int8 codes at +0, eight int32 sums of 32 codes at +256, the f32
// scale at +288 of a 320-byte block. Lane l holds elements 4l..4l+3. The scale
// is amax/127 and each code x/d, both IEEE f32 divisions (HIP's default
// division is correctly rounded; nothing here is built with fast-math),
// rounded to nearest-even by v_rndne_f32. Shared by the quantize kernel and
// the mat-vec's fused q8_K tail, so both produce the same bytes.
#pragma once

#include "xq_device.h"

namespace xq {

__device__ __forceinline__ int q8k_code(float x, float d) {
  float r = rintf(x / d);
  r = fminf(fmaxf(r, -127.0f), 127.0f);  // never active: |x/d| <= 127*(1+2^-23)
  return static_cast<int>(r);
}

// One lane's share of a block: its four packed codes, the sum of its
// sub-block's 32 codes (valid on lanes 8j), and the block scale.
struct Q8KLane {
  uint32_t packed;
  int32_t sum;
  float d;
};

__device__ __forceinline__ Q8KLane q8k_block_lane(const float4 v) {
  const float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  const float amax = wave_max(a);
  const float d = amax / 127.0f;

  int q0 = 0, q1 = 0, q2 = 0, q3 = 0;
  if (d != 0.0f) {
    q0 = q8k_code(v.x, d);
    q1 = q8k_code(v.y, d);
    q2 = q8k_code(v.z, d);
    q3 = q8k_code(v.w, d);
  }
  Q8KLane o;
  o.packed = (static_cast<uint32_t>(q0) & 0xFFu) | ((static_cast<uint32_t>(q1) & 0xFFu) << 8) |
             ((static_cast<uint32_t>(q2) & 0xFFu) << 16) |
             ((static_cast<uint32_t>(q3) & 0xFFu) << 24);
  o.sum = lane8_sum(q0 + q1 + q2 + q3);  // lanes 8j..8j+7 hold codes 32j..32j+31
  o.d = d;
  return o;
}

// Writes the whole 320-byte block at `out` (global memory or LDS).
__device__ __forceinline__ void q8k_block_wave(const float4 v, uint8_t* out, int lane) {
  const Q8KLane o = q8k_block_lane(v);
  reinterpret_cast<uint32_t*>(out)[lane] = o.packed;
  if ((lane & 7) == 0) reinterpret_cast<int32_t*>(out + 256)[lane >> 3] = o.sum;
  if (lane == 0) *reinterpret_cast<float*>(out + 288) = o.d;
  if (lane >= 1 && lane < 8) reinterpret_cast<uint32_t*>(out + 288)[lane] = 0u;  // 292..319
}

}  // namespace xq
