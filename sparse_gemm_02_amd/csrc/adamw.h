// AdamW arithmetic on one stored value (device side).  The update is Adam with
// bias-corrected moments and weight decay decoupled from the gradient
// (Loshchilov and Hutter, "Decoupled Weight Decay Regularization"), in the
// common form where the learning rate scales both the decay and the step; the
// SLoPe discussion page ("Choice of Optimizer") trains with AdamW and keeps two
// fp32 moments per stored non-zero ("Memory Footprint").
#pragma once
#include "common.h"
#include "launch.h"

namespace slope {

// p, g: the value and its gradient; m, v: the moments, updated.  Returns the
// new value in fp32 (the caller rounds it once to its storage format).  The
// operation sequence is fixed (explicit fused multiply-adds, no other
// contraction), so every kernel that inlines it rounds the same way.
__device__ __forceinline__ float adamw_apply(float p, float g, float& m, float& v, const AdamWStep& c) {
#pragma clang fp contract(off)
  m = __builtin_fmaf(c.beta1, m, c.omb1 * g);
  v = __builtin_fmaf(c.beta2, v, c.omb2 * (g * g));
  const float den = __builtin_fmaf(__builtin_sqrtf(v), c.inv_sqrt_bc2, c.eps);
  return __builtin_fmaf(-c.step_size, m / den, p * c.decay);
}

// Eight consecutive gradient values as fp32 (bf16 bits or fp32; 16-byte aligned).
__device__ __forceinline__ void load8_f32(const uint16_t* p, float out[8]) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8_f32(const _Float16* p, float out[8]) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = f16_bits_to_f32((uint16_t)(w[i] & 0xFFFFu));
    out[2 * i + 1] = f16_bits_to_f32((uint16_t)(w[i] >> 16));
  }
}
__device__ __forceinline__ void load8_f32(const float* p, float out[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[i] = a[i];
    out[4 + i] = b[i];
  }
}
__device__ __forceinline__ void store8_f32(float* p, const float in[8]) {
  *reinterpret_cast<f32x4*>(p) = f32x4{in[0], in[1], in[2], in[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{in[4], in[5], in[6], in[7]};
}

// AdamW on eight consecutive 16-bit values (bf16, or fp16 with H) held as
// four words of pairs (low half first); g, m, v point at the matching eight
// gradient / moment entries.
template <bool H, typename GT>
__device__ __forceinline__ u32x4 adamw8_16(u32x4 w, const GT* g, float* m, float* v, const AdamWStep& c) {
  typedef Fmt16<H> F;
  float gf[8], mf[8], vf[8];
  load8_f32(g, gf);
  load8_f32(m, mf);
  load8_f32(v, vf);
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = adamw_apply(F::to_f32((uint16_t)(w[i] & 0xFFFFu)), gf[2 * i], mf[2 * i], vf[2 * i], c);
    const float hi = adamw_apply(F::to_f32((uint16_t)(w[i] >> 16)), gf[2 * i + 1], mf[2 * i + 1], vf[2 * i + 1], c);
    out[i] = (uint32_t)F::from_f32(lo) | ((uint32_t)F::from_f32(hi) << 16);
  }
  store8_f32(m, mf);
  store8_f32(v, vf);
  return out;
}

}  // namespace slope
