// Device helpers shared by the gfx950 selective-scan kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;

// bf16 storage: the payload is the high half of an fp32 word.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v.bits) << 16);
}

// fp32 -> storage type; bf16 rounds to nearest even (v_cvt_pk_bf16_f32).
template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) {
  __bf16 b = static_cast<__bf16>(v);
  bf16_t r;
  r.bits = __builtin_bit_cast(uint16_t, b);
  return r;
}

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// silu(z) = z * sigmoid(z) = z / (1 + e^-z).  For z -> -inf, e^-z -> inf and
// the reciprocal goes to 0, giving -0; for z -> +inf it gives z.
__device__ __forceinline__ float silu(float z) {
  float e = fast_exp2(-z * kLog2e);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// Step size as the recurrence uses it: delta + bias, then (if asked)
// softplus(v) = log(1 + e^v) = max(v, 0) + log1p(e^-|v|).  log1p(w) is
// log(1 + w) corrected for the rounding of 1 + w: log(u) * w / (u - 1) with
// u = 1 + w (or w itself when u rounds to 1), which stays accurate for the
// small w of large |v|.
__device__ __forceinline__ float step_size(float v, float bias, bool softplus) {
  v += bias;
  if (softplus) {
    constexpr float kLn2 = 0.6931471805599453f;
    const float w = fast_exp2(-fabsf(v) * kLog2e);
    const float u = 1.0f + w;
    const float um1 = u - 1.0f;
    const float lp = um1 == 0.f ? w : __builtin_amdgcn_logf(u) * kLn2 * (w / um1);
    v = fmaxf(v, 0.f) + lp;
  }
  return v;
}

}  // namespace ssm
