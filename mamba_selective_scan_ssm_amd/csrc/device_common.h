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

}  // namespace ssm
