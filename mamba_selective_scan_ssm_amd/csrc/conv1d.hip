// Short causal convolution ahead of the scan, for gfx950.
//
// What is computed ("ggml : add GPU support for Mamba models", llama.cpp
// issue 6758: the SSM_CONV op ggml_ssm_conv(s, x, c) with the state s holding
// the d_conv - 1 previous inputs of each channel, the weights c {d_conv,
// d_inner}, the ssm_conv1d_b bias; "Clean up SSM ops directory structure -
// #6444": causal_conv1d_update for the single-token step): per (b, d) with
// the padded window xp = [state, x],
//   y_t = act(sum_k w[d][k] xp[t + k] + bias[d]),  act = identity or SiLU,
// and the new state is the last K - 1 entries of xp.
//
// Layout: x, y (B, L, D); w (D, K); bias (D); state (B, D, K-1), oldest
// first.  The convolution has no recurrence, so the prefill kernel cuts L
// into segments processed independently; a segment re-reads the K - 1 rows
// before it (the halo) or, for the first segment, the carried state.  Each
// lane owns one channel, so a wave's load or store of one token row is one
// contiguous 64-channel run.
#include "device_common.h"
#include "launch.h"

namespace ssm {
namespace {

constexpr int kConvThreads = 256;   // channels per workgroup
constexpr int kConvSeg = 64;        // tokens per segment
constexpr int kConvBatch = 16;      // token rows loaded ahead

template <typename T>
__device__ __forceinline__ float conv_ld(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  if constexpr (sizeof(T) == 2) {
    return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(
                               r, static_cast<int>(voff), static_cast<int>(soff), 0))
                           << 16);
  } else {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(voff),
                                                                static_cast<int>(soff), 0));
  }
}

template <typename T>
__device__ __forceinline__ void conv_st(float v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  if constexpr (sizeof(T) == 2) {
    __builtin_amdgcn_raw_buffer_store_b16(from_f32<bf16_t>(v).bits, r, static_cast<int>(voff),
                                          static_cast<int>(soff), 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, static_cast<int>(voff),
                                          static_cast<int>(soff), 0);
  }
}

// Grid: x = 256-channel tile, y = segment of kConvSeg tokens, z = b.
template <typename T, int K, bool ACT>
__global__ __launch_bounds__(kConvThreads) void conv1d_fwd_kernel(ConvArgs a) {
  const int64_t D = a.D, L = a.L;
  const int64_t d_raw = static_cast<int64_t>(blockIdx.x) * kConvThreads + threadIdx.x;
  const bool active = d_raw < D;
  const int64_t d = active ? d_raw : D - 1;
  const int64_t b = blockIdx.z;
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * kConvSeg;
  const int64_t t1 = (t0 + kConvSeg < L) ? t0 + kConvSeg : L;
  constexpr uint32_t kES = sizeof(T);

  float w[K];
#pragma unroll
  for (int k = 0; k < K; ++k) w[k] = a.w[d * K + k];
  const float bias = a.bias ? a.bias[d] : 0.f;

  const int64_t plane = L * D * kES;
  auto rsrc = [&](const void *p) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(static_cast<const char *>(p)) + b * plane,
                                             0, static_cast<int>(plane), 0x00020000);
  };
  const __amdgpu_buffer_rsrc_t rx = rsrc(a.x), ry = rsrc(a.y);
  const uint32_t voff = static_cast<uint32_t>(d * kES);
  const uint32_t row = static_cast<uint32_t>(D * kES);

  // window of the K - 1 inputs before t0: x rows, or the carried state
  float win[K];
#pragma unroll
  for (int j = 0; j < K - 1; ++j) {
    const int64_t t = t0 - (K - 1) + j;
    if (t >= 0) {
      win[j] = conv_ld<T>(rx, voff, static_cast<uint32_t>(t) * row);
    } else {
      win[j] = a.state_in ? a.state_in[(b * D + d) * (K - 1) + (K - 1) + t] : 0.f;
    }
  }

  for (int64_t tb = t0; tb < t1; tb += kConvBatch) {
    float xv[kConvBatch];
#pragma unroll
    for (int i = 0; i < kConvBatch; ++i)  // rows past L read 0 (range check)
      xv[i] = conv_ld<T>(rx, voff, static_cast<uint32_t>(tb + i) * row);
#pragma unroll
    for (int i = 0; i < kConvBatch; ++i) {
      win[K - 1] = xv[i];
      float v = 0.f;
#pragma unroll
      for (int k = 0; k < K; ++k) v = fmaf(w[k], win[k], v);
      v += bias;
      if (ACT) v *= __builtin_amdgcn_rcpf(1.0f + fast_exp2(-v * kLog2e));
      if (active && tb + i < t1) conv_st<T>(v, ry, voff, static_cast<uint32_t>(tb + i) * row);
#pragma unroll
      for (int k = 0; k + 1 < K; ++k) win[k] = win[k + 1];
    }
  }
}

// New state: the last K - 1 entries of [state_in, x] per (b, d).
template <typename T, int K>
__global__ __launch_bounds__(256) void conv1d_state_kernel(ConvArgs a) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= a.B * a.D) return;
  const int64_t b = i / a.D, d = i % a.D;
  const T *x = static_cast<const T *>(a.x);
#pragma unroll
  for (int j = 0; j < K - 1; ++j) {
    const int64_t t = a.L - (K - 1) + j;
    float v;
    if (t >= 0) v = to_f32(x[(b * a.L + t) * a.D + d]);
    else v = a.state_in ? a.state_in[i * (K - 1) + (K - 1) + t] : 0.f;
    a.state_out[i * (K - 1) + j] = v;
  }
}

// One decode step per (s, d): window [state, x], state shifted in place.
template <typename T, int K, bool ACT>
// grid (channel blocks, sequences): no index division; the bias is read
// unconditionally (from w when absent) so no load sits behind a branch
__global__ __launch_bounds__(256) void conv1d_update_kernel(ConvArgs a) {
  const int64_t d = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (d >= a.D) return;
  const int64_t i = static_cast<int64_t>(blockIdx.y) * a.D + d;
  float *st = a.state_out + i * (K - 1);
  const float bv = (a.bias ? a.bias : a.w)[d];
  float win[K];
#pragma unroll
  for (int k = 0; k < K - 1; ++k) win[k] = st[k];
  win[K - 1] = to_f32(static_cast<const T *>(a.x)[i]);
  float v = 0.f;
#pragma unroll
  for (int k = 0; k < K; ++k) v = fmaf(a.w[d * K + k], win[k], v);
  v += a.bias ? bv : 0.f;
  if (ACT) v *= __builtin_amdgcn_rcpf(1.0f + fast_exp2(-v * kLog2e));
  static_cast<T *>(a.y)[i] = from_f32<T>(v);
#pragma unroll
  for (int k = 0; k < K - 1; ++k) st[k] = win[k + 1];
}

template <typename T, int K>
hipError_t launch_fwd_k(const ConvArgs &a, hipStream_t s) {
  if (a.L > 0) {
    dim3 grid(static_cast<unsigned>((a.D + kConvThreads - 1) / kConvThreads),
              static_cast<unsigned>((a.L + kConvSeg - 1) / kConvSeg), static_cast<unsigned>(a.B));
    if (a.act)
      conv1d_fwd_kernel<T, K, true><<<grid, kConvThreads, 0, s>>>(a);
    else
      conv1d_fwd_kernel<T, K, false><<<grid, kConvThreads, 0, s>>>(a);
  }
  if (a.state_out) {
    const int64_t n = a.B * a.D;
    conv1d_state_kernel<T, K><<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

template <typename T, int K>
hipError_t launch_update_k(const ConvArgs &a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((a.D + 255) / 256), static_cast<unsigned>(a.B));
  if (a.act)
    conv1d_update_kernel<T, K, true><<<grid, 256, 0, s>>>(a);
  else
    conv1d_update_kernel<T, K, false><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

template <typename T, bool UPDATE>
hipError_t dispatch_k(const ConvArgs &a, hipStream_t s) {
  switch (a.K) {
#define SSM_CONV_CASE(KV) \
  case KV: return UPDATE ? launch_update_k<T, KV>(a, s) : launch_fwd_k<T, KV>(a, s);
    SSM_CONV_CASE(2) SSM_CONV_CASE(3) SSM_CONV_CASE(4) SSM_CONV_CASE(5)
    SSM_CONV_CASE(6) SSM_CONV_CASE(7) SSM_CONV_CASE(8)
#undef SSM_CONV_CASE
    default: return hipErrorNotSupported;
  }
}

}  // namespace

hipError_t launch_conv1d_fwd(const ConvArgs &a, hipStream_t s) {
  if (a.dt == DType::BF16) return dispatch_k<bf16_t, false>(a, s);
  return dispatch_k<float, false>(a, s);
}

hipError_t launch_conv1d_update(const ConvArgs &a, hipStream_t s) {
  if (a.dt == DType::BF16) return dispatch_k<bf16_t, true>(a, s);
  return dispatch_k<float, true>(a, s);
}

}  // namespace ssm
