// Decode step (selective_state_update in "Clean up SSM ops directory
// structure - #6444"): the scan body for T >= 1 tokens per sequence with the
// state (S or pool rows, D, N) fp32 read once, carried in registers over the
// T tokens, and written back in place.
//
// The step is HBM-bound on the state (read + write of S*D*N fp32), so the
// layout is chosen for the state stream: a channel's N states are N/4 lanes
// holding four consecutive states each, so one 16-byte load per lane covers
// the state tensor contiguously across the wave.  The y contraction over n is
// finished with a butterfly over those N/4 lanes.  The single-token step
// gives each thread two channels whose loads are all issued before either is
// used, so a wave keeps twice the state bytes in flight (the step is bound by
// how many bytes are in flight, not by the instruction stream).  Sizes this
// layout does not
// cover (N not a multiple of 4, or a state/A not 16-byte aligned) go to the
// per-lane scan kernel with L = T, whose lanes read and then write only their
// own state row.
#include "device_common.h"
#include "launch.h"

namespace ssm {
namespace {

constexpr int kBlock = 256;

// LPC = lanes per channel (N / 4).  TT = tokens whose inputs are loaded
// together before any of them is computed (1 for the single-token step).
template <typename T, int LPC, int TT>
__global__ __launch_bounds__(kBlock) void state_update_kernel(StepArgs a) {
  constexpr int N = 4 * LPC;
  constexpr int kCh = kBlock / LPC;  // channels per block
  const int q = threadIdx.x % LPC;
  const int64_t d_raw = static_cast<int64_t>(blockIdx.x) * kCh + threadIdx.x / LPC;
  const int64_t s = blockIdx.y;
  const int64_t D = a.D;
  const int64_t nT = TT == 1 ? 1 : a.T;
  int64_t row = s;  // state row of sequence s
  if (a.slots != nullptr) {
    const int32_t sl = a.slots[s];
    if (sl < 0 || sl >= a.pool_rows) return;  // uniform over the block
    row = sl;
  }
  const bool active = d_raw < D;
  const int64_t d = active ? d_raw : D - 1;
  const T *xp = static_cast<const T *>(a.x);
  const T *dp = static_cast<const T *>(a.delta);
  const T *zp = static_cast<const T *>(a.z);
  const T *Bp = static_cast<const T *>(a.Bm);
  const T *Cp = static_cast<const T *>(a.Cm);

  float4 *st = reinterpret_cast<float4 *>(a.state + (row * D + d) * N) + q;
  const float4 hv = *st;
  const float4 Av = reinterpret_cast<const float4 *>(a.A + d * N)[q];
  const float bias = a.delta_bias ? a.delta_bias[d] : 0.f;
  float h[4] = {hv.x, hv.y, hv.z, hv.w};
  const float Ar[4] = {Av.x, Av.y, Av.z, Av.w};

  for (int64_t t0 = 0; t0 < nT; t0 += TT) {
    // inputs of TT tokens first (indices clamped to the last token, so every
    // load is in bounds), so their latencies overlap
    float xv[TT], dv[TT], zv[TT], bv[TT][4], cv[TT][4];
#pragma unroll
    for (int k = 0; k < TT; ++k) {
      const int64_t tok = s * nT + (t0 + k < nT ? t0 + k : nT - 1);  // row of (S, T, .) inputs
      xv[k] = to_f32(xp[tok * D + d]);
      dv[k] = to_f32(dp[tok * D + d]);
      zv[k] = zp ? to_f32(zp[tok * D + d]) : 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bv[k][j] = to_f32(Bp[tok * N + 4 * q + j]);
        cv[k][j] = to_f32(Cp[tok * N + 4 * q + j]);
      }
    }
#pragma unroll
    for (int k = 0; k < TT; ++k) {
      if (t0 + k >= nT) break;
      const int64_t tok = s * nT + t0 + k;
      const float dl = step_size(dv[k], bias, a.delta_softplus);
      const float u = dl * xv[k];
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float dA = fast_exp2(dl * (Ar[j] * kLog2e));
        h[j] = fmaf(dA, h[j], u * bv[k][j]);
        acc = fmaf(cv[k][j], h[j], acc);
      }
#pragma unroll
      for (int off = LPC / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, LPC);
      if (active && q == 0) {
        float v = acc;
        if (a.D_skip) v = fmaf(a.D_skip[d], xv[k], v);
        if (zp) v *= silu(zv[k]);
        static_cast<T *>(a.y)[tok * D + d] = from_f32<T>(v);
      }
    }
  }
  if (!active) return;
  *st = make_float4(h[0], h[1], h[2], h[3]);
}

// Single-token step with CPT channels per thread: every load of the CPT
// channels (and the sequence's B/C slice, shared by them) is issued before
// any of them is used, so a wave keeps CPT times the state bytes in flight.
template <typename T, int LPC, int CPT>
__global__ __launch_bounds__(kBlock) void state_step_kernel(StepArgs a) {
  constexpr int N = 4 * LPC;
  constexpr int kCh = kBlock / LPC;  // channels per pass of the block
  const int q = threadIdx.x % LPC;
  const int64_t s = blockIdx.y;
  const int64_t D = a.D;
  int64_t row = s;
  if (a.slots != nullptr) {
    const int32_t sl = a.slots[s];
    if (sl < 0 || sl >= a.pool_rows) return;  // uniform over the block
    row = sl;
  }
  const T *xp = static_cast<const T *>(a.x);
  const T *dp = static_cast<const T *>(a.delta);
  const T *zp = static_cast<const T *>(a.z);
  float Bv[4], Cv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    Bv[j] = to_f32(static_cast<const T *>(a.Bm)[s * N + 4 * q + j]);
    Cv[j] = to_f32(static_cast<const T *>(a.Cm)[s * N + 4 * q + j]);
  }
  int64_t d[CPT];
  bool act[CPT];
  float4 hv[CPT], Av[CPT];
  float xv[CPT], dv[CPT], zv[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int64_t dr = (static_cast<int64_t>(blockIdx.x) * CPT + k) * kCh + threadIdx.x / LPC;
    act[k] = dr < D;
    d[k] = act[k] ? dr : D - 1;
    hv[k] = reinterpret_cast<const float4 *>(a.state + (row * D + d[k]) * N)[q];
    Av[k] = reinterpret_cast<const float4 *>(a.A + d[k] * N)[q];
    xv[k] = to_f32(xp[s * D + d[k]]);
    dv[k] = to_f32(dp[s * D + d[k]]);
    zv[k] = zp ? to_f32(zp[s * D + d[k]]) : 0.f;
  }
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const float dl = step_size(dv[k], a.delta_bias ? a.delta_bias[d[k]] : 0.f, a.delta_softplus);
    const float u = dl * xv[k];
    float h[4] = {hv[k].x, hv[k].y, hv[k].z, hv[k].w};
    const float Ar[4] = {Av[k].x, Av[k].y, Av[k].z, Av[k].w};
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float dA = fast_exp2(dl * (Ar[j] * kLog2e));
      h[j] = fmaf(dA, h[j], u * Bv[j]);
      acc = fmaf(Cv[j], h[j], acc);
    }
#pragma unroll
    for (int off = LPC / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, LPC);
    hv[k] = make_float4(h[0], h[1], h[2], h[3]);
    if (act[k] && q == 0) {
      float v = acc;
      if (a.D_skip) v = fmaf(a.D_skip[d[k]], xv[k], v);
      if (zp) v *= silu(zv[k]);
      static_cast<T *>(a.y)[s * D + d[k]] = from_f32<T>(v);
    }
  }
#pragma unroll
  for (int k = 0; k < CPT; ++k)
    if (act[k]) reinterpret_cast<float4 *>(a.state + (row * D + d[k]) * N)[q] = hv[k];
}

template <typename T, int LPC>
hipError_t launch_t(const StepArgs &a, hipStream_t st) {
  constexpr int kCh = kBlock / LPC;
  dim3 grid(static_cast<unsigned>((a.D + kCh - 1) / kCh), static_cast<unsigned>(a.S));
  if (a.T == 1) {
#ifndef SSM_STEP_CPT
#define SSM_STEP_CPT 2
#endif
    constexpr int kCPT = SSM_STEP_CPT;
    dim3 g1(static_cast<unsigned>((a.D + kCPT * kCh - 1) / (kCPT * kCh)), static_cast<unsigned>(a.S));
    state_step_kernel<T, LPC, kCPT><<<g1, kBlock, 0, st>>>(a);
  } else
    state_update_kernel<T, LPC, 4><<<grid, kBlock, 0, st>>>(a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dt(const StepArgs &a, hipStream_t st) {
  switch (a.vec_ok ? a.N : -1) {
    case 4: return launch_t<T, 1>(a, st);
    case 8: return launch_t<T, 2>(a, st);
    case 16: return launch_t<T, 4>(a, st);
    case 32: return launch_t<T, 8>(a, st);
    case 64: return launch_t<T, 16>(a, st);
    default: break;
  }
  // Other N or unaligned rows: the per-lane scan over the T tokens, the
  // state as both h0 and h_final (each lane reads its row before writing it).
  ScanArgs sa{};
  sa.B = a.S;
  sa.L = a.T;
  sa.D = a.D;
  sa.N = a.N;
  sa.dt = a.dt;
  sa.x = a.x;
  sa.delta = a.delta;
  sa.A = a.A;
  sa.Bm = a.Bm;
  sa.Cm = a.Cm;
  sa.D_skip = a.D_skip;
  sa.z = a.z;
  sa.h0 = a.state;
  sa.y = a.y;
  sa.h_final = a.state;
  sa.delta_bias = a.delta_bias;
  sa.delta_softplus = a.delta_softplus;
  sa.slots = a.slots;
  sa.pool_rows = a.pool_rows;
  return launch_scan_lane(sa, st);
}

}  // namespace

hipError_t launch_state_update(const StepArgs &a, hipStream_t st) {
  if (a.dt == DType::BF16) return launch_dt<bf16_t>(a, st);
  return launch_dt<float>(a, st);
}

}  // namespace ssm
