// Decode step (selective_state_update in "Clean up SSM ops directory
// structure - #6444"): the scan body for T >= 1 tokens per sequence with the
// state (S or pool rows, D, N) fp32 read once, carried in registers over the
// T tokens, and written back in place.
//
// The step is HBM-bound on the state (read + write of S*D*N fp32), so the
// layout is chosen for the state stream: a channel's N states are N/4 lanes
// holding four consecutive states each, so one 16-byte load per lane covers
// the state tensor contiguously across the wave.  The y contraction over n is
// finished with DPP sums over those N/4 lanes.  The single-token step
// gives each thread one channel of two sequences: the channel's A row (read
// by every sequence) is loaded once for both, and all loads of the thread
// are issued before any is used, so a wave keeps twice the state bytes in
// flight (the step is bound by how many bytes are in flight, not by the
// instruction stream).  Optional inputs (gate, skip, step bias) are read
// unconditionally, since a load inside a branch brings a wait that drains
// every load before it.  Sizes this layout does not
// cover (N not a multiple of 4, or a state/A not 16-byte aligned) go to the
// per-lane scan kernel with L = T, whose lanes read and then write only their
// own state row.
#include "device_common.h"
#include "launch.h"

namespace ssm {
namespace {

constexpr int kBlock = 256;

// four consecutive B or C values of a lane: one 8- (bf16) or 16-byte (fp32)
// load when the rows are aligned (V), else four element loads
template <typename T, bool V>
__device__ __forceinline__ void load4(const T *p, float *v) {
  if constexpr (V && sizeof(T) == 2) {
    const uint2 u = *reinterpret_cast<const uint2 *>(p);
    v[0] = __uint_as_float(u.x << 16);
    v[1] = __uint_as_float(u.x & 0xffff0000u);
    v[2] = __uint_as_float(u.y << 16);
    v[3] = __uint_as_float(u.y & 0xffff0000u);
  } else if constexpr (V) {
    const float4 f = *reinterpret_cast<const float4 *>(p);
    v[0] = f.x;
    v[1] = f.y;
    v[2] = f.z;
    v[3] = f.w;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = to_f32(p[j]);
  }
}

// Sum over the LPC adjacent lanes of a channel, every lane getting it, with
// DPP moves on the VALU (quad permutations, then mirrors within half rows
// and rows) rather than lane shuffles through the LDS unit.
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, true));
}
template <int LPC>
__device__ __forceinline__ float lane_group_sum(float v) {
  if constexpr (LPC >= 2) v += dpp_mov<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  if constexpr (LPC >= 4) v += dpp_mov<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  if constexpr (LPC >= 8) v += dpp_mov<0x141>(v);  // lane i <- 7 - i of the half row
  if constexpr (LPC >= 16) v += dpp_mov<0x140>(v); // lane i <- 15 - i of the row
  return v;
}

// LPC = lanes per channel (N / 4).  TT = tokens whose inputs are loaded
// together before any of them is computed (1 for the single-token step).
template <typename T, int LPC, int TT, bool BCV>
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
  // optional inputs read unconditionally (from A, or x, when absent): a load
  // in a branch would bring a wait that drains the loads issued before it
  const float bv0 = (a.delta_bias ? a.delta_bias : a.A)[d];
  const float bias = a.delta_bias ? bv0 : 0.f;
  const float skp = (a.D_skip ? a.D_skip : a.A)[d];
  const T *zsrc = zp ? zp : xp;
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
      zv[k] = to_f32(zsrc[tok * D + d]);
      load4<T, BCV>(Bp + tok * N + 4 * q, bv[k]);
      load4<T, BCV>(Cp + tok * N + 4 * q, cv[k]);
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
      acc = lane_group_sum<LPC>(acc);
      if (active && q == 0) {
        float v = acc;
        if (a.D_skip) v = fmaf(skp, xv[k], v);
        if (zp) v *= silu(zv[k]);
        static_cast<T *>(a.y)[tok * D + d] = from_f32<T>(v);
      }
    }
  }
  if (!active) return;
  *st = make_float4(h[0], h[1], h[2], h[3]);
}

// Single-token step with SPT sequences per thread for one channel: the
// channel's A row (read by every sequence) is loaded once for the SPT
// sequences, and all loads of the thread are issued before any is used.  A
// sequence whose slot is outside the pool is skipped (its loads are clamped
// to row 0 and nothing is stored).
template <typename T, int LPC, int SPT, bool BCV>
__global__ __launch_bounds__(kBlock) void state_step_seq_kernel(StepArgs a) {
  constexpr int N = 4 * LPC;
  constexpr int kCh = kBlock / LPC;  // channels per block
  const int q = threadIdx.x % LPC;
  const int64_t D = a.D, S = a.S;
  const int64_t d_raw = static_cast<int64_t>(blockIdx.x) * kCh + threadIdx.x / LPC;
  const bool act = d_raw < D;
  const int64_t d = act ? d_raw : D - 1;
  const T *xp = static_cast<const T *>(a.x);
  const T *dp = static_cast<const T *>(a.delta);
  const T *zp = static_cast<const T *>(a.z);
  const T *zsrc = zp ? zp : xp;  // optional inputs read unconditionally (see above)
  const float bv0 = (a.delta_bias ? a.delta_bias : a.A)[d];
  const float skp = (a.D_skip ? a.D_skip : a.A)[d];
  const float4 Av = reinterpret_cast<const float4 *>(a.A + d * N)[q];
  int64_t sq[SPT], row[SPT];
  bool ok[SPT];
  float4 hv[SPT];
  float xv[SPT], dv[SPT], zv[SPT], Bv[SPT][4], Cv[SPT][4];
#pragma unroll
  for (int k = 0; k < SPT; ++k) {
    const int64_t s_raw = static_cast<int64_t>(blockIdx.y) * SPT + k;
    sq[k] = s_raw < S ? s_raw : S - 1;
    ok[k] = s_raw < S;
    row[k] = sq[k];
    if (a.slots != nullptr) {
      const int32_t sl = a.slots[sq[k]];
      ok[k] = ok[k] && sl >= 0 && sl < a.pool_rows;
      row[k] = ok[k] ? sl : 0;
    }
    hv[k] = reinterpret_cast<const float4 *>(a.state + (row[k] * D + d) * N)[q];
    xv[k] = to_f32(xp[sq[k] * D + d]);
    dv[k] = to_f32(dp[sq[k] * D + d]);
    zv[k] = to_f32(zsrc[sq[k] * D + d]);
    load4<T, BCV>(static_cast<const T *>(a.Bm) + sq[k] * N + 4 * q, Bv[k]);
    load4<T, BCV>(static_cast<const T *>(a.Cm) + sq[k] * N + 4 * q, Cv[k]);
  }
  const float Ar[4] = {Av.x, Av.y, Av.z, Av.w};
#pragma unroll
  for (int k = 0; k < SPT; ++k) {
    const float dl = step_size(dv[k], a.delta_bias ? bv0 : 0.f, a.delta_softplus);
    const float u = dl * xv[k];
    float h[4] = {hv[k].x, hv[k].y, hv[k].z, hv[k].w};
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float dA = fast_exp2(dl * (Ar[j] * kLog2e));
      h[j] = fmaf(dA, h[j], u * Bv[k][j]);
      acc = fmaf(Cv[k][j], h[j], acc);
    }
    acc = lane_group_sum<LPC>(acc);
    hv[k] = make_float4(h[0], h[1], h[2], h[3]);
    if (act && ok[k] && q == 0) {
      float v = acc;
      if (a.D_skip) v = fmaf(skp, xv[k], v);
      if (zp) v *= silu(zv[k]);
      static_cast<T *>(a.y)[sq[k] * D + d] = from_f32<T>(v);
    }
  }
#pragma unroll
  for (int k = 0; k < SPT; ++k)
    if (act && ok[k]) reinterpret_cast<float4 *>(a.state + (row[k] * D + d) * N)[q] = hv[k];
}

template <typename T, int LPC, bool BCV>
hipError_t launch_tv(const StepArgs &a, hipStream_t st) {
  constexpr int kCh = kBlock / LPC;
  if (a.T == 1) {
    constexpr int kSPT = 2;
    dim3 gs(static_cast<unsigned>((a.D + kCh - 1) / kCh), static_cast<unsigned>((a.S + kSPT - 1) / kSPT));
    state_step_seq_kernel<T, LPC, kSPT, BCV><<<gs, kBlock, 0, st>>>(a);
  } else {
    dim3 grid(static_cast<unsigned>((a.D + kCh - 1) / kCh), static_cast<unsigned>(a.S));
    state_update_kernel<T, LPC, 4, BCV><<<grid, kBlock, 0, st>>>(a);
  }
  return hipGetLastError();
}

template <typename T, int LPC>
hipError_t launch_t(const StepArgs &a, hipStream_t st) {
  // a lane's 4 B (or C) values start at a multiple of 4 elements: one load
  // when the rows are aligned to 4 elements
  const uintptr_t al = 4 * sizeof(T);
  if (reinterpret_cast<uintptr_t>(a.Bm) % al == 0 && reinterpret_cast<uintptr_t>(a.Cm) % al == 0)
    return launch_tv<T, LPC, true>(a, st);
  return launch_tv<T, LPC, false>(a, st);
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
