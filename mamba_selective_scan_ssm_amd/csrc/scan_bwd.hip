// Backward of the selective scan, for gfx950.
//
// What is computed ("Adding Initial Value Support to Selective Scan Forward
// Kernel", state-spaces/mamba issue 285, the replies on the backward kernel:
// the states are recomputed by a forward scan, their gradients are carried
// backwards by a reverse scan fed with dy * C, and the gradient of the
// initial state is exp(delta_0 A) times the carried gradient at the first
// token).  With u = delta x, a = exp(delta A), h_t = a_t h_{t-1} + u_t B_t,
// q_t = sum_n C_t h_t + D x_t, y_t = q_t silu(z_t) and g_t = dy_t silu(z_t):
//   lam_t    = g_t C_t + a_{t+1} lam_{t+1}      (lam after the last token = dh_final)
//   ddelta_t = sum_n lam_t (A a_t h_{t-1} + B_t x_t), times sigmoid(delta + bias)
//              when the step size went through softplus
//   dx_t     = delta_t sum_n lam_t B_t + D g_t,   dz_t = dy_t q_t silu'(z_t)
//   dB_t     = sum_d lam_t delta_t x_t,           dC_t = sum_d g_t h_t
//   dA       = sum_{b,t} lam_t delta_t a_t h_{t-1},  dD = sum g x,  dbias = sum ddelta
//   dh0      = a_0 lam_0.
//
// Schedule.  A lane holds 4 consecutive states of a channel (N/4 lanes per
// channel, as in the decode step) and a workgroup 1024/N channels of one
// sequence.  Pass 1 runs the recurrence forward and writes the state that
// enters every 8-token segment to the workspace (skipped when the forward
// saved those states).  Pass 2 walks the segments
// backwards: it reloads a segment's entering state, recomputes the
// segment's 8 states into registers, then runs the reverse recurrence over
// them.  A segment's inputs are loaded by the whole workgroup one segment
// ahead (coalesced over channels, kept as raw bits until they are staged,
// with no load behind a branch, so the loads stay in flight through the
// current segment), converted once, and staged in LDS with the gate and
// step-size factors already applied; its per-token outputs go back through
// LDS to coalesced buffer stores that every thread issues on every path.  Sums across lanes use DPP: over a
// channel's lanes, and over half the channels of a row of 16 lanes for dB
// and dC, whose partials meet in LDS; the workgroup writes one partial per
// (token, n).  Two small kernels then add the partials of the channel tiles
// (dB, dC) and of the sequences (dA, dD, dbias) in a fixed order, so the
// result does not depend on timing (no atomics).
#include "bwd.h"
#include "device_common.h"

namespace ssm {
namespace {

constexpr int kBwdThreads = 256;
constexpr int kSeg = 8;  // tokens per checkpointed segment

__device__ __forceinline__ float sigmoid_f(float v) {
  return __builtin_amdgcn_rcpf(1.0f + fast_exp2(-v * kLog2e));
}

// Cross-lane moves on the VALU (DPP): quad permutations, row rotations and
// mirrors stay inside a row of 16 lanes.
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, true));
}
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2, 3, 0, 1]
constexpr int kRowMirror = 0x140;     // lane i <- lane 15 - i of the row
constexpr int kRowHalfMirror = 0x141; // lane i <- lane 7 - i of the half row
constexpr int kRowRor = 0x120;        // + m: rotate the row right by m lanes

// sum over the LPC adjacent lanes of a channel (all of them get it)
template <int LPC>
__device__ __forceinline__ float channel_sum(float v) {
  if constexpr (LPC >= 2) v += dpp_f<kQuadXor1>(v);
  if constexpr (LPC >= 4) v += dpp_f<kQuadXor2>(v);
  if constexpr (LPC >= 8) v += dpp_f<kRowHalfMirror>(v);
  if constexpr (LPC >= 16) v += dpp_f<kRowMirror>(v);
  return v;
}

// Partial sum over the channels of a row of 16 lanes for each state slice q
// (lanes LPC apart hold the same q): rotations by LPC, 2 LPC, ... add up a
// cyclic window of half the row's channels, so the lanes of channels 0 and
// R/2 (R = 16 / LPC channels per row) hold two sums that together cover the
// row.  With one channel per row the value is returned as is.
template <int LPC, int M = LPC>
__device__ __forceinline__ float row_half_sum(float v) {
  if constexpr (2 * M < 16) return row_half_sum<LPC, 2 * M>(v + dpp_f<kRowRor + M>(v));
  else return v;
}

__host__ __device__ constexpr int64_t bwd_nseg(int64_t L) { return (L + kSeg - 1) / kSeg; }
// states per lane.  Two per lane at N = 16 doubles the waves but needs 127
// VGPRs and 40 KB of LDS, so only 4 waves per SIMD fit and the 5 per SIMD of
// the 2.8B shape run in two rounds (5.2 ms against 4.1 ms): 4 per lane.
__host__ __device__ constexpr int64_t bwd_spl(int64_t) { return 4; }
__host__ __device__ constexpr int64_t bwd_channels_per_block(int64_t N) {
  return bwd_spl(N) * kBwdThreads / N;
}

// SPL consecutive floats (16- or 8-byte aligned)
template <int SPL>
__device__ __forceinline__ void ld_spl(const float *p, float *v) {
  if constexpr (SPL == 4) {
    const float4 r = *reinterpret_cast<const float4 *>(p);
    v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
  } else {
    const float2 r = *reinterpret_cast<const float2 *>(p);
    v[0] = r.x; v[1] = r.y;
  }
}
// The same, marked non-temporal: for the segment states, each read once
template <int SPL>
__device__ __forceinline__ void ld_spl_nt(const float *p, float *v) {
  using f32x4 = float __attribute__((ext_vector_type(4)));
  using f32x2 = float __attribute__((ext_vector_type(2)));
  if constexpr (SPL == 4) {
    const f32x4 r = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
    v[0] = r[0]; v[1] = r[1]; v[2] = r[2]; v[3] = r[3];
  } else {
    const f32x2 r = __builtin_nontemporal_load(reinterpret_cast<const f32x2 *>(p));
    v[0] = r[0]; v[1] = r[1];
  }
}
template <int SPL>
__device__ __forceinline__ void st_spl(float *p, const float *v) {
  if constexpr (SPL == 4)
    *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
  else
    *reinterpret_cast<float2 *>(p) = make_float2(v[0], v[1]);
}

// Raw inputs of kTok tokens for the workgroup, loaded into registers one
// block ahead.  Thread tid stages channel tid % kCh of the tile at tokens
// tid / kCh + e * LPC (e < kE), and B/C entries tid + e * 256 of the
// block's (kTok, N) rows.  Indices past the sequence or the channel range
// are clamped (their values are never used).
// store of one element through a buffer resource (out-of-range offsets dropped)
template <typename T>
__device__ __forceinline__ void out_st(__amdgpu_buffer_rsrc_t r, int off, float v) {
  if constexpr (sizeof(T) == 2)
    __builtin_amdgcn_raw_buffer_store_b16(from_f32<bf16_t>(v).bits, r, off, 0, 0);
  else
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}

template <typename T, int LPC, int SPL, bool kFull, int kTok = kSeg>
struct SegRegs {
  static constexpr int N = SPL * LPC;
  static constexpr int kCh = kBwdThreads / LPC;
  static constexpr int kE = (kTok * kCh + kBwdThreads - 1) / kBwdThreads;
  static constexpr int kEB = (kTok * N + kBwdThreads - 1) / kBwdThreads;
  // raw bits as loaded (bf16 in the low half): converted where they are
  // staged, so the loads stay in flight until then (a conversion here would
  // wait for them at once)
  uint32_t d[kE], x[kE], z[kFull ? kE : 1], g[kFull ? kE : 1], bb[kEB], cc[kFull ? kEB : 1];

  __device__ __forceinline__ static uint32_t raw(const T &v) {
    if constexpr (sizeof(T) == 2) return v.bits;
    else return __float_as_uint(v);
  }
  __device__ __forceinline__ static float f(uint32_t r) {
    if constexpr (sizeof(T) == 2) return __uint_as_float(r << 16);
    else return __uint_as_float(r);
  }

  __device__ __forceinline__ void load(const BwdArgs &a, int64_t b, int64_t t0, int64_t dst, int tid) {
    const T *xp = static_cast<const T *>(a.x), *dp = static_cast<const T *>(a.delta);
    const T *gp = static_cast<const T *>(a.dy);
    // z read unconditionally (x stands in when there is no gate): a load in
    // a branch brings a wait for every load issued before it
    const T *zp = a.z ? static_cast<const T *>(a.z) : xp;
    const T *Bp = static_cast<const T *>(a.Bm), *Cp = static_cast<const T *>(a.Cm);
    const int64_t L = a.L, D = a.D;
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      const int64_t t = t0 + tid / kCh + e * LPC;
      const int64_t i = (b * L + (t < L ? t : L - 1)) * D + dst;
      d[e] = raw(dp[i]);
      x[e] = raw(xp[i]);
      if constexpr (kFull) {
        z[e] = raw(zp[i]);
        g[e] = raw(gp[i]);
      }
    }
#pragma unroll
    for (int e = 0; e < kEB; ++e) {
      const int idx = (tid + e * kBwdThreads) % (kTok * N);
      const int64_t t = t0 + idx / N;
      const int64_t i = (b * L + (t < L ? t : L - 1)) * N + idx % N;
      bb[e] = raw(Bp[i]);
      if constexpr (kFull) cc[e] = raw(Cp[i]);
    }
  }
};

template <typename T, int LPC, int SPL>
__global__ __launch_bounds__(kBwdThreads, LPC == 4 ? 3 : 1) void scan_bwd_kernel(BwdArgs a) {
  constexpr int N = SPL * LPC;
  constexpr int kCh = kBwdThreads / LPC;        // channels per workgroup
  constexpr int kE = (kSeg * kCh + kBwdThreads - 1) / kBwdThreads;  // staged entries per thread
  constexpr int kEB = (kSeg * N + kBwdThreads - 1) / kBwdThreads;
  static_assert(kBwdThreads % kCh == 0, "a staging thread keeps one channel");
  // staged segment: step size, x, gradient reaching q (dy silu(z)); B, C rows
  __shared__ float s_dl[kSeg][kCh], s_x[kSeg][kCh], s_g[kSeg][kCh];
  __shared__ __attribute__((aligned(16))) float s_B[kSeg][N], s_C[kSeg][N];
  // per (token, channel): dx, ddelta before the softplus slope, q.  Lane q
  // of a channel stores entries q, q + LPC, ... (all its lanes hold the same
  // sums), rows past the third being spare, so the stores take no branch.
  constexpr int kOS = (3 + LPC - 1) / LPC;        // stores per lane and token
  __shared__ float s_o[kOS * LPC][kSeg][kCh];
  constexpr int kRowCh = 16 / LPC;                // channels per row of 16 lanes
  constexpr int kSPR = kRowCh >= 2 ? 2 : 1;       // partial sums per row
  constexpr int kSlots = 16 * kSPR;               // per workgroup
  __shared__ __attribute__((aligned(16))) float s_red[kSlots][kSeg][2 * N];  // [slot][token][B | C sums]
  __shared__ float s_db[kBwdThreads];

  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64, q = tid % LPC;
  const int64_t tile = blockIdx.x, ntile = gridDim.x, b = blockIdx.y;
  const int64_t B = a.B, L = a.L, D = a.D;
  // compute role: channel c of the tile, states 4q..4q+3
  const int c = tid / LPC;
  const int64_t d_raw = tile * kCh + c;
  const bool active = d_raw < D;
  const int64_t d = active ? d_raw : D - 1;
  // staging role: channel cs of the tile, tokens k0 + e * LPC
  const int cs = tid % kCh, k0 = tid / kCh;
  const int64_t ds_raw = tile * kCh + cs;
  const bool s_active = ds_raw < D;
  const int64_t dst = s_active ? ds_raw : D - 1;
  const float bias_s = a.delta_bias ? a.delta_bias[dst] : 0.f;
  const bool has_z = a.z != nullptr;

  const int64_t nseg = bwd_nseg(L);
  float *ck = a.ws;                      // (B, nseg, D, N) entering states
  // (B, L, ntile, 2N) dB|dC partials, after the entering states unless the
  // forward saved them (then the workspace holds no states)
  float *P = ck + (a.h_ckpt ? 0 : B * nseg * D * N);
  // the entering states: from the forward when it saved them, else pass 1
  const float *ckr = a.h_ckpt ? a.h_ckpt : ck;
  float *PA = P + B * L * ntile * 2 * N; // (B, D, N) dA partials
  float *PD = PA + B * D * N;            // (B, D) dD partials
  float *PB = PD + B * D;                // (B, D) dbias partials

  float An[SPL], A2[SPL];
  ld_spl<SPL>(a.A + d * N + SPL * q, An);
#pragma unroll
  for (int j = 0; j < SPL; ++j) A2[j] = An[j] * kLog2e;
  const float Dd = a.D_skip ? a.D_skip[d] : 0.f;

  // ---- pass 1: forward, keeping the state that enters every segment ----
  float h[SPL] = {};
  if (a.h0 != nullptr && active) ld_spl<SPL>(a.h0 + (b * D + d) * N + SPL * q, h);
  if (a.h_ckpt == nullptr) {
    // blocks of kP1 tokens (kM segments) per staging step where the staged
    // block fits in the LDS of the pass-2 partial sums, which pass 1 does
    // not use
    constexpr int kM = (2 * 4 * kSeg * kCh + 4 * kSeg * N) <= kSlots * kSeg * 2 * N ? 4 : 1;
    constexpr int kP1 = kM * kSeg;
    float (*p_dl)[kCh] = kM > 1 ? reinterpret_cast<float (*)[kCh]>(&s_red[0][0][0]) : s_dl;
    float (*p_x)[kCh] = kM > 1 ? p_dl + kP1 : s_x;
    float (*p_B)[N] = kM > 1 ? reinterpret_cast<float (*)[N]>(p_x + kP1) : s_B;
    const int64_t nblk = (L + kP1 - 1) / kP1;
    SegRegs<T, LPC, SPL, false, kP1> r;
    if (nblk > 0) r.load(a, b, 0, dst, tid);
    for (int64_t blk = 0; blk < nblk; ++blk) {
      const int64_t t0 = blk * kP1;
      const int nt = static_cast<int>(L - t0 < kP1 ? L - t0 : kP1);
      __syncthreads();  // the previous block's LDS reads are done
#pragma unroll
      for (int e = 0; e < SegRegs<T, LPC, SPL, false, kP1>::kE; ++e) {
        const int k = k0 + e * LPC;
        if (k < kP1) {  // tokens past L: zeros, as in pass 2
          const bool tok = t0 + k < L;
          p_dl[k][cs] = tok ? step_size(r.f(r.d[e]), bias_s, a.delta_softplus) : 0.f;
          p_x[k][cs] = tok ? r.f(r.x[e]) : 0.f;
        }
      }
#pragma unroll
      for (int e = 0; e < SegRegs<T, LPC, SPL, false, kP1>::kEB; ++e) {
        const int idx = tid + e * kBwdThreads;
        if (idx < kP1 * N) p_B[idx / N][idx % N] = r.f(r.bb[e]);
      }
      if (blk + 1 < nblk) r.load(a, b, t0 + kP1, dst, tid);
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kP1; ++k) {
        if (k % kSeg == 0 && active && k < nt)  // the state entering segment (t0 + k) / kSeg
          st_spl<SPL>(ck + ((b * nseg + (t0 + k) / kSeg) * D + d) * N + SPL * q, h);
        const float dl = p_dl[k][c];
        const float u = dl * p_x[k][c];
        float bv[SPL];
        ld_spl<SPL>(&p_B[k][SPL * q], bv);
#pragma unroll
        for (int j = 0; j < SPL; ++j) h[j] = fmaf(fast_exp2(dl * A2[j]), h[j], u * bv[j]);
      }
    }
  }

  // ---- pass 2: segments in reverse ----
  float lam[SPL] = {};
  if (a.dh_final != nullptr && active) ld_spl<SPL>(a.dh_final + (b * D + d) * N + SPL * q, lam);
  float dAacc[SPL] = {};
  float dDacc = 0.f, dbacc = 0.f;
  SegRegs<T, LPC, SPL, true> r;
  float hck[SPL] = {};
  // (d is clamped, so every lane's address is valid: the loads of the
  // entering states are unconditional, like the inputs')
  if (nseg > 0) {
    r.load(a, b, (nseg - 1) * kSeg, dst, tid);
    ld_spl_nt<SPL>(ckr + ((b * nseg + nseg - 1) * D + d) * N + SPL * q, hck);
  }
  for (int64_t s = nseg - 1; s >= 0; --s) {
    const int64_t t0 = s * kSeg;
    const int nt = static_cast<int>(L - t0 < kSeg ? L - t0 : kSeg);
    float slope[kE], wz[kE];  // softplus slope and dz / q of the staged entries
    __syncthreads();  // the previous segment's LDS reads are done
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      const int k = k0 + e * LPC;
      const float raw = r.f(r.d[e]);
      slope[e] = a.delta_softplus ? sigmoid_f(raw + bias_s) : 1.f;
      const float gv = r.f(r.g[e]);
      float gq = gv, w = 0.f;
      if (has_z) {
        const float zv = r.f(r.z[e]);
        const float sg = sigmoid_f(zv);
        gq = gv * zv * sg;
        w = gv * sg * fmaf(zv, 1.f - sg, 1.f);
      }
      wz[e] = w;
      if (k < kSeg) {
        // tokens past L stage zeros, through which the state and lam pass
        // unchanged (exp(0) = 1, u = g = 0), so the token loops below need no
        // branch; channels past D: no gradient flows
        const bool tok = t0 + k < L;
        s_dl[k][cs] = tok ? step_size(raw, bias_s, a.delta_softplus) : 0.f;
        s_x[k][cs] = tok ? r.f(r.x[e]) : 0.f;
        s_g[k][cs] = tok && s_active ? gq : 0.f;
      }
    }
#pragma unroll
    for (int e = 0; e < kEB; ++e) {
      const int idx = tid + e * kBwdThreads;
      if (idx < kSeg * N) {
        s_B[idx / N][idx % N] = r.f(r.bb[e]);
        s_C[idx / N][idx % N] = r.f(r.cc[e]);
      }
    }
    float H[kSeg + 1][SPL];  // H[k] = state before token t0 + k
    float aS[kSeg][SPL];     // exp(delta A) of token t0 + k
#pragma unroll
    for (int j = 0; j < SPL; ++j) H[0][j] = hck[j];
    if (s > 0) r.load(a, b, t0 - kSeg, dst, tid);
    // the state entering the previous segment, loaded every step (segment 0's
    // again at the last one): with one value per step the loop carries it in
    // the registers it is loaded into, where a merge would need a copy and
    // the copy a wait for every load and store in flight
    ld_spl_nt<SPL>(ckr + ((b * nseg + (s > 0 ? s - 1 : 0)) * D + d) * N + SPL * q, hck);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kSeg; ++k) {
      const float dl = s_dl[k][c];
      const float u = dl * s_x[k][c];
      float bv[SPL];
      ld_spl<SPL>(&s_B[k][SPL * q], bv);
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        aS[k][j] = fast_exp2(dl * A2[j]);
        H[k + 1][j] = fmaf(aS[k][j], H[k][j], u * bv[j]);
      }
    }
#pragma unroll
    for (int k = kSeg - 1; k >= 0; --k) {
      const float dl = s_dl[k][c];
      const float xv = s_x[k][c];
      const float g = s_g[k][c];
      float Bv[SPL], Cv[SPL];
      ld_spl<SPL>(&s_B[k][SPL * q], Bv);
      ld_spl<SPL>(&s_C[k][SPL * q], Cv);
      float qp = 0.f;
#pragma unroll
      for (int j = 0; j < SPL; ++j) qp = fmaf(Cv[j], H[k + 1][j], qp);
      const float qs = fmaf(Dd, xv, channel_sum<LPC>(qp));
      const float u = dl * xv;
      float v[2 * SPL];  // dB then dC contributions of the lane's states
      // ddelta = sum_n lam A a h_prev + x sum_n lam B; the second sum is dx's
      float dda = 0.f, dxp = 0.f;
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        lam[j] = fmaf(g, Cv[j], lam[j]);
        v[j] = lam[j] * u;
        v[SPL + j] = g * H[k + 1][j];
        const float w = lam[j] * (aS[k][j] * H[k][j]);
        dda = fmaf(An[j], w, dda);
        dAacc[j] = fmaf(w, dl, dAacc[j]);
        dxp = fmaf(lam[j], Bv[j], dxp);
        lam[j] *= aS[k][j];
      }
      dxp = channel_sum<LPC>(dxp);
      const float ddl = fmaf(xv, dxp, channel_sum<LPC>(dda));
      {
        const float dxv = fmaf(dl, dxp, Dd * g);
#pragma unroll
        for (int i = 0; i < kOS; ++i) {
          const int row = q + i * LPC;
          s_o[row][k][c] = row == 0 ? dxv : (row == 1 ? ddl : qs);
        }
      }
      dDacc = fmaf(g, xv, dDacc);
      const int rc = (lane % 16) / LPC;  // channel within the row
      if constexpr (LPC == 4) {
        // dB / dC over the row's 4 channels, whose parity alternates: an
        // even channel's lanes add the dB terms of the channel one over
        // (a row rotation by 4 lanes), an odd channel's lanes its dC terms.
        // Either pair of windows covers the row once, so every lane stores
        // one vector of SPL partials and no lane idles in a branch.
        const bool odd = rc & 1;
        float w[SPL];
#pragma unroll
        for (int j = 0; j < SPL; ++j) {
          const float other = odd ? v[j] : v[SPL + j];
          w[j] = (odd ? v[SPL + j] : v[j]) + dpp_f<kRowRor + 4>(other);
        }
        st_spl<SPL>(&s_red[(wave * 4 + lane / 16) * kSPR + rc / 2][k][(odd ? N : 0) + SPL * q], w);
      } else {
        // dB / dC: partial sums over the row's channels, written by the
        // lanes of the row's channels 0 and R/2
#pragma unroll
        for (int i = 0; i < 2 * SPL; ++i) v[i] = row_half_sum<LPC>(v[i]);
        if (rc % (kRowCh / kSPR) == 0) {
          float *dst = &s_red[(wave * 4 + lane / 16) * kSPR + rc / (kRowCh / kSPR)][k][SPL * q];
          st_spl<SPL>(dst, v);
          st_spl<SPL>(dst + N, v + SPL);
        }
      }
      // the scheduler may interleave two tokens; more overlap spills
      if (k % 2 == 0) __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    for (int e = tid; e < nt * 2 * N; e += kBwdThreads) {
      const int k = e / (2 * N), j = e % (2 * N);
      float v = 0.f;
#pragma unroll
      for (int r = 0; r < kSlots; ++r) v += s_red[r][k][j];
      P[((b * L + t0 + k) * ntile + tile) * 2 * N + j] = v;
    }
    // per-token outputs, stored by the staging role (coalesced over channels)
    // through buffer resources over this segment's rows: entries past the
    // segment or the channel range take an offset past the resource and are
    // dropped, and dz's resource is empty without a gate, so every thread
    // issues the same stores on every path (a store count that varies by
    // path makes the compiler wait for every load and store in flight)
    {
      constexpr uint32_t kES = sizeof(T);
      const int64_t row0 = (b * L + t0) * D;
      const int seg_bytes = static_cast<int>(static_cast<int64_t>(nt) * D * kES);
      auto rsrc = [&](void *p, int bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(static_cast<char *>(p) + row0 * kES, 0, bytes, 0x00020000);
      };
      const __amdgpu_buffer_rsrc_t rdx = rsrc(a.dx, seg_bytes), rdd = rsrc(a.ddelta, seg_bytes),
                                   rdz = rsrc(has_z ? a.dz : a.dx, has_z ? seg_bytes : 0);
#pragma unroll
      for (int e = 0; e < kE; ++e) {
        const int k = k0 + e * LPC;
        const bool ok = k < nt && s_active;
        const int kk = k < kSeg ? k : 0;
        const float ddl = s_o[1][kk][cs] * slope[e];
        const int off = ok ? static_cast<int>((static_cast<int64_t>(k) * D + ds_raw) * kES) : 0x7fffffff;
        out_st<T>(rdx, off, s_o[0][kk][cs]);
        out_st<T>(rdd, off, ddl);
        out_st<T>(rdz, off, s_o[2][kk][cs] * wz[e]);
        if (ok) dbacc += ddl;
      }
    }
  }

  // dbias partial of channel cs: the LPC staging threads of a channel add up
  s_db[tid] = dbacc;
  __syncthreads();
  if (tid < kCh && s_active) {
    float v = 0.f;
#pragma unroll
    for (int m = 0; m < LPC; ++m) v += s_db[tid + m * kCh];
    PB[b * D + ds_raw] = v;
  }
  if (!active) return;
  if (a.dh0 != nullptr)
    st_spl<SPL>(a.dh0 + (b * D + d) * N + SPL * q, lam);
  st_spl<SPL>(PA + (b * D + d) * N + SPL * q, dAacc);
  if (q == 0) PD[b * D + d] = dDacc;
}

// dB, dC: sum of the channel tiles' partials.  A workgroup per (b, t)
// row, whose partials (ntile, 2N) are contiguous: thread i reads entries i,
// i + 256, ... (coalesced), all of column i % 2N since 2N divides 256, and
// adds them in tile order; the 256 / 2N sums of a column are then added in
// order, so the result does not depend on timing.
__global__ __launch_bounds__(256) void bwd_reduce_bc_kernel(int64_t rows, int64_t N, int64_t ntile,
                                                            const float *P, float *dB, float *dC) {
  __shared__ float s_p[256];
  const int64_t N2 = 2 * N, tot = ntile * N2;
  const int tid = threadIdx.x;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const float *p = P + row * tot;
    float v = 0.f;
    int64_t e = tid;
    for (; e + 7 * 256 < tot; e += 8 * 256) {  // eight loads in flight, added in order
      float t[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) t[m] = p[e + m * 256];
#pragma unroll
      for (int m = 0; m < 8; ++m) v += t[m];
    }
    for (; e < tot; e += 256) v += p[e];
    __syncthreads();  // the previous row's sums are read
    s_p[tid] = v;
    __syncthreads();
    if (tid < N2) {
      float r = 0.f;
      for (int m = tid; m < 256; m += static_cast<int>(N2)) r += s_p[m];
      if (tid < N)
        dB[row * N + tid] = r;
      else
        dC[row * N + tid - N] = r;
    }
  }
}

// dA, dD, dbias: sum of the sequences' partials, sequences in order
__global__ __launch_bounds__(256) void bwd_reduce_param_kernel(int64_t B, int64_t D, int64_t N,
                                                               const float *PA, const float *PD,
                                                               const float *PB, float *dA, float *dD,
                                                               float *dbias) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t nA = D * N;
  if (i < nA) {
    float v = 0.f;
    for (int64_t b = 0; b < B; ++b) v += PA[b * nA + i];
    dA[i] = v;
    return;
  }
  const int64_t k = i - nA;
  const float *src = k < D ? PD : PB;
  float *dst = k < D ? dD : dbias;
  const int64_t c = k < D ? k : k - D;
  if (c >= D || dst == nullptr) return;
  float v = 0.f;
  for (int64_t b = 0; b < B; ++b) v += src[b * D + c];
  dst[c] = v;
}

template <typename T, int LPC, int SPL>
hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t s) {
  static_assert(LPC * SPL > 0, "");
  const int64_t kCh = bwd_channels_per_block(a.N);
  const int64_t ntile = (a.D + kCh - 1) / kCh;
  const int64_t nseg = bwd_nseg(a.L);
  float *P = a.ws + (a.h_ckpt ? 0 : a.B * nseg * a.D * a.N);
  float *PA = P + a.B * a.L * ntile * 2 * a.N;
  float *PD = PA + a.B * a.D * a.N;
  float *PB = PD + a.B * a.D;
  if (ntile > 0 && a.B > 0) {
    dim3 grid(static_cast<unsigned>(ntile), static_cast<unsigned>(a.B));
    scan_bwd_kernel<T, LPC, SPL><<<grid, kBwdThreads, 0, s>>>(a);
  }
  // a workgroup per (b, t) row (grid-strided past 2^20 rows); 2N (8 .. 128)
  // divides the 256 threads
  static_assert(256 % (2 * LPC * SPL) == 0, "2N must divide the reduction's 256 threads");
  const int64_t rows = a.B * a.L;
  if (rows > 0)
    bwd_reduce_bc_kernel<<<static_cast<unsigned>(rows < (1 << 20) ? rows : (1 << 20)), 256, 0, s>>>(
        rows, a.N, ntile, P, a.dB, a.dC);
  const int64_t npar = a.D * a.N + 2 * a.D;
  if (npar > 0)
    bwd_reduce_param_kernel<<<static_cast<unsigned>((npar + 255) / 256), 256, 0, s>>>(
        a.B, a.D, a.N, PA, PD, PB, a.dA, a.D_skip ? a.dD : nullptr, a.dbias);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_bwd_dt(const BwdArgs &a, hipStream_t s) {
  switch (a.N) {
    case 4: return launch_bwd_t<T, 1, 4>(a, s);
    case 8: return launch_bwd_t<T, 2, 4>(a, s);
    case 16: return launch_bwd_t<T, 4, 4>(a, s);
    case 32: return launch_bwd_t<T, 8, 4>(a, s);
    case 64: return launch_bwd_t<T, 16, 4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool scan_bwd_supported_n(int64_t N) { return N == 4 || N == 8 || N == 16 || N == 32 || N == 64; }

int64_t scan_bwd_ws_floats(int64_t B, int64_t L, int64_t D, int64_t N, bool saved_states) {
  if (!scan_bwd_supported_n(N)) return 0;
  const int64_t kCh = bwd_channels_per_block(N);
  const int64_t ntile = (D + kCh - 1) / kCh;
  return (saved_states ? 0 : B * bwd_nseg(L) * D * N) + B * L * ntile * 2 * N + B * D * N + 2 * B * D;
}

hipError_t launch_scan_bwd(const BwdArgs &a, hipStream_t s) {
  // Without saved states, the lane-split forward recomputes them into the
  // workspace (its first B * nseg * D * N floats) where its layout applies;
  // the backward then runs as if the forward had saved them, with the rest
  // of the workspace, which is where the partials already lie.  The
  // kernel's own first pass remains for the shapes the lane-split scan
  // does not take.
  static_assert(kSeg == 8, "the lane-split scan saves the state entering every 8 tokens");
  if (a.h_ckpt == nullptr && a.L > 0 && a.B > 0 && a.D > 0 && reinterpret_cast<uintptr_t>(a.ws) % 16 == 0) {
    ScanArgs f{};
    f.B = a.B; f.L = a.L; f.D = a.D; f.N = a.N; f.dt = a.dt;
    f.x = a.x; f.delta = a.delta; f.A = a.A; f.Bm = a.Bm;
    f.Cm = a.Bm;                    // not accessed in this mode
    f.y = const_cast<void *>(a.x);  // not written in this mode
    f.h0 = a.h0;
    f.delta_bias = a.delta_bias; f.delta_softplus = a.delta_softplus;
    f.h_ckpt = a.ws;
    if (scan_lanesplit_supported(f)) {
      hipError_t e = launch_scan_states(f, s);
      if (e != hipSuccess) return e;
      BwdArgs g = a;
      g.h_ckpt = a.ws;
      g.ws = a.ws + a.B * bwd_nseg(a.L) * a.D * a.N;
      return a.dt == DType::BF16 ? launch_bwd_dt<bf16_t>(g, s) : launch_bwd_dt<float>(g, s);
    }
  }
  if (a.dt == DType::BF16) return launch_bwd_dt<bf16_t>(a, s);
  return launch_bwd_dt<float>(a, s);
}

}  // namespace ssm
