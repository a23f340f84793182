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
// enters every 16-token segment to the workspace.  Pass 2 walks the
// segments backwards: it reloads a segment's entering state, recomputes the
// segment's 16 states into registers, then runs the reverse recurrence over
// them.  Per token each wave sums its channels' dB and dC contributions with
// a butterfly that leaves every (B|C, n) sum in one lane, the four waves add
// theirs through LDS, and the workgroup writes one partial per (token, n).
// Two small kernels then add the partials of the channel tiles (dB, dC) and
// of the sequences (dA, dD, dbias) in a fixed order, so the result does not
// depend on timing (no atomics).
#include "bwd.h"
#include "device_common.h"

namespace ssm {
namespace {

constexpr int kBwdThreads = 256;
constexpr int kSeg = 16;  // tokens per checkpointed segment

__device__ __forceinline__ float sigmoid_f(float v) {
  return __builtin_amdgcn_rcpf(1.0f + fast_exp2(-v * kLog2e));
}

// sum over the LPC adjacent lanes of a channel
template <int LPC>
__device__ __forceinline__ float channel_sum(float v) {
#pragma unroll
  for (int off = LPC / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, LPC);
  return v;
}

template <typename T>
__device__ __forceinline__ void load4(const T *p, float *v) {
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = to_f32(p[j]);
}

__host__ __device__ constexpr int64_t bwd_nseg(int64_t L) { return (L + kSeg - 1) / kSeg; }
__host__ __device__ constexpr int64_t bwd_channels_per_block(int64_t N) { return 4 * kBwdThreads / N; }

template <typename T, int LPC>
__global__ __launch_bounds__(kBwdThreads) void scan_bwd_kernel(BwdArgs a) {
  constexpr int N = 4 * LPC;
  constexpr int kCh = kBwdThreads / LPC;        // channels per workgroup
  constexpr int kLq = LPC == 1 ? 0 : LPC == 2 ? 1 : LPC == 4 ? 2 : LPC == 8 ? 3 : 4;
  constexpr int kCB = 6 - kLq;                   // lane bits that select the channel
  constexpr int kHalv = kCB < 3 ? kCB : 3;       // halving steps of the butterfly
  constexpr int kFull = kCB - kHalv;             // remaining summing steps
  constexpr int kCnt = 8 >> kHalv;               // sums each lane ends with
  __shared__ float s_red[4][kSeg][2 * N];        // per wave: [token][B sums | C sums]

  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64, q = tid % LPC;
  const int64_t tile = blockIdx.x, ntile = gridDim.x, b = blockIdx.y;
  const int64_t B = a.B, L = a.L, D = a.D;
  const int64_t d_raw = tile * kCh + tid / LPC;
  const bool active = d_raw < D;
  const int64_t d = active ? d_raw : D - 1;
  const int64_t nseg = bwd_nseg(L);
  const T *xp = static_cast<const T *>(a.x);
  const T *dp = static_cast<const T *>(a.delta);
  const T *zp = static_cast<const T *>(a.z);
  const T *gp = static_cast<const T *>(a.dy);
  const T *Bp = static_cast<const T *>(a.Bm);
  const T *Cp = static_cast<const T *>(a.Cm);
  float *ck = a.ws;                      // (B, nseg, D, N) entering states
  float *P = ck + B * nseg * D * N;      // (B, L, ntile, 2N) dB|dC partials
  float *PA = P + B * L * ntile * 2 * N; // (B, D, N) dA partials
  float *PD = PA + B * D * N;            // (B, D) dD partials
  float *PB = PD + B * D;                // (B, D) dbias partials

  const float4 Av = reinterpret_cast<const float4 *>(a.A + d * N)[q];
  const float An[4] = {Av.x, Av.y, Av.z, Av.w};
  float A2[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) A2[j] = An[j] * kLog2e;
  const float bias = a.delta_bias ? a.delta_bias[d] : 0.f;
  const float Dd = a.D_skip ? a.D_skip[d] : 0.f;

  // ---- pass 1: forward, keeping the state that enters every segment ----
  float h[4] = {0.f, 0.f, 0.f, 0.f};
  if (a.h0 != nullptr && active) {
    const float4 v = reinterpret_cast<const float4 *>(a.h0 + (b * D + d) * N)[q];
    h[0] = v.x; h[1] = v.y; h[2] = v.z; h[3] = v.w;
  }
  for (int64_t s = 0; s < nseg; ++s) {
    if (active)
      reinterpret_cast<float4 *>(ck + ((b * nseg + s) * D + d) * N)[q] =
          make_float4(h[0], h[1], h[2], h[3]);
    const int64_t t0 = s * kSeg;
    const int nt = static_cast<int>(L - t0 < kSeg ? L - t0 : kSeg);
    for (int k = 0; k < nt; ++k) {
      const int64_t row = b * L + t0 + k;
      const float dl = step_size(to_f32(dp[row * D + d]), bias, a.delta_softplus);
      const float u = dl * to_f32(xp[row * D + d]);
      float Bv[4];
      load4(Bp + row * N + 4 * q, Bv);
#pragma unroll
      for (int j = 0; j < 4; ++j) h[j] = fmaf(fast_exp2(dl * A2[j]), h[j], u * Bv[j]);
    }
  }

  // ---- pass 2: segments in reverse ----
  float lam[4] = {0.f, 0.f, 0.f, 0.f};
  if (a.dh_final != nullptr && active) {
    const float4 v = reinterpret_cast<const float4 *>(a.dh_final + (b * D + d) * N)[q];
    lam[0] = v.x; lam[1] = v.y; lam[2] = v.z; lam[3] = v.w;
  }
  float dAacc[4] = {0.f, 0.f, 0.f, 0.f};
  float dDacc = 0.f, dbacc = 0.f;
  for (int64_t s = nseg - 1; s >= 0; --s) {
    const int64_t t0 = s * kSeg;
    const int nt = static_cast<int>(L - t0 < kSeg ? L - t0 : kSeg);
    float H[kSeg + 1][4];  // H[k] = state before token t0 + k
    {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (active) v = reinterpret_cast<const float4 *>(ck + ((b * nseg + s) * D + d) * N)[q];
      H[0][0] = v.x; H[0][1] = v.y; H[0][2] = v.z; H[0][3] = v.w;
    }
#pragma unroll
    for (int k = 0; k < kSeg; ++k) {
      if (k < nt) {
        const int64_t row = b * L + t0 + k;
        const float dl = step_size(to_f32(dp[row * D + d]), bias, a.delta_softplus);
        const float u = dl * to_f32(xp[row * D + d]);
        float Bv[4];
        load4(Bp + row * N + 4 * q, Bv);
#pragma unroll
        for (int j = 0; j < 4; ++j) H[k + 1][j] = fmaf(fast_exp2(dl * A2[j]), H[k][j], u * Bv[j]);
      }
    }
#pragma unroll
    for (int k = kSeg - 1; k >= 0; --k) {
      if (k < nt) {
        const int64_t row = b * L + t0 + k;
        const float raw = to_f32(dp[row * D + d]);
        const float dl = step_size(raw, bias, a.delta_softplus);
        const float xv = to_f32(xp[row * D + d]);
        const float dyv = to_f32(gp[row * D + d]);
        float Bv[4], Cv[4];
        load4(Bp + row * N + 4 * q, Bv);
        load4(Cp + row * N + 4 * q, Cv);
        float qp = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) qp = fmaf(Cv[j], H[k + 1][j], qp);
        const float qs = fmaf(Dd, xv, channel_sum<LPC>(qp));
        float g = dyv, dzv = 0.f;
        if (zp != nullptr) {
          const float zv = to_f32(zp[row * D + d]);
          const float sg = sigmoid_f(zv);
          g = dyv * zv * sg;
          dzv = dyv * qs * sg * fmaf(zv, 1.f - sg, 1.f);
        }
        const float u = dl * xv;
        float v[8];
        float ddl = 0.f, dxp = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float aj = fast_exp2(dl * A2[j]);
          lam[j] = fmaf(g, Cv[j], lam[j]);
          v[j] = lam[j] * u;
          v[4 + j] = g * H[k + 1][j];
          const float p = aj * H[k][j];
          ddl = fmaf(lam[j], fmaf(An[j], p, Bv[j] * xv), ddl);
          dAacc[j] = fmaf(lam[j] * dl, p, dAacc[j]);
          dxp = fmaf(lam[j], Bv[j], dxp);
          lam[j] *= aj;
        }
        ddl = channel_sum<LPC>(ddl);
        dxp = channel_sum<LPC>(dxp);
        if (a.delta_softplus) ddl *= sigmoid_f(raw + bias);
        if (active && q == 0) {
          static_cast<T *>(a.dx)[row * D + d] = from_f32<T>(fmaf(dl, dxp, Dd * g));
          static_cast<T *>(a.ddelta)[row * D + d] = from_f32<T>(ddl);
          if (zp != nullptr) static_cast<T *>(a.dz)[row * D + d] = from_f32<T>(dzv);
        }
        dDacc = fmaf(g, xv, dDacc);
        dbacc += ddl;
        if (!active) {
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = 0.f;
        }
        // butterfly over the channel bits of the lane: halving steps leave
        // each lane with the sums of kCnt of the 8 values (indices base..),
        // the remaining steps add the rest of the wave's channels
        int base = 0;
#pragma unroll
        for (int st = 0; st < kHalv; ++st) {
          const int m = 1 << (5 - st);
          const int half = 4 >> st;
          const bool hi = (lane & m) != 0;
#pragma unroll
          for (int i = 0; i < half; ++i) {
            const float keep = hi ? v[half + i] : v[i];
            const float send = hi ? v[i] : v[half + i];
            v[i] = keep + __shfl_xor(send, m);
          }
          base += hi ? half : 0;
        }
        bool writer = true;
#pragma unroll
        for (int st = 0; st < kFull; ++st) {
          const int m = 1 << (5 - kHalv - st);
          v[0] += __shfl_xor(v[0], m);
          writer = writer && (lane & m) == 0;
        }
        if (writer) {
#pragma unroll
          for (int i = 0; i < kCnt; ++i) {
            const int idx = base + i;
            s_red[wave][k][(idx / 4) * N + 4 * q + idx % 4] = v[i];
          }
        }
      }
    }
    __syncthreads();
    for (int e = tid; e < nt * 2 * N; e += kBwdThreads) {
      const int k = e / (2 * N), j = e % (2 * N);
      P[((b * L + t0 + k) * ntile + tile) * 2 * N + j] =
          s_red[0][k][j] + s_red[1][k][j] + s_red[2][k][j] + s_red[3][k][j];
    }
    __syncthreads();
  }

  if (!active) return;
  if (a.dh0 != nullptr)
    reinterpret_cast<float4 *>(a.dh0 + (b * D + d) * N)[q] = make_float4(lam[0], lam[1], lam[2], lam[3]);
  reinterpret_cast<float4 *>(PA + (b * D + d) * N)[q] = make_float4(dAacc[0], dAacc[1], dAacc[2], dAacc[3]);
  if (q == 0) {
    PD[b * D + d] = dDacc;
    PB[b * D + d] = dbacc;
  }
}

// dB, dC: sum of the channel tiles' partials, tiles in order
__global__ __launch_bounds__(256) void bwd_reduce_bc_kernel(int64_t rows, int64_t N, int64_t ntile,
                                                            const float *P, float *dB, float *dC) {
  const int64_t N2 = 2 * N;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= rows * N2) return;
  const int64_t row = i / N2, j = i % N2;
  const float *p = P + row * ntile * N2 + j;
  float v = 0.f;
  for (int64_t t = 0; t < ntile; ++t) v += p[t * N2];
  if (j < N)
    dB[row * N + j] = v;
  else
    dC[row * N + j - N] = v;
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

template <typename T, int LPC>
hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t s) {
  const int64_t kCh = bwd_channels_per_block(a.N);
  const int64_t ntile = (a.D + kCh - 1) / kCh;
  const int64_t nseg = bwd_nseg(a.L);
  float *P = a.ws + a.B * nseg * a.D * a.N;
  float *PA = P + a.B * a.L * ntile * 2 * a.N;
  float *PD = PA + a.B * a.D * a.N;
  float *PB = PD + a.B * a.D;
  if (ntile > 0 && a.B > 0) {
    dim3 grid(static_cast<unsigned>(ntile), static_cast<unsigned>(a.B));
    scan_bwd_kernel<T, LPC><<<grid, kBwdThreads, 0, s>>>(a);
  }
  const int64_t nbc = a.B * a.L * 2 * a.N;
  if (nbc > 0)
    bwd_reduce_bc_kernel<<<static_cast<unsigned>((nbc + 255) / 256), 256, 0, s>>>(a.B * a.L, a.N, ntile, P,
                                                                              a.dB, a.dC);
  const int64_t npar = a.D * a.N + 2 * a.D;
  if (npar > 0)
    bwd_reduce_param_kernel<<<static_cast<unsigned>((npar + 255) / 256), 256, 0, s>>>(
        a.B, a.D, a.N, PA, PD, PB, a.dA, a.D_skip ? a.dD : nullptr, a.dbias);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_bwd_dt(const BwdArgs &a, hipStream_t s) {
  switch (a.N) {
    case 4: return launch_bwd_t<T, 1>(a, s);
    case 8: return launch_bwd_t<T, 2>(a, s);
    case 16: return launch_bwd_t<T, 4>(a, s);
    case 32: return launch_bwd_t<T, 8>(a, s);
    case 64: return launch_bwd_t<T, 16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool scan_bwd_supported_n(int64_t N) { return N == 4 || N == 8 || N == 16 || N == 32 || N == 64; }

int64_t scan_bwd_ws_floats(int64_t B, int64_t L, int64_t D, int64_t N) {
  if (!scan_bwd_supported_n(N)) return 0;
  const int64_t kCh = bwd_channels_per_block(N);
  const int64_t ntile = (D + kCh - 1) / kCh;
  return B * bwd_nseg(L) * D * N + B * L * ntile * 2 * N + B * D * N + 2 * B * D;
}

hipError_t launch_scan_bwd(const BwdArgs &a, hipStream_t s) {
  if (a.dt == DType::BF16) return launch_bwd_dt<bf16_t>(a, s);
  return launch_bwd_dt<float>(a, s);
}

}  // namespace ssm
