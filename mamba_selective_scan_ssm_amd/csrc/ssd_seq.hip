// Mamba-2 SSD recurrence on the vector ALU, token by token: the path for the
// shapes the matrix-core kernels of ssd.hip are not built for -- fp32
// inputs (whose 1e-5 bar the hi + lo bf16 operand split of those kernels
// cannot meet), head dims other than 64, N not a multiple of 32 and chunk
// lengths other than 64, 128 and 256 (the result does not depend on the
// chunk length: this path walks the tokens in order).
//
// What is computed ("Clean up SSM ops directory structure - #6444", the SSD
// kernels; groups as in "Tensor-parallel SSM #333"): per sequence b, head h,
// channel p and state n, with group g = h / (H / G),
//   h_t[p,n] = exp(dt_t A[h]) h_{t-1}[p,n] + dt_t B_t[g,n] x_t[h,p]
//   y_t[h,p] = (sum_n C_t[g,n] h_t[p,n] + D[h] x_t[h,p]) * silu(z_t[h,p])
// the Mamba recurrence with one A per head, so exp(dt_t A[h]) is formed once
// per (token, head) and each element costs one multiply and two FMAs.
//
// Work decomposition: a workgroup owns 64 consecutive channels c = h P + p
// of one sequence (any P, so a workgroup may span heads and groups) and its
// W waves split the N states, 16 per lane, kept in fp32 registers for the
// whole sequence.  Every lane reads its own head's dt and its own group's B
// and C (lanes of one group read the same addresses).  The waves' partial
// sums of C h meet in LDS every 8 tokens; wave w then finishes tokens
// w, w + W, ... of the block (skip term, gate, store).
#include "device_common.h"
#include "launch.h"

namespace ssm {
namespace {

constexpr int kWave = 64;
constexpr int kSPL = 16;  // states per lane
constexpr int kTB = 8;    // tokens per LDS round

template <typename T>
__device__ __forceinline__ float ld(const void *p, int64_t i) {
  return to_f32(static_cast<const T *>(p)[i]);
}

template <typename T, int W>
__global__ __launch_bounds__(kWave *W) void ssd_seq_kernel(SSDArgs a) {
  __shared__ float s_y[W][kTB][kWave];
  const int64_t H = a.H, P = a.P, G = a.G, N = a.N, L = a.L;
  const int64_t HP = H * P, HPG = H / G;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int64_t b = blockIdx.y;
  const int64_t c_raw = static_cast<int64_t>(blockIdx.x) * kWave + lane;
  const bool active = c_raw < HP;
  const int64_t c = active ? c_raw : HP - 1;
  const int64_t h = c / P, g = h / HPG;
  const int n0 = wave * kSPL;
  const float A2 = a.A[h] * kLog2e;
  const float bias = a.dt_bias ? a.dt_bias[h] : 0.f;
  const float Dh = a.D_skip ? a.D_skip[h] : 0.f;

  float hs[kSPL];
#pragma unroll
  for (int s = 0; s < kSPL; ++s) {
    const int64_t n = n0 + s;
    hs[s] = (a.h0 && n < N) ? a.h0[(b * HP + c) * N + n] : 0.f;
  }

  for (int64_t t0 = 0; t0 < L; t0 += kTB) {
#pragma unroll
    for (int j = 0; j < kTB; ++j) {
      const int64_t t = t0 + j;
      float acc = 0.f;
      if (t < L) {
        const int64_t row = b * L + t;
        const float dtv = step_size(ld<T>(a.dt, row * H + h), bias, a.dt_softplus);
        const float dA = fast_exp2(dtv * A2);
        const float u = dtv * ld<T>(a.x, row * HP + c);
        const int64_t bc = (row * G + g) * N;
#pragma unroll
        for (int s = 0; s < kSPL; ++s) {
          const int64_t n = n0 + s;
          if (n < N) {
            hs[s] = fmaf(dA, hs[s], u * ld<T>(a.Bm, bc + n));
            acc = fmaf(ld<T>(a.Cm, bc + n), hs[s], acc);
          }
        }
      }
      s_y[wave][j][lane] = acc;
    }
    __syncthreads();
    for (int j = wave; j < kTB; j += W) {
      const int64_t t = t0 + j;
      if (t < L && active) {
        float v = s_y[0][j][lane];
#pragma unroll
        for (int w = 1; w < W; ++w) v += s_y[w][j][lane];
        const int64_t i = (b * L + t) * HP + c;
        v = fmaf(Dh, ld<T>(a.x, i), v);
        if (a.z) v *= silu(ld<T>(a.z, i));
        static_cast<T *>(a.y)[i] = from_f32<T>(v);
      }
    }
    __syncthreads();
  }
  if (!active || a.h_final == nullptr) return;
#pragma unroll
  for (int s = 0; s < kSPL; ++s) {
    const int64_t n = n0 + s;
    if (n < N) a.h_final[(b * HP + c) * N + n] = hs[s];
  }
}

template <typename T>
hipError_t launch_t(const SSDArgs &a, hipStream_t s) {
  const int64_t HP = a.H * a.P;
  const dim3 grid(static_cast<unsigned>((HP + kWave - 1) / kWave), static_cast<unsigned>(a.B));
  const int w = a.N > 0 ? static_cast<int>((a.N + kSPL - 1) / kSPL) : 1;
#define SSM_SEQ_CASE(Wv) \
  case Wv: ssd_seq_kernel<T, Wv><<<grid, kWave * Wv, 0, s>>>(a); break;
  switch (w) {
    SSM_SEQ_CASE(1) SSM_SEQ_CASE(2) SSM_SEQ_CASE(3) SSM_SEQ_CASE(4) SSM_SEQ_CASE(5) SSM_SEQ_CASE(6)
    SSM_SEQ_CASE(7) SSM_SEQ_CASE(8) SSM_SEQ_CASE(9) SSM_SEQ_CASE(10) SSM_SEQ_CASE(11)
    SSM_SEQ_CASE(12) SSM_SEQ_CASE(13) SSM_SEQ_CASE(14) SSM_SEQ_CASE(15) SSM_SEQ_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef SSM_SEQ_CASE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ssd_seq(const SSDArgs &a, hipStream_t s) {
  if (a.dt_type == DType::BF16) return launch_t<bf16_t>(a, s);
  return launch_t<float>(a, s);
}

}  // namespace ssm
