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

// Staged variant, for shapes where every 64-channel block lies inside one
// group ((H / G) P a multiple of 64), so the block's channels share one row
// of B and of C per token.  Tokens move in blocks of 16: all threads load
// the next block's x, dt, z and B/C rows (raw, into registers, with clamped
// indices so no load sits behind a branch) while the current block
// computes, then convert them once into LDS; a lane reads its 16 states' B
// and C with broadcast LDS reads.  States past N see B = C = 0 and stay 0.
constexpr int kSeqTB = 16;

template <typename T>
__device__ __forceinline__ uint32_t raw_bits(const void *p, int64_t i) {
  if constexpr (sizeof(T) == 2) return static_cast<const uint16_t *>(p)[i];
  else return __float_as_uint(static_cast<const float *>(p)[i]);
}
template <typename T>
__device__ __forceinline__ float from_bits(uint32_t r) {
  if constexpr (sizeof(T) == 2) return __uint_as_float(r << 16);
  else return __uint_as_float(r);
}

template <typename T, int W, int SPL>
__global__ __launch_bounds__(kWave *W) void ssd_seq_staged_kernel(SSDArgs a) {
  constexpr int kNT = kWave * W;                              // threads
  constexpr int kNP = W * SPL;                                // N padded to the lanes' states
  constexpr int kXR = (kSeqTB * kWave + kNT - 1) / kNT;       // (token, channel) entries per thread
  constexpr int kBR = (kSeqTB * kNP + kNT - 1) / kNT;         // (token, n) entries of B (and C)
  __shared__ float s_y[W][kSeqTB][kWave];
  __shared__ float s_x[kSeqTB][kWave], s_dt[kSeqTB][kWave], s_z[kSeqTB][kWave];
  __shared__ __attribute__((aligned(16))) float s_b[kSeqTB][kNP];
  __shared__ __attribute__((aligned(16))) float s_c[kSeqTB][kNP];
  const int64_t H = a.H, P = a.P, G = a.G, N = a.N, L = a.L;
  const int64_t HP = H * P, HPG = H / G;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int64_t b = blockIdx.y;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kWave;
  // a thread's channel is c0 + lane in both roles (kNT is a multiple of 64)
  const int64_t c = c0 + lane, h = c / P;
  const int64_t g = (c0 / P) / HPG;
  const int n0 = wave * SPL;
  const float A2 = a.A[h] * kLog2e;
  const float bias = a.dt_bias ? a.dt_bias[h] : 0.f;
  const float Dh = a.D_skip ? a.D_skip[h] : 0.f;
  const bool has_z = a.z != nullptr;
  const void *zsrc = has_z ? a.z : a.x;  // read unconditionally; unused without a gate

  float hs[SPL];
#pragma unroll
  for (int s = 0; s < SPL; ++s) {
    const int64_t n = n0 + s;
    hs[s] = (a.h0 && n < N) ? a.h0[(b * HP + c) * N + n] : 0.f;
  }

  uint32_t rx[kXR], rd[kXR], rz[kXR], rb[kBR], rc[kBR];
  auto issue = [&](int64_t t0) {
#pragma unroll
    for (int k = 0; k < kXR; ++k) {
      const int j = (tid + k * kNT) / kWave;
      const int64_t t = t0 + j < L ? t0 + j : L - 1;
      const int64_t row = b * L + t;
      rx[k] = raw_bits<T>(a.x, row * HP + c);
      rd[k] = raw_bits<T>(a.dt, row * H + h);
      rz[k] = raw_bits<T>(zsrc, row * HP + c);
    }
#pragma unroll
    for (int k = 0; k < kBR; ++k) {
      const int i = tid + k * kNT;
      const int j = (i / kNP) % kSeqTB;
      const int n = i % kNP;
      const int64_t t = t0 + j < L ? t0 + j : L - 1;
      const int64_t bc = ((b * L + t) * G + g) * N + (n < N ? n : N - 1);
      rb[k] = raw_bits<T>(a.Bm, bc);
      rc[k] = raw_bits<T>(a.Cm, bc);
    }
  };
  // tokens past L stage dt = x = 0 (the state passes through unchanged)
  auto stage = [&](int64_t t0) {
#pragma unroll
    for (int k = 0; k < kXR; ++k) {
      const int i = tid + k * kNT;
      if (i < kSeqTB * kWave) {
        const int j = i / kWave;
        const bool ok = t0 + j < L;
        s_dt[j][lane] = ok ? step_size(from_bits<T>(rd[k]), bias, a.dt_softplus) : 0.f;
        s_x[j][lane] = ok ? from_bits<T>(rx[k]) : 0.f;
        s_z[j][lane] = from_bits<T>(rz[k]);
      }
    }
#pragma unroll
    for (int k = 0; k < kBR; ++k) {
      const int i = tid + k * kNT;
      if (i < kSeqTB * kNP) {
        const int j = i / kNP, n = i % kNP;
        s_b[j][n] = n < N ? from_bits<T>(rb[k]) : 0.f;
        s_c[j][n] = n < N ? from_bits<T>(rc[k]) : 0.f;
      }
    }
  };

  const int64_t nblk = (L + kSeqTB - 1) / kSeqTB;
  if (nblk > 0) issue(0);
  for (int64_t blk = 0; blk < nblk; ++blk) {
    const int64_t t0 = blk * kSeqTB;
    if (blk > 0) __syncthreads();  // the previous block's reads are done
    stage(t0);
    __syncthreads();
    if (blk + 1 < nblk) issue(t0 + kSeqTB);
#pragma unroll
    for (int j = 0; j < kSeqTB; ++j) {
      const float dtv = s_dt[j][lane];
      const float dA = fast_exp2(dtv * A2);
      const float u = dtv * s_x[j][lane];
      float acc = 0.f;
#pragma unroll
      for (int s4 = 0; s4 < SPL / 4; ++s4) {
        const float4 bv = *reinterpret_cast<const float4 *>(&s_b[j][n0 + 4 * s4]);
        const float4 cv = *reinterpret_cast<const float4 *>(&s_c[j][n0 + 4 * s4]);
        const float bb[4] = {bv.x, bv.y, bv.z, bv.w}, cc[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float &hv = hs[4 * s4 + e];
          hv = fmaf(dA, hv, u * bb[e]);
          acc = fmaf(cc[e], hv, acc);
        }
      }
      s_y[wave][j][lane] = acc;
    }
    __syncthreads();
    for (int j = wave; j < kSeqTB; j += W) {
      const int64_t t = t0 + j;
      if (t < L) {
        float v = s_y[0][j][lane];
#pragma unroll
        for (int w = 1; w < W; ++w) v += s_y[w][j][lane];
        v = fmaf(Dh, s_x[j][lane], v);
        if (has_z) v *= silu(s_z[j][lane]);
        static_cast<T *>(a.y)[(b * L + t) * HP + c] = from_f32<T>(v);
      }
    }
  }
  if (a.h_final == nullptr) return;
#pragma unroll
  for (int s = 0; s < SPL; ++s) {
    const int64_t n = n0 + s;
    if (n < N) a.h_final[(b * HP + c) * N + n] = hs[s];
  }
}

// N <= 128: 8 states per lane, so twice the waves of 16 per lane (the
// sequences' channels alone give few waves at Mamba-2 shapes); larger N: 16.
template <typename T, int SPL>
hipError_t launch_staged_spl(const SSDArgs &a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.H * a.P / kWave), static_cast<unsigned>(a.B));
  const int w = a.N > 0 ? static_cast<int>((a.N + SPL - 1) / SPL) : 1;
#define SSM_SEQ_CASE(Wv) \
  case Wv: ssd_seq_staged_kernel<T, Wv, SPL><<<grid, kWave * Wv, 0, s>>>(a); break;
  if constexpr (SPL == 8) {  // N <= 128
    switch (w) {
      SSM_SEQ_CASE(1) SSM_SEQ_CASE(2) SSM_SEQ_CASE(3) SSM_SEQ_CASE(4) SSM_SEQ_CASE(5) SSM_SEQ_CASE(6)
      SSM_SEQ_CASE(7) SSM_SEQ_CASE(8) SSM_SEQ_CASE(9) SSM_SEQ_CASE(10) SSM_SEQ_CASE(11)
      SSM_SEQ_CASE(12) SSM_SEQ_CASE(13) SSM_SEQ_CASE(14) SSM_SEQ_CASE(15) SSM_SEQ_CASE(16)
      default: return hipErrorInvalidValue;
    }
  } else {  // 128 < N <= 256
    switch (w) {
      SSM_SEQ_CASE(9) SSM_SEQ_CASE(10) SSM_SEQ_CASE(11) SSM_SEQ_CASE(12) SSM_SEQ_CASE(13)
      SSM_SEQ_CASE(14) SSM_SEQ_CASE(15) SSM_SEQ_CASE(16)
      default: return hipErrorInvalidValue;
    }
  }
#undef SSM_SEQ_CASE
  return hipGetLastError();
}

template <typename T>
hipError_t launch_staged(const SSDArgs &a, hipStream_t s) {
  return a.N <= 128 ? launch_staged_spl<T, 8>(a, s) : launch_staged_spl<T, 16>(a, s);
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
  // every 64-channel block inside one group: the staged kernel
  const bool staged = (a.H / a.G) * a.P % kWave == 0;
  if (a.dt_type == DType::BF16) return staged ? launch_staged<bf16_t>(a, s) : launch_t<bf16_t>(a, s);
  return staged ? launch_staged<float>(a, s) : launch_t<float>(a, s);
}

}  // namespace ssm
