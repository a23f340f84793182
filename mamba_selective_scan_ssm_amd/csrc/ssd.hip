// Mamba-2 SSD (state-space duality) chunked scan on the gfx950 matrix cores.
//
// The pages name the kernel family -- ssd_bmm, ssd_chunk_state,
// ssd_state_passing, ssd_chunk_scan, ssd_combined ("Clean up SSM ops
// directory structure - #6444") -- and the head/group structure (B and C
// shared by the heads of a group, "Tensor-parallel SSM #333"; groups divide
// heads, "Current Implementation of TP in MambaMixer2").  The math below is
// the Mamba recurrence with a scalar A per head, regrouped by chunks of Q
// tokens.  With a_t = dt_t A[h] and the in-chunk cumulative sum
// S_i = sum_{k<=i} a_k (inclusive, so token j's own input is not decayed):
//   chunk state   dS[p,n]   = sum_j exp(S_end - S_j) dt_j x_j[p] B_j[n]
//   state passing h_c       = exp(S_end,c) h_{c-1} + dS_c,  h_{-1} = h0
//   outputs       y_i[p]    = exp(S_i) sum_n C_i[n] h_in[p,n]              (Y_off)
//                           + sum_{j<=i} (C_i.B_j) exp(S_i - S_j) dt_j x_j[p] (Y_diag)
//                           + D x_i[p], then * silu(z_i[p])
// which is the recurrence h_t = exp(a_t) h_{t-1} + dt_t B_t x_t exactly up to
// rounding order.  All exponents are <= 0 (A < 0 is not required: the code
// never forms exp(-S_j) alone, only differences with i >= j).
//
// Three kernels (grid = chunk x head x batch for 1 and 3):
//  1. ssd_chunk_state: dS = Xw^T B on MFMA (Xw = x scaled by the decay to the
//     chunk end and dt), written fp32 to the workspace; also exp(S_end).
//  2. ssd_state_pass: per (b, h, p, n) the fp32 recurrence over chunks,
//     seeded by h0, replacing each dS_c with the state entering chunk c.
//  3. ssd_chunk_scan: CB^T = B C^T on MFMA per 32x32 block pair, masked and
//     decayed in registers, then Y += M X and Y_off = C h_in on MFMA.
//
// Precision: B, C and x arrive in bf16 and enter the MFMA unchanged (exact).
// Operands that are products computed here (the decayed scores M, the scaled
// Xw, the fp32 carried state) are split into hi + lo bf16 halves and both
// halves are multiplied (two MFMAs), giving ~16 significant bits per operand;
// accumulation is fp32.
//
// MFMA used: v_mfma_f32_32x32x16_bf16.  Operand layout (lane l, e = 0..7):
// A[i = l%32][k = 8*(l/32) + e], B[k = 8*(l/32) + e][j = l%32]; result
// register r holds D[8*(r/4) + 4*(l/32) + r%4][l%32].
#include "device_common.h"
#include "launch.h"

namespace ssm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kP = 64;        // head dim supported
constexpr int kThreads = 256;  // 4 waves

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ __bf16 bf16_bits(uint16_t u) { return __builtin_bit_cast(__bf16, u); }
__device__ __forceinline__ float bf_to_f(__bf16 v) { return static_cast<float>(v); }

// split an fp32 value into bf16 hi + lo with hi + lo ~= v to ~16 bits
__device__ __forceinline__ void split_bf16(float v, __bf16 &hi, __bf16 &lo) {
  hi = static_cast<__bf16>(v);
  lo = static_cast<__bf16>(v - static_cast<float>(hi));
}

// Inclusive prefix sum over the Q <= 256 values v (one per thread, threads
// >= Q pass 0) into s_out[0..Q).  Uses wave shuffles and one LDS round.
__device__ void block_inclusive_scan(float v, float *s_out, float *s_wave, int Q) {
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    float o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  if (lane == 63) s_wave[wave] = v;
  __syncthreads();
  float add = 0.f;
  for (int w = 0; w < wave; ++w) add += s_wave[w];
  v += add;
  if (tid < Q) s_out[tid] = v;
  __syncthreads();
}

// 16-byte load of 8 bf16 (row-major source, 16-B aligned), zero if !valid.
__device__ __forceinline__ uint4 load8_raw(const uint16_t *p, bool valid) {
  return valid ? *reinterpret_cast<const uint4 *>(p) : make_uint4(0, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 load8(const uint16_t *p, bool valid) {
  return __builtin_bit_cast(bf16x8, load8_raw(p, valid));
}
// element e (0..7) of 8 packed bf16, as its 16 raw bits in the low half
__device__ __forceinline__ uint32_t elem16(const uint4 &u, int e) {
  const uint32_t w = (e >> 1) == 0 ? u.x : (e >> 1) == 1 ? u.y : (e >> 1) == 2 ? u.z : u.w;
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}
__device__ __forceinline__ float elem_f32(const uint4 &u, int e) {
  return __uint_as_float(elem16(u, e) << 16);
}
// two bf16 (raw bits) packed low/high into one 32-bit LDS word
__device__ __forceinline__ uint32_t pack2(uint32_t lo, uint32_t hi) { return lo | (hi << 16); }

// ---------------------------------------------------------------------------
// 1. chunk states
// ---------------------------------------------------------------------------
// LDS staging of one 64-token slice, transposed so each MFMA operand lane
// reads 8 consecutive tokens: Xhi/Xlo [p][j], Bt [n][j]; rows padded.
constexpr int kSlice = 64;
constexpr int kSlicePad = kSlice + 8;

template <int N>
__global__ __launch_bounds__(kThreads) void ssd_chunk_state_kernel(SSDArgs a, float *ws_states,
                                                                     float *ws_decay) {
  const int Q = static_cast<int>(a.chunk);
  const int64_t c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t nc = gridDim.x, H = a.H, L = a.L;
  const int64_t g = h / (H / a.G);
  const int64_t t0 = c * Q;
  const int nvalid = static_cast<int>((L - t0) < Q ? (L - t0) : Q);
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64, lg = lane / 32, l32 = lane % 32;

  __shared__ float s_S[256];     // cumulative log2-decay, inclusive
  __shared__ float s_w[256];     // exp2(S_end - S_j) * dt_j
  __shared__ float s_wave[4];
  __shared__ __attribute__((aligned(16))) uint16_t s_xhi[kP * kSlicePad];
  __shared__ __attribute__((aligned(16))) uint16_t s_xlo[kP * kSlicePad];
  __shared__ __attribute__((aligned(16))) uint16_t s_bt[N * kSlicePad];

  const uint16_t *dtp = static_cast<const uint16_t *>(a.dt);
  const float A2 = a.A[h] * kLog2e;
  float dtv = 0.f;
  if (tid < nvalid) dtv = bf_to_f(bf16_bits(dtp[(b * L + t0 + tid) * H + h]));
  block_inclusive_scan(dtv * A2, s_S, s_wave, Q);
  const float S_end = s_S[Q - 1];
  if (tid < Q) s_w[tid] = fast_exp2(S_end - s_S[tid]) * dtv;
  if (tid == 0) ws_decay[(b * nc + c) * H + h] = fast_exp2(S_end);
  __syncthreads();

  constexpr int NT = N / 32;                 // n tiles
  constexpr int TPW = (NT + 3) / 4;          // n tiles per wave
  f32x16 acc[TPW][2];
#pragma unroll
  for (int q = 0; q < TPW; ++q) acc[q][0] = acc[q][1] = f32x16{};

  const uint16_t *xp = static_cast<const uint16_t *>(a.x);
  const uint16_t *Bp = static_cast<const uint16_t *>(a.Bm);

  for (int js = 0; js < Q; js += kSlice) {
    // stage x (scaled, split) and B for tokens [js, js+64), transposed
    // unit = (token pair jp, 8-wide column chunk)
    for (int u = tid; u < (kSlice / 2) * (kP / 8); u += kThreads) {
      const int jp = u / (kP / 8), pc = u % (kP / 8);
      const int j0 = js + 2 * jp;
      const int64_t base = ((b * L + t0 + j0) * H + h) * kP + pc * 8;
      const uint4 r0 = load8_raw(xp + base, j0 < nvalid);
      const uint4 r1 = load8_raw(xp + base + H * kP, j0 + 1 < nvalid);
      const float w0 = s_w[j0], w1 = s_w[j0 + 1];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        __bf16 h0v, l0v, h1v, l1v;
        split_bf16(elem_f32(r0, e) * w0, h0v, l0v);
        split_bf16(elem_f32(r1, e) * w1, h1v, l1v);
        const int off = (pc * 8 + e) * kSlicePad + 2 * jp;
        *reinterpret_cast<uint32_t *>(&s_xhi[off]) =
            pack2(__builtin_bit_cast(uint16_t, h0v), __builtin_bit_cast(uint16_t, h1v));
        *reinterpret_cast<uint32_t *>(&s_xlo[off]) =
            pack2(__builtin_bit_cast(uint16_t, l0v), __builtin_bit_cast(uint16_t, l1v));
      }
    }
    for (int u = tid; u < (kSlice / 2) * (N / 8); u += kThreads) {
      const int jp = u / (N / 8), nc8 = u % (N / 8);
      const int j0 = js + 2 * jp;
      const int64_t base = ((b * L + t0 + j0) * a.G + g) * N + nc8 * 8;
      const uint4 r0 = load8_raw(Bp + base, j0 < nvalid);
      const uint4 r1 = load8_raw(Bp + base + a.G * N, j0 + 1 < nvalid);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int off = (nc8 * 8 + e) * kSlicePad + 2 * jp;
        *reinterpret_cast<uint32_t *>(&s_bt[off]) = pack2(elem16(r0, e), elem16(r1, e));
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kSlice / 16; ++ks) {
      const int jo = ks * 16 + 8 * lg;
      bf16x8 ahi[2], alo[2];
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
        const int p = pt * 32 + l32;
        ahi[pt] = *reinterpret_cast<const bf16x8 *>(&s_xhi[p * kSlicePad + jo]);
        alo[pt] = *reinterpret_cast<const bf16x8 *>(&s_xlo[p * kSlicePad + jo]);
      }
#pragma unroll
      for (int q = 0; q < TPW; ++q) {
        const int nt = wave + 4 * q;
        if (nt < NT) {
          const int n = nt * 32 + l32;
          const bf16x8 bv = *reinterpret_cast<const bf16x8 *>(&s_bt[n * kSlicePad + jo]);
#pragma unroll
          for (int pt = 0; pt < 2; ++pt) {
            acc[q][pt] = mfma(ahi[pt], bv, acc[q][pt]);
            acc[q][pt] = mfma(alo[pt], bv, acc[q][pt]);
          }
        }
      }
    }
    __syncthreads();
  }

  float *out = ws_states + ((b * nc + c) * H + h) * (int64_t)kP * N;
#pragma unroll
  for (int q = 0; q < TPW; ++q) {
    const int nt = wave + 4 * q;
    if (nt < NT) {
#pragma unroll
      for (int pt = 0; pt < 2; ++pt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int p = pt * 32 + 8 * (r / 4) + 4 * lg + (r % 4);
          out[p * N + nt * 32 + l32] = acc[q][pt][r];
        }
    }
  }
}

// ---------------------------------------------------------------------------
// 2. state passing
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void ssd_state_pass_kernel(int64_t B, int64_t H, int64_t PN,
                                                              int64_t nc, const float *h0,
                                                              const float *ws_decay,
                                                              float *ws_states, float *h_final) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= B * H * PN) return;
  const int64_t bh = i / PN, e = i % PN;
  const int64_t b = bh / H, h = bh % H;
  float carry = h0 ? h0[i] : 0.f;
  for (int64_t c = 0; c < nc; ++c) {
    const int64_t k = ((b * nc + c) * H + h) * PN + e;
    const float dS = ws_states[k];
    ws_states[k] = carry;
    carry = fmaf(ws_decay[(b * nc + c) * H + h], carry, dS);
  }
  if (h_final) h_final[i] = carry;
}

// ---------------------------------------------------------------------------
// 3. chunk outputs
// ---------------------------------------------------------------------------
constexpr int kQPad = 256 + 8;

template <int N>
__global__ __launch_bounds__(kThreads) void ssd_chunk_scan_kernel(SSDArgs a, const float *ws_states) {
  const int Q = static_cast<int>(a.chunk);
  const int64_t c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t nc = gridDim.x, H = a.H, L = a.L, G = a.G;
  const int64_t g = h / (H / G);
  const int64_t t0 = c * Q;
  const int nvalid = static_cast<int>((L - t0) < Q ? (L - t0) : Q);
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64, lg = lane / 32, l32 = lane % 32;

  __shared__ float s_S[256];
  __shared__ float s_dt[256];
  __shared__ float s_wave[4];
  __shared__ __attribute__((aligned(16))) uint16_t s_x[kP * kQPad];  // x^T: [p][j]

  const uint16_t *dtp = static_cast<const uint16_t *>(a.dt);
  const float A2 = a.A[h] * kLog2e;
  float dtv = 0.f;
  if (tid < nvalid) dtv = bf_to_f(bf16_bits(dtp[(b * L + t0 + tid) * H + h]));
  if (tid < Q) s_dt[tid] = dtv;
  block_inclusive_scan(dtv * A2, s_S, s_wave, Q);

  const uint16_t *xp = static_cast<const uint16_t *>(a.x);
  for (int u = tid; u < (Q / 2) * (kP / 8); u += kThreads) {
    const int jp = u / (kP / 8), pc = u % (kP / 8);
    const int j0 = 2 * jp;
    const int64_t base = ((b * L + t0 + j0) * H + h) * kP + pc * 8;
    const uint4 r0 = load8_raw(xp + base, j0 < nvalid);
    const uint4 r1 = load8_raw(xp + base + H * kP, j0 + 1 < nvalid);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int off = (pc * 8 + e) * kQPad + j0;
      *reinterpret_cast<uint32_t *>(&s_x[off]) = pack2(elem16(r0, e), elem16(r1, e));
    }
  }
  __syncthreads();

  const uint16_t *Bp = static_cast<const uint16_t *>(a.Bm);
  const uint16_t *Cp = static_cast<const uint16_t *>(a.Cm);
  const float *hin = ws_states + ((b * nc + c) * H + h) * (int64_t)kP * N;
  const float Dh = a.D_skip ? a.D_skip[h] : 0.f;
  uint16_t *yp = static_cast<uint16_t *>(a.y);
  const uint16_t *zp = static_cast<const uint16_t *>(a.z);
  constexpr int KS = N / 16;   // K steps over n
  const int nIB = Q / 32;

  // wave -> i-blocks: pair a short and a long block when there are 8
  for (int slot = 0; slot < 2; ++slot) {
    int I;
    if (nIB == 8) I = slot == 0 ? wave : 7 - wave;
    else if (nIB == 4) I = slot == 0 ? wave : -1;
    else I = (slot == 0 && wave < nIB) ? wave : -1;
    if (I < 0) continue;
    const int i_lane = I * 32 + l32;            // this lane's column i in CB^T / row in C frags
    const bool i_ok = i_lane < nvalid;

    // C_I fragments (A-operand rows i for Y_off, B-operand cols i for CB^T)
    bf16x8 cf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      cf[ks] = load8(Cp + ((b * L + t0 + i_lane) * G + g) * N + ks * 16 + 8 * lg, i_ok);

    f32x16 acc[2] = {f32x16{}, f32x16{}};
    // Y_off = C h_in^T  (rows i, cols p), h_in split hi/lo
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
        const float *hr = hin + (pt * 32 + l32) * N + ks * 16 + 8 * lg;
        const float4 v0 = *reinterpret_cast<const float4 *>(hr);
        const float4 v1 = *reinterpret_cast<const float4 *>(hr + 4);
        const float hv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        bf16x8 hh, hl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          __bf16 x1, x2;
          split_bf16(hv[e], x1, x2);
          hh[e] = x1;
          hl[e] = x2;
        }
        acc[pt] = mfma(cf[ks], hh, acc[pt]);
        acc[pt] = mfma(cf[ks], hl, acc[pt]);
      }
    }
    // scale row i by exp(S_i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = I * 32 + 8 * (r / 4) + 4 * lg + (r % 4);
      const float sc = fast_exp2(s_S[i]);
      acc[0][r] *= sc;
      acc[1][r] *= sc;
    }

    // Y_diag
    const float S_i = s_S[i_lane < Q ? i_lane : Q - 1];
    for (int J = 0; J <= I; ++J) {
      const int j_lane = J * 32 + l32;
      const bool j_ok = j_lane < nvalid;
      f32x16 cb = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 bfr = load8(Bp + ((b * L + t0 + j_lane) * G + g) * N + ks * 16 + 8 * lg, j_ok);
        cb = mfma(bfr, cf[ks], cb);        // CB^T[j][i]
      }
      // M[i][j] = CB^T[j][i] * exp(S_i - S_j) * dt_j for j <= i
      bf16x8 mh[2], ml[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = J * 32 + 8 * (r / 4) + 4 * lg + (r % 4);
        float m = 0.f;
        if (j <= i_lane) m = cb[r] * fast_exp2(S_i - s_S[j]) * s_dt[j];
        __bf16 x1, x2;
        split_bf16(m, x1, x2);
        mh[r / 8][r % 8] = x1;
        ml[r / 8][r % 8] = x2;
      }
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const int jb = J * 32 + 16 * k2 + 4 * lg;
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
          const int p = pt * 32 + l32;
          const bf16x4 x0 = *reinterpret_cast<const bf16x4 *>(&s_x[p * kQPad + jb]);
          const bf16x4 x1 = *reinterpret_cast<const bf16x4 *>(&s_x[p * kQPad + jb + 8]);
          const bf16x8 xf = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
          acc[pt] = mfma(mh[k2], xf, acc[pt]);
          acc[pt] = mfma(ml[k2], xf, acc[pt]);
        }
      }
    }

    // epilogue: + D x, gate, store (rows i, cols p)
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      const int p = pt * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = I * 32 + 8 * (r / 4) + 4 * lg + (r % 4);
        if (i < nvalid) {
          const float xv = bf_to_f(bf16_bits(s_x[p * kQPad + i]));
          float v = fmaf(Dh, xv, acc[pt][r]);
          const int64_t idx = ((b * L + t0 + i) * H + h) * kP + p;
          if (zp) v *= silu(bf_to_f(bf16_bits(zp[idx])));
          yp[idx] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
        }
      }
    }
  }
}

template <int N>
hipError_t launch_n(const SSDArgs &a, void *ws, hipStream_t s) {
  const int64_t nc = (a.L + a.chunk - 1) / a.chunk;
  float *states = static_cast<float *>(ws);
  float *decay = states + a.B * nc * a.H * kP * N;
  if (a.L == 0) {
    const int64_t tot = a.B * a.H * kP * N;
    ssd_state_pass_kernel<<<static_cast<unsigned>((tot + 255) / 256), 256, 0, s>>>(
        a.B, a.H, kP * N, 0, a.h0, decay, states, a.h_final);
    return hipGetLastError();
  }
  dim3 grid(static_cast<unsigned>(nc), static_cast<unsigned>(a.H), static_cast<unsigned>(a.B));
  ssd_chunk_state_kernel<N><<<grid, kThreads, 0, s>>>(a, states, decay);
  const int64_t tot = a.B * a.H * kP * N;
  ssd_state_pass_kernel<<<static_cast<unsigned>((tot + 255) / 256), 256, 0, s>>>(
      a.B, a.H, kP * N, nc, a.h0, decay, states, a.h_final);
  ssd_chunk_scan_kernel<N><<<grid, kThreads, 0, s>>>(a, states);
  return hipGetLastError();
}

}  // namespace

int64_t ssd_ws_bytes(int64_t B, int64_t L, int64_t H, int64_t P, int64_t, int64_t N, int64_t chunk) {
  const int64_t nc = (L + chunk - 1) / chunk;
  return (B * nc * H * P * N + B * nc * H) * static_cast<int64_t>(sizeof(float));
}

hipError_t launch_ssd(const SSDArgs &a, void *ws, hipStream_t s) {
  switch (a.N) {
    case 32: return launch_n<32>(a, ws, s);
    case 64: return launch_n<64>(a, ws, s);
    case 96: return launch_n<96>(a, ws, s);
    case 128: return launch_n<128>(a, ws, s);
    case 160: return launch_n<160>(a, ws, s);
    case 192: return launch_n<192>(a, ws, s);
    case 224: return launch_n<224>(a, ws, s);
    case 256: return launch_n<256>(a, ws, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace ssm
