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
// Three kernels:
//  1. ssd_chunk_state: dS = Xw^T B on MFMA (Xw = x scaled by the decay to the
//     chunk end and dt), written fp32 to the workspace; also exp(S_end).
//     N <= 128: one workgroup per (chunk, group) looping over the group's
//     heads (the chunk's B read once); larger N: one per (chunk, head).
//  2. ssd_state_pass: per (b, h, four consecutive (p, n)) the fp32
//     recurrence over chunks, seeded by h0, replacing each dS_c with the
//     state entering chunk c.
//  3. ssd_chunk_scan: CB^T = B C^T on MFMA per 32x32 block pair, decayed in
//     registers (left of the diagonal with the decay factored at the row
//     block's first row, on it element by element and masked), then
//     Y += M X and Y_off = C h_in on MFMA.  N <= 128: one workgroup per
//     (chunk, group) looping over the heads; larger N: one per (chunk, head).
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
#include <type_traits>

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
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// split_bf16 of two values, each half converted as a pair
__device__ __forceinline__ void split_bf16x2(float a, float b, bf16x2 &hi, bf16x2 &lo) {
  hi = __builtin_convertvector(f32x2{a, b}, bf16x2);
  const uint32_t hb = __builtin_bit_cast(uint32_t, hi);
  lo = __builtin_convertvector(f32x2{a - __uint_as_float(hb << 16), b - __uint_as_float(hb & 0xffff0000u)},
                               bf16x2);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts
// by 1, 2, 4, 8 within rows of 16 lanes (lanes without a source add 0), then
// the last lane of row 0 added to row 1 and of row 2 to row 3, then that of
// row 1 to rows 2 and 3.
__device__ __forceinline__ float wave_inclusive_scan(float v) {
  auto shr = [](float x, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value, 0xf, 0xf, true));
  };
  v += shr(v, std::integral_constant<int, 0x111>{});  // row_shr:1
  v += shr(v, std::integral_constant<int, 0x112>{});  // row_shr:2
  v += shr(v, std::integral_constant<int, 0x114>{});  // row_shr:4
  v += shr(v, std::integral_constant<int, 0x118>{});  // row_shr:8
  // row_bcast:15 into rows 1 and 3, row_bcast:31 into rows 2 and 3; other
  // rows keep the 0 passed as the old value
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xc, 0xf, false));
  return v;
}

// Inclusive prefix sum over the Q <= 256 values v (one per thread, threads
// >= Q pass 0) into s_out[0..Q).  Uses DPP moves and one LDS round.
__device__ void block_inclusive_scan(float v, float *s_out, float *s_wave, int Q) {
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  v = wave_inclusive_scan(v);
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

  const uint16_t *xp = static_cast<const uint16_t *>(a.x);
  const uint16_t *Bp = static_cast<const uint16_t *>(a.Bm);
  // Raw x and B of one 64-token slice, loaded into registers one slice
  // ahead so their latency overlaps the previous slice's MFMAs.  Unit u:
  // token pair jp = u % 32 and an 8-wide column chunk u / 32, so that the
  // transposed LDS writes of the 64 lanes of a wave fall in distinct banks
  // (a token pair is one 32-bit word of a transposed row).
  constexpr int kXU = (kSlice / 2) * (kP / 8);                      // x units per slice
  constexpr int kXPer = (kXU + kThreads - 1) / kThreads;
  constexpr int kBU = (kSlice / 2) * (N / 8);                       // B units per slice
  constexpr int kBPer = (kBU + kThreads - 1) / kThreads;
  uint4 xr[kXPer][2], br[kBPer][2];
  auto load_slice = [&](int js) {
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const int u = tid + i * kThreads;
      const int jp = u % (kSlice / 2), pc = u / (kSlice / 2);
      const int j0 = js + 2 * jp;
      const int64_t base = ((b * L + t0 + j0) * H + h) * kP + pc * 8;
      xr[i][0] = load8_raw(xp + base, u < kXU && j0 < nvalid);
      xr[i][1] = load8_raw(xp + base + H * kP, u < kXU && j0 + 1 < nvalid);
    }
#pragma unroll
    for (int i = 0; i < kBPer; ++i) {
      const int u = tid + i * kThreads;
      const int jp = u % (kSlice / 2), nc8 = u / (kSlice / 2);
      const int j0 = js + 2 * jp;
      const int64_t base = ((b * L + t0 + j0) * a.G + g) * N + nc8 * 8;
      br[i][0] = load8_raw(Bp + base, u < kBU && j0 < nvalid);
      br[i][1] = load8_raw(Bp + base + a.G * N, u < kBU && j0 + 1 < nvalid);
    }
  };
  load_slice(0);

  const uint16_t *dtp = static_cast<const uint16_t *>(a.dt);
  const float A2 = a.A[h] * kLog2e;
  float dtv = 0.f;
  if (tid < nvalid)
    dtv = step_size(bf_to_f(bf16_bits(dtp[(b * L + t0 + tid) * H + h])), a.dt_bias ? a.dt_bias[h] : 0.f,
                    a.dt_softplus);
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

  for (int js = 0; js < Q; js += kSlice) {
    // stage x (scaled, split) and B for tokens [js, js+64), transposed
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const int u = tid + i * kThreads;
      if (u < kXU) {
        const int jp = u % (kSlice / 2), pc = u / (kSlice / 2);
        const int j0 = js + 2 * jp;
        const float w0 = s_w[j0], w1 = s_w[j0 + 1];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          __bf16 h0v, l0v, h1v, l1v;
          split_bf16(elem_f32(xr[i][0], e) * w0, h0v, l0v);
          split_bf16(elem_f32(xr[i][1], e) * w1, h1v, l1v);
          const int off = (pc * 8 + e) * kSlicePad + 2 * jp;
          *reinterpret_cast<uint32_t *>(&s_xhi[off]) =
              pack2(__builtin_bit_cast(uint16_t, h0v), __builtin_bit_cast(uint16_t, h1v));
          *reinterpret_cast<uint32_t *>(&s_xlo[off]) =
              pack2(__builtin_bit_cast(uint16_t, l0v), __builtin_bit_cast(uint16_t, l1v));
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kBPer; ++i) {
      const int u = tid + i * kThreads;
      if (u < kBU) {
        const int jp = u % (kSlice / 2), nc8 = u / (kSlice / 2);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int off = (nc8 * 8 + e) * kSlicePad + 2 * jp;
          *reinterpret_cast<uint32_t *>(&s_bt[off]) = pack2(elem16(br[i][0], e), elem16(br[i][1], e));
        }
      }
    }
    __syncthreads();
    if (js + kSlice < Q) load_slice(js + kSlice);
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

// Chunk states for N <= 128: one workgroup of 8 waves per (chunk, group)
// loops over the group's heads, so the chunk's B (shared by the heads of the
// group) is read once instead of once per head.  B^T is staged through LDS
// once and each wave keeps its MFMA fragments of it (its 32 states n, every
// token of the chunk) in registers for all the heads; the LDS then holds x.
// Per head: the cumulative decay, then x scaled by exp(S_end - S_j) dt_j,
// split into bf16 hi + lo and transposed into LDS, then one 32x32 output tile
// per wave over the chunk's tokens.  The next head's x and dt are loaded into
// registers while the current head computes.  The LDS use (67.6 KB) leaves
// room for two workgroups per CU, one staging while the other multiplies.
// x staging unit u (of 128 token pairs x 8 groups of 8 channels): 4
// consecutive lanes read 64 contiguous bytes of a row (p-groups 0-3 or
// 4-7) and a wave covers 16 token pairs.  The transposed 4-byte LDS writes
// of a wave fall on 64 distinct banks at a 130-dword row pitch (p-group
// stride 16 banks, token pairs consecutive), on 32 at 132 dwords.
__device__ __forceinline__ void x_unit(int u, int &jp, int &pc) {
  jp = (u / 4) % 128;
  pc = (u / 512) * 4 + u % 4;
}
constexpr int kCSThreads = 512;
constexpr int kCSPad = 256 + 8;

template <int N, int KS>  // KS = chunk / 16
__global__ __launch_bounds__(kCSThreads, 4) void ssd_chunk_state_group_kernel(SSDArgs a, float *ws_states,
                                                                              float *ws_decay) {
  constexpr int Q = 16 * KS;
  const int64_t c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int64_t nc = gridDim.x, H = a.H, L = a.L, G = a.G;
  const int64_t HPG = H / G;
  const int64_t t0 = c * Q;
  const int nvalid = static_cast<int>((L - t0) < Q ? (L - t0) : Q);
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64, lg = lane / 32, l32 = lane % 32;
  constexpr int NT = N / 32;                               // n tiles
  constexpr int kXU = (256 / 2) * (kP / 8) / kCSThreads;  // x units per thread at Q = 256
  static_assert(kXU * kCSThreads == (256 / 2) * (kP / 8), "x staging must tile");
  static_assert(N <= 2 * kP, "B^T must fit the x buffer");

  __shared__ float s_S[256];
  __shared__ float s_w[256];
  __shared__ float s_wave[kCSThreads / 64];
  // B^T ([n][j]) at the start, then (x w)^T hi ([p][j]) and lo (rows kP..)
  __shared__ __attribute__((aligned(16))) uint16_t s_buf[2 * kP * kCSPad];
  uint16_t *s_xh = s_buf, *s_xl = s_buf + kP * kCSPad;

  const uint16_t *xp = static_cast<const uint16_t *>(a.x);
  const uint16_t *Bp = static_cast<const uint16_t *>(a.Bm);
  const uint16_t *dtp = static_cast<const uint16_t *>(a.dt);

  // x of a head, raw, and its dt (one per thread)
  uint4 xr[kXU][2];
  float dtv = 0.f;
  auto prefetch = [&](int64_t h) {
#pragma unroll
    for (int k = 0; k < kXU; ++k) {
      int jp, pc;
      x_unit(tid + k * kCSThreads, jp, pc);
      const int j0 = 2 * jp;
      const int64_t base = ((b * L + t0 + j0) * H + h) * kP + pc * 8;
      xr[k][0] = load8_raw(xp + base, j0 < nvalid);
      xr[k][1] = load8_raw(xp + base + H * kP, j0 + 1 < nvalid);
    }
    dtv = tid < nvalid ? step_size(bf_to_f(bf16_bits(dtp[(b * L + t0 + tid) * H + h])),
                                   a.dt_bias ? a.dt_bias[h] : 0.f, a.dt_softplus)
                       : 0.f;
  };
  prefetch(g * HPG);

  // B^T of the chunk; unit u: token pair (u / 4) % 128, 8-wide n chunk
  // 4 (u / 512) + u % 4 (4 lanes read 64 contiguous bytes of a row)
  for (int u = tid; u < 128 * (N / 8); u += kCSThreads) {
    const int jp = (u / 4) % 128, nc8 = (u / 512) * 4 + u % 4;
    const int j0 = 2 * jp;
    const int64_t base = ((b * L + t0 + j0) * G + g) * N + nc8 * 8;
    const uint4 r0 = load8_raw(Bp + base, j0 < nvalid);
    const uint4 r1 = load8_raw(Bp + base + G * N, j0 + 1 < nvalid);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *reinterpret_cast<uint32_t *>(&s_buf[(nc8 * 8 + e) * kCSPad + j0]) = pack2(elem16(r0, e), elem16(r1, e));
  }
  __syncthreads();
  const int pt = wave % 2, nt = wave / 2;  // this wave's output tile
  const int p = pt * 32 + l32, n = nt * 32 + l32;
  bf16x8 bfr[KS];                          // B^T fragments of tokens 16 ks + 8 lg .. + 7
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    bfr[ks] = nt < NT ? *reinterpret_cast<const bf16x8 *>(&s_buf[n * kCSPad + ks * 16 + 8 * lg]) : bf16x8{};

  for (int64_t hh = 0; hh < HPG; ++hh) {
    const int64_t h = g * HPG + hh;
    const float A2 = a.A[h] * kLog2e;
    // (its barriers also end the reads of B^T and of the previous head's x)
    block_inclusive_scan(dtv * A2, s_S, s_wave, Q);
    const float S_end = s_S[Q - 1];
    if (tid < Q) s_w[tid] = fast_exp2(S_end - s_S[tid]) * dtv;
    if (tid == 0) ws_decay[(b * nc + c) * H + h] = fast_exp2(S_end);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kXU; ++k) {
      int jp, pc;
      x_unit(tid + k * kCSThreads, jp, pc);
      const int j0 = 2 * jp;
      const float w0 = j0 < Q ? s_w[j0] : 0.f, w1 = j0 + 1 < Q ? s_w[j0 + 1] : 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        __bf16 h0v, l0v, h1v, l1v;
        split_bf16(elem_f32(xr[k][0], e) * w0, h0v, l0v);
        split_bf16(elem_f32(xr[k][1], e) * w1, h1v, l1v);
        const int off = (pc * 8 + e) * kCSPad + j0;
        *reinterpret_cast<uint32_t *>(&s_xh[off]) =
            pack2(__builtin_bit_cast(uint16_t, h0v), __builtin_bit_cast(uint16_t, h1v));
        *reinterpret_cast<uint32_t *>(&s_xl[off]) =
            pack2(__builtin_bit_cast(uint16_t, l0v), __builtin_bit_cast(uint16_t, l1v));
      }
    }
    __syncthreads();
    if (hh + 1 < HPG) prefetch(h + 1);
    if (nt < NT) {
      f32x16 acc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int jo = ks * 16 + 8 * lg;
        const bf16x8 ah = *reinterpret_cast<const bf16x8 *>(&s_xh[p * kCSPad + jo]);
        const bf16x8 al = *reinterpret_cast<const bf16x8 *>(&s_xl[p * kCSPad + jo]);
        acc = mfma(ah, bfr[ks], acc);
        acc = mfma(al, bfr[ks], acc);
      }
      float *out = ws_states + ((b * nc + c) * H + h) * (int64_t)kP * N;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int pr = pt * 32 + 8 * (r / 4) + 4 * lg + (r % 4);
        out[pr * N + n] = acc[r];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 2. state passing
// ---------------------------------------------------------------------------
// Each thread carries four consecutive state elements of one (b, h) over the
// chunks, in place: the slot of chunk c receives the state entering chunk c.
// The chunk loop loads kBatch chunks' updates before it stores any carry, so
// a thread keeps kBatch 16-byte loads in flight (a load of chunk c + 1 would
// otherwise wait for the store to chunk c, which may alias it).
constexpr int kPassBatch = 8;

__global__ __launch_bounds__(256) void ssd_state_pass_kernel(int64_t B, int64_t H, int64_t PN,
                                                              int64_t nc, const float *h0,
                                                              const float *ws_decay,
                                                              float *ws_states, float *h_final) {
  const int64_t i4 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t PN4 = PN / 4;
  if (i4 >= B * H * PN4) return;
  const int64_t bh = i4 / PN4, e4 = i4 % PN4;
  const int64_t b = bh / H, h = bh % H;
  float4 carry = h0 ? reinterpret_cast<const float4 *>(h0)[i4] : make_float4(0.f, 0.f, 0.f, 0.f);
  float4 *st = reinterpret_cast<float4 *>(ws_states);
  for (int64_t c0 = 0; c0 < nc; c0 += kPassBatch) {
    float4 dS[kPassBatch];
    float dc[kPassBatch];
#pragma unroll
    for (int k = 0; k < kPassBatch; ++k) {
      if (c0 + k < nc) {
        dS[k] = st[((b * nc + c0 + k) * H + h) * PN4 + e4];
        dc[k] = ws_decay[(b * nc + c0 + k) * H + h];
      }
    }
#pragma unroll
    for (int k = 0; k < kPassBatch; ++k) {
      if (c0 + k < nc) {
        st[((b * nc + c0 + k) * H + h) * PN4 + e4] = carry;
        carry.x = fmaf(dc[k], carry.x, dS[k].x);
        carry.y = fmaf(dc[k], carry.y, dS[k].y);
        carry.z = fmaf(dc[k], carry.z, dS[k].z);
        carry.w = fmaf(dc[k], carry.w, dS[k].w);
      }
    }
  }
  if (h_final) reinterpret_cast<float4 *>(h_final)[i4] = carry;
}

// ---------------------------------------------------------------------------
// 3. chunk outputs
// ---------------------------------------------------------------------------
// One workgroup of 8 waves per (chunk, group), looping over the group's
// heads.  The chunk's B rows are staged in LDS once (row-major, as the
// A-operand of CB^T = B C^T needs them) and each wave keeps the C fragments
// of its row blocks in registers, so CB^T is recomputed per head from
// on-chip operands only.  Per head, x^T and the state entering the chunk
// (split into bf16 hi + lo) are staged in LDS; the next head's x, state and
// dt are loaded into registers while the current head computes.  Per wave
// and row block I (rows i), one 32-wide p tile:
//   Y_I = exp(S_i) C_I h_in^T + sum_{J <= I} M_IJ X_J,
//   M_IJ[i][j] = CB^T[j][i] exp(S_i - S_j) dt_j (j <= i),
// on the matrix cores with M formed in registers.  With 8 row blocks (Q =
// 256) each wave owns one row block and both p tiles, and the two waves that
// share a SIMD take blocks s and 7 - s, so every SIMD does the same 9 (I, J)
// blocks and each block's M is formed once for both tiles.
// x^T row pitch (elements): 130 dwords, so the 8-byte fragment reads of 32
// consecutive rows cover all 64 banks once
constexpr int kQPad = 256 + 4;
constexpr int kScanThreads = 512;

template <int N>
__global__ __launch_bounds__(kScanThreads, 1) void ssd_chunk_scan_kernel(SSDArgs a, const float *ws_states) {
  const int Q = static_cast<int>(a.chunk);
  const int64_t c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int64_t nc = gridDim.x, H = a.H, L = a.L, G = a.G;
  const int64_t HPG = H / G;
  const int64_t t0 = c * Q;
  const int nvalid = static_cast<int>((L - t0) < Q ? (L - t0) : Q);
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64, lg = lane / 32, l32 = lane % 32;
  constexpr int KS = N / 16;   // K steps over n
  constexpr int kNPad = N + 8;
  constexpr int kXU = (256 / 2) * (kP / 8) / kScanThreads;  // x staging units per thread (Q = 256)
  constexpr int kHTot = kP * N / 4;                          // state float4s
  constexpr int kHU = (kHTot + kScanThreads - 1) / kScanThreads;
  static_assert(kXU >= 1 && kXU * kScanThreads == (256 / 2) * (kP / 8), "x staging must tile");

  __shared__ __attribute__((aligned(16))) float s_S[256];   // in-chunk cumulative log2 decay of the current head
  __shared__ __attribute__((aligned(16))) float s_T[256];   // log2(dt_j) - S_j
  __shared__ __attribute__((aligned(16))) float s_wt[kScanThreads / 64 * 256];  // per wave: w_j
  __shared__ __attribute__((aligned(16))) uint16_t s_b[256 * kNPad];  // B rows: [j][n]
  __shared__ __attribute__((aligned(16))) uint16_t s_x[kP * kQPad];   // x^T: [p][j]
  __shared__ __attribute__((aligned(16))) uint16_t s_hh[kP * kNPad];  // h_in hi: [p][n]
  __shared__ __attribute__((aligned(16))) uint16_t s_hl[kP * kNPad];  // h_in lo

  const uint16_t *Bp = static_cast<const uint16_t *>(a.Bm);
  const uint16_t *Cp = static_cast<const uint16_t *>(a.Cm);
  const uint16_t *xp = static_cast<const uint16_t *>(a.x);
  const uint16_t *dtp = static_cast<const uint16_t *>(a.dt);
  uint16_t *yp = static_cast<uint16_t *>(a.y);
  const uint16_t *zp = static_cast<const uint16_t *>(a.z);
  const int nIB = Q / 32;

  // this wave's row block IA (IA < 0: none) and its p tiles pt0 .. pt0 +
  // npt - 1.  Wave k runs on SIMD k % 4; with 8 row blocks the two waves of
  // a SIMD take blocks s and 7 - s, each with both p tiles, so a block's
  // C B^T and decayed scores are formed once for both tiles and every SIMD
  // does the same 9 (I, J) blocks.
  int IA, pt0, npt;
  {
    const int sm = wave % 4, m = wave / 4;
    if (nIB == 8) {
      IA = (m == 0) ? sm : 7 - sm; pt0 = 0; npt = 2;
    } else if (nIB == 4) {
      IA = sm; pt0 = m; npt = 1;
    } else {
      IA = wave < 4 ? wave % 2 : -1; pt0 = (wave / 2) % 2; npt = 1;
    }
  }
  const bool active = IA >= 0;
  const int iA = (active ? IA : 0) * 32 + l32;  // C row of this lane

  // stage the chunk's B rows (zeros past the end)
  for (int u = tid; u < 256 * (N / 8); u += kScanThreads) {
    const int j = u / (N / 8), n8 = u % (N / 8);
    const uint4 v = load8_raw(Bp + ((b * L + t0 + j) * G + g) * N + n8 * 8, j < nvalid);
    *reinterpret_cast<uint4 *>(&s_b[j * kNPad + n8 * 8]) = v;
  }
  // C fragments of the row blocks (B-operand columns i of CB^T, A-operand
  // rows i of Y_off)
  bf16x8 cfA[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    cfA[ks] = load8(Cp + ((b * L + t0 + iA) * G + g) * N + ks * 16 + 8 * lg, active && iA < nvalid);
  // C B^T block (column block J of the row block whose C fragments are cf),
  // one accumulation chain over the K steps (it runs while the previous
  // block's scores are formed, so its latency is hidden).  All B fragments
  // are read from LDS before the first product.
  auto cb_block = [&](int J, const bf16x8 *cf, f32x16 &acc0) {
    bf16x8 bfr[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      bfr[ks] = *reinterpret_cast<const bf16x8 *>(&s_b[(J * 32 + l32) * kNPad + ks * 16 + 8 * lg]);
    acc0 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc0 = mfma(bfr[ks], cf[ks], acc0);
  };

  // per-head inputs in flight: x (pairs of rows, 8 columns each) and (wave
  // 0) dt of tokens 4 lane .. 4 lane + 3
  uint4 px[kXU][2];
  float pdt[4] = {0.f, 0.f, 0.f, 0.f};
  // x of one (chunk, head) through a buffer resource: row j, column p at
  // ((j * H) * P + p) * 2 bytes; rows past the valid tokens read zeros
  const int x_bytes = static_cast<int>(((nvalid - 1) * H * kP + kP) * 2);
  auto prefetch = [&](int64_t h) {
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(xp + ((b * L + t0) * H + h) * kP), 0, x_bytes, 0x00020000);
#pragma unroll
    for (int k = 0; k < kXU; ++k) {
      int jp, pc;
      x_unit(tid + k * kScanThreads, jp, pc);
      const int j0 = 2 * jp;
      const int off = (j0 * static_cast<int>(H) * kP + pc * 8) * 2;
      const auto v0 = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
      const auto v1 = __builtin_amdgcn_raw_buffer_load_b128(rx, off + static_cast<int>(H) * kP * 2, 0, 0);
      px[k][0] = make_uint4(v0[0], v0[1], v0[2], v0[3]);
      px[k][1] = make_uint4(v1[0], v1[1], v1[2], v1[3]);
    }
    if (wave == 0) {  // raw values: the step-size transform waits for the loads
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 4 * lane + e;
        pdt[e] = j < nvalid ? bf_to_f(bf16_bits(dtp[(b * L + t0 + j) * H + h])) : 0.f;
      }
    }
  };

  prefetch(g * HPG);
  __syncthreads();  // B rows staged
  for (int64_t hh = 0; hh < HPG; ++hh) {
    const int64_t h = g * HPG + hh;
    if (hh > 0) __syncthreads();  // the previous head's LDS reads are done
    // stage x^T and the state split into hi + lo
    const float *hin = ws_states + ((b * nc + c) * H + h) * (int64_t)kP * N;
    float4 ph[kHU];
#pragma unroll
    for (int k = 0; k < kHU; ++k) {
      const int u = tid + k * kScanThreads;
      ph[k] = u < kHTot ? *reinterpret_cast<const float4 *>(hin + 4 * u) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int k = 0; k < kXU; ++k) {
      int jp, pc;
      x_unit(tid + k * kScanThreads, jp, pc);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int off = (pc * 8 + e) * kQPad + 2 * jp;
        *reinterpret_cast<uint32_t *>(&s_x[off]) = pack2(elem16(px[k][0], e), elem16(px[k][1], e));
      }
    }
#pragma unroll
    for (int k = 0; k < kHU; ++k) {
      const int u = tid + k * kScanThreads;
      if (u >= kHTot) break;
      const int p = u / (N / 4), n4 = u % (N / 4);
      const float vv[4] = {ph[k].x, ph[k].y, ph[k].z, ph[k].w};
      uint32_t hw[2], lw[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        __bf16 h0v, l0v, h1v, l1v;
        split_bf16(vv[2 * e], h0v, l0v);
        split_bf16(vv[2 * e + 1], h1v, l1v);
        hw[e] = pack2(__builtin_bit_cast(uint16_t, h0v), __builtin_bit_cast(uint16_t, h1v));
        lw[e] = pack2(__builtin_bit_cast(uint16_t, l0v), __builtin_bit_cast(uint16_t, l1v));
      }
      *reinterpret_cast<uint2 *>(&s_hh[p * kNPad + 4 * n4]) = make_uint2(hw[0], hw[1]);
      *reinterpret_cast<uint2 *>(&s_hl[p * kNPad + 4 * n4]) = make_uint2(lw[0], lw[1]);
    }
    // wave 0: S = inclusive cumsum of dt A (log2 units) and T = log2(dt) - S
    if (wave == 0) {
      const float A2 = a.A[h] * kLog2e;
      const float bias = a.dt_bias ? a.dt_bias[h] : 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) pdt[e] = 4 * lane + e < nvalid ? step_size(pdt[e], bias, a.dt_softplus) : 0.f;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = pdt[e] * A2 + (e > 0 ? v[e - 1] : 0.f);
      const float run = wave_inclusive_scan(v[3]);
      const float excl = run - v[3];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float S = v[e] + excl;
        s_S[4 * lane + e] = S;
        s_T[4 * lane + e] = __builtin_amdgcn_logf(pdt[e]) - S;  // log2; dt = 0 gives -inf
      }
    }
    __syncthreads();
    if (hh + 1 < HPG) prefetch(h + 1);
    if (!active) continue;

    // one row block at a time: Y_off = exp(S_i) C_I h_in^T, then Y_diag
    // (CB^T masked and decayed into M, Y += M X_J), then + D x, gate, store
    const float Dh = a.D_skip ? a.D_skip[h] : 0.f;
    const int64_t head0 = ((b * L + t0) * H + h) * kP;  // element (token t0, head h, p 0)
    const int yz_bytes = static_cast<int>(((nvalid - 1) * H * kP + kP) * 2);
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(yp + head0, 0, yz_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(zp ? zp + head0 : yp + head0), 0, yz_bytes, 0x00020000);
    auto row_block = [&](int I, const bf16x8 *cf) {
      const int i_lane = I * 32 + l32;
      f32x16 acc[2] = {f32x16{}, f32x16{}};  // p tiles pt0, pt0 + 1
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          if (q < npt) {
            const int off = ((pt0 + q) * 32 + l32) * kNPad + ks * 16 + 8 * lg;
            const bf16x8 vh = *reinterpret_cast<const bf16x8 *>(&s_hh[off]);
            const bf16x8 vl = *reinterpret_cast<const bf16x8 *>(&s_hl[off]);
            acc[q] = mfma(cf[ks], vh, acc[q]);
            acc[q] = mfma(cf[ks], vl, acc[q]);
          }
        }
      }
      // Decay of rows i against the columns j < I0 = 32 I left of the
      // diagonal block, factored at row I0:
      //   exp2(S_i - S_j) dt_j = exp2(S_i - S_I0) * (exp2(S_I0 - S_j) dt_j),
      // both factors at most 1 (S falls along the chunk), so neither
      // overflows and one that underflows only drops a product below the
      // fp32 range.  The column factors w_j of this wave's row block are
      // tabulated once per head; Y (with the carried-in term scaled by
      // exp2(S_I0) only) takes the row factors once, before the diagonal
      // block, whose decay is formed element by element.
      const int I0 = I * 32;
      const float S_I0 = s_S[I0];
      float *wt = s_wt + wave * 256;
      {
        const float4 t = *reinterpret_cast<const float4 *>(&s_T[4 * lane]);
        const float tv[4] = {t.x, t.y, t.z, t.w};
        float w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = 4 * lane + e < I0 ? fast_exp2(S_I0 + tv[e]) : 0.f;
        *reinterpret_cast<float4 *>(&wt[4 * lane]) = make_float4(w[0], w[1], w[2], w[3]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      {
        const float e0 = fast_exp2(S_I0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          acc[0][r] *= e0;
          acc[1][r] *= e0;
        }
      }
      const float S_i = s_S[i_lane < Q ? i_lane : Q - 1];
      // software pipeline over the column blocks: the C B^T products of
      // block J + 1 run on the matrix cores while block J's M is formed
      f32x16 cn;
      cb_block(0, cf, cn);
      for (int J = 0; J <= I; ++J) {
        const f32x16 cb = cn;  // (its products were issued a block ago)
        const bool diag = J == I;
        // this block's w_j (log2(dt_j) - S_j on the diagonal) at the rows r
        // of the MFMA layout, and x fragments, read before the next block's
        // products are issued
        const float *src = diag ? s_T : wt;
        float tj[16];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const float4 t = *reinterpret_cast<const float4 *>(&src[J * 32 + 8 * r4 + 4 * lg]);
          tj[4 * r4] = t.x;
          tj[4 * r4 + 1] = t.y;
          tj[4 * r4 + 2] = t.z;
          tj[4 * r4 + 3] = t.w;
        }
        bf16x8 xf[2][2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int pl = (pt0 + (q < npt ? q : 0)) * 32 + l32;
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            const int jb = J * 32 + 16 * k2 + 4 * lg;
            const bf16x4 x0 = *reinterpret_cast<const bf16x4 *>(&s_x[pl * kQPad + jb]);
            const bf16x4 x1 = *reinterpret_cast<const bf16x4 *>(&s_x[pl * kQPad + jb + 8]);
            xf[q][k2] = bf16x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
          }
        }
        if (J < I) cb_block(J + 1, cf, cn);
        __builtin_amdgcn_sched_barrier(0);
        float m[16];
        if (!diag) {
#pragma unroll
          for (int r = 0; r < 16; ++r) m[r] = cb[r] * tj[r];
        } else {
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {  // rows I0 + 8 r4 + 4 lg + 0..3 of Y
            const float4 sv = *reinterpret_cast<const float4 *>(&s_S[I0 + 8 * r4 + 4 * lg]);
            const float su[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float u = fast_exp2(su[e] - S_I0);
              acc[0][4 * r4 + e] *= u;
              acc[1][4 * r4 + e] *= u;
            }
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = J * 32 + 8 * (r / 4) + 4 * lg + (r % 4);
            m[r] = j > i_lane ? 0.f : cb[r] * fast_exp2(S_i + tj[r]);
          }
        }
        bf16x8 mh[2], ml[2];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          bf16x2 hv, lv;
          split_bf16x2(m[r], m[r + 1], hv, lv);
          mh[r / 8][r % 8] = hv[0];
          mh[r / 8][r % 8 + 1] = hv[1];
          ml[r / 8][r % 8] = lv[0];
          ml[r / 8][r % 8 + 1] = lv[1];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          if (q < npt) {
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
              acc[q] = mfma(mh[k2], xf[q][k2], acc[q]);
              acc[q] = mfma(ml[k2], xf[q][k2], acc[q]);
            }
          }
        }
      }
      // y and z of this (chunk, head) through buffer resources with 32-bit
      // offsets: row i, column p at ((i * H) * P + p) * 2 bytes
      // (all reads of a tile are issued before its arithmetic and stores)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        if (q < npt) {
          const int pl = (pt0 + q) * 32 + l32;
          float v[16];
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {  // x of rows i = I*32 + 8 r4 + 4 lg + 0..3
            const bf16x4 xv = *reinterpret_cast<const bf16x4 *>(&s_x[pl * kQPad + I * 32 + 8 * r4 + 4 * lg]);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * r4 + e] = fmaf(Dh, static_cast<float>(xv[e]), acc[q][4 * r4 + e]);
          }
          int off[16];
#pragma unroll
          for (int r = 0; r < 16; ++r)
            off[r] = ((I * 32 + 8 * (r / 4) + 4 * lg + (r % 4)) * static_cast<int>(H) * kP + pl) * 2;
          if (zp) {
            uint32_t zb[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) zb[r] = __builtin_amdgcn_raw_buffer_load_b16(rz, off[r], 0, 0);
#pragma unroll
            for (int r = 0; r < 16; ++r) v[r] *= silu(__uint_as_float(zb[r] << 16));
          }
          // rows past the chunk's valid tokens lie past the resource: dropped
#pragma unroll
          for (int r = 0; r < 16; ++r)
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, static_cast<__bf16>(v[r])), ry,
                                                  off[r], 0, 0);
        }
      }
    };
    row_block(IA, cfA);
  }
}

// Per-(chunk, head) variant for N > 128, whose B rows do not fit in LDS
// beside x and the state: B fragments come from global memory.

// One 32-row block I of a chunk's outputs: the C_I fragments, the running
// Y accumulators (rows i, cols p in two 32-wide p tiles) and S_i.
template <int KS>
struct RowBlock {
  int I;
  int i_lane;
  bf16x8 cf[KS];
  f32x16 acc[2];
  float S_i;
};

template <int N>
__global__ __launch_bounds__(kThreads) void ssd_chunk_scan_head_kernel(SSDArgs a, const float *ws_states) {
  const int Q = static_cast<int>(a.chunk);
  const int64_t c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t nc = gridDim.x, H = a.H, L = a.L, G = a.G;
  const int64_t g = h / (H / G);
  const int64_t t0 = c * Q;
  const int nvalid = static_cast<int>((L - t0) < Q ? (L - t0) : Q);
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64, lg = lane / 32, l32 = lane % 32;
  constexpr int KS = N / 16;   // K steps over n
  constexpr int kNPad = N + 8;

  __shared__ float s_S[256];
  __shared__ float s_dt[256];
  __shared__ float s_wave[4];
  __shared__ __attribute__((aligned(16))) uint16_t s_x[kP * kQPad];   // x^T: [p][j]
  __shared__ __attribute__((aligned(16))) uint16_t s_hh[kP * kNPad];  // h_in hi: [p][n]
  __shared__ __attribute__((aligned(16))) uint16_t s_hl[kP * kNPad];  // h_in lo

  const uint16_t *dtp = static_cast<const uint16_t *>(a.dt);
  const float A2 = a.A[h] * kLog2e;
  float dtv = 0.f;
  if (tid < nvalid)
    dtv = step_size(bf_to_f(bf16_bits(dtp[(b * L + t0 + tid) * H + h])), a.dt_bias ? a.dt_bias[h] : 0.f,
                    a.dt_softplus);
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
  // the state entering the chunk, split once into bf16 hi + lo
  const float *hin = ws_states + ((b * nc + c) * H + h) * (int64_t)kP * N;
  for (int u = tid; u < kP * N / 4; u += kThreads) {
    const int p = u / (N / 4), n4 = u % (N / 4);
    const float4 v = *reinterpret_cast<const float4 *>(hin + p * N + 4 * n4);
    const float vv[4] = {v.x, v.y, v.z, v.w};
    uint32_t hw[2], lw[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      __bf16 h0v, l0v, h1v, l1v;
      split_bf16(vv[2 * e], h0v, l0v);
      split_bf16(vv[2 * e + 1], h1v, l1v);
      hw[e] = pack2(__builtin_bit_cast(uint16_t, h0v), __builtin_bit_cast(uint16_t, h1v));
      lw[e] = pack2(__builtin_bit_cast(uint16_t, l0v), __builtin_bit_cast(uint16_t, l1v));
    }
    *reinterpret_cast<uint2 *>(&s_hh[p * kNPad + 4 * n4]) = make_uint2(hw[0], hw[1]);
    *reinterpret_cast<uint2 *>(&s_hl[p * kNPad + 4 * n4]) = make_uint2(lw[0], lw[1]);
  }
  __syncthreads();

  const uint16_t *Bp = static_cast<const uint16_t *>(a.Bm);
  const uint16_t *Cp = static_cast<const uint16_t *>(a.Cm);
  const float Dh = a.D_skip ? a.D_skip[h] : 0.f;
  uint16_t *yp = static_cast<uint16_t *>(a.y);
  const uint16_t *zp = static_cast<const uint16_t *>(a.z);
  const int nIB = Q / 32;

  // wave -> row blocks: with 8 blocks a long one (7 - w) and a short one (w),
  // which share the B fragments of their common column blocks J <= w
  RowBlock<KS> rb[2];
  rb[0].I = nIB == 8 ? 7 - wave : (wave < nIB ? wave : -1);
  rb[1].I = nIB == 8 ? wave : -1;

#pragma unroll
  for (int s = 0; s < 2; ++s) {
    RowBlock<KS> &R = rb[s];
    if (R.I < 0) continue;
    R.i_lane = R.I * 32 + l32;
    const bool i_ok = R.i_lane < nvalid;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      R.cf[ks] = load8(Cp + ((b * L + t0 + R.i_lane) * G + g) * N + ks * 16 + 8 * lg, i_ok);
    R.S_i = s_S[R.i_lane < Q ? R.i_lane : Q - 1];
    // Y_off = C_I h_in^T (rows i, cols p), then row i scaled by exp(S_i)
    R.acc[0] = R.acc[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
        const int off = (pt * 32 + l32) * kNPad + ks * 16 + 8 * lg;
        const bf16x8 hh = *reinterpret_cast<const bf16x8 *>(&s_hh[off]);
        const bf16x8 hl = *reinterpret_cast<const bf16x8 *>(&s_hl[off]);
        R.acc[pt] = mfma(R.cf[ks], hh, R.acc[pt]);
        R.acc[pt] = mfma(R.cf[ks], hl, R.acc[pt]);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = R.I * 32 + 8 * (r / 4) + 4 * lg + (r % 4);
      const float sc = fast_exp2(s_S[i]);
      R.acc[0][r] *= sc;
      R.acc[1][r] *= sc;
    }
  }

  // Y_diag: for each column block J, CB^T[j][i] = B_J C_I^T on the matrix
  // cores, masked and decayed into M[i][j] = CB^T[j][i] exp(S_i - S_j) dt_j
  // (j <= i), then Y += M X_J.
  auto diag_block = [&](RowBlock<KS> &R, const f32x16 &cb, int J) {
    bf16x8 mh[2], ml[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = J * 32 + 8 * (r / 4) + 4 * lg + (r % 4);
      float m = 0.f;
      if (j <= R.i_lane) m = cb[r] * fast_exp2(R.S_i - s_S[j]) * s_dt[j];
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
        R.acc[pt] = mfma(mh[k2], xf, R.acc[pt]);
        R.acc[pt] = mfma(ml[k2], xf, R.acc[pt]);
      }
    }
  };
  const int Jmax = rb[0].I;  // rb[0] holds the larger block when there are two
  for (int J = 0; J <= Jmax; ++J) {
    const int j_lane = J * 32 + l32;
    const bool j_ok = j_lane < nvalid;
    const bool both = rb[1].I >= 0 && J <= rb[1].I;
    f32x16 cb0 = f32x16{}, cb1 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 bfr = load8(Bp + ((b * L + t0 + j_lane) * G + g) * N + ks * 16 + 8 * lg, j_ok);
      cb0 = mfma(bfr, rb[0].cf[ks], cb0);
      if (both) cb1 = mfma(bfr, rb[1].cf[ks], cb1);
    }
    diag_block(rb[0], cb0, J);
    if (both) diag_block(rb[1], cb1, J);
  }

  // epilogue: + D x, gate, store (rows i, cols p)
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    RowBlock<KS> &R = rb[s];
    if (R.I < 0) continue;
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      const int p = pt * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = R.I * 32 + 8 * (r / 4) + 4 * lg + (r % 4);
        if (i < nvalid) {
          const float xv = bf_to_f(bf16_bits(s_x[p * kQPad + i]));
          float v = fmaf(Dh, xv, R.acc[pt][r]);
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
    const int64_t tot = a.B * a.H * kP * N / 4;
    ssd_state_pass_kernel<<<static_cast<unsigned>((tot + 255) / 256), 256, 0, s>>>(
        a.B, a.H, kP * N, 0, a.h0, decay, states, a.h_final);
    return hipGetLastError();
  }
  dim3 grid(static_cast<unsigned>(nc), static_cast<unsigned>(a.H), static_cast<unsigned>(a.B));
  if constexpr (N <= 128) {
    dim3 grid_g(static_cast<unsigned>(nc), static_cast<unsigned>(a.G), static_cast<unsigned>(a.B));
    if (a.chunk == 64)
      ssd_chunk_state_group_kernel<N, 4><<<grid_g, kCSThreads, 0, s>>>(a, states, decay);
    else if (a.chunk == 128)
      ssd_chunk_state_group_kernel<N, 8><<<grid_g, kCSThreads, 0, s>>>(a, states, decay);
    else
      ssd_chunk_state_group_kernel<N, 16><<<grid_g, kCSThreads, 0, s>>>(a, states, decay);
  } else {
    ssd_chunk_state_kernel<N><<<grid, kThreads, 0, s>>>(a, states, decay);
  }
  const int64_t tot = a.B * a.H * kP * N / 4;  // float4 per thread
  ssd_state_pass_kernel<<<static_cast<unsigned>((tot + 255) / 256), 256, 0, s>>>(
      a.B, a.H, kP * N, nc, a.h0, decay, states, a.h_final);
  if constexpr (N <= 128) {
    dim3 grid_g(static_cast<unsigned>(nc), static_cast<unsigned>(a.G), static_cast<unsigned>(a.B));
    ssd_chunk_scan_kernel<N><<<grid_g, kScanThreads, 0, s>>>(a, states);
  } else {
    ssd_chunk_scan_head_kernel<N><<<grid, kThreads, 0, s>>>(a, states);
  }
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
