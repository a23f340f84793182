// Mamba-1 selective scan kernels for gfx950.
//
// What is computed ("Adding Initial Value Support to Selective Scan Forward
// Kernel", state-spaces/mamba issue 285, and "ggml : add GPU support for
// Mamba models", llama.cpp issue 6758): per (b, d, n)
//   h_t = exp(delta_t A[d,n]) h_{t-1} + delta_t B_t[n] x_t,  h_0 = h0 (or 0)
//   y_t = (sum_n C_t[n] h_t[n] + D[d] x_t) * silu(z_t)
// with the final state written to its own buffer.
//
// Layout in HBM: x, delta, z, y (B, L, D); Bm, Cm (B, L, N); A (D, N);
// h0, h_final (B, D, N).  A wave owns 64 consecutive channels of one
// sequence, so every per-token load and store of x/delta/z/y is one
// contiguous 64-element row segment, and the B/C row of a token is the same
// for the whole wave (scalar loads, shared by all 64 channels).  Each lane
// keeps its channel's N states in VGPRs for the whole token loop.
//
// Two schedules share the token-loop body:
//  * sequential: one pass over all L tokens per wave (no extra work);
//  * chunked: the L axis is cut into segments processed in parallel.  A
//    summary pass runs each segment from a zero state and records the
//    segment's affine map (prod of dA, state reached); a carry pass composes
//    the maps segment by segment from the seed (1, h0) -- the composition
//    (a1, b1) then (a2, b2) = (a2 a1, a2 b1 + b2) of the scan pair
//    (exp(delta A), state) -- and an output pass reruns each segment from its
//    incoming state to produce y.  It costs a second exp per element and is
//    used when B*D is too small to fill the chip.
#include "device_common.h"
#include "launch.h"

namespace ssm {
namespace {

constexpr int kWave = 64;
constexpr int kPrefetch = 8;  // tokens of x/delta/z kept in flight per lane

enum Mode : int { kFull = 0, kSummary = 1, kOutput = 2 };

template <typename T>
__device__ __forceinline__ T ld(const T *p) { return *p; }

// One kernel body for the three roles.  Grid: x = 64-channel tile, y =
// segment, z = sequence b.
//   kFull:    segment = all of L; h starts at h0 (or 0); writes y, h_final.
//   kSummary: h starts at 0; writes seg_a[n] = exp(A * sum delta) and
//             seg_h[n] = state reached, per (b, seg, d, n).
//   kOutput:  h starts at seg_h (overwritten with the incoming state by the
//             carry pass); writes y.
template <typename T, int NB, bool EXACT, int MODE>
__global__ __launch_bounds__(kWave) void scan_kernel(ScanArgs a, int64_t seg_len, float *seg_a,
                                                     float *seg_h) {
  const int64_t D = a.D, L = a.L;
  const int N = EXACT ? NB : static_cast<int>(a.N);
  const int lane = threadIdx.x;
  const int64_t d_raw = static_cast<int64_t>(blockIdx.x) * kWave + lane;
  const bool active = d_raw < D;
  const int64_t d = active ? d_raw : D - 1;  // clamped: loads stay in bounds
  const int64_t seg = blockIdx.y;
  const int64_t nseg = gridDim.y;
  const int64_t b = blockIdx.z;
  const int64_t t0 = seg * seg_len;
  const int64_t t1 = (t0 + seg_len < L) ? t0 + seg_len : L;

  float A2[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) A2[n] = (EXACT || n < N) ? a.A[d * N + n] * kLog2e : 0.f;

  const int64_t ws_row = ((b * nseg + seg) * D + d) * N;
  float h[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    float v = 0.f;
    if (EXACT || n < N) {
      if (MODE == kFull && a.h0 != nullptr) v = a.h0[(b * D + d) * N + n];
      if (MODE == kOutput) v = seg_h[ws_row + n];
    }
    h[n] = v;
  }

  const T *xp = static_cast<const T *>(a.x) + b * L * D + d;
  const T *dp = static_cast<const T *>(a.delta) + b * L * D + d;
  const T *zp = a.z ? static_cast<const T *>(a.z) + b * L * D + d : nullptr;
  T *yp = static_cast<T *>(a.y) + b * L * D + d;
  const T *Bp = static_cast<const T *>(a.Bm) + b * L * N;
  const T *Cp = static_cast<const T *>(a.Cm) + b * L * N;
  const float Dd = a.D_skip ? a.D_skip[d] : 0.f;
  const bool has_z = zp != nullptr;

  float dsum = 0.f;

  T xr[kPrefetch], dr[kPrefetch], zr[kPrefetch];
#pragma unroll
  for (int j = 0; j < kPrefetch; ++j) {
    int64_t t = t0 + j < t1 ? t0 + j : t1 - 1;
    if (t < t0) t = t0;  // empty segment: never used, keep in bounds
    if (t1 > t0) {
      xr[j] = ld(xp + t * D);
      dr[j] = ld(dp + t * D);
      if (MODE != kSummary && has_z) zr[j] = ld(zp + t * D);
    }
  }

  for (int64_t tb = t0; tb < t1; tb += kPrefetch) {
    T xn[kPrefetch], dn[kPrefetch], zn[kPrefetch];
    const bool more = tb + kPrefetch < t1;
    if (more) {
#pragma unroll
      for (int j = 0; j < kPrefetch; ++j) {
        int64_t t = tb + kPrefetch + j;
        t = t < t1 ? t : t1 - 1;
        xn[j] = ld(xp + t * D);
        dn[j] = ld(dp + t * D);
        if (MODE != kSummary && has_z) zn[j] = ld(zp + t * D);
      }
    }
#pragma unroll
    for (int j = 0; j < kPrefetch; ++j) {
      const int64_t t = tb + j;
      if (t < t1) {
        const float dl = to_f32(dr[j]);
        const float xv = to_f32(xr[j]);
        const float u = dl * xv;
        const T *Bt = Bp + t * N;
        const T *Ct = Cp + t * N;
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
        for (int n = 0; n < NB; ++n) {
          if (EXACT || n < N) {
            const float dA = fast_exp2(dl * A2[n]);
            h[n] = fmaf(dA, h[n], u * to_f32(Bt[n]));
            if (MODE != kSummary) {
              if (n & 1)
                acc1 = fmaf(to_f32(Ct[n]), h[n], acc1);
              else
                acc0 = fmaf(to_f32(Ct[n]), h[n], acc0);
            }
          }
        }
        if (MODE == kSummary) {
          dsum += dl;
        } else {
          float v = fmaf(Dd, xv, acc0 + acc1);
          if (has_z) v *= silu(to_f32(zr[j]));
          if (active) yp[t * D] = from_f32<T>(v);
        }
      }
    }
    if (more) {
#pragma unroll
      for (int j = 0; j < kPrefetch; ++j) {
        xr[j] = xn[j];
        dr[j] = dn[j];
        if (MODE != kSummary && has_z) zr[j] = zn[j];
      }
    }
  }

  if (!active) return;
  if (MODE == kFull && a.h_final != nullptr) {
#pragma unroll
    for (int n = 0; n < NB; ++n)
      if (EXACT || n < N) a.h_final[(b * D + d) * N + n] = h[n];
  }
  if (MODE == kSummary) {
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      if (EXACT || n < N) {
        seg_a[ws_row + n] = fast_exp2(A2[n] * dsum);
        seg_h[ws_row + n] = h[n];
      }
    }
  }
}

// Carry pass: one thread per (b, d, n); walks the segments in order,
// replacing each segment's summary state with the state entering it, and
// writes h_final.  carry <- a_seg * carry + h_seg composes the segment's
// affine map after the carry (seed (1, h0)).
__global__ __launch_bounds__(256) void scan_carry_kernel(int64_t B, int64_t D, int64_t N,
                                                          int64_t nseg, const float *h0,
                                                          const float *seg_a, float *seg_h,
                                                          float *h_final) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t DN = D * N;
  if (i >= B * DN) return;
  const int64_t b = i / DN;
  const int64_t dn = i - b * DN;
  float carry = h0 ? h0[i] : 0.f;
  for (int64_t s = 0; s < nseg; ++s) {
    const int64_t k = (b * nseg + s) * DN + dn;
    const float av = seg_a[k];
    const float hv = seg_h[k];
    seg_h[k] = carry;
    carry = fmaf(av, carry, hv);
  }
  if (h_final) h_final[i] = carry;
}

template <typename T, int NB, bool EXACT>
hipError_t launch_full_t(const ScanArgs &a, hipStream_t s) {
  dim3 grid(static_cast<unsigned>((a.D + kWave - 1) / kWave), 1, static_cast<unsigned>(a.B));
  scan_kernel<T, NB, EXACT, kFull><<<grid, kWave, 0, s>>>(a, a.L, nullptr, nullptr);
  return hipGetLastError();
}

template <typename T, int NB, bool EXACT>
hipError_t launch_chunked_t(const ScanArgs &a, int64_t seg_len, float *ws, hipStream_t s) {
  const int64_t nseg = (a.L + seg_len - 1) / seg_len;
  float *seg_a = ws;
  float *seg_h = ws + a.B * nseg * a.D * a.N;
  dim3 grid(static_cast<unsigned>((a.D + kWave - 1) / kWave), static_cast<unsigned>(nseg),
            static_cast<unsigned>(a.B));
  scan_kernel<T, NB, EXACT, kSummary><<<grid, kWave, 0, s>>>(a, seg_len, seg_a, seg_h);
  const int64_t total = a.B * a.D * a.N;
  scan_carry_kernel<<<static_cast<unsigned>((total + 255) / 256), 256, 0, s>>>(
      a.B, a.D, a.N, nseg, a.h0, seg_a, seg_h, a.h_final);
  scan_kernel<T, NB, EXACT, kOutput><<<grid, kWave, 0, s>>>(a, seg_len, seg_a, seg_h);
  return hipGetLastError();
}

// N bucket dispatch: exact instantiations for the common N, guarded buckets
// for the rest.
template <typename T, template <typename, int, bool> class F, typename... Args>
hipError_t dispatch_n(int64_t N, Args &&...args) {
  switch (N) {
    case 4: return F<T, 4, true>::run(args...);
    case 8: return F<T, 8, true>::run(args...);
    case 16: return F<T, 16, true>::run(args...);
    case 32: return F<T, 32, true>::run(args...);
    case 64: return F<T, 64, true>::run(args...);
    default: break;
  }
  if (N <= 4) return F<T, 4, false>::run(args...);
  if (N <= 8) return F<T, 8, false>::run(args...);
  if (N <= 16) return F<T, 16, false>::run(args...);
  if (N <= 32) return F<T, 32, false>::run(args...);
  return F<T, 64, false>::run(args...);
}

template <typename T, int NB, bool EXACT>
struct FullRunner {
  static hipError_t run(const ScanArgs &a, hipStream_t s) { return launch_full_t<T, NB, EXACT>(a, s); }
};
template <typename T, int NB, bool EXACT>
struct ChunkRunner {
  static hipError_t run(const ScanArgs &a, int64_t seg_len, float *ws, hipStream_t s) {
    return launch_chunked_t<T, NB, EXACT>(a, seg_len, ws, s);
  }
};

}  // namespace

hipError_t launch_scan_sequential(const ScanArgs &a, hipStream_t s) {
  if (a.dt == DType::BF16) return dispatch_n<bf16_t, FullRunner>(a.N, a, s);
  return dispatch_n<float, FullRunner>(a.N, a, s);
}

int64_t scan_chunked_ws_floats(int64_t B, int64_t L, int64_t D, int64_t N, int64_t seg_len) {
  const int64_t nseg = (L + seg_len - 1) / seg_len;
  return 2 * B * nseg * D * N;
}

hipError_t launch_scan_chunked(const ScanArgs &a, int64_t seg_len, float *ws, hipStream_t s) {
  if (a.dt == DType::BF16) return dispatch_n<bf16_t, ChunkRunner>(a.N, a, seg_len, ws, s);
  return dispatch_n<float, ChunkRunner>(a.N, a, seg_len, ws, s);
}

}  // namespace ssm
