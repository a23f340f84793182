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
// h0, h_final (B, D, N).
//
// Work decomposition (split kernel).  A workgroup owns 64 consecutive
// channels of one sequence; its W waves split the N states of those
// channels (SPL = states per lane, W * SPL >= N).  Each lane keeps its SPL
// states in VGPRs for the whole token loop, so the per-element work is the
// bare recurrence: one v_exp_f32 and four fp32 VALU ops.  Splitting N over
// waves multiplies the number of independent waves by W, which the chip
// needs (B*D/64 alone is 640 waves at the 2.8B prefill shape, fewer than
// the 1024 SIMDs).
//  * x/delta/z rows of a block of TB tokens are loaded two blocks ahead,
//    coalesced over the 64 channels, converted once, and staged in LDS as
//    delta, u = delta*x, D*x and z (fp32); every wave reads them from there.
//  * B/C rows are shared by all channels: they are staged in LDS with the
//    same two-block lead, converted to fp32 and laid out per wave, so each
//    wave reads its token's SPL B and C values with uniform-address LDS
//    reads (a broadcast to all 64 lanes).  LDS reads complete in order, so
//    the compiler can keep them in flight across tokens with partial waits
//    (scalar loads could only be waited for all at once).
//  * Each wave's partial y (its states' share of sum_n C h) goes to LDS;
//    after a barrier per block, every wave finishes 1/W of the block's
//    tokens: sums the partials, applies the gate and stores y.
//
// Schedules:
//  * sequential: one pass over all L tokens per workgroup;
//  * chunked: the L axis is cut into segments processed in parallel.  A
//    summary pass runs each segment from a zero state and records the
//    segment's affine map (prod of dA = exp(A sum delta), state reached); a
//    carry pass composes the maps segment by segment from the seed (1, h0)
//    -- the composition (a1, b1) then (a2, b2) = (a2 a1, a2 b1 + b2) of the
//    scan pair (exp(delta A), state) -- and an output pass reruns each
//    segment from its incoming state to produce y.  It costs a second exp per
//    element and is chosen when B*D is too small to fill the chip.
//
// A third, workspace-free kernel keeps all N states of a channel in one lane
// (no cross-wave reduction); the decode step uses it for shapes its
// vectorised kernel does not cover.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace ssm {
namespace {

constexpr int kWave = 64;

enum Mode : int { kFull = 0, kSummary = 1, kOutput = 2 };

template <int K>
using f32v = float __attribute__((ext_vector_type(K)));
template <int K>
using cf32v = __attribute__((address_space(4))) const f32v<K>;

// ---------------------------------------------------------------------------
// Buffer access to the per-sequence (L, D) planes of x, delta, z and y: the
// lane offset (d * bytes) is fixed for the whole kernel and the token offset
// (t * D * bytes) is a scalar, so a load or store costs no VALU address math.
// Accesses past the plane (never issued here) would return 0.
// ---------------------------------------------------------------------------
constexpr int kRsrcWord3 = 0x00020000;

template <typename T>
struct Plane {
  __amdgpu_buffer_rsrc_t r;
  __device__ Plane(const void *base, int64_t bytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0,
                                            static_cast<int>(bytes > 0x7fffffff ? 0x7fffffff : bytes),
                                            kRsrcWord3)) {}
  __device__ __forceinline__ T load(uint32_t voff, uint32_t soff) const {
    if constexpr (sizeof(T) == 2) {
      bf16_t v;
      v.bits = __builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(voff), static_cast<int>(soff), 0);
      return v;
    } else {
      return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(voff),
                                                                  static_cast<int>(soff), 0));
    }
  }
  __device__ __forceinline__ void store(T v, uint32_t voff, uint32_t soff) const {
    if constexpr (sizeof(T) == 2) {
      __builtin_amdgcn_raw_buffer_store_b16(v.bits, r, static_cast<int>(voff), static_cast<int>(soff), 0);
    } else {
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, static_cast<int>(voff),
                                            static_cast<int>(soff), 0);
    }
  }
};

// ---------------------------------------------------------------------------
// Split kernel.  Grid: x = 64-channel tile, y = segment, z = sequence b.
//   kFull:    segment = all of L; h starts at h0 (or 0); writes y, h_final.
//   kSummary: h starts at 0; writes seg_a[n] = exp(A * sum delta) and
//             seg_h[n] = state reached, per (b, seg, d, n).
//   kOutput:  h starts at seg_h (the state entering the segment, written by
//             the carry pass); writes y.
// Segment lengths are multiples of TB.  Tokens past the end of the last
// block are staged with delta = u = 0, for which dA = 1 and the update adds
// 0, so the state passes through them unchanged and no per-token branch is
// needed.
// ---------------------------------------------------------------------------
template <typename T, int SPL, int W, int TB, int MODE, bool HAS_Z>
__global__ __launch_bounds__(kWave *W) void scan_split_kernel(ScanArgs a, int64_t seg_len,
                                                              float *seg_a, float *seg_h) {
  constexpr bool kY = MODE != kSummary;
  constexpr int kNP = SPL * W;             // padded N
  constexpr int kTokPerThread = TB / W;    // x/delta/z tokens each thread stages per block
  static_assert(TB % W == 0, "W must divide the block length");
  constexpr int kBC = TB * 2 * kNP;        // B/C values per block
  constexpr int kBCPerThread = (kBC + kWave * W - 1) / (kWave * W);
  constexpr uint32_t kES = sizeof(T);

  __shared__ float2 s_du[2][TB][kWave];  // (delta, u = delta * x)
  __shared__ __attribute__((aligned(16))) float s_bc[2][TB][W][2][SPL];  // B, C per wave
  __shared__ float s_dx[3][TB][kWave];   // D[d] * x
  __shared__ float s_z[3][TB][kWave];
  __shared__ float s_y[2][W][TB][kWave];

  const int64_t D = a.D, L = a.L;
  const int N = static_cast<int>(a.N);
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int64_t d_raw = static_cast<int64_t>(blockIdx.x) * kWave + lane;
  const bool active = d_raw < D;
  const int64_t d = active ? d_raw : D - 1;
  const int64_t seg = blockIdx.y, nseg = gridDim.y, b = blockIdx.z;
  const int64_t t0 = seg * seg_len;
  const int64_t t1 = (t0 + seg_len < L) ? t0 + seg_len : L;
  const int64_t nblk = (t1 - t0 + TB - 1) / TB;
  const int n0 = wave * SPL;

  float A2[SPL], h[SPL];
  const int64_t ws_row = ((b * nseg + seg) * D + d) * N;
#pragma unroll
  for (int s = 0; s < SPL; ++s) {
    const int n = n0 + s;
    const bool ok = n < N;
    A2[s] = ok ? a.A[d * N + n] * kLog2e : 0.f;
    float v = 0.f;
    if (ok && MODE == kFull && a.h0 != nullptr) v = a.h0[(b * D + d) * N + n];
    if (ok && MODE == kOutput) v = seg_h[ws_row + n];
    h[s] = v;
  }

  const int64_t plane = L * D * kES;  // bytes of one sequence's (L, D) plane
  const Plane<T> px(static_cast<const char *>(a.x) + b * plane, plane);
  const Plane<T> pd(static_cast<const char *>(a.delta) + b * plane, plane);
  constexpr bool has_z = kY && HAS_Z;
  const Plane<T> pz(has_z ? static_cast<const char *>(a.z) + b * plane : static_cast<const char *>(a.x),
                    plane);
  const Plane<T> py(static_cast<char *>(a.y) + b * plane, plane);
  const uint32_t voff = static_cast<uint32_t>(d * kES);
  const uint32_t row_bytes = static_cast<uint32_t>(D * kES);
  const int64_t bcplane = L * N * kES;
  const Plane<T> pb(static_cast<const char *>(a.Bm) + b * bcplane, bcplane);
  const Plane<T> pc(static_cast<const char *>(a.Cm) + b * bcplane, bcplane);
  const float Dd = (a.D_skip != nullptr) ? a.D_skip[d] : 0.f;

  // This thread's share of a block's B/C values: entry e = tid + i*64W of
  // [which][token j][n] (n padded to kNP), read from (b, t, n) of B or C.
  uint32_t bc_vo[kBCPerThread];
  int bc_j[kBCPerThread], bc_n[kBCPerThread], bc_w[kBCPerThread];
  bool bc_on[kBCPerThread];
#pragma unroll
  for (int i = 0; i < kBCPerThread; ++i) {
    const int e = tid + i * kWave * W;
    bc_on[i] = e < kBC;
    const int ee = bc_on[i] ? e : 0;
    bc_w[i] = ee / (TB * kNP);
    bc_j[i] = (ee / kNP) % TB;
    bc_n[i] = ee % kNP;
    const int n = bc_n[i] < N ? bc_n[i] : N - 1;
    bc_vo[i] = static_cast<uint32_t>((bc_j[i] * N + n) * kES);
  }
  const uint32_t tok0 = static_cast<uint32_t>(t0);        // first token of the segment
  const uint32_t ntok = static_cast<uint32_t>(t1 - t0);   // tokens in the segment

  // raw inputs of two blocks in flight.  Loads run past the segment end at
  // most into the next segment or past the plane (which reads 0); stage()
  // zeroes delta and u there.
  struct RawBlock {
    T x[kTokPerThread], d[kTokPerThread], z[kTokPerThread], bc[kBCPerThread];
  };
  RawBlock raw0, raw1;

  auto issue = [&](RawBlock &r, int64_t blk) {
    const uint32_t tb = tok0 + static_cast<uint32_t>(blk) * TB;
#pragma unroll
    for (int i = 0; i < kTokPerThread; ++i) {
      const uint32_t so = (tb + wave + i * W) * row_bytes;
      r.x[i] = px.load(voff, so);
      r.d[i] = pd.load(voff, so);
      if (has_z) r.z[i] = pz.load(voff, so);
    }
    const uint32_t bso = tb * static_cast<uint32_t>(N) * kES;
#pragma unroll
    for (int i = 0; i < kBCPerThread; ++i) {
      const T vb = pb.load(bc_vo[i], bso);
      const T vc = pc.load(bc_vo[i], bso);
      r.bc[i] = bc_w[i] ? vc : vb;
    }
  };
  auto stage = [&](const RawBlock &r, int64_t blk) {
    const int b2 = static_cast<int>(blk & 1), b3 = static_cast<int>(blk % 3);
    const uint32_t jb = static_cast<uint32_t>(blk) * TB;  // block start within the segment
#pragma unroll
    for (int i = 0; i < kTokPerThread; ++i) {
      const int j = wave + i * W;
      const bool ok = jb + j < ntok;
      const float dl = ok ? to_f32(r.d[i]) : 0.f;
      const float xv = ok ? to_f32(r.x[i]) : 0.f;
      s_du[b2][j][lane] = make_float2(dl, dl * xv);
      if (kY) {
        s_dx[b3][j][lane] = Dd * xv;
        if (has_z) s_z[b3][j][lane] = to_f32(r.z[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < kBCPerThread; ++i) {
      if (bc_on[i]) {
        const int n = bc_n[i];
        s_bc[b2][bc_j[i]][n / SPL][bc_w[i]][n % SPL] = n < N ? to_f32(r.bc[i]) : 0.f;
      }
    }
  };

  float dsum = 0.f;
  // recurrence over the TB tokens of block blk
  auto run_block = [&](int64_t blk) {
    const int b2 = static_cast<int>(blk & 1);
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      const float2 du = s_du[b2][j][lane];
      float Bv[SPL], Cv[SPL];
#pragma unroll
      for (int s = 0; s < SPL; ++s) {
        Bv[s] = s_bc[b2][j][wave][0][s];
        Cv[s] = s_bc[b2][j][wave][1][s];
      }
      float acc = 0.f;
#pragma unroll
      for (int s = 0; s < SPL; ++s) {
        const float dA = fast_exp2(du.x * A2[s]);
        h[s] = fmaf(dA, h[s], du.y * Bv[s]);
        if (kY) acc = fmaf(Cv[s], h[s], acc);
      }
      if (kY) s_y[b2][wave][j][lane] = acc;
      if (MODE == kSummary) dsum += du.x;
    }
  };
  auto reduce_block = [&](int64_t blk) {
    const int b2 = static_cast<int>(blk & 1), b3 = static_cast<int>(blk % 3);
    const uint32_t jb = static_cast<uint32_t>(blk) * TB;
#pragma unroll
    for (int i = 0; i < kTokPerThread; ++i) {
      const int j = wave * kTokPerThread + i;
      const uint32_t jj = jb + j;
      float v = s_y[b2][0][j][lane];
#pragma unroll
      for (int w = 1; w < W; ++w) v += s_y[b2][w][j][lane];
      v += s_dx[b3][j][lane];
      if (has_z) v *= silu(s_z[b3][j][lane]);
      if (jj < ntok && active) py.store(from_f32<T>(v), voff, (tok0 + jj) * row_bytes);
    }
  };

  if (nblk > 0) {
    issue(raw0, 0);
    issue(raw1, 1);
    stage(raw0, 0);
    __syncthreads();
  }
  for (int64_t k = 0; k < nblk; k += 2) {
    // raw0 holds block k (already staged), raw1 holds block k+1
    issue(raw0, k + 2);
    run_block(k);
    stage(raw1, k + 1);
    __syncthreads();
    if (kY) reduce_block(k);
    if (k + 1 >= nblk) break;
    issue(raw1, k + 3);
    run_block(k + 1);
    stage(raw0, k + 2);
    __syncthreads();
    if (kY) reduce_block(k + 1);
  }

  if (!active) return;
#pragma unroll
  for (int s = 0; s < SPL; ++s) {
    const int n = n0 + s;
    if (n < N) {
      if (MODE == kFull && a.h_final != nullptr) a.h_final[(b * D + d) * N + n] = h[s];
      if (MODE == kSummary) {
        seg_a[ws_row + n] = fast_exp2(A2[s] * dsum);
        seg_h[ws_row + n] = h[s];
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

// ---------------------------------------------------------------------------
// Per-lane kernel (no workspace): one lane holds all N states of a channel.
// Used by the decode step for shapes its vectorised kernel does not cover;
// h0 and h_final may alias (each lane reads its row before writing it).
// ---------------------------------------------------------------------------
template <typename T, int NB, bool EXACT>
__global__ __launch_bounds__(kWave) void scan_lane_kernel(ScanArgs a) {
  const int64_t D = a.D, L = a.L;
  const int N = EXACT ? NB : static_cast<int>(a.N);
  const int lane = threadIdx.x;
  const int64_t d_raw = static_cast<int64_t>(blockIdx.x) * kWave + lane;
  const bool active = d_raw < D;
  const int64_t d = active ? d_raw : D - 1;
  const int64_t b = blockIdx.z;

  float A2[NB], h[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    const bool ok = EXACT || n < N;
    A2[n] = ok ? a.A[d * N + n] * kLog2e : 0.f;
    h[n] = (ok && a.h0 != nullptr) ? a.h0[(b * D + d) * N + n] : 0.f;
  }
  // B/C rows are the same for every lane: scalar loads of the raw bits
  using Bits = typename std::conditional<sizeof(T) == 2, uint16_t, float>::type;
  using BT = __attribute__((address_space(4))) const Bits;
  const BT *Bp = (const BT *)(a.Bm) + b * L * N;
  const BT *Cp = (const BT *)(a.Cm) + b * L * N;
  auto bc_f32 = [](Bits v) -> float {
    if constexpr (sizeof(T) == 2) return __uint_as_float(static_cast<uint32_t>(v) << 16);
    else return v;
  };
  const T *xp = static_cast<const T *>(a.x) + b * L * D + d;
  const T *dp = static_cast<const T *>(a.delta) + b * L * D + d;
  const T *zp = a.z ? static_cast<const T *>(a.z) + b * L * D + d : nullptr;
  T *yp = static_cast<T *>(a.y) + b * L * D + d;
  const float Dd = a.D_skip ? a.D_skip[d] : 0.f;
  for (int64_t t = 0; t < L; ++t) {
    const float dl = to_f32(dp[t * D]);
    const float xv = to_f32(xp[t * D]);
    const float u = dl * xv;
    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      if (EXACT || n < N) {
        const float dA = fast_exp2(dl * A2[n]);
        h[n] = fmaf(dA, h[n], u * bc_f32(Bp[t * N + n]));
        if (n & 1)
          acc1 = fmaf(bc_f32(Cp[t * N + n]), h[n], acc1);
        else
          acc0 = fmaf(bc_f32(Cp[t * N + n]), h[n], acc0);
      }
    }
    float v = fmaf(Dd, xv, acc0 + acc1);
    if (zp) v *= silu(to_f32(zp[t * D]));
    if (active) yp[t * D] = from_f32<T>(v);
  }
  if (!active || a.h_final == nullptr) return;
#pragma unroll
  for (int n = 0; n < NB; ++n)
    if (EXACT || n < N) a.h_final[(b * D + d) * N + n] = h[n];
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct SplitCfg {
  int spl, w;
};

// tokens per LDS stage / barrier (segment lengths are multiples of it)
#ifndef SSM_SCAN_BLOCK_TOKENS
#define SSM_SCAN_BLOCK_TOKENS 8
#endif
constexpr int kBlockTokens = SSM_SCAN_BLOCK_TOKENS;

}  // namespace

// States per lane and waves per workgroup for a given N (tuning may force spl).
static SplitCfg split_cfg(int64_t N, int spl_req) {
  if (spl_req == 2 || spl_req == 4 || spl_req == 8 || spl_req == 16) {
    int w = static_cast<int>((N + spl_req - 1) / spl_req);
    if (w < 1) w = 1;
    if (w <= 8 && (w == 1 || w == 2 || w == 4 || w == 8)) return {spl_req, w};
  }
  if (N <= 4) return {4, 1};
  if (N <= 8) return {4, 2};
  if (N <= 16) return {4, 4};
  if (N <= 32) return {8, 4};
  return {16, 4};
}

namespace {

template <typename T, int SPL, int W>
hipError_t launch_split_t(const ScanArgs &a, int64_t seg_len, float *seg_a, float *seg_h,
                          hipStream_t s) {
  constexpr int TB = kBlockTokens;
  const unsigned tiles = static_cast<unsigned>((a.D + kWave - 1) / kWave);
  if (seg_a == nullptr) {
    dim3 grid(tiles, 1, static_cast<unsigned>(a.B));
    if (a.z)
      scan_split_kernel<T, SPL, W, TB, kFull, true><<<grid, kWave * W, 0, s>>>(a, a.L, nullptr, nullptr);
    else
      scan_split_kernel<T, SPL, W, TB, kFull, false><<<grid, kWave * W, 0, s>>>(a, a.L, nullptr, nullptr);
    return hipGetLastError();
  }
  const int64_t nseg = (a.L + seg_len - 1) / seg_len;
  dim3 grid(tiles, static_cast<unsigned>(nseg), static_cast<unsigned>(a.B));
  scan_split_kernel<T, SPL, W, TB, kSummary, false><<<grid, kWave * W, 0, s>>>(a, seg_len, seg_a, seg_h);
  const int64_t total = a.B * a.D * a.N;
  scan_carry_kernel<<<static_cast<unsigned>((total + 255) / 256), 256, 0, s>>>(
      a.B, a.D, a.N, nseg, a.h0, seg_a, seg_h, a.h_final);
  if (a.z)
    scan_split_kernel<T, SPL, W, TB, kOutput, true><<<grid, kWave * W, 0, s>>>(a, seg_len, seg_a, seg_h);
  else
    scan_split_kernel<T, SPL, W, TB, kOutput, false><<<grid, kWave * W, 0, s>>>(a, seg_len, seg_a, seg_h);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch_split(const ScanArgs &a, int spl_req, int64_t seg_len, float *seg_a,
                          float *seg_h, hipStream_t s) {
  const SplitCfg c = split_cfg(a.N, spl_req);
#define SSM_CASE(S, Wv)        \
  if (c.spl == S && c.w == Wv) \
    return launch_split_t<T, S, Wv>(a, seg_len, seg_a, seg_h, s);
  SSM_CASE(4, 1) SSM_CASE(4, 2) SSM_CASE(4, 4) SSM_CASE(8, 4) SSM_CASE(16, 4)
  SSM_CASE(2, 8) SSM_CASE(2, 4) SSM_CASE(2, 2) SSM_CASE(2, 1)
  SSM_CASE(8, 1) SSM_CASE(8, 2) SSM_CASE(8, 8) SSM_CASE(16, 1) SSM_CASE(16, 2)
  SSM_CASE(4, 8)
#undef SSM_CASE
  return hipErrorNotSupported;
}

template <typename T, int NB, bool EXACT>
hipError_t launch_lane_t(const ScanArgs &a, hipStream_t s) {
  dim3 grid(static_cast<unsigned>((a.D + kWave - 1) / kWave), 1, static_cast<unsigned>(a.B));
  scan_lane_kernel<T, NB, EXACT><<<grid, kWave, 0, s>>>(a);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch_lane(const ScanArgs &a, hipStream_t s) {
  switch (a.N) {
    case 16: return launch_lane_t<T, 16, true>(a, s);
    default: break;
  }
  if (a.N <= 4) return launch_lane_t<T, 4, false>(a, s);
  if (a.N <= 8) return launch_lane_t<T, 8, false>(a, s);
  if (a.N <= 16) return launch_lane_t<T, 16, false>(a, s);
  if (a.N <= 32) return launch_lane_t<T, 32, false>(a, s);
  return launch_lane_t<T, 64, false>(a, s);
}

}  // namespace

hipError_t launch_scan_sequential(const ScanArgs &a, int spl_req, hipStream_t s) {
  if (a.dt == DType::BF16) return dispatch_split<bf16_t>(a, spl_req, 0, nullptr, nullptr, s);
  return dispatch_split<float>(a, spl_req, 0, nullptr, nullptr, s);
}

int64_t scan_chunked_ws_floats(int64_t B, int64_t L, int64_t D, int64_t N, int64_t seg_len) {
  const int64_t nseg = (L + seg_len - 1) / seg_len;
  return 2 * B * nseg * D * N;
}

hipError_t launch_scan_chunked(const ScanArgs &a, int spl_req, int64_t seg_len, float *ws,
                               hipStream_t s) {
  const int64_t nseg = (a.L + seg_len - 1) / seg_len;
  float *seg_a = ws;
  float *seg_h = ws + a.B * nseg * a.D * a.N;
  if (a.dt == DType::BF16) return dispatch_split<bf16_t>(a, spl_req, seg_len, seg_a, seg_h, s);
  return dispatch_split<float>(a, spl_req, seg_len, seg_a, seg_h, s);
}

hipError_t launch_scan_lane(const ScanArgs &a, hipStream_t s) {
  if (a.dt == DType::BF16) return dispatch_lane<bf16_t>(a, s);
  return dispatch_lane<float>(a, s);
}

}  // namespace ssm
