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

enum Mode : int { kFull = 0, kSummary = 1, kOutput = 2, kHalves = 3, kStates = 4 };

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
  __shared__ float s_xv[3][TB][kWave];   // x (for the skip term)
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
  int64_t hrow;  // state row of sequence b
  if (!scan_state_row(a, b, hrow)) return;  // uniform over the workgroup, before any barrier
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
    if (ok && MODE == kFull && a.h0 != nullptr) v = a.h0[(hrow * D + d) * N + n];
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
  const float dbias = a.delta_bias ? a.delta_bias[d] : 0.f;
  const bool dsoft = a.delta_softplus;

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
      const float dl = ok ? step_size(to_f32(r.d[i]), dbias, dsoft) : 0.f;
      const float xv = ok ? to_f32(r.x[i]) : 0.f;
      s_du[b2][j][lane] = make_float2(dl, dl * xv);
      if (kY) {
        s_xv[b3][j][lane] = xv;
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
      v = fmaf(Dd, s_xv[b3][j][lane], v);  // skip term D x
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
      if (MODE == kFull && a.h_final != nullptr) a.h_final[(hrow * D + d) * N + n] = h[s];
      if (MODE == kSummary) {
        seg_a[ws_row + n] = fast_exp2(A2[s] * dsum);
        seg_h[ws_row + n] = h[s];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Lane-split kernel.  A wave owns kCPW = 64/LPC consecutive channels; the LPC
// adjacent lanes of a channel hold SPL states each (N = LPC * SPL).  Nothing
// is shared between waves, so there is no workgroup barrier; each wave works
// through blocks of TB tokens:
//  * every lane loads two adjacent channels of one token row of x, delta and
//    z (one 32-bit load each for bf16), converts them once and writes
//    (delta, u = delta*x) per (token, channel) to wave-private LDS, from
//    which the LPC lanes of a channel read them;
//  * the block's B/C rows (shared by all channels) are loaded by the wave,
//    converted once and put in wave-private LDS laid out so lane q of a
//    channel reads its SPL values of B and of C with vector LDS reads;
//  * each lane writes its partial sum_n C h per token to wave-private LDS;
//    the lane that loaded a (token, channel pair) adds the LPC partials of
//    each channel, the skip term and the gate, and stores the pair of y.
// LDS executes one wave's instructions in order, so a wave's LDS reads see
// its own earlier LDS writes; fences at wavefront scope keep the compiler
// from reordering the cross-lane accesses.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// kBytes bytes at byte offset voff + soff of a buffer, as raw 32-bit words.
template <int kBytes>
__device__ __forceinline__ void load_words(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                           uint32_t *w) {
  const int vo = static_cast<int>(voff), so = static_cast<int>(soff);
  if constexpr (kBytes == 2) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b16(r, vo, so, 0);
  } else if constexpr (kBytes == 4) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, vo, so, 0);
  } else if constexpr (kBytes == 8) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, vo, so, 0);
    w[0] = v[0];
    w[1] = v[1];
  } else {
    static_assert(kBytes % 16 == 0, "unsupported load width");
#pragma unroll
    for (int k = 0; k < kBytes / 16; ++k) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, vo + 16 * k, so, 0);
      w[4 * k] = v[0];
      w[4 * k + 1] = v[1];
      w[4 * k + 2] = v[2];
      w[4 * k + 3] = v[3];
    }
  }
}

// element e of words holding consecutive values of type T, as fp32
template <typename T>
__device__ __forceinline__ float word_elem(const uint32_t *w, int e) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t v = w[e / 2];
    return __uint_as_float((e & 1) ? (v & 0xffff0000u) : (v << 16));
  } else {
    return __uint_as_float(w[e]);
  }
}

// CK: also write the state entering every 8-token segment to a.h_ckpt
// (B, ceil(L/8), D, N) -- what a training step's backward recomputes
// otherwise.  A block of this kernel is exactly one such segment.
// STEP: delta takes the per-channel bias and/or softplus; without it delta is
// used as loaded (rows past L load as 0, which is what they must stage).
// MODE (grid y = segment of seg_len tokens, as the split kernel's modes):
// kFull runs all of L from h0; kSummary runs its segment from 0 and writes
// seg_a = exp(A sum delta) and seg_h = the state reached, without outputs;
// kOutput runs its segment from seg_h (the state entering it) and writes y.
// kStates (with CK) runs all of L from h0 and writes only the saved states
// (no y or h_final, no loads of C or z): the backward's recomputation of them.
// seg_len is a multiple of the 32-token load cycle (TB * CYC), so only the
// last segment has a partial cycle and its rows past L lie past the plane.
// kHalves (1-D grid of J + S workgroups, J = B x channel tiles): the first
// S workgroup tasks are cut in two at seg_len, the rest run whole.  Ids
// [0, S) run the first halves, [S, J) the whole tasks, [J, J + S) the
// second halves.  With 2,560 waves on 1,024 SIMDs (2 each and 512 over)
// and S = 128, round-robin placement gives every SIMD two whole waves and
// one half, instead of 3 whole waves on half of them.  A first half stores
// the state it reaches to seg_h (B, D, N) and then sets its wave's flag in
// seg_a (a device-scope release); the second half waits for that flag
// (bounded: kSpinLimit polls, after which the state is taken as NaN, making
// the failure visible), then runs on from the state.  The state crosses the
// cut exactly, so y and h_final are bitwise those of kFull.  The waiter's
// publisher has a lower workgroup id, so it was dispatched first and never
// waits, and the wait ends.
constexpr int kSpinLimit = 1 << 20;

using f32x4 = float __attribute__((ext_vector_type(4)));

template <typename T, int LPC, int SPL, bool HAS_Z, bool CK, bool STEP, int CYC = 4, int MODE = kFull>
__global__ __launch_bounds__(kWave * 4) void scan_lanesplit_kernel(ScanArgs a, int64_t seg_len, float *seg_a,
                                                                   float *seg_h) {
  constexpr int TB = 8;                 // tokens per block
  constexpr int kCPW = kWave / LPC;     // channels per wave
  constexpr int kN = LPC * SPL;         // = N
  constexpr int kPairs = kCPW / 16;     // (token, channel pair) slots per lane per block
  constexpr int kPPR = kCPW / 2;        // channel pairs per token row
  constexpr int kPW = 2 * static_cast<int>(sizeof(T)) / 4;  // words per channel pair
  constexpr int kV = kN / 4;            // B or C values each lane converts per block
  constexpr int kWords = (kV * static_cast<int>(sizeof(T)) + 3) / 4;
  constexpr uint32_t kES = sizeof(T);
  constexpr int kCyc = CYC;             // blocks per load cycle
  static_assert(LPC == 1 || LPC == 2 || LPC == 4, "LPC must be 1, 2 or 4");
  static_assert(SPL % kV == 0, "a loader lane's values must fall in one lane's slice");
  static_assert(kPairs * 64 * 2 == TB * kCPW, "pair slots must tile the block");
  static_assert(!CK || MODE == kFull || MODE == kStates, "segment states are saved by full runs only");
  static_assert(MODE != kStates || CK, "kStates writes the saved states only");
  constexpr bool kY = MODE != kSummary && MODE != kStates;

  // per wave and block of the cycle: B/C [token][q][B|C][SPL] and
  // (delta, u) [token][channel]; per wave: partial sums [token][channel *
  // LPC + q], rows padded by 4 words so the two rows read by a group of 16
  // lanes fall in different banks
  constexpr int kRow = kCPW * LPC + 4;
  __shared__ __attribute__((aligned(16))) float s_bc[4][kCyc][TB][LPC][2][SPL];
  __shared__ __attribute__((aligned(16))) float2 s_du[4][kCyc][TB][kCPW];
  __shared__ __attribute__((aligned(16))) float s_y[4][TB][kRow];

  const int64_t D = a.D, L = a.L;
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  constexpr bool kHalf = MODE == kHalves;
  // kHalves: workgroup task j of J, split (first S) or whole
  const int64_t h_ntile = (D + 4 * kCPW - 1) / (4 * kCPW);
  const int64_t h_J = a.B * h_ntile;
  const int64_t h_S = kHalf ? static_cast<int64_t>(gridDim.x) - h_J : 0;
  const int64_t h_g = blockIdx.x;
  const int64_t h_j = h_g < h_J ? h_g : h_g - h_J;
  const int64_t d0 = kHalf ? ((h_j % h_ntile) * 4 + wave) * kCPW
                           : (static_cast<int64_t>(blockIdx.x) * 4 + wave) * kCPW;  // first channel of the wave
  const int64_t b = kHalf ? h_j / h_ntile : blockIdx.z;
  int64_t hrow;  // state row of sequence b
  if (!scan_state_row(a, b, hrow)) return;
  // kHalves: seg 0 first half, 1 second half, 2 whole
  const int64_t seg = kHalf ? (h_g < h_S ? 0 : h_g < h_J ? 2 : 1) : blockIdx.y;
  const int64_t nseg = kHalf ? 1 : gridDim.y;
  const int64_t tok0 = kHalf ? (seg == 1 ? seg_len : 0) : seg * seg_len;  // first token of the segment
  const int64_t Ls = kHalf ? (seg == 2 ? L : seg == 0 ? seg_len : L - seg_len)
                           : ((L - tok0) < seg_len ? (L - tok0) : seg_len);  // its tokens
  const uint32_t tok0_u = static_cast<uint32_t>(tok0);

  // compute role: channel c, state slice q
  const int c = lane / LPC, q = lane % LPC;
  const int64_t dc = (d0 + c < D) ? d0 + c : D - 1;
  const int64_t ws_row = ((b * nseg + seg) * D + dc) * kN + q * SPL;  // segment summaries
  // kHalves: this wave's handoff flag and this lane's handoff states
  int *hflag = kHalf ? reinterpret_cast<int *>(seg_a) + h_j * 4 + wave : nullptr;
  float *hslot = kHalf ? seg_h + (b * D + dc) * kN + q * SPL : nullptr;
  if (kHalf && seg == 1) {
    int seen = 0;
    for (int it = 0; it < kSpinLimit; ++it) {
      seen = __builtin_amdgcn_readfirstlane(__hip_atomic_load(hflag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      if (seen != 0) break;
      __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (seen == 0) {
#pragma unroll
      for (int s = 0; s < SPL; ++s) hslot[s] = __builtin_nanf("");
    }
  }
  float A2[SPL], h[SPL];
  {
    const float *Ap = a.A + dc * kN + q * SPL;
    const float *hp = MODE == kOutput ? seg_h + ws_row
                      : (kHalf && seg == 1) ? hslot
                      : ((MODE == kFull || MODE == kStates || kHalf) && a.h0) ? a.h0 + (hrow * D + dc) * kN + q * SPL
                                                           : nullptr;
#pragma unroll
    for (int s = 0; s < SPL; ++s) {
      A2[s] = Ap[s] * kLog2e;
      h[s] = hp ? hp[s] : 0.f;
    }
  }
  float dsum = 0.f;  // sum of the segment's delta (kSummary)

  // load/finish role: slot m covers token row rr[m] of a block and the
  // channel pair pp[m] (wave-local channels 2pp, 2pp+1; D is even, so a pair
  // is either wholly inside D or wholly past it)
  const int64_t plane = L * D * kES;
  const uint32_t row_bytes = static_cast<uint32_t>(D * kES);
  int rr[kPairs], pp[kPairs];
  uint32_t vo[kPairs], vo_st[kPairs];
  float Dd[kPairs][2], Db[kPairs][2];
#pragma unroll
  for (int m = 0; m < kPairs; ++m) {
    const int e = lane + 64 * m;
    rr[m] = e / kPPR;
    pp[m] = e % kPPR;
    const int64_t dp = d0 + 2 * pp[m];
    const bool on = dp < D;
    const int64_t dpc = on ? dp : D - 2;
    vo[m] = static_cast<uint32_t>(dpc * kES) + static_cast<uint32_t>(rr[m]) * row_bytes;
    // stores of pairs past D get an offset past the plane (dropped by the
    // range check); rows past L lie past the plane anyway
    vo_st[m] = on ? vo[m] : 0x80000000u;
    Dd[m][0] = a.D_skip ? a.D_skip[dpc] : 0.f;
    Dd[m][1] = a.D_skip ? a.D_skip[dpc + 1] : 0.f;
    Db[m][0] = (STEP && a.delta_bias) ? a.delta_bias[dpc] : 0.f;
    Db[m][1] = (STEP && a.delta_bias) ? a.delta_bias[dpc + 1] : 0.f;
  }
  const bool dsoft = a.delta_softplus;
  auto rsrc = [&](const void *p, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(static_cast<const char *>(p)), 0,
                                             static_cast<int>(bytes), kRsrcWord3);
  };
  const __amdgpu_buffer_rsrc_t rx = rsrc(static_cast<const char *>(a.x) + b * plane, plane);
  const __amdgpu_buffer_rsrc_t rd = rsrc(static_cast<const char *>(a.delta) + b * plane, plane);
  const __amdgpu_buffer_rsrc_t rz =
      rsrc(HAS_Z ? static_cast<const char *>(a.z) + b * plane : static_cast<const char *>(a.x), plane);
  const __amdgpu_buffer_rsrc_t ry = rsrc(static_cast<char *>(a.y) + b * plane, plane);

  // B/C: even lanes convert B, odd lanes C (the LDS writes of 16 consecutive
  // lanes then cover distinct banks); lane l handles the flat elements
  // [kV*(l/2), kV*(l/2) + kV) of a block's (TB, N) rows
  const int64_t bcplane = L * kN * kES;
  const __amdgpu_buffer_rsrc_t rb = rsrc(static_cast<const char *>(a.Bm) + b * bcplane, bcplane);
  const __amdgpu_buffer_rsrc_t rc = rsrc(static_cast<const char *>(a.Cm) + b * bcplane, bcplane);
  const int ld = lane / 2;
  const bool ld_c = lane & 1;
  const int ld_j = (kV * ld) / kN, ld_n = (kV * ld) % kN;
  const uint32_t ld_vo = static_cast<uint32_t>(kV * ld) * kES;

  const uint32_t ntok = static_cast<uint32_t>(L);
  const int64_t nblk = (Ls + TB - 1) / TB;
  const int64_t ncyc = (nblk + kCyc - 1) / kCyc;

  // segment states: the state after each block of a cycle, stored with the
  // cycle's y (the state entering segment 0 is h0, stored here)
  const bool ck_on = CK && d0 + c < D;
  float *ckp = CK ? a.h_ckpt + (b * nblk * D + dc) * kN + q * SPL : nullptr;
  float hk[CK ? kCyc : 1][SPL];
  auto store_ckpt = [&](int64_t seg, const float *v) {
    if constexpr (SPL % 4 == 0) {
#pragma unroll
      for (int s4 = 0; s4 < SPL / 4; ++s4) {
        const f32x4 sv = {v[4 * s4], v[4 * s4 + 1], v[4 * s4 + 2], v[4 * s4 + 3]};
        __builtin_nontemporal_store(sv, reinterpret_cast<f32x4 *>(ckp + seg * D * kN) + s4);
      }
    } else {
#pragma unroll
      for (int s = 0; s < SPL; ++s) ckp[seg * D * kN + s] = v[s];
    }
  };
  if (CK && ck_on && nblk > 0) store_ckpt(0, h);

  // Raw inputs of one cycle of kCyc blocks.  Two sets alternate: while one
  // cycle is computed, the next one's loads are in flight.
  struct Raw {
    uint32_t x[kCyc][kPairs][kPW], d[kCyc][kPairs][kPW], z[kCyc][kPairs][kPW];
    uint32_t b[kCyc][kWords], c[kCyc][kWords];
  };
  // Loads past the end of a plane return 0 (buffer range check), so the
  // blocks past the last one need no special case.
  auto issue = [&](Raw &w, int64_t cyc) {
#pragma unroll
    for (int u = 0; u < kCyc; ++u) {
      const uint32_t blk = static_cast<uint32_t>(cyc * kCyc + u);
      const uint32_t so = __builtin_amdgcn_readfirstlane((tok0_u + blk * TB) * row_bytes);
#pragma unroll
      for (int m = 0; m < kPairs; ++m) {
        load_words<2 * kES>(rx, vo[m], so, w.x[u][m]);
        load_words<2 * kES>(rd, vo[m], so, w.d[u][m]);
        if (HAS_Z && kY) load_words<2 * kES>(rz, vo[m], so, w.z[u][m]);
      }
      // buffer resources must be wave-uniform: every lane loads its slice
      // of both B and C and converts one of them when the cycle is staged
      const uint32_t bso = __builtin_amdgcn_readfirstlane((tok0_u + blk * TB) * kN * kES);
      load_words<kV * kES>(rb, ld_vo, bso, w.b[u]);
      if (kY) load_words<kV * kES>(rc, ld_vo, bso, w.c[u]);  // (kSummary: no outputs, no C)
    }
  };

  // convert a cycle's delta, u = delta*x and B/C into LDS; tokens past L get
  // delta = u = 0, for which dA = 1 and the state passes through unchanged
  auto stage = [&](const Raw &w, int64_t cyc) {
#pragma unroll
    for (int u = 0; u < kCyc; ++u) {
      const uint32_t tb = tok0_u + static_cast<uint32_t>(cyc * kCyc + u) * TB;
#pragma unroll
      for (int m = 0; m < kPairs; ++m) {
        float du[4];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const float xv = word_elem<T>(w.x[u][m], hh);
          float dv = word_elem<T>(w.d[u][m], hh);
          if constexpr (STEP) dv = (tb + rr[m] < ntok) ? step_size(dv, Db[m][hh], dsoft) : 0.f;
          du[2 * hh] = dv;
          du[2 * hh + 1] = dv * xv;
        }
        *reinterpret_cast<float4 *>(&s_du[wave][u][rr[m]][2 * pp[m]]) =
            make_float4(du[0], du[1], du[2], du[3]);
      }
      uint32_t bc[kWords];
#pragma unroll
      for (int k = 0; k < kWords; ++k) bc[k] = (kY && ld_c) ? w.c[u][k] : w.b[u][k];
      float *dst = &s_bc[wave][u][ld_j][ld_n / SPL][ld_c ? 1 : 0][ld_n % SPL];
#pragma unroll
      for (int e = 0; e < kV; ++e) dst[e] = word_elem<T>(bc, e);
    }
  };

  auto run_block = [&](int u) {
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      const float2 du = s_du[wave][u][j][c];
      float Bv[SPL], Cv[SPL];
#pragma unroll
      for (int s = 0; s < SPL; ++s) {
        Bv[s] = s_bc[wave][u][j][q][0][s];
        Cv[s] = s_bc[wave][u][j][q][1][s];
      }
      float acc = 0.f;
#pragma unroll
      for (int s = 0; s < SPL; ++s) {
        const float dA = fast_exp2(du.x * A2[s]);
        h[s] = fmaf(dA, h[s], du.y * Bv[s]);
        if (kY) acc = fmaf(Cv[s], h[s], acc);
      }
      if (kY) s_y[wave][j][c * LPC + q] = acc;
      if (MODE == kSummary) dsum += du.x;
    }
    if constexpr (CK) {
#pragma unroll
      for (int s = 0; s < SPL; ++s) hk[u][s] = h[s];
    }
  };

  // y of the slots of a block, packed as stored
  uint32_t yv[kCyc][kPairs][kPW];
  auto finish_block = [&](const Raw &w, int u) {
#pragma unroll
    for (int m = 0; m < kPairs; ++m) {
      float v[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const float *py = &s_y[wave][rr[m]][(2 * pp[m] + hh) * LPC];
        float t = py[0];
#pragma unroll
        for (int k = 1; k < LPC; ++k) t += py[k];
        t = fmaf(Dd[m][hh], word_elem<T>(w.x[u][m], hh), t);  // skip term D x
        if (HAS_Z) t *= silu(word_elem<T>(w.z[u][m], hh));
        v[hh] = t;
      }
      if constexpr (sizeof(T) == 2) {
        yv[u][m][0] = static_cast<uint32_t>(from_f32<T>(v[0]).bits) |
                      (static_cast<uint32_t>(from_f32<T>(v[1]).bits) << 16);
      } else {
        yv[u][m][0] = __float_as_uint(v[0]);
        yv[u][m][1] = __float_as_uint(v[1]);
      }
    }
  };
  auto store_cycle = [&](int64_t cyc) {
#pragma unroll
    for (int u = 0; u < kCyc; ++u) {
      const uint32_t so =
          __builtin_amdgcn_readfirstlane((tok0_u + static_cast<uint32_t>(cyc * kCyc + u) * TB) * row_bytes);
#pragma unroll
      for (int m = 0; m < (kY ? kPairs : 0); ++m) {
        const int vov = static_cast<int>(vo_st[m]), sov = static_cast<int>(so);
        if constexpr (sizeof(T) == 2) {
          __builtin_amdgcn_raw_buffer_store_b32(yv[u][m][0], ry, vov, sov, 0);
        } else {
          using u32x2 = uint32_t __attribute__((ext_vector_type(2)));
          const u32x2 pv = {yv[u][m][0], yv[u][m][1]};
          __builtin_amdgcn_raw_buffer_store_b64(pv, ry, vov, sov, 0);
        }
      }
      if constexpr (CK) {
        const int64_t seg = cyc * kCyc + u + 1;  // entered after block cyc * kCyc + u
        if (ck_on && seg < nblk) store_ckpt(seg, hk[u]);
      }
    }
  };

  // One cycle: stage its inputs (this waits for its loads, issued a cycle
  // earlier, and for the previous cycle's stores), store the previous
  // cycle's y, issue the next cycle's loads, then compute.  Loads and stores
  // share one counter whose waits cannot skip a pending store, so no store is
  // issued between a load and the wait for it except a whole cycle earlier.
  // nb: blocks of the cycle that hold tokens (the last cycle may have
  // fewer; its blocks past the end are neither computed nor finished -- their
  // y stores fall past the plane and the state is already final)
  auto cycle = [&](Raw &cur, Raw &nxt, int64_t cyc, int nb) {
    stage(cur, cyc);
    if ((kY || CK) && cyc > 0) store_cycle(cyc - 1);
    issue(nxt, cyc + 1);
    wave_sync_lds();
#pragma unroll
    for (int u = 0; u < kCyc; ++u) {
      if (u < nb) {
        run_block(u);
        wave_sync_lds();
        if (kY) {
          finish_block(cur, u);
          wave_sync_lds();
        }
      }
    }
  };

  Raw r0, r1;
  issue(r0, 0);
  int64_t cyc = 0;
  for (; cyc + 1 < ncyc; cyc += 2) {
    cycle(r0, r1, cyc, kCyc);
    cycle(r1, r0, cyc + 1, kCyc);
  }
  if (cyc < ncyc) {
    cycle(r0, r1, cyc, static_cast<int>(nblk - cyc * kCyc));
    ++cyc;
  }
  if ((kY || CK) && ncyc > 0) store_cycle(cyc - 1);

  if (kHalf && seg == 0) {  // publish the state reached at the cut
    if (d0 + c < D) {
#pragma unroll
      for (int s = 0; s < SPL; ++s) hslot[s] = h[s];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if (lane == 0) __hip_atomic_store(hflag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  if (d0 + c >= D) return;
  if (MODE == kSummary) {
#pragma unroll
    for (int s = 0; s < SPL; ++s) {
      seg_a[ws_row + s] = fast_exp2(A2[s] * dsum);
      seg_h[ws_row + s] = h[s];
    }
  }
  if ((MODE != kFull && !kHalf) || a.h_final == nullptr) return;
  float *hf = a.h_final + (hrow * D + dc) * kN + q * SPL;
#pragma unroll
  for (int s = 0; s < SPL; ++s) hf[s] = h[s];
}

// Carry pass: one thread per (b, d, n); walks the segments in order,
// replacing each segment's summary state with the state entering it, and
// writes h_final.  carry <- a_seg * carry + h_seg composes the segment's
// affine map after the carry (seed (1, h0)).  The summaries of kCarryBatch
// segments are loaded before any carry is stored, so that many loads are in
// flight per thread (a load of segment s + 1 would otherwise wait for the
// store to segment s).
constexpr int kCarryBatch = 8;
constexpr int kCarryThreads = 256;

__global__ __launch_bounds__(kCarryThreads) void scan_carry_kernel(int64_t B, int64_t D, int64_t N,
                                                          int64_t nseg, const float *h0,
                                                          const float *seg_a, float *seg_h,
                                                          float *h_final) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t DN = D * N;
  if (i >= B * DN) return;
  const int64_t b = i / DN;
  const int64_t dn = i - b * DN;
  float carry = h0 ? h0[i] : 0.f;
  for (int64_t s0 = 0; s0 < nseg; s0 += kCarryBatch) {
    float av[kCarryBatch], hv[kCarryBatch];
#pragma unroll
    for (int k = 0; k < kCarryBatch; ++k) {
      if (s0 + k < nseg) {
        const int64_t idx = (b * nseg + s0 + k) * DN + dn;
        av[k] = seg_a[idx];
        hv[k] = seg_h[idx];
      }
    }
#pragma unroll
    for (int k = 0; k < kCarryBatch; ++k) {
      if (s0 + k < nseg) {
        seg_h[(b * nseg + s0 + k) * DN + dn] = carry;
        carry = fmaf(av[k], carry, hv[k]);
      }
    }
  }
  if (h_final) h_final[i] = carry;
}

// Zeroes the kHalves handoff flags (a fill kernel rather than a memset, so
// the launch pair can be captured in a graph).
__global__ __launch_bounds__(256) void halves_flags_clear(int *flag, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) flag[i] = 0;
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
  int64_t hrow;  // state row of sequence b
  if (!scan_state_row(a, b, hrow)) return;

  float A2[NB], h[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    const bool ok = EXACT || n < N;
    A2[n] = ok ? a.A[d * N + n] * kLog2e : 0.f;
    h[n] = (ok && a.h0 != nullptr) ? a.h0[(hrow * D + d) * N + n] : 0.f;
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
  const float dbias = a.delta_bias ? a.delta_bias[d] : 0.f;
  for (int64_t t = 0; t < L; ++t) {
    const float dl = step_size(to_f32(dp[t * D]), dbias, a.delta_softplus);
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
    if (EXACT || n < N) a.h_final[(hrow * D + d) * N + n] = h[n];
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct SplitCfg {
  int spl, w;
};

// tokens per LDS stage / barrier (segment lengths are multiples of it)
constexpr int kBlockTokens = 8;

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
  const unsigned carry_grid = static_cast<unsigned>((total + kCarryThreads - 1) / kCarryThreads);
  scan_carry_kernel<<<carry_grid, kCarryThreads, 0, s>>>(a.B, a.D, a.N, nseg, a.h0, seg_a, seg_h, a.h_final);
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

template <typename T, int LPC, int SPL, bool STEP>
void launch_lanesplit_s(const ScanArgs &a, dim3 grid, hipStream_t s) {
  if (a.L <= 16 && a.h_ckpt == nullptr) {
    // short runs (multi-token decode): cycles of two blocks halve the LDS and
    // the registers of the input sets, so more waves stay resident to cover
    // the latency of each wave's state load and store
    if (a.z)
      scan_lanesplit_kernel<T, LPC, SPL, true, false, STEP, 2><<<grid, kWave * 4, 0, s>>>(a, a.L, nullptr, nullptr);
    else
      scan_lanesplit_kernel<T, LPC, SPL, false, false, STEP, 2><<<grid, kWave * 4, 0, s>>>(a, a.L, nullptr, nullptr);
    return;
  }
  if (a.h_ckpt) {
    if (a.z)
      scan_lanesplit_kernel<T, LPC, SPL, true, true, STEP><<<grid, kWave * 4, 0, s>>>(a, a.L, nullptr, nullptr);
    else
      scan_lanesplit_kernel<T, LPC, SPL, false, true, STEP><<<grid, kWave * 4, 0, s>>>(a, a.L, nullptr, nullptr);
  } else {
    if (a.z)
      scan_lanesplit_kernel<T, LPC, SPL, true, false, STEP><<<grid, kWave * 4, 0, s>>>(a, a.L, nullptr, nullptr);
    else
      scan_lanesplit_kernel<T, LPC, SPL, false, false, STEP><<<grid, kWave * 4, 0, s>>>(a, a.L, nullptr, nullptr);
  }
}

template <typename T, int LPC, int SPL>
hipError_t launch_states_t(const ScanArgs &a, hipStream_t s) {
  constexpr int kChPerWG = 4 * (kWave / LPC);
  dim3 grid(static_cast<unsigned>((a.D + kChPerWG - 1) / kChPerWG), 1, static_cast<unsigned>(a.B));
  if (a.delta_bias != nullptr || a.delta_softplus)
    scan_lanesplit_kernel<T, LPC, SPL, false, true, true, 4, kStates><<<grid, kWave * 4, 0, s>>>(a, a.L, nullptr,
                                                                                                nullptr);
  else
    scan_lanesplit_kernel<T, LPC, SPL, false, true, false, 4, kStates><<<grid, kWave * 4, 0, s>>>(a, a.L, nullptr,
                                                                                                 nullptr);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch_states(const ScanArgs &a, hipStream_t s) {
  switch (a.N) {
    case 4: return launch_states_t<T, 1, 4>(a, s);
    case 8: return launch_states_t<T, 2, 4>(a, s);
    case 16: return launch_states_t<T, 4, 4>(a, s);
    case 32: return launch_states_t<T, 4, 8>(a, s);
    case 64: return launch_states_t<T, 4, 16>(a, s);
    default: return hipErrorNotSupported;
  }
}

template <typename T, int LPC, int SPL>
hipError_t launch_lanesplit_t(const ScanArgs &a, hipStream_t s) {
  constexpr int kChPerWG = 4 * (kWave / LPC);
  dim3 grid(static_cast<unsigned>((a.D + kChPerWG - 1) / kChPerWG), 1, static_cast<unsigned>(a.B));
  if (a.delta_bias != nullptr || a.delta_softplus)
    launch_lanesplit_s<T, LPC, SPL, true>(a, grid, s);
  else
    launch_lanesplit_s<T, LPC, SPL, false>(a, grid, s);
  return hipGetLastError();
}

// Chunked schedule on the lane-split kernel: segment summaries, the carry
// pass, then each segment's outputs from the state entering it.
template <typename T, int LPC, int SPL, bool STEP>
void launch_lanesplit_chunked_s(const ScanArgs &a, int64_t seg_len, float *seg_a, float *seg_h,
                                hipStream_t s) {
  constexpr int kChPerWG = 4 * (kWave / LPC);
  const int64_t nseg = (a.L + seg_len - 1) / seg_len;
  dim3 grid(static_cast<unsigned>((a.D + kChPerWG - 1) / kChPerWG), static_cast<unsigned>(nseg),
            static_cast<unsigned>(a.B));
  scan_lanesplit_kernel<T, LPC, SPL, false, false, STEP, 4, kSummary><<<grid, kWave * 4, 0, s>>>(a, seg_len, seg_a,
                                                                                                 seg_h);
  const int64_t total = a.B * a.D * a.N;
  const unsigned carry_grid = static_cast<unsigned>((total + kCarryThreads - 1) / kCarryThreads);
  scan_carry_kernel<<<carry_grid, kCarryThreads, 0, s>>>(a.B, a.D, a.N, nseg, a.h0, seg_a, seg_h, a.h_final);
  if (a.z)
    scan_lanesplit_kernel<T, LPC, SPL, true, false, STEP, 4, kOutput><<<grid, kWave * 4, 0, s>>>(a, seg_len, seg_a,
                                                                                               seg_h);
  else
    scan_lanesplit_kernel<T, LPC, SPL, false, false, STEP, 4, kOutput><<<grid, kWave * 4, 0, s>>>(a, seg_len, seg_a,
                                                                                                seg_h);
}

template <typename T, int LPC, int SPL>
hipError_t launch_lanesplit_chunked_t(const ScanArgs &a, int64_t seg_len, float *seg_a, float *seg_h,
                                      hipStream_t s) {
  if (a.delta_bias != nullptr || a.delta_softplus)
    launch_lanesplit_chunked_s<T, LPC, SPL, true>(a, seg_len, seg_a, seg_h, s);
  else
    launch_lanesplit_chunked_s<T, LPC, SPL, false>(a, seg_len, seg_a, seg_h, s);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch_lanesplit_chunked(const ScanArgs &a, int64_t seg_len, float *seg_a, float *seg_h,
                                      hipStream_t s) {
  switch (a.N) {
    case 4: return launch_lanesplit_chunked_t<T, 1, 4>(a, seg_len, seg_a, seg_h, s);
    case 8: return launch_lanesplit_chunked_t<T, 2, 4>(a, seg_len, seg_a, seg_h, s);
    case 16: return launch_lanesplit_chunked_t<T, 4, 4>(a, seg_len, seg_a, seg_h, s);
    case 32: return launch_lanesplit_chunked_t<T, 4, 8>(a, seg_len, seg_a, seg_h, s);
    case 64: return launch_lanesplit_chunked_t<T, 4, 16>(a, seg_len, seg_a, seg_h, s);
    default: return hipErrorNotSupported;
  }
}

template <typename T>
hipError_t dispatch_lanesplit(const ScanArgs &a, hipStream_t s) {
  switch (a.N) {
    case 4: return launch_lanesplit_t<T, 1, 4>(a, s);
    case 8: return launch_lanesplit_t<T, 2, 4>(a, s);
    case 16: return launch_lanesplit_t<T, 4, 4>(a, s);
    case 32: return launch_lanesplit_t<T, 4, 8>(a, s);
    case 64: return launch_lanesplit_t<T, 4, 16>(a, s);
    default: return hipErrorNotSupported;
  }
}

// Halved schedule: ws holds the handoff states (B, D, N) and then one flag
// per wave of the first halves.
template <typename T, int LPC, int SPL, bool STEP>
void launch_lanesplit_halves_s(const ScanArgs &a, int64_t nsplit, float *ws, hipStream_t s) {
  constexpr int kChPerWG = 4 * (kWave / LPC);
  const int64_t tiles = (a.D + kChPerWG - 1) / kChPerWG;
  const int64_t nflag = nsplit * 4;
  float *hand = ws;
  float *flags = ws + a.B * a.D * a.N;
  halves_flags_clear<<<static_cast<unsigned>((nflag + 255) / 256), 256, 0, s>>>(reinterpret_cast<int *>(flags),
                                                                             nflag);
  const int64_t cut = ((a.L + 1) / 2 + 31) / 32 * 32;  // whole 32-token cycles
  const dim3 grid(static_cast<unsigned>(a.B * tiles + nsplit), 1, 1);
  if (a.z)
    scan_lanesplit_kernel<T, LPC, SPL, true, false, STEP, 4, kHalves><<<grid, kWave * 4, 0, s>>>(a, cut, flags, hand);
  else
    scan_lanesplit_kernel<T, LPC, SPL, false, false, STEP, 4, kHalves><<<grid, kWave * 4, 0, s>>>(a, cut, flags,
                                                                                               hand);
}

template <typename T, int LPC, int SPL>
hipError_t launch_lanesplit_halves_t(const ScanArgs &a, int64_t nsplit, float *ws, hipStream_t s) {
  if (a.delta_bias != nullptr || a.delta_softplus)
    launch_lanesplit_halves_s<T, LPC, SPL, true>(a, nsplit, ws, s);
  else
    launch_lanesplit_halves_s<T, LPC, SPL, false>(a, nsplit, ws, s);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch_lanesplit_halves(const ScanArgs &a, int64_t nsplit, float *ws, hipStream_t s) {
  switch (a.N) {
    case 4: return launch_lanesplit_halves_t<T, 1, 4>(a, nsplit, ws, s);
    case 8: return launch_lanesplit_halves_t<T, 2, 4>(a, nsplit, ws, s);
    case 16: return launch_lanesplit_halves_t<T, 4, 4>(a, nsplit, ws, s);
    case 32: return launch_lanesplit_halves_t<T, 4, 8>(a, nsplit, ws, s);
    case 64: return launch_lanesplit_halves_t<T, 4, 16>(a, nsplit, ws, s);
    default: return hipErrorNotSupported;
  }
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

bool scan_lanesplit_supported(const ScanArgs &a) {
  const bool n_ok = a.N == 4 || a.N == 8 || a.N == 16 || a.N == 32 || a.N == 64;
  auto al = [](const void *p, uintptr_t k) { return reinterpret_cast<uintptr_t>(p) % k == 0; };
  const uintptr_t pair = a.dt == DType::BF16 ? 4 : 8;  // a channel pair is loaded as one word
  const bool aligned = al(a.Bm, 16) && al(a.Cm, 16) && al(a.x, pair) && al(a.delta, pair) &&
                       al(a.y, pair) && (a.z == nullptr || al(a.z, pair));
  return n_ok && aligned && a.D % 2 == 0;
}

hipError_t launch_scan_lanesplit(const ScanArgs &a, hipStream_t s) {
  if (a.dt == DType::BF16) return dispatch_lanesplit<bf16_t>(a, s);
  return dispatch_lanesplit<float>(a, s);
}

hipError_t launch_scan_states(const ScanArgs &a, hipStream_t s) {
  if (a.dt == DType::BF16) return dispatch_states<bf16_t>(a, s);
  return dispatch_states<float>(a, s);
}

int64_t scan_halves_split(int64_t B, int64_t D, int64_t N, int64_t simds, bool forced) {
  const int64_t lpc = N == 4 ? 1 : N == 8 ? 2 : 4;
  const int64_t J = B * ((D + 4 * (kWave / lpc) - 1) / (4 * (kWave / lpc)));  // workgroup tasks
  if (forced) return J / 2 > 0 ? J / 2 : 1;
  // the waves over a whole number per SIMD, halved, give each SIMD at most
  // one half more when they number at most half the SIMDs
  const int64_t waves = 4 * J;
  if (simds <= 0 || waves <= simds) return 0;
  const int64_t r = waves % simds;
  if (r == 0 || 2 * r > simds) return 0;
  return r / 4;
}

int64_t scan_halves_ws_floats(int64_t B, int64_t D, int64_t N) {
  const int64_t lpc = N == 4 ? 1 : N == 8 ? 2 : 4;
  const int64_t tiles = (D + 4 * (kWave / lpc) - 1) / (4 * (kWave / lpc));
  return B * D * N + B * tiles * 4;  // handoff states, then the flags (at most one per wave)
}

hipError_t launch_scan_lanesplit_halves(const ScanArgs &a, int64_t nsplit, float *ws, hipStream_t s) {
  if (a.dt == DType::BF16) return dispatch_lanesplit_halves<bf16_t>(a, nsplit, ws, s);
  return dispatch_lanesplit_halves<float>(a, nsplit, ws, s);
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
  // the lane-split kernel takes segments of whole 32-token load cycles
  if (spl_req == 0 && seg_len % 32 == 0 && a.slots == nullptr && a.h_ckpt == nullptr &&
      scan_lanesplit_supported(a)) {
    if (a.dt == DType::BF16) return dispatch_lanesplit_chunked<bf16_t>(a, seg_len, seg_a, seg_h, s);
    return dispatch_lanesplit_chunked<float>(a, seg_len, seg_a, seg_h, s);
  }
  if (a.dt == DType::BF16) return dispatch_split<bf16_t>(a, spl_req, seg_len, seg_a, seg_h, s);
  return dispatch_split<float>(a, spl_req, seg_len, seg_a, seg_h, s);
}

hipError_t launch_scan_lane(const ScanArgs &a, hipStream_t s) {
  if (a.dt == DType::BF16) return dispatch_lane<bf16_t>(a, s);
  return dispatch_lane<float>(a, s);
}

}  // namespace ssm
