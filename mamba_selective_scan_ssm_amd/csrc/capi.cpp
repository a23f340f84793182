// C ABI of libssmscan.so: host-side validation, variant choice and dispatch.
// Validation is pure host code and runs before any HIP call, so a rejected
// call enqueues nothing and has no side effects.
#include "../../include/ssm_scan.h"

#include <hip/hip_runtime.h>

#include <cstdint>

#include "bwd.h"
#include "launch.h"

namespace {

using ssm::DType;

constexpr int64_t kMaxGridYZ = 65535;

bool valid_dtype(ssm_dtype dt) { return dt == SSM_F32 || dt == SSM_BF16; }
int64_t esize(ssm_dtype dt) { return dt == SSM_BF16 ? 2 : 4; }

struct Range {
  const void *p;
  int64_t bytes;
};

bool overlap(Range a, Range b) {
  if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + static_cast<uintptr_t>(b.bytes) && b0 < a0 + static_cast<uintptr_t>(a.bytes);
}

template <size_t K>
bool overlaps_any(Range out, const Range (&ins)[K]) {
  for (size_t i = 0; i < K; ++i)
    if (overlap(out, ins[i])) return true;
  return false;
}

bool tuning_ok(const ssm_tuning *t) {
  if (!t) return true;
  for (int i = 0; i < 5; ++i)
    if (t->reserved[i] != 0) return false;
  if (t->variant < 0 || t->variant > 4) return false;
  if (t->chunk_len < 0 || (t->chunk_len != 0 && (t->chunk_len < 8 || t->chunk_len % 8 != 0)))
    return false;
  const int s = t->states_per_lane;
  if (s != 0 && s != 2 && s != 4 && s != 8 && s != 16) return false;
  return true;
}

int spl_of(const ssm_tuning *t) { return t ? t->states_per_lane : 0; }

bool dopts_ok(const ssm_delta_opts *o) {
  if (!o) return true;
  for (int i = 0; i < 3; ++i)
    if (o->reserved[i] != 0) return false;
  return o->softplus == 0 || o->softplus == 1;
}
const float *dbias_of(const ssm_delta_opts *o) { return o ? o->bias : nullptr; }
bool dsoft_of(const ssm_delta_opts *o) { return o && o->softplus == 1; }

// Variant choice: a function of (L, D, N) only, so a sequence's result does
// not depend on the batch it is in.  Sequential when one sequence already
// brings enough 64-channel waves or L is short; otherwise chunked with
// segments sized so one sequence yields ~2048 waves, a multiple of 32 tokens
// (whole load cycles of the lane-split kernel).
struct Plan {
  int variant;  // 1 sequential (waves split N), 2 chunked, 3 sequential (lanes split N),
                // 4 as 3 with every wave's tokens cut in two
  int64_t seg_len;
};

Plan plan_scan(int64_t L, int64_t D, const ssm_tuning *t) {
  const int64_t wps = (D + 63) / 64;  // channel tiles per sequence
  int variant = t ? t->variant : 0;
  int64_t seg = t ? t->chunk_len : 0;
  if (variant == 0) variant = (L <= 256 || wps >= 64) ? 1 : 2;
  if (variant == 2 && seg == 0) {
    int64_t nseg = 512 / (wps > 0 ? wps : 1);  // ~512 tiles x segments per sequence
    if (nseg < 1) nseg = 1;
    seg = (L + nseg - 1) / nseg;
    seg = seg / 32 * 32;
    if (seg < 64) seg = 64;
  }
  if (variant == 2 && seg <= 0) seg = 64;
  return Plan{variant, seg};
}

ssm_status hip_status(hipError_t e) { return e == hipSuccess ? SSM_OK : SSM_ERR_HIP; }

// SIMDs of the current device (4 per CU; cached per device; 0 if the query
// fails, where the halved schedule is then not chosen automatically).
int64_t device_simds() {
  static int64_t cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 0;
  if (dev < 64) cached[dev] = 4 * static_cast<int64_t>(cus);
  return 4 * static_cast<int64_t>(cus);
}

// Whether this call takes the halved lane-split schedule (variant 4): asked
// for, or chosen automatically where the channel-sequential schedule applies
// and halving the waves evens the SIMDs' load.  Its results are bitwise
// those of variant 3, so the choice, which depends on B and on the device,
// changes no result.
// Returns the workgroup tasks to cut in two (0: not this schedule).
int64_t halves_planned(int64_t B, int64_t L, int64_t D, int64_t N, const ssm_tuning *t) {
  const Plan p = plan_scan(L, D, t);
  const bool n_ok = N == 4 || N == 8 || N == 16 || N == 32 || N == 64;
  if (!n_ok || L < 64) return 0;
  if (p.variant == 4) return ssm::scan_halves_split(B, D, N, 0, true);
  const bool auto_seq = (t == nullptr || (t->variant == 0 && t->states_per_lane == 0)) && p.variant == 1;
  return auto_seq ? ssm::scan_halves_split(B, D, N, device_simds(), false) : 0;
}

// shapes the matrix-core SSD kernels are built for
bool ssd_mfma_applies(ssm_dtype dt, int64_t P, int64_t N, int64_t chunk) {
  return dt == SSM_BF16 && P == 64 && N % 32 == 0 && N >= 32 && N <= SSM_SSD_MAX_N &&
         (chunk == 64 || chunk == 128 || chunk == 256);
}

}  // namespace

extern "C" {

ssm_status ssm_conv1d_fwd(int64_t B, int64_t L, int64_t D, int64_t K, ssm_dtype dt,
                          const void *x, const float *w, const float *bias,
                          const float *state_in, int32_t activation, void *y,
                          float *state_out, void *stream) {
  if (B < 0 || L < 0 || D < 0 || K < 0) return SSM_ERR_INVALID_ARG;
  if (!valid_dtype(dt) || (activation != 0 && activation != 1)) return SSM_ERR_INVALID_ARG;
  if (K < 2 || K > 8) return SSM_ERR_UNSUPPORTED;
  if (B == 0 || D == 0) return SSM_OK;
  if (B > kMaxGridYZ || (L + 63) / 64 > kMaxGridYZ) return SSM_ERR_UNSUPPORTED;
  const int64_t es = esize(dt);
  if ((L + 64) * D * es >= (int64_t(1) << 31)) return SSM_ERR_UNSUPPORTED;
  if (!w || (L > 0 && (!x || !y))) return SSM_ERR_INVALID_ARG;
  const int64_t nBLD = B * L * D, nSt = B * D * (K - 1);
  const Range ins[] = {{x, nBLD * es}, {w, D * K * 4}, {bias, D * 4}, {state_in, nSt * 4}};
  if (overlaps_any(Range{y, nBLD * es}, ins)) return SSM_ERR_INVALID_ARG;
  if (overlaps_any(Range{state_out, nSt * 4}, ins)) return SSM_ERR_INVALID_ARG;
  if (overlap(Range{y, nBLD * es}, Range{state_out, nSt * 4})) return SSM_ERR_INVALID_ARG;
  ssm::ConvArgs a{};
  a.B = B; a.L = L; a.D = D; a.K = K;
  a.dt = dt == SSM_BF16 ? DType::BF16 : DType::F32;
  a.x = x; a.w = w; a.bias = bias; a.state_in = state_in; a.state_out = state_out;
  a.y = y; a.act = activation == 1;
  return hip_status(ssm::launch_conv1d_fwd(a, static_cast<hipStream_t>(stream)));
}

ssm_status ssm_conv1d_update(int64_t S, int64_t D, int64_t K, ssm_dtype dt, float *state,
                             const void *x, const float *w, const float *bias,
                             int32_t activation, void *y, void *stream) {
  if (S < 0 || D < 0 || K < 0) return SSM_ERR_INVALID_ARG;
  if (!valid_dtype(dt) || (activation != 0 && activation != 1)) return SSM_ERR_INVALID_ARG;
  if (K < 2 || K > 8) return SSM_ERR_UNSUPPORTED;
  if (S > kMaxGridYZ) return SSM_ERR_UNSUPPORTED;  // one grid row per sequence
  if (S == 0 || D == 0) return SSM_OK;
  if (!state || !x || !w || !y) return SSM_ERR_INVALID_ARG;
  const int64_t es = esize(dt);
  const Range ins[] = {{x, S * D * es}, {w, D * K * 4}, {bias, D * 4}, {state, S * D * (K - 1) * 4}};
  if (overlaps_any(Range{y, S * D * es}, ins)) return SSM_ERR_INVALID_ARG;
  const Range st{state, S * D * (K - 1) * 4};
  if (overlap(st, Range{x, S * D * es}) || overlap(st, Range{w, D * K * 4}) ||
      overlap(st, Range{bias, D * 4}))
    return SSM_ERR_INVALID_ARG;
  ssm::ConvArgs a{};
  a.B = S; a.L = 1; a.D = D; a.K = K;
  a.dt = dt == SSM_BF16 ? DType::BF16 : DType::F32;
  a.x = x; a.w = w; a.bias = bias; a.state_in = state; a.state_out = state;
  a.y = y; a.act = activation == 1;
  return hip_status(ssm::launch_conv1d_update(a, static_cast<hipStream_t>(stream)));
}

const char *ssm_status_string(ssm_status s) {
  switch (s) {
    case SSM_OK: return "ok";
    case SSM_ERR_INVALID_ARG: return "invalid argument";
    case SSM_ERR_UNSUPPORTED: return "unsupported size or dtype";
    case SSM_ERR_WORKSPACE: return "workspace missing or too small";
    case SSM_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int ssm_version(void) { return 100; }  // 0.1.0

// Workspace: the segment summaries of the chunked schedule, the state
// handoff of the halved one (none otherwise).
int64_t scan_ws_floats(int64_t B, int64_t L, int64_t D, int64_t N, const ssm_tuning *t) {
  if (B <= 0 || L <= 0 || D <= 0 || N <= 0) return 0;
  const Plan p = plan_scan(L, D, t);
  if (p.variant == 2) return ssm::scan_chunked_ws_floats(B, L, D, N, p.seg_len);
  if (halves_planned(B, L, D, N, t) > 0) return ssm::scan_halves_ws_floats(B, D, N);
  return 0;
}

size_t ssm_scan_fwd_workspace_size(int64_t B, int64_t L, int64_t D, int64_t N,
                                   const ssm_tuning *tuning) {
  if (!tuning_ok(tuning) || N > SSM_SCAN_MAX_N) return 0;
  return static_cast<size_t>(scan_ws_floats(B, L, D, N, tuning)) * sizeof(float);
}

ssm_status ssm_scan_fwd(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype dt, const void *x,
                        const void *delta, const float *A, const void *Bm, const void *Cm,
                        const float *D_skip, const void *z, const float *h0, void *y,
                        float *h_final, void *workspace, size_t workspace_bytes,
                        const ssm_tuning *tuning, void *stream) {
  return ssm_scan_fwd_ex(B, L, D, N, dt, x, delta, A, Bm, Cm, D_skip, z, h0, y, h_final, workspace,
                         workspace_bytes, tuning, nullptr, stream);
}

}  // extern "C"

namespace {

// ssm_scan_fwd_ex, and ssm_scan_fwd_noalloc (own_scratch: the chunked
// schedule's segment summaries go to the library's device scratch instead of
// a caller workspace).
ssm_status scan_fwd_impl(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype dt, const void *x,
                         const void *delta, const float *A, const void *Bm, const void *Cm,
                         const float *D_skip, const void *z, const float *h0, void *y,
                         float *h_final, void *workspace, size_t workspace_bytes,
                         const ssm_tuning *tuning, const ssm_delta_opts *dopts, void *stream,
                         bool own_scratch) {
  if (B < 0 || L < 0 || D < 0 || N < 0) return SSM_ERR_INVALID_ARG;
  if (!valid_dtype(dt) || !tuning_ok(tuning) || !dopts_ok(dopts)) return SSM_ERR_INVALID_ARG;
  if (N > SSM_SCAN_MAX_N) return SSM_ERR_UNSUPPORTED;
  if (B == 0 || D == 0) return SSM_OK;
  if (B > kMaxGridYZ) return SSM_ERR_UNSUPPORTED;
  const int64_t es = esize(dt);
  // one sequence's (L, D) and (L, N) planes are addressed with 32-bit offsets
  if ((L + 64) * D * es >= (int64_t(1) << 31) || (L + 64) * N * es >= (int64_t(1) << 31))
    return SSM_ERR_UNSUPPORTED;
  const int64_t nBLD = B * L * D, nBLN = B * L * N, nBDN = B * D * N;
  if (L > 0 && (!x || !delta || !y)) return SSM_ERR_INVALID_ARG;
  if (L > 0 && N > 0 && (!Bm || !Cm)) return SSM_ERR_INVALID_ARG;
  if (N > 0 && !A) return SSM_ERR_INVALID_ARG;
  const Range ins[] = {{x, nBLD * es},   {delta, nBLD * es}, {A, D * N * 4}, {Bm, nBLN * es},
                       {Cm, nBLN * es},  {D_skip, D * 4},    {z, nBLD * es}, {h0, nBDN * 4},
                       {dbias_of(dopts), D * 4}};
  if (overlaps_any(Range{y, nBLD * es}, ins)) return SSM_ERR_INVALID_ARG;
  if (overlaps_any(Range{h_final, nBDN * 4}, ins)) return SSM_ERR_INVALID_ARG;
  if (overlap(Range{y, nBLD * es}, Range{h_final, nBDN * 4})) return SSM_ERR_INVALID_ARG;

  ssm::ScanArgs a{};
  a.B = B; a.L = L; a.D = D; a.N = N;
  a.dt = dt == SSM_BF16 ? DType::BF16 : DType::F32;
  a.x = x; a.delta = delta; a.A = A; a.Bm = Bm; a.Cm = Cm;
  a.D_skip = D_skip; a.z = z; a.h0 = h0; a.y = y; a.h_final = h_final;
  a.delta_bias = dbias_of(dopts); a.delta_softplus = dsoft_of(dopts);
  hipStream_t s = static_cast<hipStream_t>(stream);

  const Plan p = plan_scan(L, D, tuning);
  if (L == 0 || N == 0) return hip_status(ssm::launch_scan_lane(a, s));
  if (p.variant == 2) {
    if ((L + p.seg_len - 1) / p.seg_len > kMaxGridYZ) return SSM_ERR_UNSUPPORTED;
    const size_t need = static_cast<size_t>(scan_ws_floats(B, L, D, N, tuning)) * sizeof(float);
    if (own_scratch) {
      if (need > ssm::kScratchBytes) return SSM_ERR_WORKSPACE;
      const hipError_t e = ssm::scratch_device_ptr(&workspace);
      if (e != hipSuccess) return SSM_ERR_HIP;
      workspace_bytes = ssm::kScratchBytes;
    } else {
      if (!workspace || workspace_bytes < need) return SSM_ERR_WORKSPACE;
      const Range wsr{workspace, static_cast<int64_t>(need)};
      if (overlaps_any(wsr, ins) || overlap(wsr, Range{y, nBLD * es}) ||
          overlap(wsr, Range{h_final, nBDN * 4}))
        return SSM_ERR_INVALID_ARG;
    }
    return hip_status(ssm::launch_scan_chunked(a, spl_of(tuning), p.seg_len,
                                               static_cast<float *>(workspace), s));
  }
  const bool auto_variant = tuning == nullptr || tuning->variant == 0;
  const bool lanesplit_ok = ssm::scan_lanesplit_supported(a);
  const int64_t nsplit = halves_planned(B, L, D, N, tuning);
  if (p.variant == 4 || (nsplit > 0 && lanesplit_ok)) {
    if (!lanesplit_ok || nsplit == 0) return SSM_ERR_UNSUPPORTED;
    const size_t need = static_cast<size_t>(ssm::scan_halves_ws_floats(B, D, N)) * sizeof(float);
    if (own_scratch) {
      if (need > ssm::kScratchBytes) return SSM_ERR_WORKSPACE;
      const hipError_t e = ssm::scratch_device_ptr(&workspace);
      if (e != hipSuccess) return SSM_ERR_HIP;
    } else {
      if (!workspace || workspace_bytes < need) return SSM_ERR_WORKSPACE;
      const Range wsr{workspace, static_cast<int64_t>(need)};
      if (overlaps_any(wsr, ins) || overlap(wsr, Range{y, nBLD * es}) ||
          overlap(wsr, Range{h_final, nBDN * 4}))
        return SSM_ERR_INVALID_ARG;
    }
    return hip_status(ssm::launch_scan_lanesplit_halves(a, nsplit, static_cast<float *>(workspace), s));
  }
  if (p.variant == 3) {
    if (!lanesplit_ok) return SSM_ERR_UNSUPPORTED;
    return hip_status(ssm::launch_scan_lanesplit(a, s));
  }
  if (auto_variant && spl_of(tuning) == 0 && lanesplit_ok)
    return hip_status(ssm::launch_scan_lanesplit(a, s));
  return hip_status(ssm::launch_scan_sequential(a, spl_of(tuning), s));
}

}  // namespace

extern "C" {

ssm_status ssm_scan_fwd_ex(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype dt, const void *x,
                           const void *delta, const float *A, const void *Bm, const void *Cm,
                           const float *D_skip, const void *z, const float *h0, void *y,
                           float *h_final, void *workspace, size_t workspace_bytes,
                           const ssm_tuning *tuning, const ssm_delta_opts *dopts, void *stream) {
  return scan_fwd_impl(B, L, D, N, dt, x, delta, A, Bm, Cm, D_skip, z, h0, y, h_final, workspace,
                       workspace_bytes, tuning, dopts, stream, false);
}

ssm_status ssm_scan_fwd_noalloc(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype dt,
                                const void *x, const void *delta, const float *A, const void *Bm,
                                const void *Cm, const float *D_skip, const void *z, const float *h0,
                                void *y, float *h_final, const ssm_tuning *tuning,
                                const ssm_delta_opts *dopts, void *stream) {
  return scan_fwd_impl(B, L, D, N, dt, x, delta, A, Bm, Cm, D_skip, z, h0, y, h_final, nullptr, 0,
                       tuning, dopts, stream, true);
}

ssm_status ssm_scan_fwd_train(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype dt,
                              const void *x, const void *delta, const float *A, const void *Bm,
                              const void *Cm, const float *D_skip, const void *z, const float *h0,
                              void *y, float *h_final, float *h_ckpt, const ssm_delta_opts *dopts,
                              void *stream) {
  if (B < 0 || L < 0 || D < 0 || N < 0 || !valid_dtype(dt) || !dopts_ok(dopts))
    return SSM_ERR_INVALID_ARG;
  if (N > SSM_SCAN_MAX_N) return SSM_ERR_UNSUPPORTED;
  if (B == 0 || D == 0 || L == 0)  // no segment states to write
    return ssm_scan_fwd_ex(B, L, D, N, dt, x, delta, A, Bm, Cm, D_skip, z, h0, y, h_final, nullptr, 0,
                           nullptr, dopts, stream);
  if (!h_ckpt) return SSM_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(h_ckpt) % 16 != 0) return SSM_ERR_UNSUPPORTED;
  if (B > kMaxGridYZ) return SSM_ERR_UNSUPPORTED;
  const int64_t es = esize(dt);
  if ((L + 64) * D * es >= (int64_t(1) << 31) || (L + 64) * N * es >= (int64_t(1) << 31))
    return SSM_ERR_UNSUPPORTED;
  const int64_t nBLD = B * L * D, nBLN = B * L * N, nBDN = B * D * N;
  const int64_t nCk = B * ((L + 7) / 8) * D * N;
  if (!x || !delta || !y || (N > 0 && (!Bm || !Cm || !A))) return SSM_ERR_INVALID_ARG;
  const Range ins[] = {{x, nBLD * es},   {delta, nBLD * es}, {A, D * N * 4}, {Bm, nBLN * es},
                       {Cm, nBLN * es},  {D_skip, D * 4},    {z, nBLD * es}, {h0, nBDN * 4},
                       {dbias_of(dopts), D * 4}};
  const Range ry{y, nBLD * es}, rh{h_final, nBDN * 4}, rc{h_ckpt, nCk * 4};
  if (overlaps_any(ry, ins) || overlaps_any(rh, ins) || overlaps_any(rc, ins)) return SSM_ERR_INVALID_ARG;
  if (overlap(ry, rh) || overlap(ry, rc) || overlap(rh, rc)) return SSM_ERR_INVALID_ARG;
  ssm::ScanArgs a{};
  a.B = B; a.L = L; a.D = D; a.N = N;
  a.dt = dt == SSM_BF16 ? DType::BF16 : DType::F32;
  a.x = x; a.delta = delta; a.A = A; a.Bm = Bm; a.Cm = Cm;
  a.D_skip = D_skip; a.z = z; a.h0 = h0; a.y = y; a.h_final = h_final;
  a.delta_bias = dbias_of(dopts); a.delta_softplus = dsoft_of(dopts);
  a.h_ckpt = h_ckpt;
  if (!ssm::scan_lanesplit_supported(a)) return SSM_ERR_UNSUPPORTED;
  return hip_status(ssm::launch_scan_lanesplit(a, static_cast<hipStream_t>(stream)));
}

ssm_status ssm_state_update(int64_t S, int64_t D, int64_t N, ssm_dtype dt, float *state,
                            const void *x, const void *delta, const float *A, const void *Bm,
                            const void *Cm, const float *D_skip, const void *z, void *y,
                            void *stream) {
  return ssm_state_update_ex(S, D, N, dt, state, x, delta, A, Bm, Cm, D_skip, z, y, nullptr, stream);
}

ssm_status ssm_state_update_ex(int64_t S, int64_t D, int64_t N, ssm_dtype dt, float *state,
                               const void *x, const void *delta, const float *A, const void *Bm,
                               const void *Cm, const float *D_skip, const void *z, void *y,
                               const ssm_delta_opts *dopts, void *stream) {
  if (S < 0 || D < 0 || N < 0 || !valid_dtype(dt) || !dopts_ok(dopts)) return SSM_ERR_INVALID_ARG;
  if (N > SSM_SCAN_MAX_N) return SSM_ERR_UNSUPPORTED;
  if (S == 0 || D == 0) return SSM_OK;
  if (S > kMaxGridYZ) return SSM_ERR_UNSUPPORTED;
  if (!x || !delta || !y) return SSM_ERR_INVALID_ARG;
  if (N > 0 && (!state || !A || !Bm || !Cm)) return SSM_ERR_INVALID_ARG;
  const int64_t es = esize(dt);
  const Range ins[] = {{x, S * D * es},  {delta, S * D * es}, {A, D * N * 4}, {Bm, S * N * es},
                       {Cm, S * N * es}, {D_skip, D * 4},     {z, S * D * es},
                       {dbias_of(dopts), D * 4}};
  const Range st{state, S * D * N * 4};
  if (overlaps_any(Range{y, S * D * es}, ins) || overlap(Range{y, S * D * es}, st))
    return SSM_ERR_INVALID_ARG;
  if (overlaps_any(st, ins)) return SSM_ERR_INVALID_ARG;

  ssm::StepArgs a{};
  a.S = S; a.D = D; a.N = N; a.T = 1;
  a.dt = dt == SSM_BF16 ? DType::BF16 : DType::F32;
  a.state = state; a.x = x; a.delta = delta; a.A = A; a.Bm = Bm; a.Cm = Cm;
  a.D_skip = D_skip; a.z = z; a.y = y;
  a.delta_bias = dbias_of(dopts); a.delta_softplus = dsoft_of(dopts);
  // The vectorised step needs 16-byte aligned state and A rows.
  const bool aligned = (reinterpret_cast<uintptr_t>(state) % 16 == 0) &&
                       (reinterpret_cast<uintptr_t>(A) % 16 == 0);
  a.vec_ok = aligned;
  return hip_status(ssm::launch_state_update(a, static_cast<hipStream_t>(stream)));
}

// up to this many tokens per sequence a decode call runs the decode-step
// kernel; longer calls run the prefill scan kernels (the choice depends on T
// only, so a sequence's results do not depend on the other sequences)
// (measured at 256 sequences x 5120 channels, N = 16: the decode-step kernel
// takes 29 / 51 / 144 us at T = 1 / 4 / 16, the lane-split scan 64 us up to
// T = 8 and 92 us at T = 16)
constexpr int64_t kDecodeLoopMaxT = 4;

ssm_status ssm_decode_steps(int64_t S, int64_t T, int64_t D, int64_t N, ssm_dtype dt,
                            float *state_pool, int64_t pool_rows, const int32_t *slot_idx,
                            const void *x, const void *delta, const float *A, const void *Bm,
                            const void *Cm, const float *D_skip, const void *z, void *y,
                            const ssm_delta_opts *dopts, void *stream) {
  if (S < 0 || T < 0 || D < 0 || N < 0 || pool_rows < 0 || !valid_dtype(dt) || !dopts_ok(dopts))
    return SSM_ERR_INVALID_ARG;
  if (N > SSM_SCAN_MAX_N) return SSM_ERR_UNSUPPORTED;
  if (S == 0 || D == 0 || T == 0) return SSM_OK;
  if (S > kMaxGridYZ) return SSM_ERR_UNSUPPORTED;
  if (slot_idx == nullptr && pool_rows < S) return SSM_ERR_INVALID_ARG;
  const int64_t es = esize(dt);
  if ((T + 64) * D * es >= (int64_t(1) << 31) || (T + 64) * N * es >= (int64_t(1) << 31))
    return SSM_ERR_UNSUPPORTED;
  if (!x || !delta || !y) return SSM_ERR_INVALID_ARG;
  if (N > 0 && (!state_pool || !A || !Bm || !Cm)) return SSM_ERR_INVALID_ARG;
  const int64_t nX = S * T * D, nBC = S * T * N;
  const Range ins[] = {{x, nX * es},    {delta, nX * es},  {A, D * N * 4}, {Bm, nBC * es},
                       {Cm, nBC * es},  {D_skip, D * 4},   {z, nX * es},   {slot_idx, S * 4},
                       {dbias_of(dopts), D * 4}};
  const Range pool{state_pool, pool_rows * D * N * 4};
  if (overlaps_any(Range{y, nX * es}, ins) || overlap(Range{y, nX * es}, pool))
    return SSM_ERR_INVALID_ARG;
  if (overlaps_any(pool, ins)) return SSM_ERR_INVALID_ARG;
  // an empty pool: every slot lies outside it, so every sequence is skipped
  // (and no kernel may read a state row)
  if (slot_idx != nullptr && pool_rows == 0) return SSM_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T <= kDecodeLoopMaxT) {
    // the decode-step kernel, state carried in registers over the T tokens
    ssm::StepArgs a{};
    a.S = S; a.D = D; a.N = N; a.T = T;
    a.dt = dt == SSM_BF16 ? DType::BF16 : DType::F32;
    a.state = state_pool; a.x = x; a.delta = delta; a.A = A; a.Bm = Bm; a.Cm = Cm;
    a.D_skip = D_skip; a.z = z; a.y = y;
    a.delta_bias = dbias_of(dopts); a.delta_softplus = dsoft_of(dopts);
    a.slots = slot_idx; a.pool_rows = pool_rows;
    a.vec_ok = (reinterpret_cast<uintptr_t>(state_pool) % 16 == 0) &&
               (reinterpret_cast<uintptr_t>(A) % 16 == 0);
    return hip_status(ssm::launch_state_update(a, s));
  }
  // longer runs: the channel-sequential scan with the pool rows as both
  // initial and final state (each lane reads its state elements before
  // writing them)
  ssm::ScanArgs a{};
  a.B = S; a.L = T; a.D = D; a.N = N;
  a.dt = dt == SSM_BF16 ? DType::BF16 : DType::F32;
  a.x = x; a.delta = delta; a.A = A; a.Bm = Bm; a.Cm = Cm;
  a.D_skip = D_skip; a.z = z; a.h0 = state_pool; a.y = y; a.h_final = state_pool;
  a.delta_bias = dbias_of(dopts); a.delta_softplus = dsoft_of(dopts);
  a.slots = slot_idx; a.pool_rows = pool_rows;
  if (N == 0) return hip_status(ssm::launch_scan_lane(a, s));
  if (ssm::scan_lanesplit_supported(a)) return hip_status(ssm::launch_scan_lanesplit(a, s));
  return hip_status(ssm::launch_scan_sequential(a, 0, s));
}

size_t ssm_scan_bwd_workspace_size(int64_t B, int64_t L, int64_t D, int64_t N) {
  return ssm_scan_bwd_workspace_size_ex(B, L, D, N, 0);
}

size_t ssm_scan_bwd_workspace_size_ex(int64_t B, int64_t L, int64_t D, int64_t N,
                                      int32_t saved_states) {
  if (B < 0 || L < 0 || D < 0 || N < 0 || !ssm::scan_bwd_supported_n(N)) return 0;
  if (saved_states != 0 && saved_states != 1) return 0;
  return static_cast<size_t>(ssm::scan_bwd_ws_floats(B, L, D, N, saved_states == 1)) * sizeof(float);
}

ssm_status ssm_scan_bwd(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype dt,
                        const void *x, const void *delta, const float *A, const void *Bm,
                        const void *Cm, const float *D_skip, const void *z, const float *h0,
                        const void *dy, const float *dh_final, const float *h_ckpt, void *dx,
                        void *ddelta, void *dz,
                        float *dA, float *dB, float *dC, float *dD, float *dh0,
                        float *d_delta_bias, const ssm_delta_opts *dopts, void *workspace,
                        size_t workspace_bytes, void *stream) {
  if (B < 0 || L < 0 || D < 0 || N < 0 || !valid_dtype(dt) || !dopts_ok(dopts))
    return SSM_ERR_INVALID_ARG;
  if (!ssm::scan_bwd_supported_n(N)) return SSM_ERR_UNSUPPORTED;
  if (B > kMaxGridYZ) return SSM_ERR_UNSUPPORTED;
  const int64_t es = esize(dt);
  const int64_t nX = B * L * D, nBC = B * L * N, nS = B * D * N;
  if (nX > 0 && (!x || !delta || !dy || !dx || !ddelta || (z && !dz))) return SSM_ERR_INVALID_ARG;
  if (nBC > 0 && (!Bm || !Cm || !dB || !dC)) return SSM_ERR_INVALID_ARG;
  if (D * N > 0 && (!A || !dA)) return SSM_ERR_INVALID_ARG;
  if (!z && dz) return SSM_ERR_INVALID_ARG;
  auto a16 = [](const void *p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  if (!a16(A) || !a16(h0) || !a16(dh_final) || !a16(dh0) || !a16(h_ckpt)) return SSM_ERR_UNSUPPORTED;
  const size_t need = ssm_scan_bwd_workspace_size_ex(B, L, D, N, h_ckpt != nullptr ? 1 : 0);
  if (need > 0 && (!workspace || workspace_bytes < need || !a16(workspace))) return SSM_ERR_WORKSPACE;
  const Range ins[] = {{x, nX * es},     {delta, nX * es},    {A, D * N * 4},
                       {Bm, nBC * es},   {Cm, nBC * es},      {D_skip, D * 4},
                       {z, nX * es},     {h0, nS * 4},        {dy, nX * es},
                       {dh_final, nS * 4}, {dbias_of(dopts), D * 4}, {workspace, static_cast<int64_t>(need)},
                       {h_ckpt, B * ((L + 7) / 8) * D * N * 4}};
  const Range outs[] = {{dx, nX * es},  {ddelta, nX * es}, {dz, nX * es}, {dA, D * N * 4},
                        {dB, nBC * 4},  {dC, nBC * 4},     {dD, D * 4},   {dh0, nS * 4},
                        {d_delta_bias, D * 4}};
  for (const Range &o : outs) {
    if (overlaps_any(o, ins)) return SSM_ERR_INVALID_ARG;
    int same = 0;
    for (const Range &o2 : outs) same += overlap(o, o2) ? 1 : 0;
    if (same > 1) return SSM_ERR_INVALID_ARG;  // overlaps another output
  }
  ssm::BwdArgs a{};
  a.B = B; a.L = L; a.D = D; a.N = N;
  a.dt = dt == SSM_BF16 ? DType::BF16 : DType::F32;
  a.x = x; a.delta = delta; a.A = A; a.Bm = Bm; a.Cm = Cm; a.D_skip = D_skip; a.z = z;
  a.h0 = h0; a.dy = dy; a.dh_final = dh_final; a.h_ckpt = h_ckpt;
  a.delta_bias = dbias_of(dopts); a.delta_softplus = dsoft_of(dopts);
  a.dx = dx; a.ddelta = ddelta; a.dz = dz; a.dA = dA; a.dB = dB; a.dC = dC;
  a.dD = dD; a.dbias = d_delta_bias; a.dh0 = dh0;
  a.ws = static_cast<float *>(workspace);
  return hip_status(ssm::launch_scan_bwd(a, static_cast<hipStream_t>(stream)));
}

size_t ssm_ssd_fwd_workspace_size(int64_t B, int64_t L, int64_t H, int64_t P, int64_t G,
                                  int64_t N, int64_t chunk) {
  if (B <= 0 || L <= 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0 || chunk <= 0) return 0;
  // what the matrix-core path needs (bf16 inputs); the token-by-token path
  // needs none
  if (!ssd_mfma_applies(SSM_BF16, P, N, chunk)) return 0;
  return static_cast<size_t>(ssm::ssd_ws_bytes(B, L, H, P, G, N, chunk));
}

ssm_status ssm_ssd_fwd(int64_t B, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                       int64_t chunk, ssm_dtype dt, const void *x, const void *dt_in,
                       const float *A, const void *Bm, const void *Cm, const float *D_skip,
                       const void *z, const float *h0, void *y, float *h_final, void *workspace,
                       size_t workspace_bytes, void *stream) {
  return ssm_ssd_fwd_ex(B, L, H, P, G, N, chunk, dt, x, dt_in, A, Bm, Cm, D_skip, z, h0, y, h_final,
                        workspace, workspace_bytes, nullptr, stream);
}

ssm_status ssm_ssd_fwd_ex(int64_t B, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                          int64_t chunk, ssm_dtype dt, const void *x, const void *dt_in,
                          const float *A, const void *Bm, const void *Cm, const float *D_skip,
                          const void *z, const float *h0, void *y, float *h_final, void *workspace,
                          size_t workspace_bytes, const ssm_delta_opts *dopts, void *stream) {
  if (B < 0 || L < 0 || H < 0 || P < 0 || G < 0 || N < 0 || chunk < 0 || !valid_dtype(dt) ||
      !dopts_ok(dopts))
    return SSM_ERR_INVALID_ARG;
  if (N > SSM_SSD_MAX_N || chunk < 1) return SSM_ERR_UNSUPPORTED;
  if (G <= 0 || H % G != 0) return SSM_ERR_UNSUPPORTED;
  // the matrix-core kernels where they apply (x, B, C read and the states
  // moved in 16-byte pieces); the token-by-token kernel otherwise
  auto a16 = [](const void *p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  const bool mfma_path = ssd_mfma_applies(dt, P, N, chunk) && a16(x) && a16(Bm) && a16(Cm) && a16(h0) &&
                         a16(h_final) && a16(workspace);
  if (B == 0 || H == 0 || P == 0) return SSM_OK;
  const int64_t nc = (L + chunk - 1) / chunk;
  if (B > kMaxGridYZ || H > kMaxGridYZ) return SSM_ERR_UNSUPPORTED;
  if (L > 0 && (!x || !dt_in || !Bm || !Cm || !y)) return SSM_ERR_INVALID_ARG;
  if (!A) return SSM_ERR_INVALID_ARG;
  const int64_t es = esize(dt);
  const int64_t nX = B * L * H * P, nB = B * L * G * N, nS = B * H * P * N;
  const Range ins[] = {{x, nX * es},  {dt_in, B * L * H * es}, {A, H * 4},  {Bm, nB * es},
                       {Cm, nB * es}, {D_skip, H * 4},         {z, nX * es}, {h0, nS * 4},
                       {dbias_of(dopts), H * 4}};
  if (overlaps_any(Range{y, nX * es}, ins)) return SSM_ERR_INVALID_ARG;
  if (overlaps_any(Range{h_final, nS * 4}, ins)) return SSM_ERR_INVALID_ARG;
  if (overlap(Range{y, nX * es}, Range{h_final, nS * 4})) return SSM_ERR_INVALID_ARG;
  const int64_t need = mfma_path ? ssm::ssd_ws_bytes(B, L, H, P, G, N, chunk) : 0;
  if (need > 0 && (!workspace || static_cast<int64_t>(workspace_bytes) < need))
    return SSM_ERR_WORKSPACE;
  if (need > 0 && (overlaps_any(Range{workspace, need}, ins) ||
                   overlap(Range{workspace, need}, Range{y, nX * es}) ||
                   overlap(Range{workspace, need}, Range{h_final, nS * 4})))
    return SSM_ERR_INVALID_ARG;
  (void)nc;

  ssm::SSDArgs a{};
  a.B = B; a.L = L; a.H = H; a.P = P; a.G = G; a.N = N; a.chunk = chunk;
  a.dt_type = dt == SSM_BF16 ? DType::BF16 : DType::F32;
  a.x = x; a.dt = dt_in; a.A = A; a.Bm = Bm; a.Cm = Cm; a.D_skip = D_skip; a.z = z;
  a.h0 = h0; a.y = y; a.h_final = h_final;
  a.dt_bias = dbias_of(dopts); a.dt_softplus = dsoft_of(dopts);
  if (!mfma_path) return hip_status(ssm::launch_ssd_seq(a, static_cast<hipStream_t>(stream)));
  return hip_status(ssm::launch_ssd(a, workspace, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
