// Internal launcher interface between the C ABI (capi.cpp) and the kernels.
// Every launcher assumes its arguments were validated by the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

enum class DType : int { F32 = 0, BF16 = 1 };

struct ScanArgs {
  int64_t B, L, D, N;
  DType dt;
  const void *x, *delta;
  const float *A;
  const void *Bm, *Cm;
  const float *D_skip;
  const void *z;
  const float *h0;
  void *y;
  float *h_final;
  const float *delta_bias;  // (D) or null: added to delta
  bool delta_softplus;      // softplus of (delta + bias)
  // Optional state-row indirection (decode of a slot pool): sequence b reads
  // h0 and writes h_final at row slots[b] of a pool of pool_rows rows; a slot
  // outside [0, pool_rows) skips the sequence.  Sequential schedules only.
  const int32_t *slots;
  int64_t pool_rows;
  // Optional (lane-split schedule only): the state entering every 8-token
  // segment of sequence b, at ((b * ceil(L/8) + s) * D + d) * N + n.
  float *h_ckpt;
};

// State row of sequence b (false: skip the sequence).
__device__ __forceinline__ bool scan_state_row(const ScanArgs &a, int64_t b, int64_t &row) {
  row = b;
  if (a.slots == nullptr) return true;
  const int32_t sl = a.slots[b];
  if (sl < 0 || sl >= a.pool_rows) return false;
  row = sl;
  return true;
}

// Channel-sequential scan: a workgroup per (b, 64 channels), its waves
// splitting N, one pass over the L tokens.  spl_req = requested states per
// lane (0 = automatic).
hipError_t launch_scan_sequential(const ScanArgs &a, int spl_req, hipStream_t s);

// Channel-sequential scan with a channel's N states split over 1, 2 or 4
// adjacent lanes of one wave (no workgroup barrier).  Supported for N in
// {4, 8, 16, 32, 64}, even D, 16-byte aligned Bm and Cm, and x, delta, z, y
// aligned to two elements.
bool scan_lanesplit_supported(const ScanArgs &a);
hipError_t launch_scan_lanesplit(const ScanArgs &a, hipStream_t s);

// The lane-split scan writing only a.h_ckpt (the state entering every
// 8-token segment, from h0): no y, h_final, z or C.  a.y and a.Cm must
// still be valid pointers for scan_lanesplit_supported (neither is
// accessed); no slots.
hipError_t launch_scan_states(const ScanArgs &a, hipStream_t s);

// The lane-split scan with the first nsplit workgroup tasks cut in two at
// a 32-token cycle, their second halves continuing from the state the first
// halves hand over through ws (no slots, no saved states, L >= 64): bitwise
// the results of launch_scan_lanesplit.  scan_halves_split: nsplit for this
// shape on `simds` SIMDs (0: the whole-task grid is as balanced; forced:
// half the tasks, for tests).
int64_t scan_halves_split(int64_t B, int64_t D, int64_t N, int64_t simds, bool forced);
int64_t scan_halves_ws_floats(int64_t B, int64_t D, int64_t N);
hipError_t launch_scan_lanesplit_halves(const ScanArgs &a, int64_t nsplit, float *ws, hipStream_t s);

// Chunked scan: segment summaries, carry pass over segments, output pass.
// ws must hold scan_chunked_ws_floats(...) floats.
int64_t scan_chunked_ws_floats(int64_t B, int64_t L, int64_t D, int64_t N, int64_t seg_len);
hipError_t launch_scan_chunked(const ScanArgs &a, int spl_req, int64_t seg_len, float *ws,
                               hipStream_t s);

// Library-owned device scratch (scratch.hip): kScratchBytes per device, for
// entry points whose callers cannot allocate.  Sets *ptr to this device's
// copy (the current device), looking its address up on first use.
constexpr size_t kScratchBytes = size_t(16) << 20;
hipError_t scratch_device_ptr(void **ptr);

// Workspace-free scan, one lane per channel holding all N states.  h0 and
// h_final may alias (each lane reads its row before writing it).
hipError_t launch_scan_lane(const ScanArgs &a, hipStream_t s);

struct StepArgs {
  int64_t S, D, N;
  int64_t T;  // tokens per sequence (>= 1); inputs (S, T, D) and (S, T, N)
  DType dt;
  float *state;
  const void *x, *delta;
  const float *A;
  const void *Bm, *Cm;
  const float *D_skip;
  const void *z;
  void *y;
  bool vec_ok;  // state and A rows 16-byte aligned: vectorised lanes allowed
  const float *delta_bias;  // (D) or null
  bool delta_softplus;
  const int32_t *slots;     // as ScanArgs: state row of sequence s, or null
  int64_t pool_rows;
};

hipError_t launch_state_update(const StepArgs &a, hipStream_t s);

struct SSDArgs {
  int64_t B, L, H, P, G, N, chunk;
  DType dt_type;  // storage type of x, dt, Bm, Cm, z and y
  const void *x, *dt;
  const float *A;
  const void *Bm, *Cm;
  const float *D_skip;
  const void *z;
  const float *h0;
  void *y;
  float *h_final;
  const float *dt_bias;  // (H) or null: added to dt
  bool dt_softplus;      // softplus of (dt + bias)
};

// Short causal convolution.  Prefill: x, y (B, L, D); state_in/state_out
// (B, D, K-1) (either may be null; they do not overlap).  Decode step (B =
// sequences, L = 1): state_out is the state, updated in place.
struct ConvArgs {
  int64_t B, L, D, K;
  DType dt;
  const void *x;
  const float *w, *bias;
  const float *state_in;
  float *state_out;
  void *y;
  bool act;  // SiLU on the output
};

hipError_t launch_conv1d_fwd(const ConvArgs &a, hipStream_t s);
hipError_t launch_conv1d_update(const ConvArgs &a, hipStream_t s);

// SSD on the matrix cores (ssd.hip): bf16, P = 64, N a multiple of 32 up to
// 256, chunk 64, 128 or 256; workspace ssd_ws_bytes.
int64_t ssd_ws_bytes(int64_t B, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N, int64_t chunk);
hipError_t launch_ssd(const SSDArgs &a, void *ws, hipStream_t s);
// SSD token by token on the vector ALU (ssd_seq.hip): any dtype, P, N <= 256,
// no workspace.
hipError_t launch_ssd_seq(const SSDArgs &a, hipStream_t s);

}  // namespace ssm
