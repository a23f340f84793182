// Launcher interface of the selective-scan backward (scan_bwd.hip).  The
// arguments are validated by the C ABI before the launch.
#pragma once

#include "launch.h"

namespace ssm {

struct BwdArgs {
  int64_t B, L, D, N;
  DType dt;
  const void *x, *delta;
  const float *A;
  const void *Bm, *Cm;
  const float *D_skip;       // (D) or null
  const void *z;             // (B, L, D) or null
  const float *h0;           // (B, D, N) or null
  const void *dy;            // (B, L, D): gradient of the output y
  const float *dh_final;     // (B, D, N) or null: gradient of h_final
  const float *h_ckpt;       // (B, ceil(L/8), D, N) states entering each 8-token
                             // segment, saved by the forward; null: recomputed
  const float *delta_bias;   // (D) or null
  bool delta_softplus;
  void *dx, *ddelta, *dz;    // (B, L, D) in the input dtype (dz null without z)
  float *dA;                 // (D, N)
  float *dB, *dC;            // (B, L, N)
  float *dD, *dbias;         // (D) or null
  float *dh0;                // (B, D, N) or null
  float *ws;                 // scan_bwd_ws_floats(B, L, D, N, h_ckpt != null) floats
};

// Supported: N in {4, 8, 16, 32, 64}.
bool scan_bwd_supported_n(int64_t N);
// Workspace floats: the states entering every 8-token segment (unless the
// forward saved them), the dB/dC tile partials and the parameter partials.
int64_t scan_bwd_ws_floats(int64_t B, int64_t L, int64_t D, int64_t N, bool saved_states);
hipError_t launch_scan_bwd(const BwdArgs &a, hipStream_t s);

}  // namespace ssm
