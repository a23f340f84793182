// Single-token decode step (selective_state_update in "Clean up SSM ops
// directory structure - #6444"): the scan body with L = 1 and the state
// (S, D, N) fp32 read and written in place.
//
// The step is HBM-bound on the state (read + write of S*D*N fp32), so the
// layout is chosen for the state stream: a channel's N states are N/4 lanes
// holding four consecutive states each, so one 16-byte load per lane covers
// the state tensor contiguously across the wave.  The y contraction over n is
// finished with a butterfly over those N/4 lanes.  Sizes this layout does not
// cover (N not a multiple of 4, or a state/A not 16-byte aligned) go to the
// per-lane scan kernel with L = 1, whose lanes read and then write only their
// own state row.
#include "device_common.h"
#include "launch.h"

namespace ssm {
namespace {

constexpr int kBlock = 256;

// LPC = lanes per channel (N / 4).
template <typename T, int LPC>
__global__ __launch_bounds__(kBlock) void state_update_kernel(StepArgs a) {
  constexpr int N = 4 * LPC;
  constexpr int kCh = kBlock / LPC;  // channels per block
  const int q = threadIdx.x % LPC;
  const int64_t d_raw = static_cast<int64_t>(blockIdx.x) * kCh + threadIdx.x / LPC;
  const int64_t s = blockIdx.y;
  const int64_t D = a.D;
  int64_t row = s;  // state row of sequence s
  if (a.slots != nullptr) {
    const int32_t sl = a.slots[s];
    if (sl < 0 || sl >= a.pool_rows) return;  // uniform over the block
    row = sl;
  }
  const bool active = d_raw < D;
  const int64_t d = active ? d_raw : D - 1;

  float4 *st = reinterpret_cast<float4 *>(a.state + (row * D + d) * N) + q;
  const float4 hv = *st;
  const float4 Av = reinterpret_cast<const float4 *>(a.A + d * N)[q];
  const T *Bt = static_cast<const T *>(a.Bm) + s * N + 4 * q;
  const T *Ct = static_cast<const T *>(a.Cm) + s * N + 4 * q;
  const float dl = step_size(to_f32(static_cast<const T *>(a.delta)[s * D + d]),
                             a.delta_bias ? a.delta_bias[d] : 0.f, a.delta_softplus);
  const float xv = to_f32(static_cast<const T *>(a.x)[s * D + d]);
  const float u = dl * xv;

  float h[4] = {hv.x, hv.y, hv.z, hv.w};
  const float Ar[4] = {Av.x, Av.y, Av.z, Av.w};
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float dA = fast_exp2(dl * (Ar[j] * kLog2e));
    h[j] = fmaf(dA, h[j], u * to_f32(Bt[j]));
    acc = fmaf(to_f32(Ct[j]), h[j], acc);
  }
#pragma unroll
  for (int off = LPC / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, LPC);

  if (!active) return;
  *st = make_float4(h[0], h[1], h[2], h[3]);
  if (q == 0) {
    float v = acc;
    if (a.D_skip) v = fmaf(a.D_skip[d], xv, v);
    if (a.z) v *= silu(to_f32(static_cast<const T *>(a.z)[s * D + d]));
    static_cast<T *>(a.y)[s * D + d] = from_f32<T>(v);
  }
}

template <typename T, int LPC>
hipError_t launch_t(const StepArgs &a, hipStream_t st) {
  constexpr int kCh = kBlock / LPC;
  dim3 grid(static_cast<unsigned>((a.D + kCh - 1) / kCh), static_cast<unsigned>(a.S));
  state_update_kernel<T, LPC><<<grid, kBlock, 0, st>>>(a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dt(const StepArgs &a, hipStream_t st) {
  switch (a.vec_ok ? a.N : -1) {
    case 4: return launch_t<T, 1>(a, st);
    case 8: return launch_t<T, 2>(a, st);
    case 16: return launch_t<T, 4>(a, st);
    case 32: return launch_t<T, 8>(a, st);
    case 64: return launch_t<T, 16>(a, st);
    default: break;
  }
  // Other N or unaligned rows: the per-lane scan over one token, the state
  // as both h0 and h_final (each lane reads its row before writing it).
  ScanArgs sa{};
  sa.B = a.S;
  sa.L = 1;
  sa.D = a.D;
  sa.N = a.N;
  sa.dt = a.dt;
  sa.x = a.x;
  sa.delta = a.delta;
  sa.A = a.A;
  sa.Bm = a.Bm;
  sa.Cm = a.Cm;
  sa.D_skip = a.D_skip;
  sa.z = a.z;
  sa.h0 = a.state;
  sa.y = a.y;
  sa.h_final = a.state;
  sa.delta_bias = a.delta_bias;
  sa.delta_softplus = a.delta_softplus;
  sa.slots = a.slots;
  sa.pool_rows = a.pool_rows;
  return launch_scan_lane(sa, st);
}

}  // namespace

hipError_t launch_state_update(const StepArgs &a, hipStream_t st) {
  if (a.dt == DType::BF16) return launch_dt<bf16_t>(a, st);
  return launch_dt<float>(a, st);
}

}  // namespace ssm
