#!/usr/bin/env python3
"""Throughput of the selective-scan hot path on one MI355X.

A step is one ssm_scan_fwd call over the Mamba-2.8B-shaped prefill workload
(B=8, L=4096, D=5120, N=16; x/delta/z/B/C bf16, A/D fp32, fp32 state, random
h0, silu(z) gate on) with all inputs resident in HBM.  The headline value is
selective-scan elements per second, B*L*D*N / step time, in Gelem/s.

The JSON line also carries
* roofline: the scan kernel against the ceiling that binds it (measured live
  with HIP events on the launch stream), plus its algorithmic HBM bandwidth
  against the 8 TB/s peak;
* cpu_baseline: the fp64 CPU oracle (untuned, threads over channels) timed
  on a bounded sample of the same workload, and on one core;
* copy_GBs: a plain elementwise kernel reading and writing 1 GiB each, the
  practical ceiling the HBM-bound rates are also given against (copy_frac);
* rows: the other hot-path entry points measured the same way -- the decode
  step (S=256, D=5120, N=16, 128 steps), the Mamba-2 SSD chunked scan
  (B=2, L=8192, H=80, P=64, N=128, G=8, chunk 256) and the width-4 causal
  convolution ahead of the scan (B=8, L=4096, D=5120) with its decode step.
  Launches of tens of microseconds (the decode steps, pool decode, the
  convolution's decode step) are timed as HIP-graph replays of 32-64 calls,
  since the host's per-call cost exceeds theirs; the eager per-call event
  time and the host-driven wall time are given beside them.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# fp32 VALU lane rate from 157.3 TFLOP/s (FMA = 2 flops) and the
# transcendental unit at a quarter of it (8 lanes/clk/SIMD * 1024 SIMDs * 2.4 GHz)
VALU_LANE_OPS = 157.3e12 / 2
TRANS_LANE_OPS = VALU_LANE_OPS / 4
# per scan element: dA = exp2(delta*A2) -> 1 mul + 1 exp; u*B -> 1 mul;
# h = dA*h + u*B -> 1 fma; y += C*h -> 1 fma.  6 flops + 1 transcendental.
SCAN_VALU_PER_ELEM, SCAN_TRANS_PER_ELEM, SCAN_FLOPS_PER_ELEM = 4, 1, 6
SCAN_ELEM_PEAK = 1.0 / (SCAN_VALU_PER_ELEM / VALU_LANE_OPS + SCAN_TRANS_PER_ELEM / TRANS_LANE_OPS)
# backward, per element at least: the forward recurrence again (3 VALU) and
# one exp(delta A); the adjoint g*C + lam (1), lam*u for dB (1), g*h for dC
# (1), C*h for q (1), p = a*h_prev (1), ddelta += lam (A p + B x) (3),
# dA += (lam delta) p (2), dx += lam B (1), lam *= a (1): 15 VALU + 1 exp
BWD_VALU_PER_ELEM, BWD_TRANS_PER_ELEM = 15, 1
BWD_ELEM_PEAK = 1.0 / (BWD_VALU_PER_ELEM / VALU_LANE_OPS + BWD_TRANS_PER_ELEM / TRANS_LANE_OPS)


# the kernel sources behind each measured entry point: counters taken on
# other sources are not reported
_COMMON = ["launch.h", "device_common.h"]
KERNEL_SOURCES = {
    "scan_fwd": ["scan_fwd.hip"] + _COMMON,
    "state_update": ["state_update.hip"] + _COMMON,
    "ssd_fwd": ["ssd.hip"] + _COMMON,
    "conv1d_fwd": ["conv1d.hip"] + _COMMON,
    "conv1d_update": ["conv1d.hip"] + _COMMON,
    "decode_steps_T1": ["state_update.hip"] + _COMMON,
    "decode_steps_T4": ["state_update.hip"] + _COMMON,
    "decode_steps_T16": ["state_update.hip"] + _COMMON,
    "scan_bwd": ["scan_bwd.hip", "bwd.h"] + _COMMON,
}


def csrc_hash(entry: str) -> str:
    """sha256 (first 16 hex digits) over the kernel sources of an entry."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "mamba_selective_scan_ssm_amd", "csrc")
    for f in sorted(KERNEL_SOURCES[entry]):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic(entry: str, field: str = "bytes_per_launch"):
    """HBM bytes per launch (or per call) from the committed rocprofv3 --pmc
    runs, if they were taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        with open(p) as f:
            t = json.load(f)
        e = t.get(entry)
        if not e or e.get("csrc_hash") != csrc_hash(entry):
            return None
        return float(e[field])
    except (OSError, ValueError, KeyError):
        return None


def scan_alg_bytes(B, L, D, N, es, gate=True, h0=True, hf=True):
    """Algorithmic HBM bytes of one scan: every input read once, outputs written once."""
    b = B * L * D * es * (3 if gate else 2)      # x, delta, (z)
    b += B * L * D * es                          # y
    b += 2 * B * L * N * es                      # Bm, Cm
    b += D * N * 4 + D * 4                       # A, D_skip
    b += B * D * N * 4 * ((1 if h0 else 0) + (1 if hf else 0))
    return float(b)


def time_calls(fn, steps, warmup, torch):
    """Mean time of `fn` (ms) with HIP events on the current stream, bracketed by syncs."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(s)
        fn()
        b.record(s)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    per = [a.elapsed_time(b) for a, b in ev]
    return float(np.mean(per)), float(np.min(per)), wall


def time_graph(fn, calls, replays, torch):
    """Per-call GPU time of `fn` (ms) with the host out of the loop: `calls`
    calls captured in one HIP graph, replayed `replays` times with HIP events
    around each replay on the stream it is launched on.  For launches of a
    few tens of microseconds the host's own per-call cost exceeds the
    kernel's, so events around eager calls also time the GPU waiting for the
    next launch."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(replays)]
    for a, b in ev:
        a.record(s)
        g.replay()
        b.record(s)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) / calls for a, b in ev]
    del g
    return float(np.mean(per)), float(np.min(per))


def upload(t, torch):
    if isinstance(t, np.ndarray):
        return torch.from_numpy(np.ascontiguousarray(t, dtype=np.float32)).cuda()
    if t.bf16 is not None:
        return torch.from_numpy(t.bf16.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(t.f32)).cuda()


def cpu_baseline(inp, n_seq: int):
    import oracle
    threads = min(16, oracle.default_threads())
    D = inp.D
    ch = np.arange(n_seq * D, dtype=np.int64)          # every channel of the first n_seq sequences
    t0 = time.perf_counter()
    oracle.scan(inp.x.f32, inp.delta.f32, inp.A, inp.Bm.f32, inp.Cm.f32, inp.D_skip, inp.z.f32,
                inp.h0, channels=ch, threads=threads)
    dt = time.perf_counter() - t0
    elems = n_seq * inp.L * D * inp.N
    # the same oracle on one core, over the first 512 channels of sequence 0
    ch1 = np.arange(512, dtype=np.int64)
    t1 = time.perf_counter()
    oracle.scan(inp.x.f32, inp.delta.f32, inp.A, inp.Bm.f32, inp.Cm.f32, inp.D_skip, inp.z.f32,
                inp.h0, channels=ch1, threads=1)
    dt1 = time.perf_counter() - t1
    return {"value": elems / dt / 1e9, "unit": "Gelem/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_seq} of {inp.B} sequences (all {D} channels, L={inp.L}, N={inp.N}), "
                      f"fp64 sequential recurrence, {dt:.2f} s wall",
            "one_core": {"value": len(ch1) * inp.L * inp.N / dt1 / 1e9, "unit": "Gelem/s",
                         "sample": f"512 channels of sequence 0, L={inp.L}, N={inp.N}, {dt1:.2f} s"}}


def copy_bandwidth(torch, nbytes=1 << 30):
    """GB/s of a plain device elementwise kernel reading and writing nbytes
    each (torch's multiply), timed like the hot-path rows: the practical
    ceiling the HBM-bound rows are also reported against."""
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    mean_ms, _, _ = time_calls(lambda: torch.mul(a, 1.5, out=b), 20, 5, torch)
    del a, b
    return 2 * nbytes / (mean_ms * 1e-3) / 1e9


def bench_decode(torch, ssm, gen, steps_meas=128):
    dec = gen.make_workload("decode_256x5120_bf16")
    S, D, N = dec.S, dec.D, dec.N
    state = upload(dec.state0, torch)
    xs, ds, zs, bs, cs = (upload(getattr(dec, k), torch) for k in ("x", "delta", "z", "Bm", "Cm"))
    A, Ds = upload(dec.A, torch), upload(dec.D_skip, torch)
    y = torch.empty((S, D), dtype=torch.bfloat16, device="cuda")
    it = [0]

    def one():
        t = it[0] % dec.steps
        it[0] += 1
        ssm.state_update(state, xs[t], ds[t], A, bs[t], cs[t], Ds, zs[t], y=y)

    ev_ms, _, wall_ms = time_calls(one, steps_meas, 8, torch)
    mean_ms, min_ms = time_graph(one, 32, 8, torch)
    alg = S * D * N * 4 * 2 + S * D * 2 * 4 + 2 * S * N * 2 + D * N * 4 + D * 4
    # the 84 MB state fits the 256 MB last-level (Infinity) cache; a model
    # steps one such state per layer, so also time six states used in turn
    # (504 MB), as six layers of one decode step would
    states = [state.clone() for _ in range(6)]
    it2 = [0]

    def rotated():
        i = it2[0]
        it2[0] += 1
        t = (i // 6) % dec.steps
        ssm.state_update(states[i % 6], xs[t], ds[t], A, bs[t], cs[t], Ds, zs[t], y=y)

    rot_ms, _ = time_graph(rotated, 36, 8, torch)
    del states
    return {"workload": "decode_256x5120_bf16 (S=256, D=5120, N=16, bf16, fp32 state)",
            "kernel_ms_per_step": mean_ms, "kernel_ms_per_step_min": min_ms,
            "eager_event_ms_per_step": ev_ms, "wall_ms_per_step": wall_ms,
            "Gelem_per_s": S * D * N / (mean_ms * 1e-3) / 1e9,
            "alg_bytes_per_step": alg, "hbm_GBs": alg / (mean_ms * 1e-3) / 1e9,
            "hbm_frac": alg / (mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "traffic_bytes_per_step": load_traffic("state_update"),
            "six_states_in_turn": {"kernel_ms_per_step": rot_ms, "hbm_GBs": alg / (rot_ms * 1e-3) / 1e9,
                                   "hbm_frac": alg / (rot_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}}


def bench_ssd(torch, ssm, gen, steps=10):
    w = gen.make_workload("ssd_mamba2_bf16")
    t = {k: upload(getattr(w, k), torch) for k in ("x", "dt", "Bm", "Cm")}
    A, Ds, h0 = upload(w.A, torch), upload(w.D_skip, torch), upload(w.h0, torch)
    ws_n = ssm.ssd_fwd_workspace_size(w.B, w.L, w.H, w.P, w.G, w.N, w.chunk)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")
    y = torch.empty((w.B, w.L, w.H, w.P), dtype=torch.bfloat16, device="cuda")
    hf = torch.empty((w.B, w.H, w.P, w.N), dtype=torch.float32, device="cuda")

    def one():
        ssm.ssd_fwd(t["x"], t["dt"], A, t["Bm"], t["Cm"], Ds, None, h0, chunk=w.chunk, y=y,
                    h_final=hf, workspace=ws)

    try:
        one()
    except Exception as e:  # not built for this configuration
        return {"workload": "ssd_mamba2_bf16", "error": str(e)}
    mean_ms, min_ms, wall_ms = time_calls(one, steps, 10, torch)
    B, L, H, P, G, N = w.B, w.L, w.H, w.P, w.G, w.N
    alg = (B * L * H * P * 2 * 2 + B * L * H * 2 + 2 * B * L * G * N * 2 + H * 8
           + 2 * B * H * P * N * 4)
    flops = 2.0 * B * L * (w.chunk * G * N + w.chunk * H * P + 2 * H * P * N)  # dense chunked GEMMs
    return {"workload": "ssd_mamba2_bf16 (B=2, L=8192, H=80, P=64, N=128, G=8, chunk=256)",
            "ms": mean_ms, "Gelem_per_s": B * L * H * P * N / (mean_ms * 1e-3) / 1e9,
            "alg_bytes": alg, "hbm_GBs": alg / (mean_ms * 1e-3) / 1e9,
            "hbm_frac": alg / (mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "dense_gemm_TFLOPs": flops / (mean_ms * 1e-3) / 1e12,
            "mfma_frac_bf16": flops / (mean_ms * 1e-3) / 2.5e15, "workspace_bytes": ws_n,
            "traffic_bytes": load_traffic("ssd_fwd", "bytes_per_call")}


def bench_conv(torch, ssm, gen, steps=50):
    """Width-4 causal convolution ahead of the 2.8B-shaped scan (prefill) and
    its decode step; both HBM-bound."""
    c = gen.make_workload("conv_mamba2p8b_bf16")
    B, L, D, K = c.B, c.L, c.D, c.K
    x, w, bias, s0 = upload(c.x, torch), upload(c.w, torch), upload(c.bias, torch), upload(c.state0, torch)
    y = torch.empty((B, L, D), dtype=torch.bfloat16, device="cuda")
    st = torch.empty((B, D, K - 1), dtype=torch.float32, device="cuda")

    def one():
        ssm.conv1d_fwd(x, w, bias, s0, y=y, state_out=st)

    mean_ms, min_ms, _ = time_calls(one, steps, 10, torch)
    alg = B * L * D * 2 * 2 + D * K * 4 + D * 4 + 2 * B * D * (K - 1) * 4
    out = {"workload": "conv_mamba2p8b_bf16 (B=8, L=4096, D=5120, K=4, bf16, SiLU)",
           "ms": mean_ms, "alg_bytes": alg, "hbm_GBs": alg / (mean_ms * 1e-3) / 1e9,
           "hbm_frac": alg / (mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "traffic_bytes": load_traffic("conv1d_fwd", "bytes_per_call")}
    d = gen.make_workload("conv_decode_256x5120_bf16")
    S, Dd, Kd = d.S, d.D, d.K
    state = upload(d.state0, torch)
    xs = upload(d.x, torch)
    wd, bd = upload(d.w, torch), upload(d.bias, torch)
    yd = torch.empty((S, Dd), dtype=torch.bfloat16, device="cuda")
    it = [0]

    def step():
        t = it[0] % d.steps
        it[0] += 1
        ssm.conv1d_update(state, xs[t], wd, bd, y=yd)

    dev_ms, _, dwall = time_calls(step, 128, 8, torch)
    dm, _ = time_graph(step, 64, 8, torch)
    dalg = S * Dd * (Kd - 1) * 4 * 2 + S * Dd * 2 * 2 + Dd * Kd * 4 + Dd * 4
    out["decode"] = {"workload": "conv_decode_256x5120_bf16 (S=256, D=5120, K=4)",
                     "kernel_ms_per_step": dm, "eager_event_ms_per_step": dev_ms,
                     "wall_ms_per_step": dwall, "alg_bytes_per_step": dalg,
                     "hbm_GBs": dalg / (dm * 1e-3) / 1e9,
                     "hbm_frac": dalg / (dm * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "traffic_bytes_per_step": load_traffic("conv1d_update", "bytes_per_call")}
    return out


def bench_bwd(torch, ssm, gen, steps=10):
    """Backward of the 2.8B-shaped prefill scan (ssm_scan_bwd): all gradients
    (dx, ddelta, dz, dA, dB, dC, dD, dh0) for dy and dh_final."""
    inp = gen.make_workload("mamba2p8b_prefill_bf16")
    B, L, D, N = inp.B, inp.L, inp.D, inp.N
    gr = gen.make_grads(B, L, D, N, dtype="bf16", seed=1008)
    t = {k: upload(getattr(inp, k), torch) for k in ("x", "delta", "z", "Bm", "Cm")}
    A, Ds, h0 = upload(inp.A, torch), upload(inp.D_skip, torch), upload(inp.h0, torch)
    dy, dhf = upload(gr.dy, torch), upload(gr.dh_final, torch)
    ws = torch.empty(ssm.scan_bwd_workspace_size(B, L, D, N), dtype=torch.uint8, device="cuda")
    del inp, gr

    def one():
        ssm.scan_bwd(t["x"], t["delta"], A, t["Bm"], t["Cm"], Ds, t["z"], h0, dy, dhf, workspace=ws)

    ms, min_ms, wall = time_calls(one, steps, 3, torch)
    elems = B * L * D * N
    io = B * L * D * 2 * 7 + B * L * N * (2 * 2 + 4 * 2) + D * N * 4 * 2 + D * 4 * 2 + B * D * N * 4 * 3
    rate = elems / (ms * 1e-3)
    # a training step's pair: the forward saving the 8-token segment states,
    # then the backward reading them instead of recomputing them
    saved = {}

    def fwd_train():
        saved["ck"] = ssm.scan_fwd_train(t["x"], t["delta"], A, t["Bm"], t["Cm"], Ds, t["z"], h0)[2]

    fms, _, _ = time_calls(fwd_train, steps, 3, torch)
    ck = saved["ck"]

    def bwd_saved():
        ssm.scan_bwd(t["x"], t["delta"], A, t["Bm"], t["Cm"], Ds, t["z"], h0, dy, dhf, workspace=ws, h_ckpt=ck)

    bms, _, _ = time_calls(bwd_saved, steps, 3, torch)
    return {"workload": "mamba2p8b_prefill_bf16 backward (B=8, L=4096, D=5120, N=16, bf16, all gradients)",
            "ms": ms, "ms_min": min_ms, "Gelem_per_s": rate / 1e9, "alg_bytes": io,
            "hbm_GBs": io / (ms * 1e-3) / 1e9, "hbm_frac": io / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "alu_frac": rate / BWD_ELEM_PEAK, "alu_peak_Telem_s": BWD_ELEM_PEAK / 1e12,
            "workspace_bytes": ws.numel(), "traffic_bytes": load_traffic("scan_bwd", "bytes_per_call"),
            "with_saved_states": {"fwd_train_ms": fms, "bwd_ms": bms, "step_ms": fms + bms,
                                  "bwd_alu_frac": elems / (bms * 1e-3) / BWD_ELEM_PEAK,
                                  "saved_state_bytes": ck.numel() * 4}}


def bench_pool_decode(torch, ssm, gen, steps=128):
    """Decode from a state pool (ssm_decode_steps): 256 sequences on scattered
    rows of a 512-row pool; 1, 4 and 16 tokens per call."""
    w = gen.make_workload("pool_decode_256x5120_bf16")
    tk = w.tokens
    S, T, D, N = tk.B, tk.L, tk.D, tk.N
    pool = upload(w.pool, torch)
    slots = torch.from_numpy(w.slots).cuda()
    t = {k: upload(getattr(tk, k), torch) for k in ("x", "delta", "z", "Bm", "Cm")}
    A, Ds = upload(tk.A, torch), upload(tk.D_skip, torch)
    out = {"workload": f"pool_decode_256x5120_bf16 (S={S}, D={D}, N={N}, pool {w.pool.shape[0]} rows, "
                       "scattered slots, bf16, fp32 state)"}
    for tt in (1, 4, T):
        tok = {k: v[:, :tt].contiguous() for k, v in t.items()}
        y = torch.empty((S, tt, D), dtype=torch.bfloat16, device="cuda")

        def one():
            ssm.decode_steps(pool, tok["x"], tok["delta"], A, tok["Bm"], tok["Cm"], Ds, tok["z"],
                             slots=slots, y=y)

        ev_ms, _, wall = time_calls(one, steps, 8, torch)
        ms, _ = time_graph(one, 32, 8, torch)
        alg = S * D * N * 4 * 2 + S * tt * D * 2 * 4 + 2 * S * tt * N * 2 + D * N * 4 + D * 4 + S * 4
        out[f"T{tt}"] = {"kernel_ms_per_call": ms, "eager_event_ms_per_call": ev_ms,
                         "wall_ms_per_call": wall, "tokens_per_call": S * tt,
                         "alg_bytes_per_call": alg, "hbm_GBs": alg / (ms * 1e-3) / 1e9,
                         "hbm_frac": alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "us_per_token_step": ms * 1e3 / tt,
                         "traffic_bytes_per_call": load_traffic(f"decode_steps_T{tt}", "bytes_per_call")}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--no-rows", action="store_true", help="skip the decode and SSD rows")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seqs", type=int, default=8)
    ap.add_argument("--only", choices=["scan", "decode", "ssd", "conv", "pool", "bwd"], default=None,
                    help="time one hot-path entry point only (for profiling); prints its row")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 1 GiB device copy (read 1 GiB, write 1 GiB) so a "
                         "counter run can scale FETCH_SIZE/WRITE_SIZE")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(channels and sequences are independent; see the sharding notes).", file=sys.stderr)
        sys.exit(2)

    import torch

    import mamba_selective_scan_ssm_amd as ssm
    import ssm_inputs as gen

    if args.copy_calib:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)   # elementwise copy kernel: 1 GiB read + 1 GiB written
        torch.cuda.synchronize()
        del src, dst
    if args.only == "decode":
        print(json.dumps({"decode": bench_decode(torch, ssm, gen)}))
        return
    if args.only == "ssd":
        print(json.dumps({"ssd": bench_ssd(torch, ssm, gen, steps=args.steps)}))
        return
    if args.only == "bwd":
        print(json.dumps({"bwd": bench_bwd(torch, ssm, gen, steps=args.steps)}))
        return
    if args.only == "pool":
        print(json.dumps({"pool_decode": bench_pool_decode(torch, ssm, gen, steps=args.steps)}))
        return
    if args.only == "conv":
        print(json.dumps({"conv": bench_conv(torch, ssm, gen, steps=args.steps)}))
        return

    name = "mamba2p8b_prefill_bf16"
    inp = gen.make_workload(name)
    B, L, D, N = inp.B, inp.L, inp.D, inp.N
    t = {k: upload(getattr(inp, k), torch) for k in ("x", "delta", "z", "Bm", "Cm")}
    A, Ds, h0 = upload(inp.A, torch), upload(inp.D_skip, torch), upload(inp.h0, torch)
    y = torch.empty((B, L, D), dtype=torch.bfloat16, device="cuda")
    hf = torch.empty((B, D, N), dtype=torch.float32, device="cuda")
    ws_n = ssm.scan_fwd_workspace_size(B, L, D, N)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")

    def step():
        ssm.scan_fwd(t["x"], t["delta"], A, t["Bm"], t["Cm"], Ds, t["z"], h0, y=y, h_final=hf,
                     workspace=ws)

    mean_ms, min_ms, wall_ms = time_calls(step, args.steps, args.warmup, torch)
    elems = B * L * D * N
    value = elems / (wall_ms * 1e-3) / 1e9
    alg = scan_alg_bytes(B, L, D, N, 2)
    kern_s = mean_ms * 1e-3
    hbm_gbs = alg / kern_s / 1e9
    elem_rate = elems / kern_s
    traffic = load_traffic("scan_fwd")
    roofline = {
        "bound": "alu",
        "achieved": elem_rate * SCAN_FLOPS_PER_ELEM / 1e12,
        "peak": SCAN_ELEM_PEAK * SCAN_FLOPS_PER_ELEM / 1e12,
        "unit": "TFLOP/s",
        "frac": elem_rate / SCAN_ELEM_PEAK,
        "traffic": traffic,
        "kernel_ms": mean_ms,
        "kernel_ms_min": min_ms,
        "hbm": {"achieved": hbm_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": hbm_gbs / HBM_PEAK_GBS, "alg_bytes_per_launch": alg},
        "note": "per element 4 fp32 VALU ops + 1 v_exp_f32; ALU ceiling "
                f"{SCAN_ELEM_PEAK / 1e12:.2f} Telem/s is below the HBM ceiling "
                f"{HBM_PEAK_GBS * 1e9 / (alg / elems) / 1e12:.2f} Telem/s",
    }
    out = {
        "metric": "selective-scan Gelem/s (B*L*D*N) + achieved HBM GB/s vs peak on 1 MI355X",
        "value": value, "unit": "Gelem/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall_ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "mamba-2.8B-shaped prefill selective scan", "B": B, "L": L, "D": D,
                   "N": N, "inputs": "x/delta/z/B/C bf16, A/D fp32, fp32 state, random h0, gate on",
                   "parallelism": "single GPU"},
        "hbm_GBs": hbm_gbs, "hbm_frac": hbm_gbs / HBM_PEAK_GBS,
        "roofline": roofline,
    }
    if not args.no_rows and args.only is None:
        copy_gbs = copy_bandwidth(torch)
        out["copy_GBs"] = copy_gbs
        out["roofline"]["hbm"]["frac_of_copy"] = hbm_gbs / copy_gbs
        out["rows"] = {"decode": bench_decode(torch, ssm, gen), "ssd": bench_ssd(torch, ssm, gen, steps=20),
                       "conv": bench_conv(torch, ssm, gen), "pool_decode": bench_pool_decode(torch, ssm, gen),
                       "bwd": bench_bwd(torch, ssm, gen)}
        for row in out["rows"].values():  # HBM rates also as a fraction of the copy
            for r in [row] + [v for v in row.values() if isinstance(v, dict)]:
                if "hbm_GBs" in r:
                    r["copy_frac"] = r["hbm_GBs"] / copy_gbs
    if not args.no_cpu and args.only is None:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seqs)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
