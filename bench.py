#!/usr/bin/env python3
"""Throughput of the selective-scan hot path on one MI355X.

A step is one ssm_scan_fwd call over the Mamba-2.8B-shaped prefill workload
(B=8, L=4096, D=5120, N=16; x/delta/z/B/C bf16, A/D fp32, fp32 state, random
h0, silu(z) gate on) with all inputs resident in HBM.  The headline value is
selective-scan elements per second, B*L*D*N / step time, in Gelem/s.

The JSON line also carries
* roofline: the scan kernel against the HBM roofline (algorithmic bytes per
  launch / kernel time, measured live with HIP events on the launch stream,
  against 8 TB/s), with the measured HBM traffic from rocprofv3 counters and,
  under "alu", the issue-rate ceiling of the method's instruction mix and
  the kernel's own mix from its VALU counters;
* cpu_baseline: the fp64 CPU oracle (untuned, threads over channels) timed
  on the same workload, and on one core;
* copy_GBs: a plain elementwise kernel reading and writing 1 GiB each, the
  practical ceiling the HBM-bound rates are also given against (copy_frac);
* rows: the other configurations and hot-path entry points measured the same
  way -- the tiny scan (B=1, L=64, D=16, N=4, fp32) and the Mamba-130M-shaped
  scan (B=1, L=2048, D=1536, N=16, fp32) under every schedule, the decode step
  (S=256, D=5120, N=16, 128 steps), the Mamba-2 SSD chunked scan (B=2,
  L=8192, H=80, P=64, N=128, G=8, chunk 256), the width-4 causal convolution
  ahead of the scan (B=8, L=4096, D=5120) with its decode step, pool decode
  and the backward.  Launches of tens of microseconds are timed as HIP-graph
  replays, since the host's per-call cost exceeds theirs; the eager per-call
  event time and the host-driven wall time are given beside them.  The rows
  run before the headline steps, which therefore start on a warm device.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
       python bench.py --summarize DIR   (rocprofv3 output -> profiles/)
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
BF16_MFMA_PEAK = 2.5e15
# gfx950 issue model: 256 CUs x 4 SIMDs, each SIMD issuing one wave64 fp32
# VALU op per quad cycle (16 lanes x 4 cycles) at 2.4 GHz.  The VALU counters
# of the kernels here charge v_exp_f32 two quad cycles (SQ_ACTIVE_INST_VALU
# minus SQ_INSTS_VALU equals SQ_INSTS_VALU_TRANS_F32) and let two plain VALU
# ops of different waves share one quad cycle (SQ_ACTIVE_INST_VALU2); a
# transcendental never shares one.
SIMDS, CLOCK_HZ = 1024, 2.4e9
CLOCK_WARMUP_S = 0.5  # untimed headline steps before the warm-up steps (clock ramp)
# per scan element: dA = exp2(delta*A2) -> 1 mul + 1 exp; u*B -> 1 mul;
# h = dA*h + u*B -> 1 fma; y += C*h -> 1 fma.  4 VALU + 1 transcendental.
SCAN_VALU_PER_ELEM, SCAN_TRANS_PER_ELEM = 4, 1


def issue_ceiling(valu, trans, paired):
    """Elements per second if every SIMD issued only this mix, back to back:
    plain ops one quad cycle each (half when every one pairs), transcendentals
    two."""
    quads = valu / (2.0 if paired else 1.0) + 2.0 * trans
    return SIMDS * CLOCK_HZ * 64 / (4.0 * quads)


SCAN_ELEM_FLOOR = issue_ceiling(SCAN_VALU_PER_ELEM, SCAN_TRANS_PER_ELEM, False)   # 6.55 Telem/s
SCAN_ELEM_PAIRED = issue_ceiling(SCAN_VALU_PER_ELEM, SCAN_TRANS_PER_ELEM, True)   # 9.83 Telem/s
# backward, per element at least: the forward recurrence again (3 VALU) and
# one exp(delta A); the adjoint g*C + lam (1), lam*u for dB (1), g*h for dC
# (1), C*h for q (1), p = a*h_prev (1), ddelta += lam (A p + B x) (3),
# dA += (lam delta) p (2), dx += lam B (1), lam *= a (1): 15 VALU + 1 exp
BWD_VALU_PER_ELEM, BWD_TRANS_PER_ELEM = 15, 1
BWD_ELEM_PEAK = issue_ceiling(BWD_VALU_PER_ELEM, BWD_TRANS_PER_ELEM, False)


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
    "decode_steps_T16": ["scan_fwd.hip"] + _COMMON,
    "scan_bwd": ["scan_bwd.hip", "bwd.h", "scan_fwd.hip"] + _COMMON,
    "scan_fwd_130m": ["scan_fwd.hip"] + _COMMON,
}


def csrc_hash(entry: str) -> str:
    """sha256 (first 16 hex digits) over the kernel sources of an entry."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "mamba_selective_scan_ssm_amd", "csrc")
    for f in sorted(KERNEL_SOURCES[entry]):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_entry(entry: str):
    """The committed rocprofv3 figures of an entry point (profiles/traffic.json),
    if they were taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        with open(p) as f:
            e = json.load(f).get(entry)
    except (OSError, ValueError):
        return None
    if not e or e.get("csrc_hash") != csrc_hash(entry):
        return None
    return e


def load_traffic(entry: str, field: str = "bytes_per_launch"):
    """HBM bytes per launch (or per call) from the committed rocprofv3 --pmc
    runs, if they were taken on the current kernel sources; else None."""
    e = load_entry(entry)
    try:
        return None if e is None else float(e[field])
    except (KeyError, TypeError, ValueError):
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
    """Mean and min time of `fn` (ms) with HIP events on the current stream,
    bracketed by syncs, and the wall-clock time per call."""
    mean, mn, _, wall = time_calls_full(fn, steps, warmup, torch)
    return mean, mn, wall


def time_calls_full(fn, steps, warmup, torch):
    """time_calls with the median too: (mean, min, median, wall) in ms."""
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
    return float(np.mean(per)), float(np.min(per)), float(np.median(per)), wall


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
    """The fp64 oracle as it stands, on the first n_seq sequences of the
    workload (all channels, whole L), threads over channels: as many threads as
    the CPUs this process may run on, at most 16 -- the host share that goes
    with one GPU on the machines this runs on (the count used is reported).
    Then the same oracle on one core over 512 channels."""
    import oracle
    affinity = oracle.default_threads()
    threads = min(16, affinity)
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
                      f"fp64 sequential recurrence, {dt:.2f} s wall, {dt * threads:.1f} thread-s",
            "host_cpus": os.cpu_count(), "affinity_cpus": affinity,
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


def scan_inputs(inp, torch):
    t = {k: upload(getattr(inp, k), torch) for k in ("x", "delta", "z", "Bm", "Cm")}
    return t, upload(inp.A, torch), upload(inp.D_skip, torch), upload(inp.h0, torch)


def bench_tiny(torch, ssm, gen):
    """The tiny fp32 scan (B=1, L=64, D=16, N=4, gate on): one launch, bound
    by launch latency rather than by any unit of the chip."""
    inp = gen.make_workload("tiny_fp32")
    B, L, D, N = inp.B, inp.L, inp.D, inp.N
    t, A, Ds, h0 = scan_inputs(inp, torch)
    y = torch.empty((B, L, D), dtype=torch.float32, device="cuda")
    hf = torch.empty((B, D, N), dtype=torch.float32, device="cuda")

    def one():
        ssm.scan_fwd(t["x"], t["delta"], A, t["Bm"], t["Cm"], Ds, t["z"], h0, y=y, h_final=hf)

    ev_ms, _, wall = time_calls(one, 64, 8, torch)
    ms, _ = time_graph(one, 64, 8, torch)
    alg = scan_alg_bytes(B, L, D, N, 4)
    return {"workload": "tiny_fp32 (B=1, L=64, D=16, N=4, fp32, gate on, random h0)",
            "kernel_us_per_call": ms * 1e3, "eager_event_us_per_call": ev_ms * 1e3,
            "wall_us_per_call": wall * 1e3, "alg_bytes": alg, "bound": "launch"}


def bench_130m(torch, ssm, gen, steps=50):
    """The Mamba-130M-shaped fp32 scan (B=1, L=2048, D=1536, N=16, gate on,
    random h0) under the automatic schedule and each schedule forced: at 24
    channel tiles per sequence the choice between the channel-sequential
    kernels and the chunked one is what this row measures."""
    inp = gen.make_workload("mamba130m_fp32")
    B, L, D, N = inp.B, inp.L, inp.D, inp.N
    t, A, Ds, h0 = scan_inputs(inp, torch)
    y = torch.empty((B, L, D), dtype=torch.float32, device="cuda")
    hf = torch.empty((B, D, N), dtype=torch.float32, device="cuda")
    alg = scan_alg_bytes(B, L, D, N, 4)
    out = {"workload": "mamba130m_fp32 (B=1, L=2048, D=1536, N=16, fp32, gate on, random h0)",
           "alg_bytes": alg, "traffic_bytes": load_traffic("scan_fwd_130m", "bytes_per_call")}
    names = {0: "auto", 1: "workgroup", 2: "chunked", 3: "lanesplit"}
    for v in (0, 1, 2, 3):
        ws_n = ssm.scan_fwd_workspace_size(B, L, D, N, variant=v)
        ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")

        def one():
            ssm.scan_fwd(t["x"], t["delta"], A, t["Bm"], t["Cm"], Ds, t["z"], h0, y=y, h_final=hf,
                         variant=v, workspace=ws)

        ms, min_ms, _ = time_calls(one, steps, 10, torch)
        gr_ms, _ = time_graph(one, 32, 8, torch)
        out[names[v]] = {"kernel_ms": gr_ms, "eager_event_ms": ms, "eager_event_ms_min": min_ms,
                         "Gelem_per_s": B * L * D * N / (gr_ms * 1e-3) / 1e9,
                         "hbm_GBs": alg / (gr_ms * 1e-3) / 1e9,
                         "hbm_frac": alg / (gr_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "workspace_bytes": ws_n}
    return out


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
    mean_ms, min_ms, med_ms, wall_ms = time_calls_full(one, steps, 10, torch)
    B, L, H, P, G, N = w.B, w.L, w.H, w.P, w.G, w.N
    alg = (B * L * H * P * 2 * 2 + B * L * H * 2 + 2 * B * L * G * N * 2 + H * 8
           + 2 * B * H * P * N * 4)
    Q = w.chunk
    # the method's matrix work: C.B^T and (scores).X inside each chunk on
    # their causal (lower) halves, the chunk states and the carried-in term
    flops = 2.0 * B * L * (Q * G * N / 2 + Q * H * P / 2 + 2 * H * P * N)
    e = load_entry("ssd_fwd") or {}
    return {"workload": "ssd_mamba2_bf16 (B=2, L=8192, H=80, P=64, N=128, G=8, chunk=256)",
            "ms": mean_ms, "ms_min": min_ms, "ms_median": med_ms,
            "Gelem_per_s": B * L * H * P * N / (mean_ms * 1e-3) / 1e9,
            "alg_bytes": alg, "hbm_GBs": alg / (mean_ms * 1e-3) / 1e9,
            "hbm_frac": alg / (mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "causal_matrix_GFLOP": flops / 1e9,
            "matrix_TFLOPs": flops / (mean_ms * 1e-3) / 1e12,
            "mfma_frac_bf16": flops / (mean_ms * 1e-3) / BF16_MFMA_PEAK,
            "mfma_busy_counter": e.get("mfma_busy"), "workspace_bytes": ws_n,
            "traffic_bytes": load_traffic("ssd_fwd", "bytes_per_call"),
            "fp32_token_path": bench_ssd_f32(torch, ssm, w)}


def bench_ssd_f32(torch, ssm, w, steps=5):
    """The same SSD workload in fp32 (the bf16 values widened), which runs the
    token-by-token VALU kernel: one multiply and two FMAs per element."""
    f = {k: torch.from_numpy(getattr(w, k).f32).cuda() for k in ("x", "dt", "Bm", "Cm")}
    A, Ds, h0 = upload(w.A, torch), upload(w.D_skip, torch), upload(w.h0, torch)
    y = torch.empty((w.B, w.L, w.H, w.P), dtype=torch.float32, device="cuda")
    hf = torch.empty((w.B, w.H, w.P, w.N), dtype=torch.float32, device="cuda")

    def one():
        ssm.ssd_fwd(f["x"], f["dt"], A, f["Bm"], f["Cm"], Ds, None, h0, chunk=w.chunk, y=y, h_final=hf)

    mean_ms, min_ms, _ = time_calls(one, steps, 2, torch)
    B, L, H, P, G, N = w.B, w.L, w.H, w.P, w.G, w.N
    elems = B * L * H * P * N
    alg = B * L * H * P * 4 * 2 + B * L * H * 4 + 2 * B * L * G * N * 4 + 2 * B * H * P * N * 4
    floor = SIMDS * CLOCK_HZ / 4 / 3 * 64  # 3 plain VALU ops per element, one per quad cycle
    del f, y, hf
    return {"workload": "ssd_mamba2 in fp32 (B=2, L=8192, H=80, P=64, N=128, G=8)",
            "ms": mean_ms, "ms_min": min_ms, "Gelem_per_s": elems / (mean_ms * 1e-3) / 1e9,
            "hbm_GBs": alg / (mean_ms * 1e-3) / 1e9,
            "issue_floor_Telem_s": floor / 1e12,
            "frac_of_issue_floor": elems / (mean_ms * 1e-3) / floor}


def bench_ppl_context(torch, ssm, gen):
    """Context shape, not a target: the perplexity run on the llama.cpp page
    as one scan call (4 sequences of 512 tokens, d_inner 1536, d_state 16,
    fp32 as ggml computes it), timed as graph replays."""
    inp = gen.make_scan(4, 512, 1536, 16, dtype="f32", seed=1100)
    t, A, Ds, h0 = scan_inputs(inp, torch)
    y = torch.empty((4, 512, 1536), dtype=torch.float32, device="cuda")
    hf = torch.empty((4, 1536, 16), dtype=torch.float32, device="cuda")

    def one():
        ssm.scan_fwd(t["x"], t["delta"], A, t["Bm"], t["Cm"], Ds, t["z"], h0, y=y, h_final=hf)

    ms, min_ms = time_graph(one, 16, 8, torch)
    elems = 4 * 512 * 1536 * 16
    alg = scan_alg_bytes(4, 512, 1536, 16, 4)
    return {"workload": "ppl_ctx (B=4, L=512, D=1536, N=16, fp32, gate on)", "kernel_ms": ms,
            "kernel_ms_min": min_ms, "Gelem_per_s": elems / (ms * 1e-3) / 1e9,
            "hbm_GBs": alg / (ms * 1e-3) / 1e9, "tokens_per_s": 4 * 512 / (ms * 1e-3)}


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

    mean_ms, min_ms, med_ms, _ = time_calls_full(one, steps, 10, torch)
    alg = B * L * D * 2 * 2 + D * K * 4 + D * 4 + 2 * B * D * (K - 1) * 4
    out = {"workload": "conv_mamba2p8b_bf16 (B=8, L=4096, D=5120, K=4, bf16, SiLU)",
           "ms": mean_ms, "ms_min": min_ms, "ms_median": med_ms,
           "alg_bytes": alg, "hbm_GBs": alg / (mean_ms * 1e-3) / 1e9,
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

    ms, min_ms, med_ms, wall = time_calls_full(one, steps, 3, torch)
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
            "ms": ms, "ms_min": min_ms, "ms_median": med_ms, "Gelem_per_s": rate / 1e9, "alg_bytes": io,
            "hbm_GBs": io / (ms * 1e-3) / 1e9, "hbm_frac": io / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "alu_frac": rate / BWD_ELEM_PEAK, "alu_peak_Telem_s": BWD_ELEM_PEAK / 1e12,
            "workspace_bytes": ws.numel(), "traffic_bytes": load_traffic("scan_bwd", "bytes_per_call"),
            "with_saved_states": {"fwd_train_ms": fms, "bwd_ms": bms, "step_ms": fms + bms,
                                  "bwd_alu_frac": elems / (bms * 1e-3) / BWD_ELEM_PEAK,
                                  "saved_state_bytes": ck.numel() * 4}}


def bench_pool_decode(torch, ssm, gen, steps=128, only_tokens=None):
    """Decode from a state pool (ssm_decode_steps): 256 sequences on scattered
    rows of a 512-row pool; 1, 4 and 16 tokens per call (or only_tokens)."""
    w = gen.make_workload("pool_decode_256x5120_bf16")
    tk = w.tokens
    S, T, D, N = tk.B, tk.L, tk.D, tk.N
    pool = upload(w.pool, torch)
    slots = torch.from_numpy(w.slots).cuda()
    t = {k: upload(getattr(tk, k), torch) for k in ("x", "delta", "z", "Bm", "Cm")}
    A, Ds = upload(tk.A, torch), upload(tk.D_skip, torch)
    out = {"workload": f"pool_decode_256x5120_bf16 (S={S}, D={D}, N={N}, pool {w.pool.shape[0]} rows, "
                       "scattered slots, bf16, fp32 state)"}
    for tt in (1, 4, T) if only_tokens is None else (only_tokens,):
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


# ---------------------------------------------------------------------------
# rocprofv3 output -> profiles/*.md and profiles/traffic.json
# ---------------------------------------------------------------------------
# Each entry was profiled from the repository root on the GPU machine (after
# `cd /tmp && export TMPDIR=/tmp`) into <DIR>/<entry>/<pass>/ with
#   kt: rocprofv3 --kernel-trace --stats --output-format csv -d <DIR>/<entry>/kt -o kt -- python3 bench.py --only <only> <timed args>
#   f:  rocprofv3 --pmc FETCH_SIZE --output-format csv -d <DIR>/<entry>/f -o f -- python3 bench.py --only <only> <short args> --copy-calib
#   w:  the same with --pmc WRITE_SIZE
#   v:  --pmc VALU_COUNTERS (entries with "valu")
#   m:  --pmc MFMA_COUNTERS (entries with "mfma")
VALU_COUNTERS = ["SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_VALU2",
                 "SQ_INSTS_LDS", "SQ_WAVES", "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE"]
MFMA_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU",
                 "SQ_ACTIVE_INST_VALU", "SQ_INSTS_LDS", "SQ_WAVES", "GRBM_GUI_ACTIVE"]
PROFILE_ENTRIES = {
    # entry: dict(only=--only, t=timed args, s=short args, file=summary file, title, k=kernel name
    #   patterns of one call, elems=elements per call (per-element counter figures), extra=extra
    #   passes, run=directory of the profiled run when another entry's run also covers this one)
    "scan_fwd": dict(only="scan", t="--steps 100 --warmup 30 --no-cpu", s="--steps 2 --warmup 1 --no-cpu",
                     file="scan_lanesplit_mamba2p8b_prefill_bf16.md",
                     title="Mamba-1 prefill selective scan, B=8 L=4096 D=5120 N=16, bf16 inputs, fp32 state "
                           "(ssm_scan_fwd)",
                     k=["scan_lanesplit_kernel"], elems=8 * 4096 * 5120 * 16, extra="v"),
    "scan_fwd_130m": dict(only="m130", t="--steps 50", s="--steps 2", file="scan_mamba130m_fp32.md",
                          title="Mamba-1 scan, B=1 L=2048 D=1536 N=16, fp32, every schedule (ssm_scan_fwd)",
                          k=["scan_split_kernel", "scan_carry_kernel", "scan_lanesplit_kernel"],
                          elems=2048 * 1536 * 16),
    "state_update": dict(only="decode", t="", s="", file="state_update_decode_256x5120_bf16.md",
                         title="decode step, S=256 D=5120 N=16, bf16 inputs, fp32 state (ssm_state_update)",
                         k=["state_step"]),
    "ssd_fwd": dict(only="ssd", t="--steps 20", s="--steps 2", file="ssd_chunked_mamba2_bf16.md",
                    title="Mamba-2 SSD chunked scan, B=2 L=8192 H=80 P=64 N=128 G=8 chunk 256, bf16 "
                          "(ssm_ssd_fwd)",
                    k=["ssd_"], extra="m"),
    "conv1d_fwd": dict(only="conv", t="--steps 50", s="--steps 2", file="conv1d_mamba2p8b_bf16.md",
                       title="causal convolution K=4, B=8 L=4096 D=5120 bf16 (ssm_conv1d_fwd)",
                       k=["conv1d_fwd_kernel", "conv1d_state_kernel"]),
    "conv1d_update": dict(only="conv", t="--steps 50", s="--steps 2", file="conv1d_mamba2p8b_bf16.md",
                          title="convolution decode step K=4, S=256 D=5120 bf16 (ssm_conv1d_update)",
                          k=["conv1d_update_kernel"], run="conv1d_fwd"),
    "decode_steps_T1": dict(only="pool", t="--steps 64 --pool-tokens 1", s="--steps 2 --pool-tokens 1",
                            file="decode_steps_pool_256x5120_bf16.md",
                            title="pool decode, 256 of 512 rows, D=5120 N=16 bf16, T=1 token per call "
                                  "(ssm_decode_steps)", k=["state_"]),
    "decode_steps_T4": dict(only="pool", t="--steps 64 --pool-tokens 4", s="--steps 2 --pool-tokens 4",
                            file="decode_steps_pool_256x5120_bf16.md",
                            title="pool decode, T=4 tokens per call (ssm_decode_steps)", k=["state_"]),
    "decode_steps_T16": dict(only="pool", t="--steps 64 --pool-tokens 16", s="--steps 2 --pool-tokens 16",
                             file="decode_steps_pool_256x5120_bf16.md",
                             title="pool decode, T=16 tokens per call (ssm_decode_steps; the lane-split scan "
                                   "kernel)", k=["scan_lanesplit"]),
    "scan_bwd": dict(only="bwd", t="--steps 10", s="--steps 1", file="scan_bwd_mamba2p8b_prefill_bf16.md",
                     title="selective-scan backward, B=8 L=4096 D=5120 N=16, bf16, all gradients (ssm_scan_bwd)",
                     # the backward kernels, and the states-only launch of the lane-split scan that
                     # recomputes the segment states when the forward saved none
                     k=["scan_bwd_kernel", "bwd_reduce",
                        "scan_lanesplit_kernel<ssm::bf16_t, 4, 4, false, true, false, 4, 4>"],
                     elems=8 * 4096 * 5120 * 16, extra="v"),
}


# kernels of one call under the automatic schedule, where a profiled run
# also times other schedules (short names, prefix match); default: all
CALL_KERNELS = {
    # the bf16 call's three kernels; the same run also times the fp32 token path
    "ssd_fwd": ["ssd_chunk_state", "ssd_state_pass", "ssd_chunk_scan"],
    "scan_fwd_130m": ["scan_lanesplit_kernel<float, 4, 4, false, false, false, 4, 1>", "scan_carry_kernel",
                      "scan_lanesplit_kernel<float, 4, 4, true, false, false, 4, 2>"],
}


def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _find(dirpath, suffix):
    if not os.path.isdir(dirpath):
        return None
    for root, _, files in os.walk(dirpath):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    return None


def _counters(path):
    """{dispatch id: (kernel name, {counter: value})} from a counter_collection.csv."""
    out = {}
    if path is None:
        return out
    for r in _csv_rows(path):
        d = int(r["Dispatch_Id"])
        name = r["Kernel_Name"]
        out.setdefault(d, (name, {}))[1][r["Counter_Name"]] = float(r["Counter_Value"])
    return out


def _calibration(disp, counter):
    """KiB the copy calibration kernel (torch's elementwise multiply: 1 GiB
    read and 1 GiB written) reported."""
    for name, c in disp.values():
        if "MulFunctor" in name and counter in c:
            return c[counter]
    return None


def _short(name, n=110):
    """Kernel name without 'void', namespaces and the parameter list."""
    name = name.replace("void ", "").replace("(anonymous namespace)::", "").replace("ssm::", "")
    if name.endswith(")") and "(" in name:
        name = name[:name.rindex("(")]
    return name if len(name) <= n else name[:n] + "..."


def _entry_section(src, entry, p, rec):
    """Markdown lines for one profiled entry; fills rec (its traffic.json record)."""
    base = os.path.join(src, p.get("run", entry))
    kpat, extra, elems, only = p["k"], p.get("extra", ""), p.get("elems"), p["only"]
    match = lambda name: any(k in name for k in kpat)
    trace_p = _find(os.path.join(base, "kt"), "kernel_trace.csv")
    durs = {}
    for r in _csv_rows(trace_p):
        if match(r["Kernel_Name"]):
            durs.setdefault(r["Kernel_Name"], []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    fetch = _counters(_find(os.path.join(base, "f"), "counter_collection.csv"))
    write = _counters(_find(os.path.join(base, "w"), "counter_collection.csv"))
    fcal, wcal = _calibration(fetch, "FETCH_SIZE"), _calibration(write, "WRITE_SIZE")
    fs = (1 << 30) / fcal if fcal else None   # bytes per KiB of counter
    ws_ = (1 << 30) / wcal if wcal else None

    def per_kernel(disp, counter):
        acc = {}
        for name, c in disp.values():
            if counter in c and match(name):
                acc.setdefault(name, []).append(c[counter])
        return {k: sum(v) / len(v) for k, v in acc.items()}

    f_k, w_k = per_kernel(fetch, "FETCH_SIZE"), per_kernel(write, "WRITE_SIZE")
    lines = [f"# rocprofv3: {p['title']}", ""]
    lines.append("MI355X (gfx950).  Kernel source hash (sha256, first 16 hex digits, over "
                 + ", ".join(KERNEL_SOURCES[entry]) + " in mamba_selective_scan_ssm_amd/csrc, "
                 f"as bench.py computes it): `{csrc_hash(entry)}`.  Commands, from the repository root on "
                 "the GPU machine after `cd /tmp && export TMPDIR=/tmp`:")
    lines.append("")
    cmd = lambda c: "`" + " ".join(c.split()) + "`"
    lines.append("* kernel trace: " + cmd(f"rocprofv3 --kernel-trace --stats --output-format csv -d <out>/kt "
                                          f"-o kt -- python3 bench.py --only {only} {p['t']}"))
    lines.append(f"* HBM reads: `rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/f -o f "
                 f"-- python3 bench.py --only {only} {p['s']} --copy-calib`".replace("  ", " "))
    lines.append("* HBM writes: the same with `--pmc WRITE_SIZE`")
    if "v" in extra:
        lines.append(f"* VALU counters: `rocprofv3 --pmc {' '.join(VALU_COUNTERS)} --output-format csv "
                     f"-d <out>/v -o v -- python3 bench.py --only {only} {p['s']}`".replace("  ", " "))
    if "m" in extra:
        lines.append(f"* matrix-core counters: `rocprofv3 --pmc {' '.join(MFMA_COUNTERS)} --output-format csv "
                     f"-d <out>/m -o m -- python3 bench.py --only {only} {p['s']}`".replace("  ", " "))
    lines.append("")
    if fcal and wcal:
        lines.append(f"Counter calibration: `--copy-calib` runs one elementwise copy that reads 1 GiB and "
                     f"writes 1 GiB; it read FETCH_SIZE {fcal:.0f} KiB and WRITE_SIZE {wcal:.0f} KiB, so "
                     f"FETCH_SIZE is scaled by {1048576 / fcal:.3f} and WRITE_SIZE by {1048576 / wcal:.3f} "
                     "to give bytes.")
        lines.append("")
    lines.append("| kernel | calls | avg us | min us | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch "
                 "| HBM bytes/dispatch (scaled) |")
    lines.append("|---|---|---|---|---|---|---|")
    for name, d in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        fk, wk = f_k.get(name), w_k.get(name)
        hb = (fk * fs + wk * ws_) if (fk is not None and wk is not None and fs and ws_) else None
        lines.append(f"| `{_short(name)}` | {len(d)} | {sum(d) / len(d):.1f} | {min(d):.1f} | "
                     f"{'' if fk is None else f'{fk:.0f}'} | {'' if wk is None else f'{wk:.0f}'} | "
                     f"{'' if hb is None else f'{hb / 1e6:.2f} MB'} |")
    lines.append("")
    if "v" in extra:
        disp = _counters(_find(os.path.join(base, "v"), "counter_collection.csv"))
        last = {}
        for d, (name, c) in sorted(disp.items()):
            if match(name) and "SQ_INSTS_VALU" in c:
                last[name] = c
        if last:
            lines.append("VALU counters (the last dispatch of each kernel; per wave64 element slot = per 64 "
                         "elements):")
            lines.append("")
            lines.append("| kernel | VALU insts | of which v_exp etc. (TRANS_F32) | VALU quad cycles "
                         "(ACTIVE_INST_VALU) | dual-issue quad cycles (ACTIVE_INST_VALU2) | LDS insts | waves "
                         "| VALU busy (quad cycles x 4 / (1024 SIMDs x GUI cycles / 8 XCDs)) |")
            lines.append("|---|---|---|---|---|---|---|---|")
        for name, c in last.items():
            gui = c.get("GRBM_GUI_ACTIVE", 0) / 8
            busy = c["SQ_ACTIVE_INST_VALU"] * 4 / (1024 * gui) if gui else float("nan")
            ew = elems / 64 if elems else None
            lines.append(f"| `{_short(name, 70)}` | {c['SQ_INSTS_VALU']:.4g}"
                         + (f" ({c['SQ_INSTS_VALU'] / ew:.2f}/elem-wave)" if ew else "")
                         + f" | {c['SQ_INSTS_VALU_TRANS_F32']:.4g}"
                         + (f" ({c['SQ_INSTS_VALU_TRANS_F32'] / ew:.3f})" if ew else "")
                         + f" | {c['SQ_ACTIVE_INST_VALU']:.4g} | {c['SQ_ACTIVE_INST_VALU2']:.4g}"
                         + f" ({2 * c['SQ_ACTIVE_INST_VALU2'] / c['SQ_INSTS_VALU']:.2f} of VALU insts paired)"
                         + f" | {c['SQ_INSTS_LDS']:.4g} | {c['SQ_WAVES']:.0f} | {busy:.2f} |")
            if ew and entry == "scan_fwd":
                rec["valu"] = {"valu_per_elem_wave": c["SQ_INSTS_VALU"] / ew,
                               "trans_per_elem_wave": c["SQ_INSTS_VALU_TRANS_F32"] / ew,
                               "paired_quads_per_elem_wave": c["SQ_ACTIVE_INST_VALU2"] / ew,
                               "valu_busy": busy}
        lines.append("")
    if "m" in extra:
        disp = _counters(_find(os.path.join(base, "m"), "counter_collection.csv"))
        last = {}
        for d, (name, c) in sorted(disp.items()):
            if match(name) and "SQ_VALU_MFMA_BUSY_CYCLES" in c:
                last[name] = c
        if last:
            lines.append("Matrix-core counters (last dispatch of each kernel):")
            lines.append("")
            lines.append("| kernel | MFMA busy cycles | MFMA busy (/ (1024 SIMDs x GUI cycles / 8)) "
                         "| bf16 MFMA MOPs (x512 flops) | VALU insts | LDS insts | waves |")
            lines.append("|---|---|---|---|---|---|---|")
        tot_busy, tot_gui = 0.0, 0.0
        for name, c in last.items():
            gui = c.get("GRBM_GUI_ACTIVE", 0) / 8
            mb = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * gui) if gui else float("nan")
            if entry not in CALL_KERNELS or any(_short(name).startswith(k) for k in CALL_KERNELS[entry]):
                tot_busy += c["SQ_VALU_MFMA_BUSY_CYCLES"]
                tot_gui += gui
            lines.append(f"| `{_short(name, 70)}` | {c['SQ_VALU_MFMA_BUSY_CYCLES']:.4g} | {mb:.3f} | "
                         f"{c['SQ_INSTS_VALU_MFMA_MOPS_BF16']:.4g} "
                         f"({c['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512 / 1e9:.1f} GFLOP) | "
                         f"{c['SQ_INSTS_VALU']:.4g} | {c['SQ_INSTS_LDS']:.4g} | {c['SQ_WAVES']:.0f} |")
        if tot_gui:
            rec["mfma_busy"] = tot_busy / (1024 * tot_gui)
            lines.append("")
            lines.append(f"Over the call's kernels: matrix cores busy {100 * rec['mfma_busy']:.1f}% "
                         "of SIMD-cycles.")
        lines.append("")
    # HBM bytes per call: each of the call's kernels once
    per_call, ok = 0.0, bool(f_k or w_k)
    for name in set(f_k) | set(w_k):
        if entry in CALL_KERNELS and not any(_short(name).startswith(k) for k in CALL_KERNELS[entry]):
            continue
        if name in f_k and name in w_k and fs and ws_:
            per_call += f_k[name] * fs + w_k[name] * ws_
        else:
            ok = False
    if ok:
        rec["bytes_per_call"] = per_call
        rec["bytes_per_launch"] = per_call
        which = (" under the automatic schedule (" + ", ".join(CALL_KERNELS[entry]) + ")"
                 if entry in CALL_KERNELS else "")
        lines.append(f"HBM traffic of one call{which} (each of its kernels once): {per_call / 1e6:.2f} MB.")
        lines.append("")
    return lines


def summarize_profiles(src):
    prof_dir = os.path.join(ROOT, "profiles")
    tj_path = os.path.join(prof_dir, "traffic.json")
    traffic = json.load(open(tj_path)) if os.path.exists(tj_path) else {}
    traffic["note"] = ("csrc_hash: sha256 over the entry's kernel sources (bench.KERNEL_SOURCES); "
                       "bytes: FETCH_SIZE and WRITE_SIZE scaled by the copy calibration")
    files = {}
    for entry, p in PROFILE_ENTRIES.items():
        if _find(os.path.join(src, p.get("run", entry), "kt"), "kernel_trace.csv") is None:
            continue
        rec = {"csrc_hash": csrc_hash(entry)}
        files.setdefault(p["file"], []).append(_entry_section(src, entry, p, rec))
        traffic[entry] = rec
    for fname, sections in files.items():
        with open(os.path.join(prof_dir, fname), "w") as f:
            f.write("\n".join(l for s in sections for l in s))
        print("wrote", fname)
    with open(tj_path, "w") as f:
        json.dump(traffic, f, indent=1)
    print("wrote traffic.json")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--no-rows", action="store_true", help="skip the other configurations and entry points")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seqs", type=int, default=8)
    ap.add_argument("--only", choices=["scan", "tiny", "m130", "decode", "ssd", "conv", "pool", "bwd"],
                    default=None, help="time one hot-path entry point only (for profiling); prints its row")
    ap.add_argument("--pool-tokens", type=int, choices=[1, 4, 16], default=None,
                    help="with --only pool: time this many tokens per call only (for profiling)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 1 GiB device copy (read 1 GiB, write 1 GiB) so a "
                         "counter run can scale FETCH_SIZE/WRITE_SIZE")
    ap.add_argument("--summarize", metavar="DIR", default=None,
                    help="turn the rocprofv3 output under DIR into profiles/*.md and traffic.json")
    args = ap.parse_args()
    if args.summarize:
        summarize_profiles(args.summarize)
        return
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
    single = {"tiny": ("tiny_fp32", lambda: bench_tiny(torch, ssm, gen)),
              "m130": ("mamba130m_fp32", lambda: bench_130m(torch, ssm, gen, steps=args.steps)),
              "decode": ("decode", lambda: bench_decode(torch, ssm, gen)),
              "ssd": ("ssd", lambda: bench_ssd(torch, ssm, gen, steps=args.steps)),
              "bwd": ("bwd", lambda: bench_bwd(torch, ssm, gen, steps=args.steps)),
              "pool": ("pool_decode", lambda: bench_pool_decode(torch, ssm, gen, steps=args.steps,
                                                                 only_tokens=args.pool_tokens)),
              "conv": ("conv", lambda: bench_conv(torch, ssm, gen, steps=args.steps))}
    if args.only in single:
        key, fn = single[args.only]
        print(json.dumps({key: fn()}))
        return

    # the other configurations and entry points first: besides their own
    # figures they leave the device warm for the headline steps
    rows, copy_gbs = None, None
    if not args.no_rows and args.only is None:
        copy_gbs = copy_bandwidth(torch)
        rows = {"tiny_fp32": bench_tiny(torch, ssm, gen), "mamba130m_fp32": bench_130m(torch, ssm, gen),
                "decode": bench_decode(torch, ssm, gen), "ssd": bench_ssd(torch, ssm, gen, steps=20),
                "conv": bench_conv(torch, ssm, gen), "pool_decode": bench_pool_decode(torch, ssm, gen),
                "bwd": bench_bwd(torch, ssm, gen), "ppl_context": bench_ppl_context(torch, ssm, gen)}
        for row in rows.values():  # HBM rates also as a fraction of the copy
            for r in [row] + [v for v in row.values() if isinstance(v, dict)]:
                if "hbm_GBs" in r:
                    r["copy_frac"] = r["hbm_GBs"] / copy_gbs
        torch.cuda.empty_cache()

    name = "mamba2p8b_prefill_bf16"
    inp = gen.make_workload(name)
    B, L, D, N = inp.B, inp.L, inp.D, inp.N
    t, A, Ds, h0 = scan_inputs(inp, torch)
    y = torch.empty((B, L, D), dtype=torch.bfloat16, device="cuda")
    hf = torch.empty((B, D, N), dtype=torch.float32, device="cuda")
    ws_n = ssm.scan_fwd_workspace_size(B, L, D, N)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")

    def step():
        ssm.scan_fwd(t["x"], t["delta"], A, t["Bm"], t["Cm"], Ds, t["z"], h0, y=y, h_final=hf,
                     workspace=ws)

    # The GPU clock ramps up under sustained load (from ~1.9 to ~2.37 GHz over
    # the first few dozen launches after an idle spell, such as the host-side
    # input generation above; profiles/scan_lanesplit_clock_*.md): run the
    # step untimed for CLOCK_WARMUP_S first, so the W warm-up and K timed
    # steps see the steady clock whatever W is.
    t_end = time.perf_counter() + CLOCK_WARMUP_S
    while time.perf_counter() < t_end:
        for _ in range(16):
            step()
        torch.cuda.synchronize()
    mean_ms, min_ms, med_ms, wall_ms = time_calls_full(step, args.steps, args.warmup, torch)
    elems = B * L * D * N
    value = elems / (wall_ms * 1e-3) / 1e9
    alg = scan_alg_bytes(B, L, D, N, 2)
    kern_s = mean_ms * 1e-3
    hbm_gbs = alg / kern_s / 1e9
    elem_rate = elems / kern_s
    e = load_entry("scan_fwd") or {}
    mix = e.get("valu")
    alu = {"achieved_Telem_s": elem_rate / 1e12,
           "method_floor_Telem_s": SCAN_ELEM_FLOOR / 1e12,
           "method_floor_paired_Telem_s": SCAN_ELEM_PAIRED / 1e12,
           "frac_of_floor": elem_rate / SCAN_ELEM_FLOOR,
           "kernel_mix": mix,
           "note": "4 fp32 VALU + 1 v_exp_f32 per element; one VALU op per SIMD quad cycle, "
                   "v_exp_f32 two, at 2.4 GHz on 1024 SIMDs; 'paired': every plain op dual-issued"}
    if mix:
        quads = mix["valu_per_elem_wave"] - mix["trans_per_elem_wave"] + 2 * mix["trans_per_elem_wave"] \
            - mix["paired_quads_per_elem_wave"]
        alu["kernel_mix_ceiling_Telem_s"] = SIMDS * CLOCK_HZ * 64 / (4 * quads) / 1e12
    roofline = {
        "bound": "hbm",
        "achieved": hbm_gbs,
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": hbm_gbs / HBM_PEAK_GBS,
        "traffic": e.get("bytes_per_launch"),
        "alg_bytes_per_launch": alg,
        "kernel_ms": mean_ms,
        "kernel_ms_min": min_ms,
        "kernel_ms_median": med_ms,
        "alu": alu,
    }
    out = {
        "metric": "selective-scan Gelem/s (B*L*D*N) + achieved HBM GB/s vs peak on 1 MI355X",
        "value": value, "unit": "Gelem/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "clock_warmup_s": CLOCK_WARMUP_S,
        "ms_per_step": wall_ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "mamba-2.8B-shaped prefill selective scan", "B": B, "L": L, "D": D,
                   "N": N, "inputs": "x/delta/z/B/C bf16, A/D fp32, fp32 state, random h0, gate on",
                   "parallelism": "single GPU"},
        "hbm_GBs": hbm_gbs, "hbm_frac": hbm_gbs / HBM_PEAK_GBS,
        "roofline": roofline,
    }
    if rows is not None:
        out["copy_GBs"] = copy_gbs
        out["roofline"]["frac_of_copy"] = hbm_gbs / copy_gbs
        out["rows"] = rows
    if not args.no_cpu and args.only is None:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seqs)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
