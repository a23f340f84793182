"""Seeded synthetic inputs for the selective scan, shared by the HIP path's
tests and bench and by the CPU oracle's tests.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the scan's arithmetic (no discretisation, no recurrence, no
contraction, no gate).

Workloads and value laws
------------------------
The shapes follow the (B, L, D, N) problem statement of the ggml SSM_SCAN op
("ggml : add GPU support for Mamba models", compilade's test patch: d_state,
d_inner, n_seq_tokens, n_seqs) and the Mamba/Mamba-2 model sizes named in the
workload table below.  Value laws for every workload:

* x, B, C, z ~ N(0, 1)
* delta = softplus(0.5 * g - 1), g ~ N(0, 1)   (positive step sizes)
* A = -exp(u), u ~ U(log 1, log 16)            (per (d, n); per head for SSD)
* D ~ N(0, 1)
* h0 ~ N(0, 0.5)  (standard deviation 0.5)

Each tensor draws from its own child of ``SeedSequence(seed)`` so adding a
tensor never shifts the values of another.  bf16 workloads draw in fp32 and
round to bf16 with round-to-nearest-even; the fp32 view of the rounded bits is
what any consumer computes with.

Layouts (row-major, last index fastest)
---------------------------------------
Mamba-1 scan:  x, delta, z, y: (B, L, D); Bm, Cm: (B, L, N); A: (D, N);
               D_skip: (D,); h0, h_final: (B, D, N).
Decode:        per step x, delta, z: (S, D); Bm, Cm: (S, N); state (S, D, N).
Mamba-2 SSD:   x, z, y: (B, L, H, P); dt: (B, L, H); Bm, Cm: (B, L, G, N);
               A, D_skip: (H,); h0, h_final: (B, H, P, N).
Causal conv:   x, y: (B, L, D); w: (D, K); bias: (D,); state: (B, D, K-1)
               (decode: x per step (S, D), state (S, D, K-1)).

The short causal convolution's inputs draw from streams of their own:
x ~ N(0, 1) and state ~ N(0, 1) (the state holds earlier inputs); weights
and bias ~ U(-1/sqrt(K), 1/sqrt(K)), the range of a freshly initialised
depthwise convolution of width K.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

# child-stream index of every tensor: fixed forever so values never shift
_STREAMS = ("x", "delta", "z", "Bm", "Cm", "A", "D", "h0")


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even).

    Returns the bf16 payload as uint16.  Inputs are finite by construction.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact fp32 value of a bf16 payload (uint16)."""
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _children(seed: int):
    kids = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {name: np.random.default_rng(k) for name, k in zip(_STREAMS, kids)}


def _normal(rng, shape, std=1.0):
    v = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return v


def _softplus_delta(rng, shape):
    g = rng.standard_normal(size=shape, dtype=np.float32)
    g *= np.float32(0.5)
    g -= np.float32(1.0)
    # softplus(v) = log(1 + e^v); v <= ~3 here so no overflow concern
    np.exp(g, out=g)
    np.log1p(g, out=g)
    return g


def _neg_exp_uniform(rng, shape):
    u = rng.uniform(math.log(1.0), math.log(16.0), size=shape).astype(np.float32)
    return -np.exp(u).astype(np.float32)


@dataclasses.dataclass
class Tensor:
    """One input: fp32 values (exact values any consumer computes with) and,
    for bf16 storage, the bf16 payload those values came from."""

    f32: np.ndarray
    bf16: np.ndarray | None = None

    @property
    def shape(self):
        return self.f32.shape


def _store(v: np.ndarray, dtype: str) -> Tensor:
    if dtype == "bf16":
        b = bf16_round(v)
        return Tensor(bf16_to_f32(b), b)
    return Tensor(np.ascontiguousarray(v, dtype=np.float32))


# ---------------------------------------------------------------------------
# Mamba-1 selective scan inputs
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class ScanInputs:
    B: int
    L: int
    D: int
    N: int
    dtype: str                 # storage dtype of x, delta, z, Bm, Cm (and y)
    x: Tensor
    delta: Tensor
    A: np.ndarray              # fp32 (D, N)
    Bm: Tensor
    Cm: Tensor
    D_skip: np.ndarray | None  # fp32 (D,)
    z: Tensor | None
    h0: np.ndarray | None      # fp32 (B, D, N)


def make_scan(B, L, D, N, *, dtype="f32", seed=0, gate=True, h0=True, d_skip=True) -> ScanInputs:
    r = _children(seed)
    x = _store(_normal(r["x"], (B, L, D)), dtype)
    delta = _store(_softplus_delta(r["delta"], (B, L, D)), dtype)
    z = _store(_normal(r["z"], (B, L, D)), dtype) if gate else None
    Bm = _store(_normal(r["Bm"], (B, L, N)), dtype)
    Cm = _store(_normal(r["Cm"], (B, L, N)), dtype)
    A = _neg_exp_uniform(r["A"], (D, N))
    Ds = _normal(r["D"], (D,)) if d_skip else None
    hh = _normal(r["h0"], (B, D, N), std=0.5) if h0 else None
    return ScanInputs(B, L, D, N, dtype, x, delta, A, Bm, Cm, Ds, z, hh)


# ---------------------------------------------------------------------------
# Decode (single-token state update) inputs: a sequence of per-step inputs
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class DecodeInputs:
    S: int          # independent sequences
    D: int
    N: int
    steps: int
    dtype: str
    x: Tensor       # (steps, S, D)
    delta: Tensor   # (steps, S, D)
    z: Tensor | None
    Bm: Tensor      # (steps, S, N)
    Cm: Tensor      # (steps, S, N)
    A: np.ndarray   # (D, N)
    D_skip: np.ndarray | None
    state0: np.ndarray  # fp32 (S, D, N)


def make_decode(S, D, N, steps, *, dtype="bf16", seed=0, gate=True) -> DecodeInputs:
    r = _children(seed)
    x = _store(_normal(r["x"], (steps, S, D)), dtype)
    delta = _store(_softplus_delta(r["delta"], (steps, S, D)), dtype)
    z = _store(_normal(r["z"], (steps, S, D)), dtype) if gate else None
    Bm = _store(_normal(r["Bm"], (steps, S, N)), dtype)
    Cm = _store(_normal(r["Cm"], (steps, S, N)), dtype)
    A = _neg_exp_uniform(r["A"], (D, N))
    Ds = _normal(r["D"], (D,))
    s0 = _normal(r["h0"], (S, D, N), std=0.5)
    return DecodeInputs(S, D, N, steps, dtype, x, delta, z, Bm, Cm, A, Ds, s0)


# ---------------------------------------------------------------------------
# Mamba-2 SSD inputs
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class SSDInputs:
    B: int
    L: int
    H: int
    P: int
    G: int
    N: int
    chunk: int
    dtype: str
    x: Tensor        # (B, L, H, P)
    dt: Tensor       # (B, L, H)
    A: np.ndarray    # fp32 (H,)
    Bm: Tensor       # (B, L, G, N)
    Cm: Tensor       # (B, L, G, N)
    D_skip: np.ndarray | None  # fp32 (H,)
    z: Tensor | None  # (B, L, H, P)
    h0: np.ndarray | None  # fp32 (B, H, P, N)


def make_ssd(B, L, H, P, G, N, *, chunk=256, dtype="bf16", seed=0, gate=False, h0=True,
             d_skip=True) -> SSDInputs:
    r = _children(seed)
    x = _store(_normal(r["x"], (B, L, H, P)), dtype)
    dt = _store(_softplus_delta(r["delta"], (B, L, H)), dtype)
    z = _store(_normal(r["z"], (B, L, H, P)), dtype) if gate else None
    Bm = _store(_normal(r["Bm"], (B, L, G, N)), dtype)
    Cm = _store(_normal(r["Cm"], (B, L, G, N)), dtype)
    A = _neg_exp_uniform(r["A"], (H,))
    Ds = _normal(r["D"], (H,)) if d_skip else None
    hh = _normal(r["h0"], (B, H, P, N), std=0.5) if h0 else None
    return SSDInputs(B, L, H, P, G, N, chunk, dtype, x, dt, A, Bm, Cm, Ds, z, hh)


# ---------------------------------------------------------------------------
# Short causal convolution inputs
# ---------------------------------------------------------------------------

_CONV_STREAMS = ("conv_x", "conv_w", "conv_bias", "conv_state")


def _conv_children(seed: int):
    # children after the scan's, so the scan streams of a seed never move
    kids = np.random.SeedSequence(seed).spawn(len(_STREAMS) + len(_CONV_STREAMS))[len(_STREAMS):]
    return {name: np.random.default_rng(k) for name, k in zip(_CONV_STREAMS, kids)}


def _uniform_sym(rng, shape, bound):
    return rng.uniform(-bound, bound, size=shape).astype(np.float32)


@dataclasses.dataclass
class ConvInputs:
    B: int
    L: int
    D: int
    K: int
    dtype: str                 # storage dtype of x (and y)
    x: Tensor                  # (B, L, D)
    w: np.ndarray              # fp32 (D, K)
    bias: np.ndarray | None    # fp32 (D,)
    state0: np.ndarray | None  # fp32 (B, D, K-1)


def make_conv(B, L, D, K, *, dtype="bf16", seed=0, bias=True, state=True) -> ConvInputs:
    r = _conv_children(seed)
    bound = 1.0 / math.sqrt(K)
    x = _store(_normal(r["conv_x"], (B, L, D)), dtype)
    w = _uniform_sym(r["conv_w"], (D, K), bound)
    bb = _uniform_sym(r["conv_bias"], (D,), bound) if bias else None
    st = _normal(r["conv_state"], (B, D, K - 1)) if state else None
    return ConvInputs(B, L, D, K, dtype, x, w, bb, st)


@dataclasses.dataclass
class ConvDecodeInputs:
    S: int
    D: int
    K: int
    steps: int
    dtype: str
    x: Tensor               # (steps, S, D)
    w: np.ndarray           # fp32 (D, K)
    bias: np.ndarray        # fp32 (D,)
    state0: np.ndarray      # fp32 (S, D, K-1)


def make_conv_decode(S, D, K, steps, *, dtype="bf16", seed=0) -> ConvDecodeInputs:
    r = _conv_children(seed)
    bound = 1.0 / math.sqrt(K)
    x = _store(_normal(r["conv_x"], (steps, S, D)), dtype)
    w = _uniform_sym(r["conv_w"], (D, K), bound)
    bb = _uniform_sym(r["conv_bias"], (D,), bound)
    st = _normal(r["conv_state"], (S, D, K - 1))
    return ConvDecodeInputs(S, D, K, steps, dtype, x, w, bb, st)


# ---------------------------------------------------------------------------
# The workloads, by what they are
# ---------------------------------------------------------------------------

WORKLOADS = {
    # tiny fp32 scan checked against brute-force closed forms
    "tiny_fp32": dict(kind="scan", B=1, L=64, D=16, N=4, dtype="f32", gate=True, seed=1000),
    # Mamba-130M-shaped layer scan, fp32, silu(z) gate on
    "mamba130m_fp32": dict(kind="scan", B=1, L=2048, D=1536, N=16, dtype="f32", gate=True, seed=1001),
    # Mamba-2.8B-shaped prefill scan, bf16 inputs, fp32 state, gate on, random h0
    "mamba2p8b_prefill_bf16": dict(kind="scan", B=8, L=4096, D=5120, N=16, dtype="bf16", gate=True,
                                   seed=1002),
    # decode: 256 sequences, 128 single-token steps, bf16 per-step inputs, fp32 state
    "decode_256x5120_bf16": dict(kind="decode", S=256, D=5120, N=16, steps=128, dtype="bf16",
                                 gate=True, seed=1003),
    # Mamba-2 SSD chunked scan, bf16 inputs, fp32 state, random h0
    "ssd_mamba2_bf16": dict(kind="ssd", B=2, L=8192, H=80, P=64, G=8, N=128, chunk=256,
                            dtype="bf16", gate=False, seed=1004),
    # the width-4 causal convolution ahead of the 2.8B-shaped prefill scan
    "conv_mamba2p8b_bf16": dict(kind="conv", B=8, L=4096, D=5120, K=4, dtype="bf16", seed=1005),
    # its decode step: 256 sequences, 128 single-token steps
    "conv_decode_256x5120_bf16": dict(kind="conv_decode", S=256, D=5120, K=4, steps=128,
                                      dtype="bf16", seed=1006),
    # decode from a state pool: 256 sequences on scattered rows of a 512-row
    # pool, up to 16 tokens each (prefix-cached serving; the first token
    # alone is one decode step)
    "pool_decode_256x5120_bf16": dict(kind="pool_decode", S=256, T=16, D=5120, N=16, pool_rows=512,
                                      dtype="bf16", seed=1007),
}


_GRAD_STREAMS = ("grad_dy", "grad_dh")


@dataclasses.dataclass
class GradInputs:
    dy: Tensor               # (B, L, D) gradient of the scan output, storage dtype
    dh_final: np.ndarray     # fp32 (B, D, N) gradient of the final state


def make_grads(B, L, D, N, *, dtype="bf16", seed=0) -> GradInputs:
    """Loss gradients for the scan backward: dy ~ N(0, 1), dh_final ~ N(0, 0.5)."""
    kids = np.random.SeedSequence(seed).spawn(len(_STREAMS) + len(_CONV_STREAMS) + len(_GRAD_STREAMS))
    r = {n: np.random.default_rng(k) for n, k in zip(_GRAD_STREAMS, kids[-len(_GRAD_STREAMS):])}
    return GradInputs(_store(_normal(r["grad_dy"], (B, L, D)), dtype), _normal(r["grad_dh"], (B, D, N), std=0.5))


@dataclasses.dataclass
class PoolDecodeInputs:
    tokens: ScanInputs      # (S, T, .) per-sequence tokens; tokens.h0 is None
    pool: np.ndarray        # fp32 (pool_rows, D, N) state pool
    slots: np.ndarray       # int32 (S,) distinct pool rows, scattered


def make_pool_decode(S, T, D, N, pool_rows, *, dtype="bf16", seed=0) -> PoolDecodeInputs:
    tok = make_scan(S, T, D, N, dtype=dtype, seed=seed, h0=False)
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(len(_STREAMS) + 1)[-1])
    pool = _normal(rng, (pool_rows, D, N), std=0.5)
    slots = rng.permutation(pool_rows)[:S].astype(np.int32)
    return PoolDecodeInputs(tok, pool, slots)


def make_workload(name: str, **overrides):
    w = dict(WORKLOADS[name])
    w.update(overrides)
    kind = w.pop("kind")
    if kind == "scan":
        return make_scan(w["B"], w["L"], w["D"], w["N"], dtype=w["dtype"], seed=w["seed"],
                         gate=w["gate"], h0=w.get("h0", True))
    if kind == "decode":
        return make_decode(w["S"], w["D"], w["N"], w["steps"], dtype=w["dtype"], seed=w["seed"],
                           gate=w["gate"])
    if kind == "ssd":
        return make_ssd(w["B"], w["L"], w["H"], w["P"], w["G"], w["N"], chunk=w["chunk"],
                        dtype=w["dtype"], seed=w["seed"], gate=w["gate"], h0=w.get("h0", True))
    if kind == "conv":
        return make_conv(w["B"], w["L"], w["D"], w["K"], dtype=w["dtype"], seed=w["seed"])
    if kind == "pool_decode":
        return make_pool_decode(w["S"], w["T"], w["D"], w["N"], w["pool_rows"], dtype=w["dtype"],
                                seed=w["seed"])
    if kind == "conv_decode":
        return make_conv_decode(w["S"], w["D"], w["K"], w["steps"], dtype=w["dtype"], seed=w["seed"])
    raise ValueError(kind)
