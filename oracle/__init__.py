"""CPU oracle for the Mamba selective scan -- TEST INFRASTRUCTURE ONLY.

A thin ctypes wrapper around ``oracle.c``: the plain sequential fp64
recurrence (see that file's header for what is computed and which passage of
the pages each step follows).  Only the test suite, ``__graft_entry__.smoke()``
and the bench's ``cpu_baseline`` leg may import this package.  It does not
import the HIP library, and the HIP library never imports it.

Every function takes numpy arrays of fp32 values (the exact values the GPU
path consumes, bf16 inputs already widened) and returns fp64 results.
Channels are independent, so the wrapper splits a channel list over threads;
each thread runs the unmodified sequential C code on its share.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11"]

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        i64, fp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
        lib.oracle_scan.argtypes = [i64, i64, i64, i64] + [fp] * 8 + [fp, i64, dp, dp, fp, ctypes.c_int]
        lib.oracle_scan.restype = None
        lib.oracle_scan_bwd.argtypes = [i64] * 4 + [fp] * 10 + [fp, ctypes.c_int, fp, i64] + [dp] * 9
        lib.oracle_scan_bwd.restype = None
        lib.oracle_state_update.argtypes = [i64, i64, i64, dp] + [fp] * 7 + [dp, fp, ctypes.c_int]
        lib.oracle_state_update.restype = None
        lib.oracle_ssd.argtypes = [i64] * 6 + [fp] * 8 + [fp, i64, dp, dp, fp, ctypes.c_int]
        lib.oracle_ssd.restype = None
        lib.oracle_conv1d.argtypes = [i64] * 4 + [fp] * 4 + [ctypes.c_int, dp, dp]
        lib.oracle_conv1d.restype = None
        lib.oracle_conv1d_update.argtypes = [i64] * 3 + [dp] + [fp] * 3 + [ctypes.c_int, dp]
        lib.oracle_conv1d_update.restype = None
        _lib = lib
    return _lib


def _f32(a):
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def _run_channels(fn, channels: np.ndarray, L: int, N: int, threads: int):
    """Split `channels` over threads; fn(ch_slice, y_slice, h_slice) fills outputs."""
    n = len(channels)
    y = np.empty((n, L), dtype=np.float64)
    h = np.empty((n, N), dtype=np.float64)
    if n == 0:
        return y, h
    threads = max(1, min(threads, n))
    bounds = np.linspace(0, n, threads + 1).astype(np.int64)

    def work(i):
        a, b = bounds[i], bounds[i + 1]
        if b > a:
            fn(channels[a:b], y[a:b], h[a:b])

    if threads == 1:
        work(0)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, range(threads)))
    return y, h


def scan(x, delta, A, Bm, Cm, D_skip=None, z=None, h0=None, channels=None, threads=None,
         delta_bias=None, delta_softplus=False):
    """Mamba-1 selective scan.

    Shapes: x, delta, z (B, L, D); Bm, Cm (B, L, N); A (D, N); D_skip (D,);
    h0 (B, D, N).  With ``channels=None`` returns y (B, L, D) and h_final
    (B, D, N) in fp64; otherwise ``channels`` lists flat indices b*D + d and
    the result is y (k, L), h_final (k, N) for those channels.  The step
    size is delta (+ delta_bias (D,)) (then softplus when delta_softplus).
    """
    lib = _load()
    x, delta, A, Bm, Cm = map(_f32, (x, delta, A, Bm, Cm))
    delta_bias = _f32(delta_bias)
    D_skip, z, h0 = map(_f32, (D_skip, z, h0))
    B, L, D = x.shape
    N = A.shape[1]
    full = channels is None
    ch = np.arange(B * D, dtype=np.int64) if full else np.ascontiguousarray(channels, dtype=np.int64)
    threads = threads or default_threads()

    def fn(c, ys, hs):
        lib.oracle_scan(B, L, D, N, _ptr(x), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm),
                        _ptr(D_skip), _ptr(z), _ptr(h0), c.ctypes.data, len(c),
                        ys.ctypes.data, hs.ctypes.data, _ptr(delta_bias), int(bool(delta_softplus)))

    y, h = _run_channels(fn, ch, L, N, threads)
    if full:
        return y.reshape(B, D, L).transpose(0, 2, 1).copy(), h.reshape(B, D, N)
    return y, h


def scan_bwd(x, delta, A, Bm, Cm, D_skip=None, z=None, h0=None, dy=None, dh_final=None,
             delta_bias=None, delta_softplus=False, channels=None, threads=None):
    """Gradients of ``scan`` for the output gradient dy (B, L, D) and the
    final-state gradient dh_final (B, D, N) (None = zero).

    Returns a dict of fp64 arrays: dx, ddelta, dz -- (B, L, D), or (k, L) for
    the k requested ``channels`` (flat b*D + d) -- and dh0 -- (B, D, N) or
    (k, N); dA (D, N), dD (D,), dbias (D,), dB and dC (B, L, N) summed over
    the requested channels only (all channels when ``channels`` is None).
    dz is None without a gate, dD None without D_skip.
    """
    lib = _load()
    x, delta, A, Bm, Cm, dy = map(_f32, (x, delta, A, Bm, Cm, dy))
    D_skip, z, h0, dh_final, delta_bias = map(_f32, (D_skip, z, h0, dh_final, delta_bias))
    B, L, D = x.shape
    N = A.shape[1]
    full = channels is None
    ch = np.arange(B * D, dtype=np.int64) if full else np.ascontiguousarray(channels, dtype=np.int64)
    n = len(ch)
    threads = max(1, min(threads or default_threads(), max(n, 1)))
    dx = np.zeros((n, L))
    ddl = np.zeros((n, L))
    dz = np.zeros((n, L))
    dh0 = np.zeros((n, N))
    bounds = np.linspace(0, n, threads + 1).astype(np.int64)
    acc = [dict(dA=np.zeros((D, N)), dD=np.zeros(D), dbias=np.zeros(D), dB=np.zeros((B, L, N)),
                dC=np.zeros((B, L, N))) for _ in range(threads)]

    def work(i):
        a, b = bounds[i], bounds[i + 1]
        if b <= a:
            return
        c = ch[a:b]
        r = acc[i]
        lib.oracle_scan_bwd(B, L, D, N, _ptr(x), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm),
                            _ptr(D_skip), _ptr(z), _ptr(h0), _ptr(dy), _ptr(dh_final),
                            _ptr(delta_bias), int(bool(delta_softplus)), c.ctypes.data, len(c),
                            dx[a:b].ctypes.data, ddl[a:b].ctypes.data, dz[a:b].ctypes.data,
                            dh0[a:b].ctypes.data, r["dA"].ctypes.data, r["dD"].ctypes.data,
                            r["dbias"].ctypes.data, r["dB"].ctypes.data, r["dC"].ctypes.data)

    if threads == 1:
        work(0)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, range(threads)))
    out = {k: sum(r[k] for r in acc) for k in ("dA", "dD", "dbias", "dB", "dC")}
    if full:
        tr = lambda v: v.reshape(B, D, L).transpose(0, 2, 1).copy()
        out.update(dx=tr(dx), ddelta=tr(ddl), dz=tr(dz) if z is not None else None, dh0=dh0.reshape(B, D, N))
    else:
        out.update(dx=dx, ddelta=ddl, dz=dz if z is not None else None, dh0=dh0)
    if D_skip is None:
        out["dD"] = None
    return out


def state_update(state, x, delta, A, Bm, Cm, D_skip=None, z=None, delta_bias=None,
                 delta_softplus=False):
    """One decode step.  state (S, D, N) fp64 is updated in place; returns y (S, D)."""
    lib = _load()
    assert state.dtype == np.float64 and state.flags.c_contiguous
    x, delta, A, Bm, Cm, D_skip, z, delta_bias = map(_f32, (x, delta, A, Bm, Cm, D_skip, z, delta_bias))
    S, D = x.shape
    N = A.shape[1]
    y = np.empty((S, D), dtype=np.float64)
    lib.oracle_state_update(S, D, N, state.ctypes.data, _ptr(x), _ptr(delta), _ptr(A),
                            _ptr(Bm), _ptr(Cm), _ptr(D_skip), _ptr(z), y.ctypes.data,
                            _ptr(delta_bias), int(bool(delta_softplus)))
    return y


def ssd(x, dt, A, Bm, Cm, D_skip=None, z=None, h0=None, channels=None, threads=None,
        dt_bias=None, dt_softplus=False):
    """Mamba-2 SSD recurrence.

    Shapes: x, z (B, L, H, P); dt (B, L, H); A, D_skip (H,); Bm, Cm
    (B, L, G, N); h0 (B, H, P, N).  With ``channels=None`` returns y
    (B, L, H, P) and h_final (B, H, P, N); otherwise ``channels`` lists flat
    indices (b*H + h)*P + p and the result is y (k, L), h_final (k, N).
    """
    lib = _load()
    x, dt, A, Bm, Cm, D_skip, z, h0, dt_bias = map(_f32, (x, dt, A, Bm, Cm, D_skip, z, h0, dt_bias))
    B, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    if H % G != 0:
        raise ValueError("heads must be a multiple of groups")
    full = channels is None
    ch = np.arange(B * H * P, dtype=np.int64) if full else np.ascontiguousarray(channels, dtype=np.int64)
    threads = threads or default_threads()

    def fn(c, ys, hs):
        lib.oracle_ssd(B, L, H, P, G, N, _ptr(x), _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm),
                       _ptr(D_skip), _ptr(z), _ptr(h0), c.ctypes.data, len(c),
                       ys.ctypes.data, hs.ctypes.data, _ptr(dt_bias), int(bool(dt_softplus)))

    y, h = _run_channels(fn, ch, L, N, threads)
    if full:
        return (y.reshape(B, H, P, L).transpose(0, 3, 1, 2).copy(), h.reshape(B, H, P, N))
    return y, h


def conv1d(x, w, bias=None, state0=None, act=False):
    """Short causal convolution (width K) ahead of the scan.

    Shapes: x (B, L, D); w (D, K); bias (D,); state0 (B, D, K-1), the K-1
    previous inputs of each channel, oldest first (zeros when None).  Returns
    y (B, L, D) and the new state (B, D, K-1), both fp64.
    """
    lib = _load()
    x, w, bias, state0 = map(_f32, (x, w, bias, state0))
    B, L, D = x.shape
    K = w.shape[1]
    y = np.empty((B, L, D), dtype=np.float64)
    st = np.empty((B, D, K - 1), dtype=np.float64)
    lib.oracle_conv1d(B, L, D, K, _ptr(x), _ptr(w), _ptr(bias), _ptr(state0), int(bool(act)),
                      y.ctypes.data, st.ctypes.data)
    return y, st


def conv1d_update(state, x, w, bias=None, act=False):
    """One decode step of the causal convolution.  state (S, D, K-1) fp64 is
    updated in place; returns y (S, D)."""
    lib = _load()
    assert state.dtype == np.float64 and state.flags.c_contiguous
    x, w, bias = map(_f32, (x, w, bias))
    S, D = x.shape
    K = w.shape[1]
    y = np.empty((S, D), dtype=np.float64)
    lib.oracle_conv1d_update(S, D, K, state.ctypes.data, _ptr(x), _ptr(w), _ptr(bias),
                             int(bool(act)), y.ctypes.data)
    return y
