"""GPU parity of ssm_state_update (single-token decode) against the oracle.

The decode workload carries an fp32 state over single-token steps whose
inputs are slices of one (steps, S, D) array; the GPU's y at every step and
its final state are compared with the oracle scan over the same tokens.
"""

import numpy as np
import pytest
import torch

import ssm_inputs as gen
from tests.helpers import assert_close, to_dev, to_np

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _tr(v):  # (steps, S, ...) -> (S, steps, ...)
    return np.ascontiguousarray(np.swapaxes(v, 0, 1))


def run_decode(dec, steps=None):
    import mamba_selective_scan_ssm_amd as ssm
    steps = steps or dec.steps
    state = to_dev(dec.state0).clone()
    xs, ds, zs, bs, cs = (to_dev(getattr(dec, k)) for k in ("x", "delta", "z", "Bm", "Cm"))
    A, Ds = to_dev(dec.A), to_dev(dec.D_skip)
    ys = []
    for t in range(steps):
        ys.append(ssm.state_update(state, xs[t], ds[t], A, bs[t], cs[t], Ds, zs[t]))
    torch.cuda.synchronize()
    return np.stack([to_np(y) for y in ys], 1), to_np(state)   # y (S, steps, D)


@pytest.mark.parametrize("S,D,N,steps,dtype", [
    (4, 200, 16, 20, "bf16"),
    (3, 130, 16, 12, "f32"),
    (2, 64, 4, 9, "f32"),
    (2, 96, 8, 9, "bf16"),
    (2, 70, 32, 9, "f32"),
    (2, 64, 64, 9, "bf16"),
    (2, 50, 5, 9, "f32"),       # N not a multiple of 4: per-lane path
    (2, 33, 1, 9, "bf16"),
])
def test_decode_small_full(oracle_mod, S, D, N, steps, dtype):
    dec = gen.make_decode(S, D, N, steps, dtype=dtype, seed=300 + D + N)
    _say("decode", S, D, N, steps, dtype)
    y, st = run_decode(dec)
    ry, rh = oracle_mod.scan(_tr(dec.x.f32), _tr(dec.delta.f32), dec.A, _tr(dec.Bm.f32),
                             _tr(dec.Cm.f32), dec.D_skip, _tr(dec.z.f32), dec.state0)
    assert_close(y, ry, dtype, "y")
    assert_close(st, rh, dtype, "state")


def test_decode_256x5120_whole(oracle_mod):
    """The full decode workload: 256 sequences, D=5120, N=16, 128 steps; every
    channel's y at every step and the whole final state against the oracle
    scan over the same 128 tokens."""
    dec = gen.make_workload("decode_256x5120_bf16")
    _say("decode_256x5120_bf16 full size, whole tensors")
    y, st = run_decode(dec)
    ry, rh = oracle_mod.scan(_tr(dec.x.f32), _tr(dec.delta.f32), dec.A, _tr(dec.Bm.f32),
                             _tr(dec.Cm.f32), dec.D_skip, _tr(dec.z.f32), dec.state0)
    assert_close(y, ry, "bf16", "y")
    assert_close(st, rh, "bf16", "state")


def test_decode_matches_scan_of_one_token(oracle_mod):
    """A decode step and a one-token prefill agree (two different kernels)."""
    import mamba_selective_scan_ssm_amd as ssm
    dec = gen.make_decode(6, 300, 16, 1, dtype="f32", seed=31)
    _say("decode vs scan L=1")
    y_step, st = run_decode(dec)
    y_scan, hf = ssm.scan_fwd(to_dev(_tr(dec.x.f32)), to_dev(_tr(dec.delta.f32)), to_dev(dec.A),
                              to_dev(_tr(dec.Bm.f32)), to_dev(_tr(dec.Cm.f32)), to_dev(dec.D_skip),
                              to_dev(_tr(dec.z.f32)), to_dev(dec.state0))
    assert_close(y_step, to_np(y_scan), "f32", "y")
    assert_close(st, to_np(hf), "f32", "state")


def test_decode_unaligned_state_uses_per_lane_path(oracle_mod):
    """A state that is not 16-byte aligned takes the per-lane path and stays correct."""
    import mamba_selective_scan_ssm_amd as ssm
    dec = gen.make_decode(2, 80, 16, 3, dtype="f32", seed=32)
    _say("decode unaligned")
    buf = torch.zeros(1 + 2 * 80 * 16, device="cuda")
    state = buf[1:].view(2, 80, 16)
    state.copy_(to_dev(dec.state0))
    xs, ds, zs, bs, cs = (to_dev(getattr(dec, k)) for k in ("x", "delta", "z", "Bm", "Cm"))
    ys = [ssm.state_update(state, xs[t], ds[t], to_dev(dec.A), bs[t], cs[t], to_dev(dec.D_skip), zs[t])
          for t in range(3)]
    torch.cuda.synchronize()
    ry, rh = oracle_mod.scan(_tr(dec.x.f32), _tr(dec.delta.f32), dec.A, _tr(dec.Bm.f32),
                             _tr(dec.Cm.f32), dec.D_skip, _tr(dec.z.f32), dec.state0)
    assert_close(np.stack([to_np(y) for y in ys], 1), ry, "f32", "y")
    assert_close(to_np(state), rh, "f32", "state")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_unaligned_bc_element_loads(oracle_mod, dtype):
    """B and C rows offset by one element (not 4-element aligned) take the
    element-load path of the vectorised step, single- and multi-token, and
    agree bit for bit with the aligned rows."""
    import mamba_selective_scan_ssm_amd as ssm
    S, D, N, T = 3, 96, 16, 5
    dec = gen.make_decode(S, D, N, T, dtype=dtype, seed=33)
    _say("decode unaligned B/C", dtype)

    def shifted(t):  # same values, one element past an aligned start
        buf = torch.zeros(t.numel() + 1, dtype=t.dtype, device=t.device)
        v = buf[1:].view(t.shape)
        v.copy_(t)
        return v

    xs, ds, zs, bs, cs = (to_dev(getattr(dec, k)) for k in ("x", "delta", "z", "Bm", "Cm"))
    A, Ds = to_dev(dec.A), to_dev(dec.D_skip)
    outs = {}
    for name, mk in (("aligned", lambda t: t), ("shifted", shifted)):
        st1 = to_dev(dec.state0).clone()
        y1 = [ssm.state_update(st1, xs[t], ds[t], A, mk(bs[t].contiguous()), mk(cs[t].contiguous()), Ds, zs[t])
              for t in range(T)]
        stT = to_dev(dec.state0).clone()
        tr = lambda v: v.transpose(0, 1).contiguous()  # (S, T, ...)
        yT = ssm.decode_steps(stT, tr(xs), tr(ds), A, mk(tr(bs)), mk(tr(cs)), Ds, tr(zs))
        torch.cuda.synchronize()
        outs[name] = (torch.stack(y1, 1), st1, yT, stT)
    for a, b in zip(outs["aligned"], outs["shifted"]):
        assert torch.equal(a, b)
    ry, rh = oracle_mod.scan(_tr(dec.x.f32), _tr(dec.delta.f32), dec.A, _tr(dec.Bm.f32),
                             _tr(dec.Cm.f32), dec.D_skip, _tr(dec.z.f32), dec.state0)
    y1, st1, yT, stT = outs["shifted"]
    assert_close(to_np(y1), ry, dtype, "y single-token")
    assert_close(to_np(st1), rh, dtype, "state single-token")
    assert_close(to_np(yT), ry, dtype, "y multi-token")
    assert_close(to_np(stT), rh, dtype, "state multi-token")


def test_decode_batch_invariance_bitwise():
    import mamba_selective_scan_ssm_amd as ssm
    dec = gen.make_decode(5, 640, 16, 4, dtype="bf16", seed=33)
    _say("decode batch invariance")
    ys, st = run_decode(dec)
    for s in (0, 3):
        one = gen.DecodeInputs(1, dec.D, dec.N, dec.steps, dec.dtype,
                               *(gen.Tensor(getattr(dec, k).f32[:, s:s + 1],
                                            getattr(dec, k).bf16[:, s:s + 1].copy())
                                 for k in ("x", "delta", "z", "Bm", "Cm")),
                               dec.A, dec.D_skip, dec.state0[s:s + 1].copy())
        y1, s1 = run_decode(one)
        np.testing.assert_array_equal(y1[0], ys[s])
        np.testing.assert_array_equal(s1[0], st[s])
