"""HIP-graph replays of the decode entry points, which bench.py times as
graph replays: a graph of several in-place steps, replayed three times with
the same steps run eagerly between the replays, matches the eager run bit
for bit after every replay (states and outputs)."""

import numpy as np
import pytest
import torch

import ssm_inputs as gen
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu

STEPS = 4


def _say(*a):
    print("[case]", *a, flush=True)


def _replays_match(step, state0, y_shape, y_dtype):
    """step(state, t, y) runs token t in place on `state`, writing y."""
    scratch = state0.clone()
    ys_w = [torch.empty(y_shape, dtype=y_dtype, device="cuda") for _ in range(STEPS)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for t in range(STEPS):
            step(scratch, t, ys_w[t])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    sg, se = state0.clone(), state0.clone()
    ys_g = [torch.empty(y_shape, dtype=y_dtype, device="cuda") for _ in range(STEPS)]
    ys_e = [torch.empty(y_shape, dtype=y_dtype, device="cuda") for _ in range(STEPS)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(STEPS):
            step(sg, t, ys_g[t])
    sg.copy_(state0)
    torch.cuda.synchronize()
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        for t in range(STEPS):
            step(se, t, ys_e[t])
        torch.cuda.synchronize()
        assert torch.equal(sg, se), f"state after replay {rep}"
        for t in range(STEPS):
            assert torch.equal(ys_g[t], ys_e[t]), f"y of step {t} after replay {rep}"
    # the steps moved the state: the check compares work actually done
    assert not torch.equal(se, state0)
    del g


def test_graph_state_update():
    import mamba_selective_scan_ssm_amd as ssm
    d = gen.make_decode(16, 320, 16, STEPS, dtype="bf16", seed=1500)
    xs, ds, zs, bs, cs = (to_dev(getattr(d, k)) for k in ("x", "delta", "z", "Bm", "Cm"))
    A, Ds = to_dev(d.A), to_dev(d.D_skip)
    _say("graph state_update")
    _replays_match(lambda st, t, y: ssm.state_update(st, xs[t], ds[t], A, bs[t], cs[t], Ds, zs[t], y=y),
                   to_dev(d.state0), (d.S, d.D), torch.bfloat16)


def test_graph_pool_decode():
    import mamba_selective_scan_ssm_amd as ssm
    w = gen.make_pool_decode(12, 2, 320, 16, 40, dtype="bf16", seed=1501)
    tk = w.tokens
    tok = {k: to_dev(getattr(tk, k)) for k in ("x", "delta", "z", "Bm", "Cm")}
    A, Ds = to_dev(tk.A), to_dev(tk.D_skip)
    slots = torch.from_numpy(w.slots).cuda()
    _say("graph decode_steps")
    _replays_match(lambda st, t, y: ssm.decode_steps(st, tok["x"], tok["delta"], A, tok["Bm"], tok["Cm"], Ds,
                                                     tok["z"], slots=slots, y=y),
                   to_dev(w.pool), (tk.B, tk.L, tk.D), torch.bfloat16)


def test_graph_conv_update():
    import mamba_selective_scan_ssm_amd as ssm
    d = gen.make_conv_decode(16, 320, 4, STEPS, dtype="bf16", seed=1502)
    xs, wd, bd = to_dev(d.x), to_dev(d.w), to_dev(d.bias)
    _say("graph conv1d_update")
    _replays_match(lambda st, t, y: ssm.conv1d_update(st, xs[t], wd, bd, y=y),
                   to_dev(d.state0), (d.S, d.D), torch.bfloat16)
