"""GPU parity of ssm_decode_steps: decode tokens for sequences whose states are
rows of a pool, addressed through a slot index (prefix caching's state
gather/scatter and batch-invariant decode, Megatron-LM pull request 6444).

Every check gathers the pool rows the slots name, runs the oracle scan over
the T tokens from them, and compares y and the rows written back; pool rows
no slot names, and y rows of skipped sequences, must come back bit for bit.
"""

import dataclasses

import numpy as np
import pytest
import torch

import ssm_inputs as gen
from tests.helpers import assert_close, to_dev, to_np

pytestmark = pytest.mark.gpu

SENTINEL = 7.0


def _say(*a):
    print("[case]", *a, flush=True)


def _pool(rows, D, N, seed):
    return (np.random.default_rng(seed).normal(0.0, 0.5, (rows, D, N))).astype(np.float32)


def _run(inp, pool_np, slots, **kw):
    import mamba_selective_scan_ssm_amd as ssm
    pool = to_dev(pool_np)
    sl = None if slots is None else torch.tensor(slots, dtype=torch.int32, device="cuda")
    y = to_dev(inp.x).clone().fill_(SENTINEL)
    ssm.decode_steps(pool, to_dev(inp.x), to_dev(inp.delta), to_dev(inp.A), to_dev(inp.Bm),
                     to_dev(inp.Cm), to_dev(inp.D_skip), to_dev(inp.z), slots=sl, y=y, **kw)
    torch.cuda.synchronize()
    return y, pool


def _check_against_oracle(oracle_mod, inp, pool_np, slots, y, pool, dtype, **kw):
    slots = np.asarray(slots)
    live = np.nonzero((slots >= 0) & (slots < pool_np.shape[0]))[0]
    rows = slots[live]
    sub = lambda t: None if t is None else t.f32[live]
    ry, rh = oracle_mod.scan(sub(inp.x), sub(inp.delta), inp.A, sub(inp.Bm), sub(inp.Cm), inp.D_skip,
                             sub(inp.z), pool_np[rows], **kw)
    yn, pn = to_np(y), to_np(pool)
    assert_close(yn[live], ry, dtype, "y")
    assert_close(pn[rows], rh, dtype, "pool rows")
    dead = np.setdiff1d(np.arange(len(slots)), live)
    assert (yn[dead] == SENTINEL).all(), "skipped sequences had y written"
    untouched = np.setdiff1d(np.arange(pool_np.shape[0]), rows)
    assert np.array_equal(pn[untouched], pool_np[untouched].astype(np.float64)), "unnamed pool rows changed"


@pytest.mark.parametrize("T", [1, 5, 16, 40])   # 40: the prefill kernels' path
@pytest.mark.parametrize("N,dtype", [(16, "bf16"), (16, "f32"), (5, "f32"), (64, "bf16")])
def test_slots_permuted_subset(oracle_mod, T, N, dtype):
    S, D, P = 6, 130, 10
    inp = gen.make_scan(S, T, D, N, dtype=dtype, seed=700 + T + N)
    pool_np = _pool(P, D, N, 701 + N)
    slots = [7, 2, -1, 9, 0, 12]          # 12 >= pool_rows: skipped as well
    _say("decode_steps slots", T, N, dtype)
    y, pool = _run(inp, pool_np, slots)
    _check_against_oracle(oracle_mod, inp, pool_np, slots, y, pool, dtype)


@pytest.mark.parametrize("T", [1, 8])
def test_slots_with_delta_transform(oracle_mod, T):
    S, D, N, P = 4, 256, 16, 9
    inp = gen.make_scan(S, T, D, N, dtype="bf16", seed=710 + T)
    raw = gen._store((inp.delta.f32 * 6.0 - 3.0).astype(np.float32), "bf16")
    inp.delta = raw
    bias = np.random.default_rng(711).normal(0.0, 1.0, D).astype(np.float32)
    pool_np = _pool(P, D, N, 712)
    slots = [3, 8, 1, 5]
    _say("decode_steps slots + softplus", T)
    y, pool = _run(inp, pool_np, slots, delta_bias=to_dev(bias), delta_softplus=True)
    _check_against_oracle(oracle_mod, inp, pool_np, slots, y, pool, "bf16", delta_bias=bias,
                          delta_softplus=True)


@pytest.mark.parametrize("T,N", [(1, 16), (4, 16), (4, 5), (5, 16), (12, 16), (16, 5), (40, 16), (40, 5)])
def test_identity_slots_match_single_call_kernels(T, N):
    """slot_idx = NULL: up to 4 tokens the results are bitwise those of T
    successive ssm_state_update calls; longer calls bitwise ssm_scan_fwd
    (variant 1) with h0 = h_final = the state."""
    import mamba_selective_scan_ssm_amd as ssm
    S, D = 5, 320
    inp = gen.make_scan(S, T, D, N, dtype="bf16", seed=720 + T + N)
    pool_np = _pool(S, D, N, 721)
    _say("decode_steps identity vs single-call kernels", T, N)
    y, pool = _run(inp, pool_np, None)
    st = to_dev(pool_np)
    x, dl, Bm, Cm, z = (to_dev(getattr(inp, k)) for k in ("x", "delta", "Bm", "Cm", "z"))
    A, Ds = to_dev(inp.A), to_dev(inp.D_skip)
    if T <= 4:
        ry = torch.stack([ssm.state_update(st, x[:, t].contiguous(), dl[:, t].contiguous(), A,
                                           Bm[:, t].contiguous(), Cm[:, t].contiguous(), Ds,
                                           z[:, t].contiguous()) for t in range(T)], 1)
        rh = st
    else:
        ry, rh = ssm.scan_fwd(x, dl, A, Bm, Cm, Ds, z, st, variant=1)
    torch.cuda.synchronize()
    assert torch.equal(y, ry)
    assert torch.equal(pool, rh)


@pytest.mark.parametrize("T", [1, 6, 24])
def test_batch_invariance(T):
    """A sequence's y and state do not depend on which other sequences share
    the call: run it alone, then among 7 others on other slots."""
    S, D, N, P = 8, 512, 16, 16
    inp = gen.make_scan(S, T, D, N, dtype="bf16", seed=730 + T)
    pool_np = _pool(P, D, N, 731)
    slots = [11, 4, 0, 15, 9, 2, 7, 13]
    _say("decode_steps batch invariance", T)
    y_all, pool_all = _run(inp, pool_np, slots)
    for s in (0, 3, 7):
        cut = lambda t: gen.Tensor(t.f32[s:s + 1], None if t.bf16 is None else t.bf16[s:s + 1])
        one = dataclasses.replace(inp, B=1, **{k: cut(getattr(inp, k)) for k in ("x", "delta", "Bm", "Cm", "z")})
        y1, pool1 = _run(one, pool_np, [slots[s]])
        assert torch.equal(y1[0], y_all[s])
        assert torch.equal(pool1[slots[s]], pool_all[slots[s]])


@pytest.mark.parametrize("T", [1, 4, 16])
def test_pool_decode_256x5120_whole(oracle_mod, T):
    """The timed pool-decode workload (256 sequences on scattered rows of a
    512-row pool, D=5120, N=16, bf16) at T = 1, 4 and 16 tokens per call: all
    of y and every written pool row against the oracle, untouched rows
    bitwise unchanged."""
    w = gen.make_workload("pool_decode_256x5120_bf16")
    cut = lambda t: gen.Tensor(np.ascontiguousarray(t.f32[:, :T]),
                               None if t.bf16 is None else np.ascontiguousarray(t.bf16[:, :T]))
    inp = dataclasses.replace(w.tokens, L=T, **{k: cut(getattr(w.tokens, k))
                                                for k in ("x", "delta", "Bm", "Cm", "z")})
    P = w.pool.shape[0]
    slots, pool_np = w.slots, w.pool
    _say("pool_decode_256x5120_bf16", T)
    y, pool = _run(inp, pool_np, slots.tolist())
    ry, rh = oracle_mod.scan(inp.x.f32, inp.delta.f32, inp.A, inp.Bm.f32, inp.Cm.f32, inp.D_skip,
                             inp.z.f32, pool_np[slots])
    assert_close(to_np(y), ry, "bf16", "y")
    pn = pool.cpu().numpy()
    assert_close(pn[slots], rh, "bf16", "pool rows")
    untouched = np.setdiff1d(np.arange(P), slots)
    assert np.array_equal(pn[untouched], pool_np[untouched])
