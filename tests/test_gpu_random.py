"""Seeded randomized parity: shapes, dtypes and options drawn from a fixed
generator (so every run checks the same cases) for every entry point,
against the oracle.  Complements the hand-picked cases of the other files
with odd sizes: L and D not multiples of the tiles, one token, one channel.
"""

import numpy as np
import pytest
import torch

import ssm_inputs as gen
from tests.helpers import assert_close, to_dev, to_np

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(2024)
SCAN_CASES = [dict(B=int(RNG.integers(1, 4)), L=int(RNG.choice([1, 2, 7, 33, 100, 257, 300])),
                   D=int(RNG.choice([1, 2, 31, 64, 66, 130, 200])), N=int(RNG.choice([1, 4, 5, 8, 16, 32, 64])),
                   dtype=str(RNG.choice(["f32", "bf16"])), variant=int(RNG.choice([0, 1, 2, 3])),
                   gate=bool(RNG.integers(0, 2)), h0=bool(RNG.integers(0, 2)), seed=3000 + i)
              for i in range(24)]


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("case", SCAN_CASES, ids=lambda c: "B{B}L{L}D{D}N{N}{dtype}v{variant}".format(**c))
def test_random_scan(oracle_mod, case):
    import mamba_selective_scan_ssm_amd as ssm
    c = case
    inp = gen.make_scan(c["B"], c["L"], c["D"], c["N"], dtype=c["dtype"], seed=c["seed"], gate=c["gate"],
                        h0=c["h0"])
    _say("random scan", c)
    args = (to_dev(inp.x), to_dev(inp.delta), to_dev(inp.A), to_dev(inp.Bm), to_dev(inp.Cm),
            to_dev(inp.D_skip), to_dev(inp.z), to_dev(inp.h0))
    try:
        y, hf = ssm.scan_fwd(*args, variant=c["variant"], chunk_len=16 if c["variant"] == 2 else 0)
    except ssm.SSMError as e:
        # the lane-split schedule covers N in {4, 8, 16, 32, 64}, even D and aligned rows only
        assert c["variant"] == 3 and e.code == 2, e
        return
    torch.cuda.synchronize()
    ry, rh = oracle_mod.scan(inp.x.f32, inp.delta.f32, inp.A, inp.Bm.f32, inp.Cm.f32, inp.D_skip,
                             None if inp.z is None else inp.z.f32, inp.h0)
    assert_close(to_np(y), ry, c["dtype"], "y")
    assert_close(to_np(hf), rh, c["dtype"], "h_final")


BWD_CASES = [dict(B=int(RNG.integers(1, 3)), L=int(RNG.choice([1, 7, 8, 9, 40, 65])),
                  D=int(RNG.choice([1, 3, 64, 65, 130])), N=int(RNG.choice([4, 8, 16, 32, 64])),
                  dtype=str(RNG.choice(["f32", "bf16"])), gate=bool(RNG.integers(0, 2)),
                  softplus=bool(RNG.integers(0, 2)), seed=3100 + i) for i in range(18)]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "B{B}L{L}D{D}N{N}{dtype}".format(**c))
def test_random_bwd(oracle_mod, case):
    import mamba_selective_scan_ssm_amd as ssm
    c = case
    inp = gen.make_scan(c["B"], c["L"], c["D"], c["N"], dtype=c["dtype"], seed=c["seed"], gate=c["gate"])
    gr = gen.make_grads(c["B"], c["L"], c["D"], c["N"], dtype=c["dtype"], seed=c["seed"] + 1)
    bias = None
    if c["softplus"]:
        inp.delta = gen._store((inp.delta.f32 * 6.0 - 3.0).astype(np.float32), c["dtype"])
        bias = np.random.default_rng(c["seed"]).normal(0.0, 1.0, c["D"]).astype(np.float32)
    _say("random bwd", c)
    out = ssm.scan_bwd(to_dev(inp.x), to_dev(inp.delta), to_dev(inp.A), to_dev(inp.Bm), to_dev(inp.Cm),
                       to_dev(inp.D_skip), to_dev(inp.z), to_dev(inp.h0), to_dev(gr.dy), to_dev(gr.dh_final),
                       delta_bias=None if bias is None else to_dev(bias), delta_softplus=c["softplus"],
                       want_dbias=True)
    torch.cuda.synchronize()
    r = oracle_mod.scan_bwd(inp.x.f32, inp.delta.f32, inp.A, inp.Bm.f32, inp.Cm.f32, inp.D_skip,
                            None if inp.z is None else inp.z.f32, inp.h0, gr.dy.f32, gr.dh_final,
                            delta_bias=bias, delta_softplus=c["softplus"])
    for k in ("dx", "ddelta", "dz", "dA", "dB", "dC", "dD", "dh0", "dbias"):
        if r.get(k) is not None:
            assert_close(to_np(out[k]), r[k], c["dtype"], k)


POOL_CASES = [dict(S=int(RNG.integers(1, 6)), T=int(RNG.choice([1, 2, 5, 16, 17, 30])),
                   D=int(RNG.choice([2, 31, 64, 100])), N=int(RNG.choice([4, 5, 16, 64])),
                   dtype=str(RNG.choice(["f32", "bf16"])), seed=3200 + i) for i in range(16)]


@pytest.mark.parametrize("case", POOL_CASES, ids=lambda c: "S{S}T{T}D{D}N{N}{dtype}".format(**c))
def test_random_pool_decode(oracle_mod, case):
    import mamba_selective_scan_ssm_amd as ssm
    c = case
    inp = gen.make_scan(c["S"], c["T"], c["D"], c["N"], dtype=c["dtype"], seed=c["seed"], h0=False)
    rng = np.random.default_rng(c["seed"])
    P = c["S"] + 3
    pool = rng.normal(0.0, 0.5, (P, c["D"], c["N"])).astype(np.float32)
    slots = rng.permutation(P)[:c["S"]].astype(np.int32)
    _say("random pool decode", c)
    pool_d = to_dev(pool)
    y = ssm.decode_steps(pool_d, to_dev(inp.x), to_dev(inp.delta), to_dev(inp.A), to_dev(inp.Bm),
                         to_dev(inp.Cm), to_dev(inp.D_skip), to_dev(inp.z),
                         slots=torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    ry, rh = oracle_mod.scan(inp.x.f32, inp.delta.f32, inp.A, inp.Bm.f32, inp.Cm.f32, inp.D_skip, inp.z.f32,
                             pool[slots])
    assert_close(to_np(y), ry, c["dtype"], "y")
    pn = to_np(pool_d)
    assert_close(pn[slots], rh, c["dtype"], "pool rows")
    rest = np.setdiff1d(np.arange(P), slots)
    assert np.array_equal(pn[rest], pool[rest].astype(np.float64))


CONV_CASES = [dict(B=int(RNG.integers(1, 4)), L=int(RNG.choice([1, 3, 64, 65, 200])),
                   D=int(RNG.choice([1, 7, 256, 300])), K=int(RNG.integers(2, 9)),
                   dtype=str(RNG.choice(["f32", "bf16"])), seed=3300 + i) for i in range(10)]


@pytest.mark.parametrize("case", CONV_CASES, ids=lambda c: "B{B}L{L}D{D}K{K}{dtype}".format(**c))
def test_random_conv(oracle_mod, case):
    import mamba_selective_scan_ssm_amd as ssm
    c = case
    cv = gen.make_conv(c["B"], c["L"], c["D"], c["K"], dtype=c["dtype"], seed=c["seed"])
    _say("random conv", c)
    y, st = ssm.conv1d_fwd(to_dev(cv.x), to_dev(cv.w), to_dev(cv.bias), to_dev(cv.state0))
    torch.cuda.synchronize()
    ry, rs = oracle_mod.conv1d(cv.x.f32, cv.w, cv.bias, cv.state0, act=True)
    assert_close(to_np(y), ry, c["dtype"], "y")
    assert np.array_equal(to_np(st), rs)


def _ssd_case(i):
    G = int(RNG.choice([1, 2]))
    return dict(B=int(RNG.integers(1, 3)), L=int(RNG.choice([1, 63, 64, 65, 200, 300])), G=G,
                H=G * int(RNG.integers(1, 4)), N=int(RNG.choice([32, 64, 96, 128, 160, 256])),
                chunk=int(RNG.choice([64, 128, 256])), gate=bool(RNG.integers(0, 2)), seed=3400 + i)


SSD_CASES = [_ssd_case(i) for i in range(18)]


@pytest.mark.parametrize("case", SSD_CASES, ids=lambda c: "B{B}L{L}H{H}G{G}N{N}c{chunk}".format(**c))
def test_random_ssd(oracle_mod, case):
    import mamba_selective_scan_ssm_amd as ssm
    c = case
    w = gen.make_ssd(c["B"], c["L"], c["H"], 64, c["G"], c["N"], chunk=c["chunk"], dtype="bf16",
                     seed=c["seed"], gate=c["gate"])
    _say("random ssd", c)
    y, hf = ssm.ssd_fwd(to_dev(w.x), to_dev(w.dt), to_dev(w.A), to_dev(w.Bm), to_dev(w.Cm), to_dev(w.D_skip),
                        to_dev(w.z), to_dev(w.h0), chunk=c["chunk"])
    torch.cuda.synchronize()
    ry, rh = oracle_mod.ssd(w.x.f32, w.dt.f32, w.A, w.Bm.f32, w.Cm.f32, w.D_skip,
                            None if w.z is None else w.z.f32, w.h0)
    assert_close(to_np(y), ry, "bf16", "y")
    assert_close(to_np(hf), rh, "bf16", "h_final")


DEC_CASES = [dict(S=int(RNG.integers(1, 20)), D=int(RNG.choice([2, 31, 64, 100, 130, 320])),
                  N=int(RNG.choice([1, 4, 5, 8, 16, 32, 64])), dtype=str(RNG.choice(["f32", "bf16"])),
                  gate=bool(RNG.integers(0, 2)), softplus=bool(RNG.integers(0, 2)), seed=3500 + i)
             for i in range(14)]


@pytest.mark.parametrize("case", DEC_CASES, ids=lambda c: "S{S}D{D}N{N}{dtype}".format(**c))
def test_random_state_update(oracle_mod, case):
    """Three single-token steps in place against the oracle's own decode step
    (step-size bias and softplus drawn too)."""
    import mamba_selective_scan_ssm_amd as ssm
    c = case
    dec = gen.make_decode(c["S"], c["D"], c["N"], 3, dtype=c["dtype"], seed=c["seed"], gate=c["gate"])
    delta, bias = dec.delta, None
    if c["softplus"]:
        delta = gen._store((dec.delta.f32 * 6.0 - 3.0).astype(np.float32), c["dtype"])
        bias = np.random.default_rng(c["seed"]).normal(0.0, 1.0, c["D"]).astype(np.float32)
    _say("random state_update", c)
    st = to_dev(dec.state0)
    xs, ds, bs, cs, zs = (to_dev(v) for v in (dec.x, delta, dec.Bm, dec.Cm, dec.z))
    A, Ds = to_dev(dec.A), to_dev(dec.D_skip)
    bias_d = None if bias is None else to_dev(bias)
    rs = dec.state0.astype(np.float64).copy()
    for t in range(3):
        y = ssm.state_update(st, xs[t], ds[t], A, bs[t], cs[t], Ds, None if zs is None else zs[t],
                             delta_bias=bias_d, delta_softplus=c["softplus"])
        torch.cuda.synchronize()
        ry = oracle_mod.state_update(rs, dec.x.f32[t], delta.f32[t], dec.A, dec.Bm.f32[t], dec.Cm.f32[t],
                                     dec.D_skip, None if dec.z is None else dec.z.f32[t],
                                     delta_bias=bias, delta_softplus=c["softplus"])
        assert_close(to_np(y), ry, c["dtype"], f"y step {t}")
    assert_close(to_np(st), rs, c["dtype"], "state")


CONVU_CASES = [dict(S=int(RNG.integers(1, 20)), D=int(RNG.choice([1, 7, 256, 300])), K=int(RNG.integers(2, 9)),
                    dtype=str(RNG.choice(["f32", "bf16"])), seed=3600 + i) for i in range(8)]


@pytest.mark.parametrize("case", CONVU_CASES, ids=lambda c: "S{S}D{D}K{K}{dtype}".format(**c))
def test_random_conv_update(oracle_mod, case):
    """Three decode steps of the convolution in place against the oracle's."""
    import mamba_selective_scan_ssm_amd as ssm
    c = case
    d = gen.make_conv_decode(c["S"], c["D"], c["K"], 3, dtype=c["dtype"], seed=c["seed"])
    _say("random conv1d_update", c)
    st, xs = to_dev(d.state0), to_dev(d.x)
    wd, bd = to_dev(d.w), to_dev(d.bias)
    rs = d.state0.astype(np.float64).copy()
    for t in range(3):
        y = ssm.conv1d_update(st, xs[t], wd, bd)
        torch.cuda.synchronize()
        ry = oracle_mod.conv1d_update(rs, d.x.f32[t], d.w, d.bias, act=True)
        assert_close(to_np(y), ry, c["dtype"], f"y step {t}")
    assert np.array_equal(to_np(st), rs)


def _ssd_token_case(i):
    G = int(RNG.choice([1, 2]))
    return dict(B=int(RNG.integers(1, 3)), L=int(RNG.choice([1, 15, 16, 17, 100, 257])), G=G,
                H=G * int(RNG.integers(1, 5)), P=int(RNG.choice([8, 16, 24, 32, 48, 64, 96, 128])),
                N=int(RNG.choice([1, 5, 16, 33, 64, 128, 200])), chunk=int(RNG.choice([37, 64, 100])),
                dtype=str(RNG.choice(["f32", "bf16"])), gate=bool(RNG.integers(0, 2)),
                softplus=bool(RNG.integers(0, 2)), seed=3700 + i)


SSD_TOKEN_CASES = [_ssd_token_case(i) for i in range(16)]


@pytest.mark.parametrize("case", SSD_TOKEN_CASES,
                         ids=lambda c: "B{B}L{L}H{H}P{P}G{G}N{N}c{chunk}{dtype}".format(**c))
def test_random_ssd_token_path(oracle_mod, case):
    """SSD shapes and dtypes the matrix-core kernels are not built for (any P,
    any N, fp32, odd chunk lengths), with and without the dt bias + softplus:
    the token-by-token kernels, staged or plain by the group alignment."""
    import mamba_selective_scan_ssm_amd as ssm
    c = case
    w = gen.make_ssd(c["B"], c["L"], c["H"], c["P"], c["G"], c["N"], chunk=c["chunk"], dtype=c["dtype"],
                     seed=c["seed"], gate=c["gate"])
    bias = np.random.default_rng(c["seed"] + 1).normal(0.0, 0.5, c["H"]).astype(np.float32) \
        if c["softplus"] else None
    _say("random ssd token path", c)
    y, hf = ssm.ssd_fwd(to_dev(w.x), to_dev(w.dt), to_dev(w.A), to_dev(w.Bm), to_dev(w.Cm), to_dev(w.D_skip),
                        to_dev(w.z), to_dev(w.h0), chunk=c["chunk"],
                        dt_bias=None if bias is None else to_dev(bias), dt_softplus=c["softplus"])
    torch.cuda.synchronize()
    ry, rh = oracle_mod.ssd(w.x.f32, w.dt.f32, w.A, w.Bm.f32, w.Cm.f32, w.D_skip,
                            None if w.z is None else w.z.f32, w.h0, dt_bias=bias, dt_softplus=c["softplus"])
    assert_close(to_np(y), ry, c["dtype"], "y")
    assert_close(to_np(hf), rh, c["dtype"], "h_final")
