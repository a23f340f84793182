"""GPU parity of the fused step-size transform (delta + bias, then softplus)
in the scan, the decode step and SSD, against the oracle's transform."""

import numpy as np
import pytest
import torch

import ssm_inputs as gen
from tests.helpers import assert_close, to_dev, to_np

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _raw_and_bias(inp_delta, n, seed):
    """Pre-activation step sizes spanning negative and large values, and a bias."""
    rng = np.random.default_rng(seed)
    raw = (inp_delta * 6.0 - 3.0).astype(np.float32)
    bias = rng.normal(0.0, 1.0, n).astype(np.float32)
    return raw, bias


@pytest.mark.parametrize("variant,chunk", [(0, 0), (1, 0), (2, 16), (2, 64), (3, 0)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("softplus", [False, True])
def test_scan_delta_transform(oracle_mod, variant, chunk, dtype, softplus):
    import mamba_selective_scan_ssm_amd as ssm
    inp = gen.make_scan(2, 300, 192, 16, dtype=dtype, seed=600 + variant)
    raw, bias = _raw_and_bias(inp.delta.f32, inp.D, 601)
    if not softplus:
        raw = np.abs(raw) * 0.2                         # keep delta + bias positive-ish
        bias = np.abs(bias) * 0.1
    raw_t = gen._store(raw, dtype)
    _say("scan delta transform", variant, chunk, dtype, softplus)
    y, hf = ssm.scan_fwd(to_dev(inp.x), to_dev(raw_t), to_dev(inp.A), to_dev(inp.Bm), to_dev(inp.Cm),
                         to_dev(inp.D_skip), to_dev(inp.z), to_dev(inp.h0), variant=variant,
                         chunk_len=chunk, delta_bias=to_dev(bias), delta_softplus=softplus)
    torch.cuda.synchronize()
    ry, rh = oracle_mod.scan(inp.x.f32, raw_t.f32, inp.A, inp.Bm.f32, inp.Cm.f32, inp.D_skip, inp.z.f32,
                             inp.h0, delta_bias=bias, delta_softplus=softplus)
    assert_close(to_np(y), ry, dtype, "y")
    assert_close(to_np(hf), rh, dtype, "h_final")


def test_decode_delta_transform(oracle_mod):
    import mamba_selective_scan_ssm_amd as ssm
    dec = gen.make_decode(32, 640, 16, 12, dtype="bf16", seed=610)
    raw, bias = _raw_and_bias(dec.delta.f32, dec.D, 611)
    raw_t = gen._store(raw, "bf16")
    _say("decode delta transform")
    state = to_dev(dec.state0)
    xs, ds, zs, bs, cs = (to_dev(v) for v in (dec.x, raw_t, dec.z, dec.Bm, dec.Cm))
    ys = [ssm.state_update(state, xs[t], ds[t], to_dev(dec.A), bs[t], cs[t], to_dev(dec.D_skip), zs[t],
                           delta_bias=to_dev(bias), delta_softplus=True) for t in range(dec.steps)]
    torch.cuda.synchronize()
    tr = lambda a: a.transpose(1, 0, 2)
    ry, rh = oracle_mod.scan(tr(dec.x.f32), tr(raw_t.f32), dec.A, tr(dec.Bm.f32), tr(dec.Cm.f32),
                             dec.D_skip, tr(dec.z.f32), dec.state0, delta_bias=bias, delta_softplus=True)
    assert_close(to_np(torch.stack(ys, 1)), ry, "bf16", "y")
    assert_close(to_np(state), rh, "bf16", "state")


@pytest.mark.parametrize("chunk", [64, 256])
def test_ssd_dt_transform(oracle_mod, chunk):
    import mamba_selective_scan_ssm_amd as ssm
    w = gen.make_ssd(1, 600, 4, 64, 2, 128, chunk=chunk, dtype="bf16", seed=620)
    raw, hb = _raw_and_bias(w.dt.f32, w.H, 621)
    raw_t = gen._store(raw, "bf16")
    _say("ssd dt transform", chunk)
    y, hf = ssm.ssd_fwd(to_dev(w.x), to_dev(raw_t), to_dev(w.A), to_dev(w.Bm), to_dev(w.Cm),
                        to_dev(w.D_skip), None, to_dev(w.h0), chunk=chunk, dt_bias=to_dev(hb),
                        dt_softplus=True)
    torch.cuda.synchronize()
    ry, rh = oracle_mod.ssd(w.x.f32, raw_t.f32, w.A, w.Bm.f32, w.Cm.f32, w.D_skip, None, w.h0,
                            dt_bias=hb, dt_softplus=True)
    assert_close(to_np(y), ry, "bf16", "y")
    assert_close(to_np(hf), rh, "bf16", "h_final")


def test_scan_variants_bitwise_with_transform():
    import mamba_selective_scan_ssm_amd as ssm
    inp = gen.make_scan(2, 100, 256, 16, dtype="bf16", seed=630)
    raw, bias = _raw_and_bias(inp.delta.f32, inp.D, 631)
    raw_t = gen._store(raw, "bf16")
    _say("variants bitwise with transform")
    args = [to_dev(inp.x), to_dev(raw_t), to_dev(inp.A), to_dev(inp.Bm), to_dev(inp.Cm),
            to_dev(inp.D_skip), to_dev(inp.z), to_dev(inp.h0)]
    a = ssm.scan_fwd(*args, variant=1, delta_bias=to_dev(bias), delta_softplus=True)
    b = ssm.scan_fwd(*args, variant=3, delta_bias=to_dev(bias), delta_softplus=True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
