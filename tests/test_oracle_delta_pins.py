"""Pins of the oracle's step-size transform: delta + delta_bias, then the
optional softplus (-m "not gpu").

The transformed step size is checked through closed forms that do not share
the oracle's code: with A = 0 the state is h0 + cumsum(delta' B x) (numpy),
where delta' comes from numpy's logaddexp; the decode chain equals the scan;
SSD with a per-head bias equals the Mamba-1 scan on expanded inputs.
"""

import numpy as np
import pytest

import ssm_inputs as gen


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.sqrt(np.mean(b * b)), 1e-300))


def _bias(D, seed):
    return np.random.default_rng(seed).normal(0.0, 1.5, D).astype(np.float32)


@pytest.mark.parametrize("softplus", [False, True])
def test_zero_A_closed_form_with_bias(oracle_mod, softplus):
    inp = gen.make_scan(2, 40, 12, 6, dtype="f32", seed=40, gate=False)
    bias = _bias(inp.D, 41)
    raw = inp.delta.f32.astype(np.float64) - 1.0          # include negative pre-activations
    raw32 = raw.astype(np.float32)
    A0 = np.zeros_like(inp.A)
    y, hf = oracle_mod.scan(inp.x.f32, raw32, A0, inp.Bm.f32, inp.Cm.f32, inp.D_skip, None, inp.h0,
                            delta_bias=bias, delta_softplus=softplus)
    v = raw32.astype(np.float64) + bias.astype(np.float64)
    dl = np.logaddexp(0.0, v) if softplus else v
    dBx = dl[..., None] * inp.Bm.f32[:, :, None, :] * inp.x.f32[..., None]
    h = inp.h0[:, None].astype(np.float64) + np.cumsum(dBx, axis=1)
    ref_y = (np.einsum("btn,btdn->btd", inp.Cm.f32.astype(np.float64), h)
             + inp.D_skip.astype(np.float64) * inp.x.f32)
    assert _rel(hf, h[:, -1]) < 1e-12
    assert _rel(y, ref_y) < 1e-12


def test_softplus_tail_is_identity(oracle_mod):
    """Far above 0, softplus(v) = v to double precision: a huge bias with and
    without the softplus gives the same scan."""
    inp = gen.make_scan(1, 20, 8, 4, dtype="f32", seed=42, gate=True)
    bias = np.full(inp.D, 40.0, np.float32)
    small_A = (inp.A * 1e-3).astype(np.float32)               # keep exp(delta A) away from 0
    a = oracle_mod.scan(inp.x.f32, inp.delta.f32, small_A, inp.Bm.f32, inp.Cm.f32, inp.D_skip,
                        inp.z.f32, inp.h0, delta_bias=bias, delta_softplus=True)
    b = oracle_mod.scan(inp.x.f32, inp.delta.f32, small_A, inp.Bm.f32, inp.Cm.f32, inp.D_skip,
                        inp.z.f32, inp.h0, delta_bias=bias, delta_softplus=False)
    assert _rel(a[0], b[0]) < 1e-12 and _rel(a[1], b[1]) < 1e-12


def test_decode_chain_with_bias_softplus_equals_scan(oracle_mod):
    dec = gen.make_decode(3, 10, 4, 15, dtype="bf16", seed=43, gate=True)
    bias = _bias(dec.D, 44)
    state = dec.state0.astype(np.float64).copy()
    ys = [oracle_mod.state_update(state, dec.x.f32[t], dec.delta.f32[t], dec.A, dec.Bm.f32[t],
                                  dec.Cm.f32[t], dec.D_skip, dec.z.f32[t], delta_bias=bias,
                                  delta_softplus=True) for t in range(dec.steps)]
    tr = lambda a: a.transpose(1, 0, 2)
    y, hf = oracle_mod.scan(tr(dec.x.f32), tr(dec.delta.f32), dec.A, tr(dec.Bm.f32), tr(dec.Cm.f32),
                            dec.D_skip, tr(dec.z.f32), dec.state0, delta_bias=bias, delta_softplus=True)
    np.testing.assert_array_equal(np.stack(ys, 1), y)
    np.testing.assert_array_equal(state, hf)


def test_ssd_dt_bias_equals_mamba1_expanded(oracle_mod):
    B, L, H, P, G, N = 1, 17, 4, 3, 2, 8
    s = gen.make_ssd(B, L, H, P, G, N, dtype="bf16", seed=45, gate=False)
    hb = _bias(H, 46)
    y, hf = oracle_mod.ssd(s.x.f32, s.dt.f32, s.A, s.Bm.f32, s.Cm.f32, s.D_skip, None, s.h0,
                           dt_bias=hb, dt_softplus=True)
    hpg = H // G
    for g in range(G):
        heads = list(range(g * hpg, (g + 1) * hpg))
        x = s.x.f32[:, :, heads].reshape(B, L, hpg * P)
        dl = np.repeat(s.dt.f32[:, :, heads], P, axis=2)
        A = np.repeat(s.A[heads], P)[:, None].repeat(N, axis=1)
        Ds = np.repeat(s.D_skip[heads], P)
        h0 = s.h0[:, heads].reshape(B, hpg * P, N)
        db = np.repeat(hb[heads], P)
        y1, h1 = oracle_mod.scan(x, dl, A, s.Bm.f32[:, :, g], s.Cm.f32[:, :, g], Ds, None, h0,
                                 delta_bias=db, delta_softplus=True)
        np.testing.assert_array_equal(y[:, :, heads].reshape(B, L, hpg * P), y1)
        np.testing.assert_array_equal(hf[:, heads].reshape(B, hpg * P, N), h1)
