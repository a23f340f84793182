"""Pins of the oracle's scan backward (-m "not gpu").

The gradients are checked against things other than their own formulas:
central finite differences of the FORWARD oracle for every entry of every
input (the loss is J = sum dy*y + sum dh_final*h_final, evaluated in fp64);
the mamba page's statement that the gradient of the initial state is
exp(delta_0 A) times the gradient reaching the state after the first token,
with that gradient measured by finite differences of the forward oracle on
the remaining tokens; and the split-sequence hand-off, where the backward of
the second half seeds the first half through dh_final.
"""

import numpy as np
import pytest

import ssm_inputs as gen


def _loss(oracle_mod, inp, dy, dhf, **kw):
    y, hf = oracle_mod.scan(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], inp["D_skip"],
                            inp["z"], inp["h0"], threads=1, **kw)
    J = float(np.sum(dy.astype(np.float64) * y))
    if dhf is not None:
        J += float(np.sum(dhf.astype(np.float64) * hf))
    return J


def _case(seed, gate=True, d_skip=True, h0=True, softplus=False):
    w = gen.make_scan(2, 6, 3, 4, dtype="f32", seed=seed, gate=gate, h0=h0, d_skip=d_skip)
    rng = np.random.default_rng(seed + 1)
    inp = dict(x=w.x.f32.copy(), delta=w.delta.f32.copy(), A=w.A.copy(), Bm=w.Bm.f32.copy(),
               Cm=w.Cm.f32.copy(), D_skip=None if w.D_skip is None else w.D_skip.copy(),
               z=None if w.z is None else w.z.f32.copy(), h0=None if w.h0 is None else w.h0.copy())
    kw = {}
    if softplus:
        inp["delta"] = (inp["delta"] * 6.0 - 3.0).astype(np.float32)   # raw values of both signs
        kw = dict(delta_bias=rng.normal(0.0, 1.0, 3).astype(np.float32), delta_softplus=True)
    dy = rng.normal(size=(2, 6, 3)).astype(np.float32)
    dhf = rng.normal(size=(2, 3, 4)).astype(np.float32)
    return inp, dy, dhf, kw


def _fd(oracle_mod, inp, dy, dhf, kw, name, idx, eps=2.0 ** -12):
    """Central difference of J with respect to one fp32 entry."""
    if name == "delta_bias":
        arr = kw["delta_bias"]
    else:
        arr = inp[name]
    v0 = arr[idx]
    vp, vm = np.float32(v0 + eps), np.float32(v0 - eps)
    arr[idx] = vp
    jp = _loss(oracle_mod, inp, dy, dhf, **kw)
    arr[idx] = vm
    jm = _loss(oracle_mod, inp, dy, dhf, **kw)
    arr[idx] = v0
    return (jp - jm) / (float(vp) - float(vm))


GRAD_OF = {"x": "dx", "delta": "ddelta", "z": "dz", "A": "dA", "Bm": "dB", "Cm": "dC",
           "D_skip": "dD", "h0": "dh0", "delta_bias": "dbias"}


@pytest.mark.parametrize("gate,d_skip,h0,softplus", [
    (True, True, True, False),
    (True, True, True, True),
    (False, False, False, False),
    (False, True, True, True),
])
def test_every_gradient_matches_finite_differences(oracle_mod, gate, d_skip, h0, softplus):
    inp, dy, dhf, kw = _case(11 + 2 * gate + d_skip, gate, d_skip, h0, softplus)
    g = oracle_mod.scan_bwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], inp["D_skip"],
                            inp["z"], inp["h0"], dy, dhf, threads=1, **kw)
    names = ["x", "delta", "A", "Bm", "Cm"] + (["z"] if gate else []) + (["D_skip"] if d_skip else []) \
        + (["h0"] if h0 else []) + (["delta_bias"] if softplus else [])
    for name in names:
        arr = kw["delta_bias"] if name == "delta_bias" else inp[name]
        ana = np.asarray(g[GRAD_OF[name]])
        fd = np.zeros(arr.shape)
        for idx in np.ndindex(*arr.shape):
            fd[idx] = _fd(oracle_mod, inp, dy, dhf, kw, name, idx)
        scale = max(float(np.max(np.abs(fd))), 1e-3)
        err = float(np.max(np.abs(ana - fd))) / scale
        assert err < 1e-5, f"d{name}: max error {err:.2e} of scale {scale:.3g}"
    if not h0:
        assert np.isfinite(g["dh0"]).all()


def test_initial_state_gradient_is_decayed_adjoint(oracle_mod):
    """dh0 = exp(delta_0 A) * (g_0 C_0 + dJ_tail/dh), with dJ_tail/dh from
    finite differences of the forward oracle run on tokens 1.. from h."""
    inp, dy, dhf, _ = _case(31)
    g = oracle_mod.scan_bwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], inp["D_skip"],
                            inp["z"], inp["h0"], dy, dhf, threads=1)
    B, L, D = inp["x"].shape
    N = inp["A"].shape[1]
    # state after token 0 and the gate-scaled output gradient at token 0
    _, h1 = oracle_mod.scan(*(inp[k][:, :1] for k in ("x", "delta")), inp["A"],
                            *(inp[k][:, :1] for k in ("Bm", "Cm")), inp["D_skip"], inp["z"][:, :1],
                            inp["h0"], threads=1)
    z0 = inp["z"][:, 0].astype(np.float64)
    g0 = dy[:, 0].astype(np.float64) * z0 / (1.0 + np.exp(-z0))            # (B, D)
    tail = {k: (inp[k][:, 1:].copy() if k in ("x", "delta", "Bm", "Cm", "z") else inp[k])
            for k in inp}
    lam0 = np.zeros((B, D, N))
    for b in range(B):
        for d in range(D):
            for n in range(N):
                # J_tail is affine in its initial state: an exact difference quotient
                hp = h1.copy()
                hp[b, d, n] += 1.0
                hm = h1.copy()
                hm[b, d, n] -= 1.0
                tp = dict(tail, h0=hp.astype(np.float32))
                tm = dict(tail, h0=hm.astype(np.float32))
                jp = _loss(oracle_mod, tp, dy[:, 1:], dhf)
                jm = _loss(oracle_mod, tm, dy[:, 1:], dhf)
                step = float(np.float32(hp[b, d, n])) - float(np.float32(hm[b, d, n]))
                lam0[b, d, n] = (jp - jm) / step + g0[b, d] * inp["Cm"][b, 0, n]
    dA0 = np.exp(inp["delta"][:, 0, :, None].astype(np.float64) * inp["A"][None].astype(np.float64))
    want = dA0 * lam0
    assert np.max(np.abs(g["dh0"] - want)) <= 1e-9 * max(1.0, np.max(np.abs(want)))


def test_split_sequence_hand_off(oracle_mod):
    """Backward over L equals the second half's backward (with dh_final)
    followed by the first half's, seeded with the second half's dh0 and
    started from the first half's final state."""
    w = gen.make_scan(2, 40, 5, 8, dtype="f32", seed=41)
    rng = np.random.default_rng(42)
    dy = rng.normal(size=(2, 40, 5)).astype(np.float32)
    dhf = rng.normal(size=(2, 5, 8)).astype(np.float32)
    full = oracle_mod.scan_bwd(w.x.f32, w.delta.f32, w.A, w.Bm.f32, w.Cm.f32, w.D_skip, w.z.f32, w.h0, dy, dhf)
    cut = 17
    sl1, sl2 = (slice(None), slice(0, cut)), (slice(None), slice(cut, None))
    a = lambda t, s: np.ascontiguousarray(t.f32[s])
    _, hmid = oracle_mod.scan(a(w.x, sl1), a(w.delta, sl1), w.A, a(w.Bm, sl1), a(w.Cm, sl1), w.D_skip,
                              a(w.z, sl1), w.h0)
    g2 = oracle_mod.scan_bwd(a(w.x, sl2), a(w.delta, sl2), w.A, a(w.Bm, sl2), a(w.Cm, sl2), w.D_skip,
                             a(w.z, sl2), hmid.astype(np.float32), dy[:, cut:], dhf)
    g1 = oracle_mod.scan_bwd(a(w.x, sl1), a(w.delta, sl1), w.A, a(w.Bm, sl1), a(w.Cm, sl1), w.D_skip,
                             a(w.z, sl1), w.h0, dy[:, :cut], g2["dh0"].astype(np.float32))
    # dh0 of the second half passes through fp32 above: compare at fp32 resolution
    tol = lambda r: 1e-5 * max(1.0, float(np.max(np.abs(r))))
    for k in ("dx", "ddelta", "dz", "dB", "dC"):
        got = np.concatenate([g1[k], g2[k]], axis=1)
        assert np.max(np.abs(got - full[k])) <= tol(full[k]), k
    for k in ("dA", "dD"):
        assert np.max(np.abs(g1[k] + g2[k] - full[k])) <= tol(full[k]), k
    assert np.max(np.abs(g1["dh0"] - full["dh0"])) <= tol(full["dh0"])


def test_channel_subset_accumulates_only_its_channels(oracle_mod):
    """Gradients for a list of channels equal the full call's rows, and the
    summed gradients split exactly over a partition of the channels."""
    w = gen.make_scan(2, 12, 4, 4, dtype="f32", seed=51)
    dy = np.random.default_rng(52).normal(size=(2, 12, 4)).astype(np.float32)
    args = (w.x.f32, w.delta.f32, w.A, w.Bm.f32, w.Cm.f32, w.D_skip, w.z.f32, w.h0, dy)
    full = oracle_mod.scan_bwd(*args, threads=1)
    p1 = oracle_mod.scan_bwd(*args, channels=[0, 3, 5, 6], threads=1)
    p2 = oracle_mod.scan_bwd(*args, channels=[1, 2, 4, 7], threads=1)
    b, d = np.array([0, 0, 1, 1]), np.array([0, 3, 1, 2])
    assert np.array_equal(p1["dx"], full["dx"][b, :, d])
    assert np.array_equal(p1["dh0"], full["dh0"][b, d])
    for k in ("dA", "dD", "dbias", "dB", "dC"):
        assert np.allclose(p1[k] + p2[k], full[k], rtol=1e-13, atol=1e-13), k
