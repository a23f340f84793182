"""Pins for the CPU oracle: checks against things other than the oracle itself.

The pages print no numeric worked example of a scan, so the oracle is pinned
by closed forms of the recurrence ("Adding Initial Value Support to Selective
Scan Forward Kernel", opening question and the running-prefix replies),
special cases that reduce to textbook or library routines (numpy.cumsum,
scipy.signal.lfilter, scipy.special.expit), a hand-worked example
(tests/golden/scan_hand_example.txt), the associativity of the affine scan
pair (exp(delta*A), state), and the invariances the pages rely on: results do
not depend on how a batch is split ("-b must not change the output", llama.cpp
issue 6758) nor on where the sequence is split when the final state is fed
back as the initial state.
"""

import os

import numpy as np
import pytest
import scipy.signal
import scipy.special

import ssm_inputs as gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(np.sqrt(np.mean(b * b)), 1e-300)
    return float(np.max(np.abs(a - b)) / scale)


# --------------------------------------------------------------------------
# independent closed forms (numpy, no loop over the recurrence)
# --------------------------------------------------------------------------

def closed_form_segment(x, delta, A, Bm, Cm, D_skip, z, h0):
    """h_t = e^{A S_t} h0 + sum_{k<=t} e^{A (S_t - S_k)} delta_k B_k x_k,
    S_t = sum_{j<=t} delta_j (segment sums, O(L^2) per state)."""
    x, delta, Bm, Cm = (np.asarray(v, np.float64) for v in (x, delta, Bm, Cm))
    A = np.asarray(A, np.float64)
    Bsz, L, D = x.shape
    N = A.shape[1]
    S = np.cumsum(delta, axis=1)                                    # (B, L, D)
    # decay[b, t, k, d, n] = exp(A[d,n] * (S_t - S_k)) for k <= t
    diff = S[:, :, None, :] - S[:, None, :, :]                      # (B, t, k, D)
    causal = np.tril(np.ones((L, L), dtype=bool))[None, :, :, None]
    diff = np.where(causal, diff, 0.0)
    decay = np.exp(diff[..., None] * A[None, None, None, :, :])     # (B,t,k,D,N)
    decay = np.where(causal[..., None], decay, 0.0)
    dBx = delta[:, :, :, None] * Bm[:, :, None, :] * x[:, :, :, None]  # (B,k,D,N)
    h = np.einsum("btkdn,bkdn->btdn", decay, dBx)
    if h0 is not None:
        h = h + np.exp(S[..., None] * A[None, None]) * np.asarray(h0, np.float64)[:, None]
    y = np.einsum("btn,btdn->btd", Cm, h)
    if D_skip is not None:
        y = y + np.asarray(D_skip, np.float64)[None, None, :] * x
    if z is not None:
        zz = np.asarray(z, np.float64)
        y = y * zz * scipy.special.expit(zz)
    return y, h[:, -1]


def closed_form_product(x, delta, A, Bm, Cm, D_skip, z, h0):
    """h_t = (prod_{j<=t} dA_j) h0 + sum_k (prod_{k<j<=t} dA_j) dBx_k, with the
    products taken explicitly over exp(delta_j A) (the brute-force form)."""
    x, delta, Bm, Cm = (np.asarray(v, np.float64) for v in (x, delta, Bm, Cm))
    A = np.asarray(A, np.float64)
    Bsz, L, D = x.shape
    dA = np.exp(delta[..., None] * A[None, None])                   # (B, L, D, N)
    dBx = delta[..., None] * Bm[:, :, None, :] * x[..., None]
    hs = []
    for t in range(L):
        acc = np.zeros_like(dA[:, 0])
        if h0 is not None:
            acc = acc + np.prod(dA[:, : t + 1], axis=1) * np.asarray(h0, np.float64)
        for k in range(t + 1):
            acc = acc + np.prod(dA[:, k + 1: t + 1], axis=1) * dBx[:, k]
        hs.append(acc)
    h = np.stack(hs, axis=1)
    y = np.einsum("btn,btdn->btd", Cm, h)
    if D_skip is not None:
        y = y + np.asarray(D_skip, np.float64) * x
    if z is not None:
        zz = np.asarray(z, np.float64)
        y = y * zz * scipy.special.expit(zz)
    return y, h[:, -1]


def _scan_args(inp, gate=True, h0=True):
    return dict(x=inp.x.f32, delta=inp.delta.f32, A=inp.A, Bm=inp.Bm.f32, Cm=inp.Cm.f32,
                D_skip=inp.D_skip, z=(inp.z.f32 if (gate and inp.z is not None) else None),
                h0=(inp.h0 if h0 else None))


@pytest.mark.parametrize("gate", [False, True])
@pytest.mark.parametrize("h0", [False, True])
def test_closed_form_tiny(oracle_mod, gate, h0):
    """The tiny fp32 workload (B=1, L=64, D=16, N=4) against both closed forms."""
    inp = gen.make_workload("tiny_fp32")
    args = _scan_args(inp, gate, h0)
    y, hf = oracle_mod.scan(**args)
    y1, h1 = closed_form_segment(**args)
    assert _rel(y, y1) < 1e-11 and _rel(hf, h1) < 1e-11
    if not gate:
        y2, h2 = closed_form_product(**args)
        assert _rel(y, y2) < 1e-11 and _rel(hf, h2) < 1e-11


def test_closed_form_backend_ops_shape(oracle_mod):
    """llama.cpp's test-backend-ops SSM_SCAN shape: d_state 16, d_inner 1536,
    7 tokens, 2 sequences (compilade's test patch), with random h0."""
    inp = gen.make_scan(2, 7, 1536, 16, dtype="f32", seed=7, gate=True)
    args = _scan_args(inp)
    y, hf = oracle_mod.scan(**args)
    y1, h1 = closed_form_segment(**args)
    assert _rel(y, y1) < 1e-11 and _rel(hf, h1) < 1e-11


def test_hand_example(oracle_mod):
    vals = {}
    with open(os.path.join(GOLDEN, "scan_hand_example.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            k, v = line.split(":", 1)
            vals[k.strip()] = np.array([float(t) for t in v.split()])
    L, N = 3, 2
    args = dict(x=vals["x"].reshape(1, L, 1), delta=vals["delta"].reshape(1, L, 1),
                A=vals["A"].reshape(1, N), Bm=vals["Bm"].reshape(1, L, N),
                Cm=vals["Cm"].reshape(1, L, N), D_skip=vals["D_skip"],
                h0=vals["h0"].reshape(1, 1, N))
    y, hf = oracle_mod.scan(**args)
    np.testing.assert_allclose(y.ravel(), vals["y"], rtol=1e-6)
    np.testing.assert_allclose(hf.ravel(), vals["h_final"], rtol=1e-6)
    yz, hz = oracle_mod.scan(**args, z=vals["z"].reshape(1, L, 1))
    np.testing.assert_allclose(yz.ravel(), vals["y"] * vals["gate_factor"], rtol=1e-6)
    np.testing.assert_array_equal(hz, hf)


def test_zero_delta_holds_state(oracle_mod):
    """delta = 0: dA = 1 and dBx = 0, so h_t = h0 and y_t = C_t.h0 + D x_t."""
    inp = gen.make_scan(2, 33, 24, 8, dtype="f32", seed=3, gate=False)
    args = _scan_args(inp, gate=False)
    args["delta"] = np.zeros_like(args["delta"])
    y, hf = oracle_mod.scan(**args)
    np.testing.assert_array_equal(hf, inp.h0.astype(np.float64))
    ref = np.einsum("btn,bdn->btd", inp.Cm.f32.astype(np.float64), inp.h0.astype(np.float64))
    ref += inp.D_skip.astype(np.float64) * inp.x.f32
    assert _rel(y, ref) < 1e-14


def test_zero_A_is_cumsum(oracle_mod):
    """A = 0: dA = 1, so h_t = h0 + cumsum_k(delta_k B_k x_k) (numpy.cumsum)."""
    inp = gen.make_scan(2, 40, 12, 6, dtype="f32", seed=4, gate=False)
    args = _scan_args(inp, gate=False)
    args["A"] = np.zeros_like(args["A"])
    y, hf = oracle_mod.scan(**args)
    dBx = (inp.delta.f32.astype(np.float64)[..., None] * inp.Bm.f32[:, :, None, :]
           * inp.x.f32[..., None])
    h = inp.h0[:, None].astype(np.float64) + np.cumsum(dBx, axis=1)
    ref_y = (np.einsum("btn,btdn->btd", inp.Cm.f32.astype(np.float64), h)
             + inp.D_skip.astype(np.float64) * inp.x.f32)
    assert _rel(hf, h[:, -1]) < 1e-12
    assert _rel(y, ref_y) < 1e-12


def test_zero_x_is_pure_decay(oracle_mod):
    """x = 0: dBx = 0, so h_t = exp(A S_t) h0 -- pins that h0 enters as the
    state before step 1 (pair (1, h0)), not as a decay factor (pair (h0, 0))."""
    inp = gen.make_scan(1, 50, 10, 5, dtype="f32", seed=5, gate=False)
    args = _scan_args(inp, gate=False)
    args["x"] = np.zeros_like(args["x"])
    y, hf = oracle_mod.scan(**args)
    S = np.cumsum(inp.delta.f32.astype(np.float64), axis=1)
    h = np.exp(S[..., None] * inp.A[None, None]) * inp.h0[:, None]
    ref_y = np.einsum("btn,btdn->btd", inp.Cm.f32.astype(np.float64), h)
    assert _rel(hf, h[:, -1]) < 1e-12
    assert _rel(y, ref_y) < 1e-12


def test_constant_delta_A_is_lfilter(oracle_mod):
    """delta and A constant: h_t = a h_{t-1} + b_t, a first-order IIR filter,
    evaluated by scipy.signal.lfilter with the initial condition a*h0."""
    L, D, N = 64, 3, 4
    inp = gen.make_scan(1, L, D, N, dtype="f32", seed=6, gate=False)
    args = _scan_args(inp, gate=False)
    dl = np.float32(0.37)
    args["delta"] = np.full_like(args["delta"], dl)
    y, hf = oracle_mod.scan(**args)
    for d in range(D):
        for n in range(N):
            a = np.exp(np.float64(dl) * np.float64(inp.A[d, n]))
            b = np.float64(dl) * inp.Bm.f32[0, :, n].astype(np.float64) * inp.x.f32[0, :, d]
            h, _ = scipy.signal.lfilter([1.0], [1.0, -a], b, zi=[a * inp.h0[0, d, n]])
            assert abs(h[-1] - hf[0, d, n]) <= 1e-12 * max(1.0, abs(h[-1]))


def test_gate_is_silu(oracle_mod):
    """The gate multiplies the ungated output by silu(z) = z * sigmoid(z)."""
    inp = gen.make_scan(2, 20, 9, 4, dtype="f32", seed=8, gate=True)
    g, hg = oracle_mod.scan(**_scan_args(inp, gate=True))
    u, hu = oracle_mod.scan(**_scan_args(inp, gate=False))
    zz = inp.z.f32.astype(np.float64)
    assert _rel(g, u * zz * scipy.special.expit(zz)) < 1e-14
    np.testing.assert_array_equal(hg, hu)


def test_split_sequence_bitwise(oracle_mod):
    """Scanning L1 then L2 with h_final fed back as h0 equals one scan of L1+L2."""
    inp = gen.make_scan(2, 96, 20, 8, dtype="f32", seed=9, gate=True)
    a = _scan_args(inp)
    y, hf = oracle_mod.scan(**a)
    L1 = 37

    def part(sl, h0):
        return oracle_mod.scan(x=a["x"][:, sl], delta=a["delta"][:, sl], A=a["A"],
                               Bm=a["Bm"][:, sl], Cm=a["Cm"][:, sl], D_skip=a["D_skip"],
                               z=a["z"][:, sl], h0=h0)

    y1, h1 = part(slice(0, L1), a["h0"])
    # the split point's state is fed back exactly (fp64 kept as fp64 here by
    # re-running the second half from the fp64 state through the step function)
    state = h1.copy()
    ys = []
    for t in range(L1, 96):
        ys.append(oracle_mod.state_update(state, a["x"][:, t], a["delta"][:, t], a["A"],
                                          a["Bm"][:, t], a["Cm"][:, t], a["D_skip"], a["z"][:, t]))
    np.testing.assert_array_equal(np.concatenate([y1, np.stack(ys, 1)], axis=1), y)
    np.testing.assert_array_equal(state, hf)
    # and through the scan itself with an fp32-representable split state
    h1_32 = h1.astype(np.float32)
    y2, h2 = part(slice(L1, 96), h1_32)
    state = h1_32.astype(np.float64)
    for t in range(L1, 96):
        yy = oracle_mod.state_update(state, a["x"][:, t], a["delta"][:, t], a["A"],
                                     a["Bm"][:, t], a["Cm"][:, t], a["D_skip"], a["z"][:, t])
        np.testing.assert_array_equal(yy, y2[:, t - L1])
    np.testing.assert_array_equal(state, h2)


def test_batch_invariance_bitwise(oracle_mod):
    """Each sequence of a batch gives bitwise the same result alone."""
    inp = gen.make_scan(3, 25, 14, 6, dtype="f32", seed=10, gate=True)
    a = _scan_args(inp)
    y, hf = oracle_mod.scan(**a)
    for b in range(3):
        sl = slice(b, b + 1)
        yb, hb = oracle_mod.scan(x=a["x"][sl], delta=a["delta"][sl], A=a["A"], Bm=a["Bm"][sl],
                                 Cm=a["Cm"][sl], D_skip=a["D_skip"], z=a["z"][sl], h0=a["h0"][sl])
        np.testing.assert_array_equal(yb, y[sl])
        np.testing.assert_array_equal(hb, hf[sl])


def test_channel_sampling_matches_full(oracle_mod):
    inp = gen.make_scan(2, 30, 11, 5, dtype="f32", seed=11, gate=True)
    a = _scan_args(inp)
    y, hf = oracle_mod.scan(**a)
    ch = np.array([0, 5, 11, 21])
    ys, hs = oracle_mod.scan(**a, channels=ch)
    for k, c in enumerate(ch):
        b, d = divmod(int(c), 11)
        np.testing.assert_array_equal(ys[k], y[b, :, d])
        np.testing.assert_array_equal(hs[k], hf[b, d])


def test_threads_do_not_change_results(oracle_mod):
    inp = gen.make_scan(2, 30, 40, 4, dtype="f32", seed=12, gate=True)
    a = _scan_args(inp)
    y1, h1 = oracle_mod.scan(**a, threads=1)
    y4, h4 = oracle_mod.scan(**a, threads=5)
    np.testing.assert_array_equal(y1, y4)
    np.testing.assert_array_equal(h1, h4)


def test_chunked_affine_composition(oracle_mod):
    """The scan pair (a, b) = (exp(delta*A), delta*B*x) composes as
    (a1, b1) then (a2, b2) = (a2*a1, a2*b1 + b2) with identity (1, 0); per-chunk
    aggregates carried across chunks from the seed (1, h0) reproduce the
    sequential state at every chunk boundary.  This pins the associativity the
    chunked GPU scans rely on."""
    inp = gen.make_scan(1, 120, 6, 4, dtype="f32", seed=13, gate=False)
    a = _scan_args(inp, gate=False)
    dl = inp.delta.f32.astype(np.float64)[0]
    aa = np.exp(dl[..., None] * inp.A[None])                          # (L, D, N)
    bb = dl[..., None] * inp.Bm.f32[0][:, None, :] * inp.x.f32[0][..., None]
    Q = 16
    carry_a, carry_b = np.ones((6, 4)), inp.h0[0].astype(np.float64)  # seed (1, h0)
    bounds = []
    for c0 in range(0, 120, Q):
        ca, cb = np.ones((6, 4)), np.zeros((6, 4))                    # identity (1, 0)
        for t in range(c0, min(c0 + Q, 120)):
            ca, cb = aa[t] * ca, aa[t] * cb + bb[t]
        carry_a, carry_b = ca * carry_a, ca * carry_b + cb
        bounds.append(carry_b.copy())
    for i, c1 in enumerate(range(Q, 121, Q)):
        _, h = oracle_mod.scan(x=a["x"][:, :c1], delta=a["delta"][:, :c1], A=a["A"],
                               Bm=a["Bm"][:, :c1], Cm=a["Cm"][:, :c1], h0=a["h0"])
        assert _rel(h[0], bounds[i]) < 1e-12
    _, hf = oracle_mod.scan(**a)
    assert _rel(hf[0], bounds[-1]) < 1e-12


def test_step_equals_scan_of_one(oracle_mod):
    inp = gen.make_scan(4, 1, 19, 8, dtype="f32", seed=14, gate=True)
    a = _scan_args(inp)
    y, hf = oracle_mod.scan(**a)
    state = inp.h0.astype(np.float64).copy()
    ys = oracle_mod.state_update(state, a["x"][:, 0], a["delta"][:, 0], a["A"], a["Bm"][:, 0],
                                 a["Cm"][:, 0], a["D_skip"], a["z"][:, 0])
    np.testing.assert_array_equal(ys, y[:, 0])
    np.testing.assert_array_equal(state, hf)


def test_decode_steps_equal_scan(oracle_mod):
    """128-step-style decode chain equals the scan over the same tokens (bitwise)."""
    dec = gen.make_decode(5, 13, 16, 24, dtype="bf16", seed=15)
    state = dec.state0.astype(np.float64).copy()
    ys = [oracle_mod.state_update(state, dec.x.f32[t], dec.delta.f32[t], dec.A, dec.Bm.f32[t],
                                  dec.Cm.f32[t], dec.D_skip, dec.z.f32[t]) for t in range(24)]
    tr = lambda v: np.ascontiguousarray(np.swapaxes(v, 0, 1))
    y, hf = oracle_mod.scan(tr(dec.x.f32), tr(dec.delta.f32), dec.A, tr(dec.Bm.f32), tr(dec.Cm.f32),
                            dec.D_skip, tr(dec.z.f32), dec.state0)
    np.testing.assert_array_equal(np.stack(ys, 1), y)
    np.testing.assert_array_equal(state, hf)


def test_empty_sequence(oracle_mod):
    inp = gen.make_scan(2, 0, 5, 3, dtype="f32", seed=16, gate=True)
    y, hf = oracle_mod.scan(**_scan_args(inp))
    assert y.shape == (2, 0, 5)
    np.testing.assert_array_equal(hf, inp.h0.astype(np.float64))


def test_nan_stays_in_its_channel(oracle_mod):
    inp = gen.make_scan(2, 16, 8, 4, dtype="f32", seed=17, gate=True)
    a = _scan_args(inp)
    a["x"] = a["x"].copy()
    a["x"][1, 5, 3] = np.nan
    y, hf = oracle_mod.scan(**a)
    bad = ~np.isfinite(y)
    assert bad[1, 5:, 3].all()
    bad[1, 5:, 3] = False
    assert not bad.any()


# --------------------------------------------------------------------------
# Mamba-2 SSD
# --------------------------------------------------------------------------

def _ssd_args(s):
    return dict(x=s.x.f32, dt=s.dt.f32, A=s.A, Bm=s.Bm.f32, Cm=s.Cm.f32, D_skip=s.D_skip,
                z=(s.z.f32 if s.z is not None else None), h0=s.h0)


def test_ssd_equals_mamba1_on_expanded_inputs(oracle_mod):
    """With A[d, n] = A[head(d)], delta[b,t,d] = dt[b,t,head(d)] and each group's
    B/C, the SSD recurrence is the Mamba-1 recurrence over the group's H/G*P
    channels (bitwise: the same operations in the same order)."""
    B, L, H, P, G, N = 2, 21, 6, 4, 3, 8
    s = gen.make_ssd(B, L, H, P, G, N, dtype="bf16", seed=20, gate=True)
    y, hf = oracle_mod.ssd(**_ssd_args(s))
    hpg = H // G
    for g in range(G):
        heads = range(g * hpg, (g + 1) * hpg)
        x = s.x.f32[:, :, heads].reshape(B, L, hpg * P)
        z = s.z.f32[:, :, heads].reshape(B, L, hpg * P)
        dl = np.repeat(s.dt.f32[:, :, heads], P, axis=2)
        A = np.repeat(s.A[list(heads)], P)[:, None].repeat(N, axis=1)
        Ds = np.repeat(s.D_skip[list(heads)], P)
        h0 = s.h0[:, heads].reshape(B, hpg * P, N)
        y1, h1 = oracle_mod.scan(x, dl, A, s.Bm.f32[:, :, g], s.Cm.f32[:, :, g], Ds, z, h0)
        np.testing.assert_array_equal(y[:, :, heads].reshape(B, L, hpg * P), y1)
        np.testing.assert_array_equal(hf[:, heads].reshape(B, hpg * P, N), h1)


def ssd_quadratic_form(x, dt, A, Bm, Cm, D_skip, z, h0):
    """The state-space-duality (masked attention-like) form of the SSD layer:
    y_i = sum_{j<=i} (C_i . B_j) exp(S_i - S_j) dt_j x_j + exp(S_i) C_i . h0
          + D x_i, S_i = sum_{k<=i} dt_k A (per head), evaluated with dense
    matrices -- a different arithmetic path from the recurrence."""
    x, dt, Bm, Cm = (np.asarray(v, np.float64) for v in (x, dt, Bm, Cm))
    Bsz, L, H, P = x.shape
    G = Bm.shape[2]
    hpg = H // G
    y = np.zeros_like(x)
    hfin = np.zeros((Bsz, H, P, Bm.shape[3]))
    mask = np.tril(np.ones((L, L), dtype=bool))
    for b in range(Bsz):
        for h in range(H):
            g = h // hpg
            S = np.cumsum(dt[b, :, h] * A[h])
            Lmat = np.where(mask, np.exp(np.where(mask, S[:, None] - S[None, :], 0.0)), 0.0)
            CB = Cm[b, :, g] @ Bm[b, :, g].T
            M = CB * Lmat * dt[b, None, :, h]
            y[b, :, h] = M @ x[b, :, h]
            hfin[b, h] = (x[b, :, h].T * (np.exp(S[-1] - S) * dt[b, :, h])) @ Bm[b, :, g]
            if h0 is not None:
                y[b, :, h] += np.exp(S)[:, None] * (Cm[b, :, g] @ np.asarray(h0, np.float64)[b, h].T)
                hfin[b, h] += np.exp(S[-1]) * h0[b, h]
            if D_skip is not None:
                y[b, :, h] += D_skip[h] * x[b, :, h]
    if z is not None:
        zz = np.asarray(z, np.float64)
        y = y * zz * scipy.special.expit(zz)
    return y, hfin


@pytest.mark.parametrize("gate", [False, True])
def test_ssd_quadratic_form(oracle_mod, gate):
    s = gen.make_ssd(2, 40, 4, 8, 2, 16, dtype="bf16", seed=21, gate=gate)
    a = _ssd_args(s)
    y, hf = oracle_mod.ssd(**a)
    y1, h1 = ssd_quadratic_form(**a)
    assert _rel(y, y1) < 1e-11 and _rel(hf, h1) < 1e-11


def test_ssd_channel_sampling(oracle_mod):
    s = gen.make_ssd(2, 17, 4, 3, 2, 5, dtype="f32", seed=22, gate=True)
    a = _ssd_args(s)
    y, hf = oracle_mod.ssd(**a)
    ch = np.array([0, 7, 13, 23])
    ys, hs = oracle_mod.ssd(**a, channels=ch)
    for k, c in enumerate(ch):
        p = c % 3
        h = (c // 3) % 4
        b = c // 12
        np.testing.assert_array_equal(ys[k], y[b, :, h, p])
        np.testing.assert_array_equal(hs[k], hf[b, h, p])
