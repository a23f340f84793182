"""GPU parity of ssm_scan_bwd (gradients of the selective scan) against the
oracle's backward, on the same seeded inputs and loss gradients.

Every case is compared whole: small cases (ragged L across 8-token
segments, D across channel tiles, every supported N, gate / skip / h0 /
dh_final / step-size transform on and off) and the 2.8B-shaped case at the
size the bench times.
"""

import numpy as np
import pytest
import torch

import ssm_inputs as gen
from tests.helpers import assert_close, to_dev, to_np

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _run(inp, gr, dtype, gate=True, d_skip=True, h0=True, dhf=True, bias=None, softplus=False, **kw):
    import mamba_selective_scan_ssm_amd as ssm
    out = ssm.scan_bwd(to_dev(inp.x), to_dev(inp.delta), to_dev(inp.A), to_dev(inp.Bm), to_dev(inp.Cm),
                       to_dev(inp.D_skip) if d_skip else None, to_dev(inp.z) if gate else None,
                       to_dev(inp.h0) if h0 else None, to_dev(gr.dy), to_dev(gr.dh_final) if dhf else None,
                       delta_bias=None if bias is None else to_dev(bias), delta_softplus=softplus,
                       want_dh0=True, want_dbias=True, **kw)
    torch.cuda.synchronize()
    return {k: (None if v is None else to_np(v)) for k, v in out.items()}


def _oracle(oracle_mod, inp, gr, gate=True, d_skip=True, h0=True, dhf=True, bias=None, softplus=False,
            channels=None):
    return oracle_mod.scan_bwd(inp.x.f32, inp.delta.f32, inp.A, inp.Bm.f32, inp.Cm.f32,
                               inp.D_skip if d_skip else None, inp.z.f32 if gate else None,
                               inp.h0 if h0 else None, gr.dy.f32, gr.dh_final if dhf else None,
                               delta_bias=bias, delta_softplus=softplus, channels=channels)


def _compare(g, r, dtype, keys=("dx", "ddelta", "dz", "dA", "dB", "dC", "dD", "dh0", "dbias")):
    for k in keys:
        if r.get(k) is None:
            continue
        assert_close(g[k], r[k], dtype, k)


@pytest.mark.parametrize("B,L,D,N,dtype", [
    (2, 37, 70, 16, "f32"),     # ragged segment and channel tile
    (1, 64, 64, 16, "bf16"),
    (2, 50, 33, 4, "f32"),
    (1, 33, 40, 8, "bf16"),
    (2, 20, 48, 32, "f32"),
    (1, 17, 20, 64, "bf16"),
    (3, 5, 130, 16, "f32"),     # shorter than one segment
])
def test_bwd_shapes(oracle_mod, B, L, D, N, dtype):
    inp = gen.make_scan(B, L, D, N, dtype=dtype, seed=800 + L + N)
    gr = gen.make_grads(B, L, D, N, dtype=dtype, seed=801 + L)
    _say("scan_bwd", B, L, D, N, dtype)
    _compare(_run(inp, gr, dtype), _oracle(oracle_mod, inp, gr), dtype)


@pytest.mark.parametrize("gate,d_skip,h0,dhf", [
    (False, True, True, True), (True, False, True, True), (True, True, False, False), (False, False, False, True),
])
def test_bwd_optional_terms(oracle_mod, gate, d_skip, h0, dhf):
    inp = gen.make_scan(2, 40, 96, 16, dtype="f32", seed=820)
    gr = gen.make_grads(2, 40, 96, 16, dtype="f32", seed=821)
    _say("scan_bwd optional terms", gate, d_skip, h0, dhf)
    opts = dict(gate=gate, d_skip=d_skip, h0=h0, dhf=dhf)
    g = _run(inp, gr, "f32", **opts)
    r = _oracle(oracle_mod, inp, gr, **opts)
    _compare(g, r, "f32")
    if not gate:
        assert g["dz"] is None
    if not d_skip:
        assert g["dD"] is None


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_delta_transform(oracle_mod, dtype):
    inp = gen.make_scan(2, 45, 64, 16, dtype=dtype, seed=830)
    inp.delta = gen._store((inp.delta.f32 * 6.0 - 3.0).astype(np.float32), dtype)
    bias = np.random.default_rng(831).normal(0.0, 1.0, 64).astype(np.float32)
    gr = gen.make_grads(2, 45, 64, 16, dtype=dtype, seed=832)
    _say("scan_bwd softplus", dtype)
    _compare(_run(inp, gr, dtype, bias=bias, softplus=True),
             _oracle(oracle_mod, inp, gr, bias=bias, softplus=True), dtype)


def test_bwd_empty_sequence_and_no_channels(oracle_mod):
    import mamba_selective_scan_ssm_amd as ssm
    inp = gen.make_scan(2, 0, 64, 16, dtype="f32", seed=840)
    gr = gen.make_grads(2, 0, 64, 16, dtype="f32", seed=841)
    _say("scan_bwd L=0")
    g = _run(inp, gr, "f32")
    assert np.array_equal(g["dh0"], gr.dh_final.astype(np.float64))
    assert not g["dA"].any() and not g["dD"].any() and not g["dbias"].any()
    assert g["dx"].shape == (2, 0, 64) and g["dB"].shape == (2, 0, 16)
    inp = gen.make_scan(2, 10, 0, 16, dtype="f32", seed=842)
    _say("scan_bwd D=0")
    out = ssm.scan_bwd(to_dev(inp.x), to_dev(inp.delta), to_dev(inp.A), to_dev(inp.Bm), to_dev(inp.Cm),
                       None, None, None, to_dev(inp.x))
    torch.cuda.synchronize()
    assert not out["dB"].any() and not out["dC"].any()


def test_bwd_reproducible():
    """Sums are taken in a fixed order: two calls agree bit for bit."""
    inp = gen.make_scan(2, 70, 200, 16, dtype="bf16", seed=850)
    gr = gen.make_grads(2, 70, 200, 16, dtype="bf16", seed=851)
    _say("scan_bwd reproducible")
    a = _run(inp, gr, "bf16")
    b = _run(inp, gr, "bf16")
    for k in a:
        if a[k] is not None:
            assert np.array_equal(a[k], b[k]), k


def test_bwd_mamba2p8b_whole(oracle_mod):
    """The 2.8B-shaped prefill (B=8, L=4096, D=5120, N=16, bf16) as the bench
    times it: every gradient whole -- dx, ddelta, dz (B, L, D), dh0, dA, dD,
    the bias gradient, and dB, dC (B, L, N) for all sequences."""
    inp = gen.make_workload("mamba2p8b_prefill_bf16")
    B, L, D, N = inp.B, inp.L, inp.D, inp.N
    gr = gen.make_grads(B, L, D, N, dtype="bf16", seed=1008)
    _say("scan_bwd mamba2p8b full size, whole tensors")
    g = _run(inp, gr, "bf16")
    r = _oracle(oracle_mod, inp, gr)
    _compare(g, r, "bf16")
    # the training pair the bench also times: forward saving the segment
    # states, backward reading them -- bitwise the backward above
    import mamba_selective_scan_ssm_amd as ssm
    dev = [to_dev(v) for v in (inp.x, inp.delta, inp.A, inp.Bm, inp.Cm, inp.D_skip, inp.z, inp.h0)]
    _, _, ck = ssm.scan_fwd_train(*dev)
    g2 = ssm.scan_bwd(*dev, to_dev(gr.dy), to_dev(gr.dh_final), want_dbias=True, h_ckpt=ck)
    torch.cuda.synchronize()
    for k, v in g2.items():
        if v is not None:
            assert np.array_equal(to_np(v), g[k]), k


@pytest.mark.parametrize("L,N,dtype", [(37, 16, "f32"), (64, 16, "bf16"), (20, 32, "f32"), (9, 4, "bf16"),
                                       (16, 64, "f32")])
def test_saved_segment_states(oracle_mod, L, N, dtype):
    """ssm_scan_fwd_train: y and h_final bitwise those of the lane-split
    forward; its segment states equal the oracle's state after 8s tokens; the
    backward reading them is bitwise the backward that recomputes them."""
    import mamba_selective_scan_ssm_amd as ssm
    B, D = 2, 96
    inp = gen.make_scan(B, L, D, N, dtype=dtype, seed=870 + L + N)
    gr = gen.make_grads(B, L, D, N, dtype=dtype, seed=871 + L)
    dev = {k: to_dev(getattr(inp, k)) for k in ("x", "delta", "A", "Bm", "Cm", "D_skip", "z", "h0")}
    args = (dev["x"], dev["delta"], dev["A"], dev["Bm"], dev["Cm"], dev["D_skip"], dev["z"], dev["h0"])
    _say("scan_fwd_train", L, N, dtype)
    y, hf, ck = ssm.scan_fwd_train(*args)
    y3, hf3 = ssm.scan_fwd(*args, variant=3)
    torch.cuda.synchronize()
    assert torch.equal(y, y3) and torch.equal(hf, hf3)
    nseg = (L + 7) // 8
    assert ck.shape == (B, nseg, D, N)
    ckn = to_np(ck)
    assert np.array_equal(ckn[:, 0], inp.h0.astype(np.float64))
    for sg in sorted({1, nseg // 2, nseg - 1} - {0}):
        cut = lambda t: np.ascontiguousarray(t.f32[:, :8 * sg])
        _, hs = oracle_mod.scan(cut(inp.x), cut(inp.delta), inp.A, cut(inp.Bm), cut(inp.Cm), inp.D_skip,
                                cut(inp.z), inp.h0)
        assert_close(ckn[:, sg], hs, dtype, f"segment state {sg}")
    g0 = ssm.scan_bwd(*args, to_dev(gr.dy), to_dev(gr.dh_final), want_dbias=True)
    g1 = ssm.scan_bwd(*args, to_dev(gr.dy), to_dev(gr.dh_final), want_dbias=True, h_ckpt=ck)
    torch.cuda.synchronize()
    for k in g0:
        if g0[k] is not None:
            assert torch.equal(g0[k], g1[k]), k


def test_bwd_max_plane_size(oracle_mod):
    """One sequence whose (L, D) planes are just under the 2 GiB the boundary
    accepts (L = 209600, D = 5120, bf16).  dy is nonzero on sampled channels
    only (the last one included) and dh_final is zero, so every other
    channel's gradient is exactly zero and dB, dC sum over the sampled
    channels: all of them are compared with the oracle over the whole
    sequence, and the other channels' dx, ddelta, dz checked to be zero on a
    band of channels.  Inputs drawn on the GPU (seeded); A, D, h0 from the
    input generator."""
    import mamba_selective_scan_ssm_amd as ssm
    L, D, N = 209600, 5120, 16
    assert (L + 64) * D * 2 < 2 ** 31
    small = gen.make_scan(1, 1, D, N, dtype="bf16", seed=484)
    _say("bwd max plane size", L, D, N)
    g = torch.Generator(device="cuda").manual_seed(485)

    def normal(shape):
        return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)

    x, z = normal((1, L, D)), normal((1, L, D))
    dl = torch.nn.functional.softplus(
        0.5 * torch.randn((1, L, D), generator=g, device="cuda", dtype=torch.float32) - 1.0).to(torch.bfloat16)
    Bm, Cm = normal((1, L, N)), normal((1, L, N))
    sel = [0, 77, 2048, 5119]
    idx = torch.tensor(sel, device="cuda")
    dy = torch.zeros((1, L, D), dtype=torch.bfloat16, device="cuda")
    dy[:, :, idx] = normal((1, L, len(sel)))
    A, Ds, h0 = to_dev(small.A), to_dev(small.D_skip), to_dev(small.h0)
    out = ssm.scan_bwd(x, dl, A, Bm, Cm, Ds, z, h0, dy, None, want_dh0=True)
    torch.cuda.synchronize()
    take = lambda t: t.index_select(2, idx).float().cpu().numpy()
    r = oracle_mod.scan_bwd(take(x), take(dl), small.A[sel], Bm.float().cpu().numpy(), Cm.float().cpu().numpy(),
                            small.D_skip[sel], take(z), small.h0[:, sel], take(dy), None)
    for k in ("dx", "ddelta", "dz"):
        assert_close(to_np(out[k].index_select(2, idx)), r[k], "bf16", k)
    assert_close(to_np(out["dh0"][:, idx]), r["dh0"], "bf16", "dh0")
    assert_close(to_np(out["dA"][idx]), r["dA"], "bf16", "dA")
    assert_close(to_np(out["dD"][idx]), r["dD"], "bf16", "dD")
    assert_close(to_np(out["dB"]), r["dB"], "bf16", "dB")
    assert_close(to_np(out["dC"]), r["dC"], "bf16", "dC")
    band = slice(100, 164)  # channels without gradient
    for k in ("dx", "ddelta", "dz"):
        assert not (out[k][:, :, band] != 0).any(), k
