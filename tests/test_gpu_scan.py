"""GPU parity of ssm_scan_fwd against the CPU oracle (same seeded inputs).

Each case prints its name, seed and shape before touching the GPU.
"""

import numpy as np
import pytest
import torch

import ssm_inputs as gen
from tests.helpers import assert_close, to_dev, to_np

pytestmark = pytest.mark.gpu

VARIANTS = [(1, 0), (2, 8), (2, 64), (3, 0)]  # (variant, chunk_len)
LANESPLIT_N = (4, 8, 16, 32, 64)  # N the lane-split kernel (variant 3) is built for


def _say(*a):
    print("[case]", *a, flush=True)


def run_gpu(inp, gate=True, h0=True, variant=0, chunk_len=0, d_skip=True):
    x = to_dev(inp.x)
    y, hf = __import__("mamba_selective_scan_ssm_amd").scan_fwd(
        x, to_dev(inp.delta), to_dev(inp.A), to_dev(inp.Bm), to_dev(inp.Cm),
        to_dev(inp.D_skip) if d_skip else None, to_dev(inp.z) if gate else None,
        to_dev(inp.h0) if h0 else None, variant=variant, chunk_len=chunk_len)
    torch.cuda.synchronize()
    return to_np(y), to_np(hf)


def run_oracle(oracle_mod, inp, gate=True, h0=True, channels=None, d_skip=True):
    return oracle_mod.scan(inp.x.f32, inp.delta.f32, inp.A, inp.Bm.f32, inp.Cm.f32,
                           inp.D_skip if d_skip else None, inp.z.f32 if gate else None,
                           inp.h0 if h0 else None, channels=channels)


@pytest.mark.parametrize("variant,chunk", VARIANTS)
@pytest.mark.parametrize("gate", [False, True])
@pytest.mark.parametrize("h0", [False, True])
def test_tiny_fp32(oracle_mod, variant, chunk, gate, h0):
    inp = gen.make_workload("tiny_fp32")
    _say("tiny_fp32", variant, chunk, gate, h0)
    y, hf = run_gpu(inp, gate, h0, variant, chunk)
    ry, rh = run_oracle(oracle_mod, inp, gate, h0)
    assert_close(y, ry, "f32", "y")
    assert_close(hf, rh, "f32", "h_final")


@pytest.mark.parametrize("variant,chunk", [(0, 0), (1, 0), (2, 0), (2, 128), (3, 0)])
@pytest.mark.parametrize("h0", [False, True])
def test_mamba130m_fp32(oracle_mod, variant, chunk, h0):
    inp = gen.make_workload("mamba130m_fp32")
    _say("mamba130m_fp32", variant, chunk, h0)
    y, hf = run_gpu(inp, True, h0, variant, chunk)
    ry, rh = run_oracle(oracle_mod, inp, True, h0)
    assert_close(y, ry, "f32", "y")
    assert_close(hf, rh, "f32", "h_final")


@pytest.mark.parametrize("variant,chunk", [(0, 0), (1, 0), (2, 0), (3, 0)])
def test_mamba130m_split_sequence(oracle_mod, variant, chunk):
    """Two calls of L/2 with h_final fed back as h0 equal one oracle scan of L."""
    import mamba_selective_scan_ssm_amd as ssm
    inp = gen.make_workload("mamba130m_fp32")
    _say("mamba130m split", variant, chunk)
    t = {k: to_dev(getattr(inp, k)) for k in ("x", "delta", "z", "Bm", "Cm")}
    A, Ds, h0 = to_dev(inp.A), to_dev(inp.D_skip), to_dev(inp.h0)
    half = inp.L // 2
    parts = []
    h = h0
    for sl in (slice(0, half), slice(half, inp.L)):
        y, h = ssm.scan_fwd(t["x"][:, sl].contiguous(), t["delta"][:, sl].contiguous(), A,
                            t["Bm"][:, sl].contiguous(), t["Cm"][:, sl].contiguous(), Ds,
                            t["z"][:, sl].contiguous(), h, variant=variant, chunk_len=chunk)
        parts.append(y)
    torch.cuda.synchronize()
    y = to_np(torch.cat(parts, 1))
    ry, rh = run_oracle(oracle_mod, inp)
    assert_close(y, ry, "f32", "y")
    assert_close(to_np(h), rh, "f32", "h_final")


def test_mamba2p8b_prefill_bf16_whole(oracle_mod):
    """Full-size 2.8B-shaped prefill in the bench's launch configuration:
    every y (B, L, D) and every h_final (B, D, N) against the oracle."""
    inp = gen.make_workload("mamba2p8b_prefill_bf16")
    _say("mamba2p8b_prefill_bf16 full size, whole tensors")
    y, hf = run_gpu(inp)
    ry, rh = run_oracle(oracle_mod, inp)
    assert_close(y, ry, "bf16", "y")
    assert_close(hf, rh, "bf16", "h_final")


SHAPES = [
    # (B, L, D, N, dtype) -- llama.cpp's test-backend-ops SSM_SCAN shape first
    (2, 7, 1536, 16, "f32"),
    (8, 1024, 256, 16, "f32"),      # "more tokens and more sequences" (1024 tokens, 8 seqs)
    (3, 37, 1500, 16, "bf16"),      # D not a multiple of 64, odd L
    (2, 300, 100, 4, "f32"),
    (2, 300, 100, 5, "f32"),        # N off the exact buckets
    (1, 19, 70, 1, "bf16"),
    (1, 50, 64, 64, "f32"),
    (2, 1, 130, 16, "bf16"),        # single token
    (2, 513, 96, 8, "bf16"),
]


@pytest.mark.parametrize("B,L,D,N,dtype", SHAPES)
@pytest.mark.parametrize("variant,chunk", [(0, 0), (1, 0), (2, 16), (3, 0)])
def test_shapes(oracle_mod, B, L, D, N, dtype, variant, chunk):
    import mamba_selective_scan_ssm_amd as ssm
    inp = gen.make_scan(B, L, D, N, dtype=dtype, seed=100 + L + D + N)
    _say("shape", B, L, D, N, dtype, variant, chunk)
    if variant == 3 and N not in LANESPLIT_N:
        with pytest.raises(ssm.SSMError):
            run_gpu(inp, variant=variant, chunk_len=chunk)
        return
    y, hf = run_gpu(inp, variant=variant, chunk_len=chunk)
    ry, rh = run_oracle(oracle_mod, inp)
    assert_close(y, ry, dtype, "y")
    assert_close(hf, rh, dtype, "h_final")


def test_no_skip_no_gate_no_h0(oracle_mod):
    inp = gen.make_scan(2, 40, 80, 16, dtype="f32", seed=21)
    _say("no D, no z, no h0")
    y, hf = run_gpu(inp, gate=False, h0=False, d_skip=False)
    ry, rh = run_oracle(oracle_mod, inp, gate=False, h0=False, d_skip=False)
    assert_close(y, ry, "f32", "y")
    assert_close(hf, rh, "f32", "h_final")


def test_empty_sequence_returns_h0(oracle_mod):
    inp = gen.make_scan(2, 0, 70, 16, dtype="f32", seed=22)
    _say("L=0")
    y, hf = run_gpu(inp)
    assert y.shape == (2, 0, 70)
    np.testing.assert_array_equal(hf, inp.h0.astype(np.float64))
    y, hf = run_gpu(inp, h0=False)
    np.testing.assert_array_equal(hf, 0.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_batch_invariance_bitwise(dtype):
    """A sequence gives bitwise the same y and h_final alone or in a batch."""
    import mamba_selective_scan_ssm_amd as ssm
    inp = gen.make_scan(3, 300, 1536, 16, dtype=dtype, seed=23)
    _say("batch invariance", dtype)
    t = {k: to_dev(getattr(inp, k)) for k in ("x", "delta", "z", "Bm", "Cm")}
    A, Ds, h0 = to_dev(inp.A), to_dev(inp.D_skip), to_dev(inp.h0)
    y, hf = ssm.scan_fwd(t["x"], t["delta"], A, t["Bm"], t["Cm"], Ds, t["z"], h0)
    for b in range(3):
        sl = slice(b, b + 1)
        yb, hb = ssm.scan_fwd(t["x"][sl], t["delta"][sl], A, t["Bm"][sl], t["Cm"][sl], Ds,
                              t["z"][sl], h0[sl])
        assert torch.equal(yb, y[sl]) and torch.equal(hb, hf[sl])


def test_repeat_determinism():
    import mamba_selective_scan_ssm_amd as ssm
    inp = gen.make_scan(2, 777, 640, 16, dtype="bf16", seed=24)
    _say("determinism")
    t = {k: to_dev(getattr(inp, k)) for k in ("x", "delta", "z", "Bm", "Cm")}
    A, Ds, h0 = to_dev(inp.A), to_dev(inp.D_skip), to_dev(inp.h0)
    for variant in (1, 2, 3):
        outs = [ssm.scan_fwd(t["x"], t["delta"], A, t["Bm"], t["Cm"], Ds, t["z"], h0,
                             variant=variant) for _ in range(3)]
        for y, hf in outs[1:]:
            assert torch.equal(y, outs[0][0]) and torch.equal(hf, outs[0][1])


def test_chunk_length_invariance(oracle_mod):
    """Different segmentations agree with each other within the tolerance."""
    import mamba_selective_scan_ssm_amd as ssm
    inp = gen.make_scan(1, 1000, 192, 16, dtype="f32", seed=25)
    _say("chunk invariance")
    ry, rh = run_oracle(oracle_mod, inp)
    for ch in (8, 24, 200, 1000):
        y, hf = run_gpu(inp, variant=2, chunk_len=ch)
        assert_close(y, ry, "f32", f"y chunk {ch}")
        assert_close(hf, rh, "f32", f"h chunk {ch}")


def test_guard_bands_untouched():
    """Outputs are written exactly in place: NaN guards around y and h_final stay NaN."""
    import mamba_selective_scan_ssm_amd as ssm
    inp = gen.make_scan(2, 45, 100, 16, dtype="bf16", seed=26)
    _say("guard bands")
    t = {k: to_dev(getattr(inp, k)) for k in ("x", "delta", "z", "Bm", "Cm")}
    A, Ds, h0 = to_dev(inp.A), to_dev(inp.D_skip), to_dev(inp.h0)
    G = 4096
    for variant in (1, 2, 3):
        ybuf = torch.full((G + 2 * 45 * 100 + G,), float("nan"), dtype=torch.bfloat16, device="cuda")
        hbuf = torch.full((G + 2 * 100 * 16 + G,), float("nan"), dtype=torch.float32, device="cuda")
        y = ybuf[G:G + 2 * 45 * 100].view(2, 45, 100)
        hf = hbuf[G:G + 2 * 100 * 16].view(2, 100, 16)
        ssm.scan_fwd(t["x"], t["delta"], A, t["Bm"], t["Cm"], Ds, t["z"], h0, y=y, h_final=hf,
                     variant=variant, chunk_len=16)
        torch.cuda.synchronize()
        assert torch.isnan(ybuf[:G]).all() and torch.isnan(ybuf[-G:]).all()
        assert torch.isnan(hbuf[:G]).all() and torch.isnan(hbuf[-G:]).all()
        assert torch.isfinite(y.float()).all() and torch.isfinite(hf).all()


def test_nan_stays_in_its_channel():
    import mamba_selective_scan_ssm_amd as ssm
    inp = gen.make_scan(2, 64, 128, 16, dtype="f32", seed=27)
    _say("nan confinement")
    x = inp.x.f32.copy()
    x[1, 10, 77] = np.nan
    y, hf = ssm.scan_fwd(to_dev(x), to_dev(inp.delta), to_dev(inp.A), to_dev(inp.Bm),
                         to_dev(inp.Cm), to_dev(inp.D_skip), to_dev(inp.z), to_dev(inp.h0))
    bad = ~torch.isfinite(y).cpu().numpy()
    assert bad[1, 10:, 77].all()
    bad[1, 10:, 77] = False
    assert not bad.any()
    hb = ~torch.isfinite(hf).cpu().numpy()
    assert hb[1, 77].all()
    hb[1, 77] = False
    assert not hb.any()


def test_rejects_non_contiguous():
    import mamba_selective_scan_ssm_amd as ssm
    inp = gen.make_scan(1, 16, 64, 16, dtype="f32", seed=28)
    xz = torch.randn(1, 16, 128, device="cuda")
    with pytest.raises(ValueError):
        ssm.scan_fwd(xz[..., :64], to_dev(inp.delta), to_dev(inp.A), to_dev(inp.Bm),
                     to_dev(inp.Cm))


KERNEL_PAIR_SHAPES = [
    (2, 300, 1536, 16, "bf16"), (3, 37, 1500, 16, "f32"), (2, 77, 200, 4, "bf16"),
    (1, 129, 96, 8, "f32"), (2, 65, 130, 32, "bf16"), (1, 50, 64, 64, "f32"),
]


@pytest.mark.parametrize("B,L,D,N,dtype", KERNEL_PAIR_SHAPES)
@pytest.mark.parametrize("gate", [False, True])
def test_lanesplit_matches_wavesplit_bitwise(B, L, D, N, dtype, gate):
    """The two channel-sequential kernels (states split over waves, variant 1;
    over lanes, variant 3) do the same fp32 operations in the same order, so
    the automatic choice between them (which also depends on the alignment of
    Bm and Cm) never changes a result."""
    import mamba_selective_scan_ssm_amd as ssm
    inp = gen.make_scan(B, L, D, N, dtype=dtype, seed=300 + L + N)
    _say("lanesplit vs wavesplit", B, L, D, N, dtype, gate)
    t = {k: to_dev(getattr(inp, k)) for k in ("x", "delta", "z", "Bm", "Cm")}
    A, Ds, h0 = to_dev(inp.A), to_dev(inp.D_skip), to_dev(inp.h0)
    z = t["z"] if gate else None
    y1, h1 = ssm.scan_fwd(t["x"], t["delta"], A, t["Bm"], t["Cm"], Ds, z, h0, variant=1)
    y3, h3 = ssm.scan_fwd(t["x"], t["delta"], A, t["Bm"], t["Cm"], Ds, z, h0, variant=3)
    assert torch.equal(y1, y3) and torch.equal(h1, h3)


# Chunked schedule with segments of whole 32-token cycles: its summary and
# output passes run on the lane-split kernel (N in LANESPLIT_N, aligned rows).
CHUNKED_LANESPLIT_SHAPES = [
    (1, 1000, 192, 16, "f32", 96),    # ragged last segment
    (2, 333, 130, 8, "bf16", 32),     # D not a multiple of 64
    (1, 257, 64, 4, "f32", 64),       # one token in the last segment
    (1, 300, 96, 32, "bf16", 128),
    (1, 200, 64, 64, "f32", 32),
    (3, 96, 128, 16, "bf16", 96),     # a single segment
]


@pytest.mark.parametrize("B,L,D,N,dtype,chunk", CHUNKED_LANESPLIT_SHAPES)
@pytest.mark.parametrize("gate,h0", [(True, True), (False, False)])
def test_chunked_lanesplit_shapes(oracle_mod, B, L, D, N, dtype, chunk, gate, h0):
    inp = gen.make_scan(B, L, D, N, dtype=dtype, seed=700 + L + N + chunk)
    _say("chunked lane-split", B, L, D, N, dtype, chunk, gate, h0)
    y, hf = run_gpu(inp, gate, h0, variant=2, chunk_len=chunk)
    ry, rh = run_oracle(oracle_mod, inp, gate, h0)
    assert_close(y, ry, dtype, "y")
    assert_close(hf, rh, dtype, "h_final")


@pytest.mark.parametrize("B,L,D,N,dtype,chunk", CHUNKED_LANESPLIT_SHAPES)
def test_chunked_lanesplit_matches_wavesplit_bitwise(B, L, D, N, dtype, chunk):
    """The chunked schedule gives the same bits whether its passes run on the
    lane-split kernel (automatic) or on the wave-split kernel (asked for with
    an explicit states-per-lane): both do the same fp32 operations in the
    same order, segment by segment."""
    import mamba_selective_scan_ssm_amd as ssm
    inp = gen.make_scan(B, L, D, N, dtype=dtype, seed=750 + L + N)
    _say("chunked lane-split vs wave-split", B, L, D, N, dtype, chunk)
    t = {k: to_dev(getattr(inp, k)) for k in ("x", "delta", "z", "Bm", "Cm")}
    A, Ds, h0 = to_dev(inp.A), to_dev(inp.D_skip), to_dev(inp.h0)
    spl = 4 if N <= 16 else N // 4  # the lane-split kernel's states per lane
    y1, h1 = ssm.scan_fwd(t["x"], t["delta"], A, t["Bm"], t["Cm"], Ds, t["z"], h0, variant=2,
                          chunk_len=chunk)
    y2, h2 = ssm.scan_fwd(t["x"], t["delta"], A, t["Bm"], t["Cm"], Ds, t["z"], h0, variant=2,
                          chunk_len=chunk, states_per_lane=spl)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


# Halved schedule (variant 4): every wave's tokens cut in two at a 32-token
# cycle, the second half continuing from the state the first hands over.
HALVED_SHAPES = [
    (2, 500, 256, 16, "bf16"),
    (3, 777, 130, 8, "f32"),      # D not a multiple of the workgroup's channels
    (1, 300, 512, 32, "bf16"),
    (4, 96, 64, 16, "f32"),       # cut at token 64 of 96
    (5, 1000, 192, 4, "f32"),
    (1, 65, 128, 64, "bf16"),     # a one-token second half
]


@pytest.mark.parametrize("B,L,D,N,dtype", HALVED_SHAPES)
@pytest.mark.parametrize("gate,h0", [(True, True), (False, False)])
def test_halved_matches_lanesplit_bitwise(B, L, D, N, dtype, gate, h0):
    """The halved schedule hands the fp32 state across its cut exactly, so y
    and h_final are bitwise those of whole-sequence waves (variant 3)."""
    import mamba_selective_scan_ssm_amd as ssm
    inp = gen.make_scan(B, L, D, N, dtype=dtype, seed=800 + L + N)
    _say("halved vs lane-split", B, L, D, N, dtype, gate, h0)
    t = {k: to_dev(getattr(inp, k)) for k in ("x", "delta", "z", "Bm", "Cm")}
    A, Ds = to_dev(inp.A), to_dev(inp.D_skip)
    z = t["z"] if gate else None
    hz = to_dev(inp.h0) if h0 else None
    y3, h3 = ssm.scan_fwd(t["x"], t["delta"], A, t["Bm"], t["Cm"], Ds, z, hz, variant=3)
    y4, h4 = ssm.scan_fwd(t["x"], t["delta"], A, t["Bm"], t["Cm"], Ds, z, hz, variant=4)
    assert torch.equal(y3, y4) and torch.equal(h3, h4)


def test_halved_with_delta_transform(oracle_mod):
    import mamba_selective_scan_ssm_amd as ssm
    inp = gen.make_scan(2, 500, 256, 16, dtype="bf16", seed=820)
    bias = np.random.default_rng(821).normal(0.0, 0.5, inp.D).astype(np.float32)
    _say("halved, delta bias + softplus")
    t = {k: to_dev(getattr(inp, k)) for k in ("x", "delta", "z", "Bm", "Cm")}
    args = (t["x"], t["delta"], to_dev(inp.A), t["Bm"], t["Cm"], to_dev(inp.D_skip), t["z"], to_dev(inp.h0))
    kw = dict(delta_bias=to_dev(bias), delta_softplus=True)
    y3, h3 = ssm.scan_fwd(*args, variant=3, **kw)
    y4, h4 = ssm.scan_fwd(*args, variant=4, **kw)
    assert torch.equal(y3, y4) and torch.equal(h3, h4)
    ry, rh = oracle_mod.scan(inp.x.f32, inp.delta.f32, inp.A, inp.Bm.f32, inp.Cm.f32, inp.D_skip, inp.z.f32,
                             inp.h0, delta_bias=bias, delta_softplus=True)
    assert_close(to_np(y4), ry, "bf16", "y")
    assert_close(to_np(h4), rh, "bf16", "h_final")


def test_halved_where_it_does_not_apply():
    import mamba_selective_scan_ssm_amd as ssm
    for (B, L, D, N) in ((1, 50, 64, 16), (2, 300, 100, 5)):
        inp = gen.make_scan(B, L, D, N, dtype="f32", seed=830 + N)
        _say("halved unsupported", B, L, D, N)
        with pytest.raises(ssm.SSMError):
            run_gpu(inp, variant=4)


def test_mamba2p8b_prefill_auto_is_halved_bitwise():
    """At the 2.8B shape (2,560 waves of 16 channels on 1,024 SIMDs) the
    automatic choice is the halved schedule: bitwise whole-sequence waves."""
    import mamba_selective_scan_ssm_amd as ssm
    inp = gen.make_workload("mamba2p8b_prefill_bf16")
    _say("2.8B shape: automatic (halved) vs whole-sequence waves")
    assert ssm.scan_fwd_workspace_size(inp.B, inp.L, inp.D, inp.N) > 0
    t = {k: to_dev(getattr(inp, k)) for k in ("x", "delta", "z", "Bm", "Cm")}
    args = (t["x"], t["delta"], to_dev(inp.A), t["Bm"], t["Cm"], to_dev(inp.D_skip), t["z"], to_dev(inp.h0))
    y0, h0 = ssm.scan_fwd(*args)
    y3, h3 = ssm.scan_fwd(*args, variant=3)
    assert torch.equal(y0, y3) and torch.equal(h0, h3)


def test_unaligned_bc_falls_back_bitwise():
    """B/C views that are not 16-byte aligned take the wave-split kernel and
    give the same bits as aligned copies (which take the lane-split one)."""
    import mamba_selective_scan_ssm_amd as ssm
    inp = gen.make_scan(1, 90, 256, 16, dtype="bf16", seed=29)
    _say("unaligned B/C")
    t = {k: to_dev(getattr(inp, k)) for k in ("x", "delta", "z", "Bm", "Cm")}
    A, Ds, h0 = to_dev(inp.A), to_dev(inp.D_skip), to_dev(inp.h0)
    n = t["Bm"].numel()
    bbuf = torch.empty(n + 1, dtype=t["Bm"].dtype, device="cuda")
    cbuf = torch.empty(n + 1, dtype=t["Cm"].dtype, device="cuda")
    bu = bbuf[1:].view(t["Bm"].shape)
    cu = cbuf[1:].view(t["Cm"].shape)
    bu.copy_(t["Bm"])
    cu.copy_(t["Cm"])
    assert bu.data_ptr() % 16 != 0
    ya, ha = ssm.scan_fwd(t["x"], t["delta"], A, t["Bm"], t["Cm"], Ds, t["z"], h0)
    yu, hu = ssm.scan_fwd(t["x"], t["delta"], A, bu, cu, Ds, t["z"], h0)
    assert torch.equal(ya, yu) and torch.equal(ha, hu)
    with pytest.raises(ssm.SSMError):
        ssm.scan_fwd(t["x"], t["delta"], A, bu, cu, Ds, t["z"], h0, variant=3)


def test_max_plane_size(oracle_mod):
    """One sequence whose (L, D) planes are just under the 2 GiB the boundary
    accepts (L = 209600, D = 5120, bf16: the largest buffer offsets the
    kernels form), through the automatic (lane-split) and the chunked
    schedules, against the oracle on sampled channels over the whole
    sequence -- the last channel included, whose last token sits at the
    largest offset.  The inputs are drawn on the GPU (seeded) with the laws of
    the other workloads; A, D and h0 come from the input generator."""
    import mamba_selective_scan_ssm_amd as ssm
    L, D, N = 209600, 5120, 16
    assert (L + 64) * D * 2 < 2 ** 31
    small = gen.make_scan(1, 1, D, N, dtype="bf16", seed=480)
    _say("max plane size", L, D, N)
    g = torch.Generator(device="cuda").manual_seed(481)

    def normal(shape):
        return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)

    x, z = normal((1, L, D)), normal((1, L, D))
    dl = torch.nn.functional.softplus(
        0.5 * torch.randn((1, L, D), generator=g, device="cuda", dtype=torch.float32) - 1.0).to(torch.bfloat16)
    Bm, Cm = normal((1, L, N)), normal((1, L, N))
    A, Ds, h0 = to_dev(small.A), to_dev(small.D_skip), to_dev(small.h0)
    sel = [0, 1, 63, 64, 2047, 4000, 5118, 5119]
    idx = torch.tensor(sel, device="cuda")
    take = lambda t: t.index_select(2, idx).float().cpu().numpy()
    ry, rh = oracle_mod.scan(take(x), take(dl), small.A[sel], Bm.float().cpu().numpy(),
                             Cm.float().cpu().numpy(), small.D_skip[sel], take(z), small.h0[:, sel])
    for variant in (0, 2):
        _say("max plane size, variant", variant)
        y, hf = ssm.scan_fwd(x, dl, A, Bm, Cm, Ds, z, h0, variant=variant)
        torch.cuda.synchronize()
        assert_close(to_np(y.index_select(2, idx)), ry, "bf16", f"y variant {variant}")
        assert_close(to_np(hf[:, idx]), rh, "bf16", f"h_final variant {variant}")
        del y, hf
