"""GPU parity of ssm_ssd_fwd (Mamba-2 SSD chunked scan) against the oracle's
SSD recurrence on the same seeded inputs (bf16 inputs, fp32 state)."""

import numpy as np
import pytest
import torch

import ssm_inputs as gen
from tests.helpers import assert_close, to_dev, to_np

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def run_gpu(w, gate=None, h0=True, chunk=None):
    import mamba_selective_scan_ssm_amd as ssm
    z = w.z if gate is None else (w.z if gate else None)
    y, hf = ssm.ssd_fwd(to_dev(w.x), to_dev(w.dt), to_dev(w.A), to_dev(w.Bm), to_dev(w.Cm),
                        to_dev(w.D_skip), to_dev(z) if z is not None else None,
                        to_dev(w.h0) if (h0 and w.h0 is not None) else None,
                        chunk=chunk or w.chunk)
    torch.cuda.synchronize()
    return to_np(y), to_np(hf)


def run_oracle(oracle_mod, w, h0=True, channels=None):
    return oracle_mod.ssd(w.x.f32, w.dt.f32, w.A, w.Bm.f32, w.Cm.f32, w.D_skip,
                          w.z.f32 if w.z is not None else None, w.h0 if h0 else None,
                          channels=channels)


@pytest.mark.parametrize("B,L,H,G,N,chunk,gate", [
    (1, 256, 4, 2, 128, 256, False),     # one full chunk
    (2, 1000, 4, 1, 128, 256, False),    # ragged last chunk, one group
    (1, 640, 10, 2, 128, 128, True),     # gate on, chunk 128
    (1, 300, 3, 3, 64, 64, False),       # chunk 64, N 64, one head per group
    (1, 333, 2, 1, 32, 128, False),      # N 32
    (1, 270, 2, 2, 256, 256, False),     # N 256
    (2, 7, 4, 2, 128, 256, True),        # fewer tokens than a chunk
    (1, 600, 4, 2, 64, 256, True),       # chunk 256 at N 64, gate on
    (2, 530, 4, 4, 32, 256, False),      # chunk 256 at N 32, one head per group
    (1, 300, 6, 2, 96, 256, False),      # chunk 256 at N 96
])
def test_ssd_small(oracle_mod, B, L, H, G, N, chunk, gate):
    w = gen.make_ssd(B, L, H, 64, G, N, chunk=chunk, dtype="bf16", seed=400 + L + N, gate=gate)
    _say("ssd", B, L, H, G, N, chunk, gate)
    y, hf = run_gpu(w)
    ry, rh = run_oracle(oracle_mod, w)
    assert_close(y, ry, "bf16", "y")
    assert_close(hf, rh, "bf16", "h_final")


def test_ssd_no_h0(oracle_mod):
    w = gen.make_ssd(1, 512, 4, 64, 2, 128, chunk=256, dtype="bf16", seed=410)
    _say("ssd no h0")
    y, hf = run_gpu(w, h0=False)
    ry, rh = run_oracle(oracle_mod, w, h0=False)
    assert_close(y, ry, "bf16", "y")
    assert_close(hf, rh, "bf16", "h_final")


def test_ssd_chunk_invariance(oracle_mod):
    """Chunk lengths 64/128/256 all agree with the (chunk-free) recurrence."""
    w = gen.make_ssd(1, 768, 4, 64, 2, 128, chunk=256, dtype="bf16", seed=411)
    ry, rh = run_oracle(oracle_mod, w)
    for ch in (64, 128, 256):
        _say("ssd chunk", ch)
        y, hf = run_gpu(w, chunk=ch)
        assert_close(y, ry, "bf16", f"y chunk {ch}")
        assert_close(hf, rh, "bf16", f"h chunk {ch}")


@pytest.mark.parametrize("chunk", [64, 256])
def test_ssd_decay_extremes(oracle_mod, chunk):
    """Heads in different decay regimes: strong (dt 4, A -16: the decay
    across a 32-token block underflows fp32), nearly none (dt 1e-3, A
    -0.01), sparse large steps that reset the state inside a block, and the
    default mix -- the off-diagonal decay is formed from factors split at
    block starts and the diagonal block's directly."""
    w = gen.make_ssd(1, 600, 4, 64, 2, 128, chunk=chunk, dtype="bf16", seed=413)
    dt = w.dt.f32.copy()
    rng = np.random.default_rng(414)
    dt[:, :, 0] = 4.0
    dt[:, :, 1] = 1e-3
    dt[:, :, 2] = np.where(rng.random(dt.shape[:2]) < 0.05, 8.0, 0.01)
    w.dt = gen._store(dt.astype(np.float32), "bf16")
    w.A = np.array([-16.0, -0.01, -8.0, w.A[3]], np.float32)
    _say("ssd decay extremes", chunk)
    y, hf = run_gpu(w)
    assert np.isfinite(y).all() and np.isfinite(hf).all()
    ry, rh = run_oracle(oracle_mod, w)
    assert_close(y, ry, "bf16", "y")
    assert_close(hf, rh, "bf16", "h_final")


def test_ssd_empty_sequence():
    w = gen.make_ssd(1, 0, 4, 64, 2, 128, chunk=256, dtype="bf16", seed=412)
    _say("ssd L=0")
    y, hf = run_gpu(w)
    assert y.shape == (1, 0, 4, 64)
    np.testing.assert_array_equal(hf, w.h0.astype(np.float64))


def test_ssd_mamba2_full_whole(oracle_mod):
    """The full Mamba-2 workload (B=2, L=8192, H=80, P=64, N=128, G=8,
    chunk 256) in the bench's launch configuration: every y (B, L, H, P) and
    every final state (B, H, P, N) against the oracle."""
    w = gen.make_workload("ssd_mamba2_bf16")
    _say("ssd_mamba2_bf16 full size, whole tensors")
    y, hf = run_gpu(w)
    ry, rh = run_oracle(oracle_mod, w)
    assert_close(y, ry, "bf16", "y")
    assert_close(hf, rh, "bf16", "h_final")


def test_ssd_determinism():
    import mamba_selective_scan_ssm_amd as ssm
    w = gen.make_ssd(1, 600, 4, 64, 2, 128, chunk=256, dtype="bf16", seed=413)
    _say("ssd determinism")
    args = [to_dev(w.x), to_dev(w.dt), to_dev(w.A), to_dev(w.Bm), to_dev(w.Cm), to_dev(w.D_skip),
            None, to_dev(w.h0)]
    a = ssm.ssd_fwd(*args)
    b = ssm.ssd_fwd(*args)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# Shapes the matrix-core kernels are not built for take the token-by-token
# kernels (ssd_seq.hip): fp32 inputs, head dims other than 64, N not a
# multiple of 32, other chunk lengths, x not 16-byte aligned.  Where every
# 64-channel block lies in one group ((H / G) P a multiple of 64) the staged
# kernel runs, otherwise (P 16 with 3 heads per group, P 24) the plain one.
@pytest.mark.parametrize("B,L,H,P,G,N,chunk,dtype,gate", [
    (1, 200, 4, 64, 2, 64, 64, "f32", False),     # fp32, at the fp32 bar
    (2, 300, 6, 32, 3, 128, 256, "f32", True),    # fp32, P 32, gate
    (1, 130, 3, 16, 1, 48, 128, "f32", False),    # P 16 (four heads per 64 channels), N 48
    (2, 257, 4, 128, 2, 128, 256, "bf16", True),  # P 128
    (1, 99, 5, 24, 5, 16, 256, "bf16", False),    # P 24 (workgroups span heads), N 16, G = H
    (1, 300, 4, 64, 2, 128, 100, "bf16", False),  # chunk 100
    (1, 0, 2, 32, 1, 32, 64, "f32", False),       # empty sequence
    (1, 150, 2, 64, 1, 256, 64, "f32", True),     # N 256: 16 waves per workgroup
    (2, 77, 4, 32, 2, 48, 64, "f32", False),      # N 48 (3 waves), ragged 16-token block
])
def test_ssd_token_path(oracle_mod, B, L, H, P, G, N, chunk, dtype, gate):
    w = gen.make_ssd(B, L, H, P, G, N, chunk=chunk, dtype=dtype, seed=450 + L + P + N, gate=gate)
    _say("ssd token path", B, L, H, P, G, N, chunk, dtype, gate)
    y, hf = run_gpu(w)
    ry, rh = run_oracle(oracle_mod, w)
    assert y.shape == (B, L, H, P)
    assert_close(y, ry, dtype, "y")
    assert_close(hf, rh, dtype, "h_final")


def test_ssd_unaligned_x_takes_token_path(oracle_mod):
    """x one element off 16-byte alignment: the token-by-token kernel, same results."""
    import mamba_selective_scan_ssm_amd as ssm
    w = gen.make_ssd(1, 300, 4, 64, 2, 128, chunk=256, dtype="bf16", seed=470)
    _say("ssd unaligned x")
    xs = to_dev(w.x)
    buf = torch.empty(xs.numel() + 1, dtype=xs.dtype, device="cuda")
    x_off = buf[1:].view_as(xs)
    x_off.copy_(xs)
    y, hf = ssm.ssd_fwd(x_off, to_dev(w.dt), to_dev(w.A), to_dev(w.Bm), to_dev(w.Cm), to_dev(w.D_skip),
                        None, to_dev(w.h0), chunk=w.chunk)
    torch.cuda.synchronize()
    ry, rh = run_oracle(oracle_mod, w)
    assert_close(to_np(y), ry, "bf16", "y")
    assert_close(to_np(hf), rh, "bf16", "h_final")


def test_ssd_token_path_dt_transform(oracle_mod):
    """dt bias per head and softplus on the token-by-token path (fp32)."""
    import mamba_selective_scan_ssm_amd as ssm
    w = gen.make_ssd(2, 150, 4, 32, 2, 64, chunk=64, dtype="f32", seed=471)
    bias = np.random.default_rng(472).normal(0.0, 0.5, 4).astype(np.float32)
    _say("ssd token path dt transform")
    y, hf = ssm.ssd_fwd(to_dev(w.x), to_dev(w.dt), to_dev(w.A), to_dev(w.Bm), to_dev(w.Cm), to_dev(w.D_skip),
                        None, to_dev(w.h0), chunk=w.chunk, dt_bias=to_dev(bias), dt_softplus=True)
    torch.cuda.synchronize()
    ry, rh = oracle_mod.ssd(w.x.f32, w.dt.f32, w.A, w.Bm.f32, w.Cm.f32, w.D_skip, None, w.h0,
                            dt_bias=bias, dt_softplus=True)
    assert_close(to_np(y), ry, "f32", "y")
    assert_close(to_np(hf), rh, "f32", "h_final")
