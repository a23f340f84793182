"""GPU parity of the short causal convolution (ssm_conv1d_fwd and
ssm_conv1d_update) against the oracle's conv1d on the same seeded inputs."""

import numpy as np
import pytest
import torch

import ssm_inputs as gen
from tests.helpers import assert_close, to_dev, to_np

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def run_gpu(c, act=True, bias=True, state=True):
    import mamba_selective_scan_ssm_amd as ssm
    y, st = ssm.conv1d_fwd(to_dev(c.x), to_dev(c.w), to_dev(c.bias) if bias else None,
                           to_dev(c.state0) if state else None,
                           activation="silu" if act else None)
    torch.cuda.synchronize()
    return to_np(y), to_np(st)


def run_oracle(oracle_mod, c, act=True, bias=True, state=True):
    return oracle_mod.conv1d(c.x.f32, c.w, c.bias if bias else None, c.state0 if state else None,
                             act=act)


@pytest.mark.parametrize("B,L,D,K", [
    (2, 7, 1536, 4),       # the SSM_CONV test shape of the llama.cpp page
    (2, 130, 300, 4),      # ragged L (not a multiple of 8 or 64) and D
    (1, 64, 256, 3),
    (3, 65, 70, 2),
    (1, 200, 64, 8),
    (2, 2, 33, 4),         # L < K - 1: the new state mixes old state and inputs
    (1, 1, 10, 4),
])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv_shapes(oracle_mod, B, L, D, K, dtype):
    c = gen.make_conv(B, L, D, K, dtype=dtype, seed=500 + L + D + K)
    for act, bias, state in ((True, True, True), (False, False, False), (True, False, True)):
        _say("conv", B, L, D, K, dtype, act, bias, state)
        y, st = run_gpu(c, act, bias, state)
        ry, rs = run_oracle(oracle_mod, c, act, bias, state)
        assert_close(y, ry, dtype, "y")
        np.testing.assert_array_equal(st, rs)   # the state holds input values: exact


def test_conv_empty_sequence():
    c = gen.make_conv(2, 0, 40, 4, dtype="bf16", seed=510)
    _say("conv L=0")
    y, st = run_gpu(c)
    assert y.shape == (2, 0, 40)
    np.testing.assert_array_equal(st, c.state0.astype(np.float64))
    y, st = run_gpu(c, state=False)
    np.testing.assert_array_equal(st, 0.0)


def test_conv_full_size_whole(oracle_mod):
    """The width-4 convolution of the 2.8B-shaped prefill (B=8, L=4096,
    D=5120, bf16), in the bench's launch configuration: every y and every new
    state entry against the oracle."""
    c = gen.make_workload("conv_mamba2p8b_bf16")
    _say("conv_mamba2p8b_bf16 full size, whole tensors")
    y, st = run_gpu(c)
    ry, rs = oracle_mod.conv1d(c.x.f32, c.w, c.bias, c.state0, act=True)
    assert_close(y, ry, "bf16", "y")
    np.testing.assert_array_equal(st, rs)


def test_conv_split_sequence_bitwise():
    """Two calls with the state carried equal one call, bit for bit."""
    import mamba_selective_scan_ssm_amd as ssm
    c = gen.make_conv(2, 300, 520, 4, dtype="bf16", seed=511)
    _say("conv split sequence")
    x, w, b, s0 = to_dev(c.x), to_dev(c.w), to_dev(c.bias), to_dev(c.state0)
    y, st = ssm.conv1d_fwd(x, w, b, s0)
    y1, s1 = ssm.conv1d_fwd(x[:, :77].contiguous(), w, b, s0)
    y2, s2 = ssm.conv1d_fwd(x[:, 77:].contiguous(), w, b, s1)
    assert torch.equal(torch.cat([y1, y2], 1), y) and torch.equal(s2, st)


@pytest.mark.parametrize("dtype,D", [("f32", 600), ("bf16", 0), ("f32", 602), ("bf16", 302)])
def test_conv_decode_matches_oracle_and_prefill(oracle_mod, dtype, D):
    """Single-token steps (128 at 256 x 5120 bf16 -- D = 0 here -- fewer at
    the other sizes; D not a multiple of 4 takes the one-channel-per-thread
    kernel) against the oracle's convolution over the same tokens, and
    bitwise against the GPU prefill of the whole sequence."""
    import mamba_selective_scan_ssm_amd as ssm
    if D == 0:
        d = gen.make_workload("conv_decode_256x5120_bf16")
    else:
        d = gen.make_conv_decode(16, D, 4, 40, dtype=dtype, seed=512 + D)
    _say("conv decode", dtype, d.S, d.D, d.steps)
    state = to_dev(d.state0)
    w, b = to_dev(d.w), to_dev(d.bias)
    xs = to_dev(d.x)
    ys = [ssm.conv1d_update(state, xs[t], w, b) for t in range(d.steps)]
    torch.cuda.synchronize()
    y_dec = torch.stack(ys, 1)                     # (S, steps, D)
    x_seq = xs.transpose(0, 1).contiguous()        # (S, steps, D)
    y_pre, s_pre = ssm.conv1d_fwd(x_seq, w, b, to_dev(d.state0))
    assert torch.equal(y_dec, y_pre) and torch.equal(state, s_pre)
    S = d.S if D else 8                            # oracle on a subset of sequences
    ry, rs = oracle_mod.conv1d(d.x.f32.transpose(1, 0, 2)[:S], d.w, d.bias, d.state0[:S], act=True)
    assert_close(to_np(y_dec[:S]), ry, dtype, "y")
    np.testing.assert_array_equal(to_np(state[:S]), rs)


def test_conv_rejects_bad_arguments():
    import mamba_selective_scan_ssm_amd as ssm
    c = gen.make_conv(1, 16, 64, 4, dtype="f32", seed=513)
    x = to_dev(c.x)
    with pytest.raises(ssm.SSMError):
        ssm.conv1d_fwd(x, to_dev(c.w), None, None, y=x)      # y on x
    with pytest.raises(ValueError):
        ssm.conv1d_fwd(torch.randn(1, 16, 128, device="cuda")[..., :64], to_dev(c.w))


def test_conv_max_plane_size(oracle_mod):
    """One sequence whose (L, D) planes are just under the 2 GiB the boundary
    accepts (L = 209600, D = 5120, bf16), against the oracle on sampled
    channels over the whole sequence (the last channel's last token sits at
    the largest offset); the new state of those channels too.  x is drawn on
    the GPU (seeded); w, bias and the state come from the input generator."""
    import mamba_selective_scan_ssm_amd as ssm
    L, D, K = 209600, 5120, 4
    assert (L + 64) * D * 2 < 2 ** 31
    c = gen.make_conv(1, 1, D, K, dtype="bf16", seed=482)
    _say("conv max plane size", L, D, K)
    g = torch.Generator(device="cuda").manual_seed(483)
    x = torch.randn((1, L, D), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    sel = [0, 1, 255, 256, 3000, 5119]
    idx = torch.tensor(sel, device="cuda")
    ry, rs = oracle_mod.conv1d(x.index_select(2, idx).float().cpu().numpy(), c.w[sel], c.bias[sel],
                               c.state0[:, sel], act=True)
    y, st = ssm.conv1d_fwd(x, to_dev(c.w), to_dev(c.bias), to_dev(c.state0), activation="silu")
    torch.cuda.synchronize()
    assert_close(to_np(y.index_select(2, idx)), ry, "bf16", "y")
    assert_close(to_np(st[:, idx]), rs, "bf16", "state")
