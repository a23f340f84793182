"""Pins of the CPU oracle's short causal convolution (-m "not gpu").

The oracle's conv1d is checked against things other than itself: numpy's
convolve on the padded window, special kernels whose output is a plain copy
or shift of the input, the hand-worked example in tests/golden, SciPy's
logistic for the SiLU, the carried state across split sequences, and the
decode step chained over a sequence.
"""

import os

import numpy as np
import pytest
import scipy.special

import ssm_inputs as gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            vals[k.strip()] = np.array([float(t) for t in v.split()])
    return vals


def test_hand_example(oracle_mod):
    g = _golden("conv_hand_example.txt")
    x = g["x"].reshape(1, 2, 1).astype(np.float32)
    w = g["w"].reshape(1, 3).astype(np.float32)
    st = g["state"].reshape(1, 1, 2).astype(np.float32)
    b = g["bias"].astype(np.float32)
    y, s = oracle_mod.conv1d(x, w, b, st)
    np.testing.assert_allclose(y.ravel(), g["y"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(s.ravel(), g["state_out"], rtol=0, atol=0)
    ya, _ = oracle_mod.conv1d(x, w, b, st, act=True)
    np.testing.assert_allclose(ya.ravel(), g["y"] * scipy.special.expit(g["y"]), rtol=1e-14)


@pytest.mark.parametrize("K", [2, 3, 4])
@pytest.mark.parametrize("with_state", [False, True])
def test_matches_numpy_convolve(oracle_mod, K, with_state):
    c = gen.make_conv(2, 37, 11, K, dtype="f32", seed=10 + K, bias=False, state=with_state)
    y, st = oracle_mod.conv1d(c.x.f32, c.w, None, c.state0)
    for b in range(c.B):
        for d in range(c.D):
            head = c.state0[b, d].astype(np.float64) if with_state else np.zeros(K - 1)
            xp = np.concatenate([head, c.x.f32[b, :, d].astype(np.float64)])
            ref = np.convolve(xp, c.w[d, ::-1].astype(np.float64), mode="valid")
            np.testing.assert_allclose(y[b, :, d], ref, rtol=1e-12, atol=1e-12)
            np.testing.assert_array_equal(st[b, d], xp[-(K - 1):])


def test_identity_and_shift_kernels(oracle_mod):
    c = gen.make_conv(2, 20, 6, 4, dtype="f32", seed=21)
    K = c.K
    eye_last = np.zeros((c.D, K), np.float32)
    eye_last[:, K - 1] = 1.0
    y, _ = oracle_mod.conv1d(c.x.f32, eye_last, c.bias, c.state0)
    np.testing.assert_allclose(y, c.x.f32 + c.bias[None, None, :].astype(np.float64), rtol=0, atol=1e-15)
    eye_first = np.zeros((c.D, K), np.float32)
    eye_first[:, 0] = 1.0
    y, _ = oracle_mod.conv1d(c.x.f32, eye_first, None, c.state0)
    # y_t = xp[t]: the state for t < K-1, then x shifted by K-1 tokens
    np.testing.assert_array_equal(y[:, : K - 1, :], c.state0.transpose(0, 2, 1).astype(np.float64))
    np.testing.assert_array_equal(y[:, K - 1:, :], c.x.f32[:, : c.L - (K - 1), :].astype(np.float64))


def test_silu_matches_expit(oracle_mod):
    c = gen.make_conv(1, 25, 9, 4, dtype="f32", seed=22)
    y, _ = oracle_mod.conv1d(c.x.f32, c.w, c.bias, c.state0)
    ya, _ = oracle_mod.conv1d(c.x.f32, c.w, c.bias, c.state0, act=True)
    np.testing.assert_allclose(ya, y * scipy.special.expit(y), rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("L1", [1, 2, 3, 10])
def test_split_sequence_bitwise(oracle_mod, L1):
    c = gen.make_conv(2, 17, 5, 4, dtype="f32", seed=23)
    y, st = oracle_mod.conv1d(c.x.f32, c.w, c.bias, c.state0, act=True)
    y1, s1 = oracle_mod.conv1d(c.x.f32[:, :L1], c.w, c.bias, c.state0, act=True)
    y2, s2 = oracle_mod.conv1d(c.x.f32[:, L1:], c.w, c.bias, s1.astype(np.float32), act=True)
    # the carried state is made of input values, so it is exact in fp32
    np.testing.assert_array_equal(np.concatenate([y1, y2], axis=1), y)
    np.testing.assert_array_equal(s2, st)


def test_short_sequence_state_mixes_old_and_new(oracle_mod):
    c = gen.make_conv(1, 2, 3, 4, dtype="f32", seed=24)
    _, st = oracle_mod.conv1d(c.x.f32, c.w, None, c.state0)
    # L = 2 < K - 1 = 3: the new state keeps the newest old entry then both inputs
    exp = np.concatenate([c.state0[0, :, 2:], c.x.f32[0].T], axis=1).astype(np.float64)
    np.testing.assert_array_equal(st[0], exp)


def test_empty_sequence(oracle_mod):
    c = gen.make_conv(2, 0, 3, 4, dtype="f32", seed=25)
    y, st = oracle_mod.conv1d(c.x.f32, c.w, c.bias, c.state0)
    assert y.shape == (2, 0, 3)
    np.testing.assert_array_equal(st, c.state0.astype(np.float64))


def test_decode_chain_equals_prefill(oracle_mod):
    d = gen.make_conv_decode(3, 7, 4, 12, dtype="f32", seed=26)
    state = d.state0.astype(np.float64).copy()
    ys = [oracle_mod.conv1d_update(state, d.x.f32[t], d.w, d.bias, act=True) for t in range(d.steps)]
    x_seq = d.x.f32.transpose(1, 0, 2)               # (S, steps, D)
    y, st = oracle_mod.conv1d(x_seq, d.w, d.bias, d.state0, act=True)
    np.testing.assert_array_equal(np.stack(ys, axis=1), y)
    np.testing.assert_array_equal(state, st)
