"""Pins for O9, the causal convolution step in front of the decode.

ReplaySSM blog (section 3.1) has the decode path update the causal
convolution first; SGLang PR #36821 (Technical principle) writes the step as
x_hat_t = SiLU(w * x_{t-3:t}). O9 is checked against references that do not
reuse its code: numpy's full convolution of the whole input sequence (which
fixes the tap order and the window shift), single-tap filters that reduce to
SiLU of the input or of the input W-1 steps back, the SiLU identity
SiLU(x) - SiLU(-x) = x and its known values, and the padding rules.
"""
import math

import numpy as np
import pytest

from oracle import conv_update


def silu(x):
    return x / (1.0 + np.exp(-x))


@pytest.mark.parametrize("W", [2, 3, 4])
def test_sequence_equals_numpy_convolution(W):
    """T steps from a zero window equal SiLU of the causal convolution of the
    whole sequence: np.convolve(x[:, c], w[c, ::-1])[t] = sum_i w[c, i] x[t-W+1+i]."""
    rng = np.random.default_rng(W)
    T, C, N = 9, 12, 3
    xs = rng.standard_normal((T, C))
    w = rng.standard_normal((C, W))
    state = np.zeros((N, W - 1, C))
    slot = np.array([2])
    for t in range(T):
        y = conv_update(xs[t][None, :], w, state, slot)
        for c in range(C):
            ref = np.convolve(xs[:, c], w[c, ::-1])[t]
            assert abs(y[0, c] - ref / (1 + math.exp(-ref))) <= 1e-12 * (1 + abs(ref))
    # the window then holds the last W-1 inputs, oldest first
    assert np.array_equal(state[2], xs[T - W + 1:])
    assert np.all(state[:2] == 0)


def test_single_tap_filters():
    rng = np.random.default_rng(5)
    T, C, W = 7, 8, 4
    xs = rng.standard_normal((T, C))
    for tap, delay in ((W - 1, 0), (0, W - 1), (1, W - 2)):
        w = np.zeros((C, W))
        w[:, tap] = 1.0
        state = np.zeros((1, W - 1, C))
        for t in range(T):
            y = conv_update(xs[t][None, :], w, state, np.array([0]))
            want = silu(xs[t - delay]) if t >= delay else np.zeros(C)
            assert np.allclose(y[0], want, rtol=0, atol=1e-15)


def test_silu_identity_and_values():
    """SiLU(x) - SiLU(-x) = x; SiLU(0) = 0; SiLU(1) = 1/(1 + e^-1)."""
    C = 5
    x = np.array([[0.0, 1.0, -2.5, 30.0, -30.0]])
    w = np.zeros((C, 2))
    w[:, 1] = 1.0
    yp = conv_update(x, w, np.zeros((1, 1, C)), np.array([0]))
    yn = conv_update(-x, w, np.zeros((1, 1, C)), np.array([0]))
    assert np.allclose(yp - yn, x, rtol=0, atol=1e-14)
    assert yp[0, 0] == 0.0
    assert abs(yp[0, 1] - 1.0 / (1.0 + math.exp(-1.0))) <= 1e-16
    assert abs(yp[0, 3] - 30.0) < 1e-11 and abs(yp[0, 4]) < 1e-11


def test_padding_rows_and_slot_mapping():
    rng = np.random.default_rng(8)
    B, N, C, W = 4, 5, 8, 3
    x = rng.standard_normal((B, C))
    w = rng.standard_normal((C, W))
    state = rng.standard_normal((N, W - 1, C))
    before = state.copy()
    slot = np.array([3, -1, 0, 7])           # a padding row and a slot past the pool
    y = conv_update(x, w, state, slot)
    assert np.all(y[1] == 0) and np.all(y[3] == 0)
    for s in (1, 2, 4):
        assert np.array_equal(state[s], before[s])
    # rows 0 and 2 moved their windows by one input
    assert np.array_equal(state[3][:-1], before[3][1:]) and np.array_equal(state[3][-1], x[0])
    assert np.array_equal(state[0][:-1], before[0][1:]) and np.array_equal(state[0][-1], x[2])
    acc = sum(w[:, i] * np.concatenate([before[3], x[0][None]])[i] for i in range(W))
    assert np.allclose(y[0], silu(acc), rtol=0, atol=1e-14)
