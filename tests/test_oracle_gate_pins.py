"""Pins for O10, the gate activations in front of a per-key-gate decode.

SGLang PR #36821 (Technical principle) forms the per-channel log-decay as
g = l * sigma(e^A (a + b_dt)) and the delta-rule strength as beta = sigma(b).
O10 is checked against references that do not reuse its code: sigma(0) = 1/2,
the logistic written through tanh, sigma(x) + sigma(-x) = 1, the limits of g
(l and 0), a shift between a and dt_bias, e^A = 2 for A = log 2, and a
per-element loop over heads and channels.
"""
import math

import numpy as np

from oracle import kda_gates


def logistic(x):
    return 0.5 * (1.0 + math.tanh(0.5 * x))


def test_zero_argument_gives_half_the_bound():
    B, T, Hv, dk = 2, 1, 3, 8
    rng = np.random.default_rng(1)
    dt = rng.standard_normal((Hv, dk))
    a = np.broadcast_to(-dt, (B, T, Hv, dk))
    g, beta = kda_gates(a, np.zeros((B, T, Hv)), rng.standard_normal(Hv), dt, -5.0)
    assert np.all(g == -2.5) and np.all(beta == 0.5)


def test_per_element_loop_with_tanh_logistic():
    rng = np.random.default_rng(2)
    B, T, Hv, dk, lb = 2, 3, 4, 8, -5.0
    a = rng.standard_normal((B, T, Hv, dk)) * 2
    b = rng.standard_normal((B, T, Hv)) * 3
    A = rng.normal(-0.5, 1.0, Hv)
    dt = rng.standard_normal((Hv, dk))
    g, beta = kda_gates(a, b, A, dt, lb)
    for i in range(B):
        for t in range(T):
            for h in range(Hv):
                assert abs(beta[i, t, h] - logistic(b[i, t, h])) <= 1e-15
                for c in range(dk):
                    want = lb * logistic(math.exp(A[h]) * (a[i, t, h, c] + dt[h, c]))
                    assert abs(g[i, t, h, c] - want) <= 1e-14


def test_symmetry_limits_shift_and_scale():
    Hv, dk = 2, 4
    x = np.linspace(-6, 6, Hv * dk).reshape(1, 1, Hv, dk)
    zeros = np.zeros((Hv, dk))
    g_p, b_p = kda_gates(x, x[..., 0], np.zeros(Hv), zeros, -1.0)
    g_n, b_n = kda_gates(-x, -x[..., 0], np.zeros(Hv), zeros, -1.0)
    assert np.allclose(g_p + g_n, -1.0, rtol=0, atol=1e-15)      # sigma(x) + sigma(-x) = 1
    assert np.allclose(b_p + b_n, 1.0, rtol=0, atol=1e-15)
    big = np.full((1, 1, Hv, dk), 50.0)
    g_hi, _ = kda_gates(big, np.zeros((1, 1, Hv)), np.zeros(Hv), zeros, -5.0)
    g_lo, _ = kda_gates(-big, np.zeros((1, 1, Hv)), np.zeros(Hv), zeros, -5.0)
    assert np.allclose(g_hi, -5.0, atol=1e-15) and np.all(np.abs(g_lo) < 1e-20)
    # a and dt_bias enter only through their sum
    rng = np.random.default_rng(3)
    a = rng.standard_normal((1, 2, Hv, dk))
    dt = rng.standard_normal((Hv, dk))
    g1, _ = kda_gates(a, np.zeros((1, 2, Hv)), np.zeros(Hv), dt, -3.0)
    g2, _ = kda_gates(a + 0.25, np.zeros((1, 2, Hv)), np.zeros(Hv), dt - 0.25, -3.0)
    assert np.allclose(g1, g2, rtol=1e-15, atol=1e-15)
    # A = log 2 doubles the argument
    g3, _ = kda_gates(a, np.zeros((1, 2, Hv)), np.full(Hv, math.log(2.0)), dt, -3.0)
    g4, _ = kda_gates(2 * a, np.zeros((1, 2, Hv)), np.zeros(Hv), 2 * dt, -3.0)
    assert np.allclose(g3, g4, rtol=1e-14, atol=1e-15)
    # more positive a moves g towards the bound (g < 0, decreasing)
    assert np.all(np.diff(g_p.reshape(-1)) < 0)
