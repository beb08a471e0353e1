"""Pins for O8, the decode's front end (q/k L2-normalisation, q scaling).

SGLang PR #28451 (Modifications) hands the decode q already L2-normalised and
scaled; the fused front end does that in the kernel. The oracle's O8 is checked
against closed forms that do not reuse its code: a Pythagorean vector whose
norm is exact, the norm and direction of the result computed with math.hypot
and cross products, invariance under positive scaling, the zero vector, and
the agreement of O8-then-O1 with O1 on inputs normalised by hand.
"""
import math

import numpy as np
import pytest

from oracle import QK_NORM_EPS, gdn_step, l2norm_qk, rel_err


def test_pythagorean_vector():
    """[3, 4, 0, 0] has norm 5: k = [3, 4, 0, 0] / sqrt(25 + eps) and q the
    same times 4^-1/2 = 1/2."""
    x = np.array([[3.0, 4.0, 0.0, 0.0]])
    q, k = l2norm_qk(x, x)
    f = 1.0 / math.sqrt(25.0 + 1e-6)
    assert np.allclose(k[0], [3 * f, 4 * f, 0, 0], rtol=0, atol=1e-15)
    assert np.allclose(q[0], [1.5 * f, 2 * f, 0, 0], rtol=0, atol=1e-15)


@pytest.mark.parametrize("dk", [32, 64, 128, 256])
def test_norm_direction_and_scale(dk):
    rng = np.random.default_rng(dk)
    x = rng.standard_normal((5, 3, dk)) * rng.uniform(0.1, 10.0, (5, 3, 1))
    q, k = l2norm_qk(x, x)
    for i in range(5):
        for h in range(3):
            r = math.hypot(*x[i, h])
            want = r / math.sqrt(r * r + 1e-6)
            assert abs(math.hypot(*k[i, h]) - want) <= 1e-14
            assert abs(math.hypot(*q[i, h]) - want / math.sqrt(dk)) <= 1e-14
            # parallel to the input, same orientation
            c = np.outer(k[i, h], x[i, h])
            assert np.allclose(c, c.T, rtol=0, atol=1e-12)
            assert float(k[i, h] @ x[i, h]) > 0


def test_scaling_invariance_and_zero_vector():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 2, 16))
    q1, k1 = l2norm_qk(x, x)
    q2, k2 = l2norm_qk(1e3 * x, 7.5e2 * x)
    assert np.allclose(k1, k2, rtol=1e-6, atol=0)
    assert np.allclose(q1, q2, rtol=1e-6, atol=0)
    z = np.zeros((1, 1, 8))
    qz, kz = l2norm_qk(z, z)
    assert np.all(qz == 0) and np.all(kz == 0) and QK_NORM_EPS == 1e-6


def test_front_end_then_step_equals_step_on_normalised_inputs():
    """O8 composed with O1 equals O1 fed with q/|q|/sqrt(dk), k/|k| computed
    by hand (eps only moves the result by about eps/|x|^2)."""
    rng = np.random.default_rng(9)
    B, N, Hv, Hk, dk, dv = 2, 2, 4, 2, 16, 8
    S = 0.1 * rng.standard_normal((N, Hv, dv, dk))
    slot = np.array([1, 0], np.int32)
    q = rng.standard_normal((B, Hk, dk))
    k = rng.standard_normal((B, Hk, dk))
    v = rng.standard_normal((B, Hv, dv))
    g = -np.logaddexp(0.0, -rng.normal(2.0, 1.0, (B, Hv)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, Hv))))
    qn, kn = l2norm_qk(q, k)
    qh = q / np.linalg.norm(q, axis=-1, keepdims=True) / math.sqrt(dk)
    kh = k / np.linalg.norm(k, axis=-1, keepdims=True)
    S1, S2 = S.copy(), S.copy()
    o1 = gdn_step(S1, slot, qn, kn, v, g, beta)
    o2 = gdn_step(S2, slot, qh, kh, v, g, beta)
    assert rel_err(o1, o2) < 1e-7 and rel_err(S1, S2) < 1e-7
