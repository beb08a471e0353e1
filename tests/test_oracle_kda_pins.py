"""Pins for the per-key-gate (KDA) part of the CPU oracle (runs without a GPU).

SGLang PR #28451 (Modifications, item 7) describes KDA as the GDN delta rule
with the decay taken per key channel: S' = S Diag(a) + d k^T, a = exp(g) over
the dk channels; the ring keeps one g per channel, the replay's decay products
run channel by channel and fold onto the stored keys, and the token's own
decay folds into q and k. Each test below checks O6 / O7 and the per-key
ReplayModel against something that does not reuse their code: exact rational
arithmetic, explicitly composed transition matrices, the scalar-gate oracle
(already pinned on its own) for channel-constant gates, closed forms for
special keys and gates, and an exact-rounding model of the fold.
"""
import math
from fractions import Fraction as Fr

import numpy as np
import pytest

from oracle import (ReplayModel, fold_f32, fold_kda_f32, gdn_step, kda_step, rel_err,
                    window_ref)
from test_oracle_pins import PYTH, rn32, unit_rows


def kda_problem(rng, B=2, N=3, Hv=4, Hk=2, dk=6, dv=5, steps=7):
    S0 = 0.1 * rng.standard_normal((N, Hv, dv, dk))
    slot = rng.permutation(N)[:B].astype(np.int32)
    toks = []
    for _ in range(steps):
        q = unit_rows(rng.standard_normal((B, Hk, dk))) * dk ** -0.5
        k = unit_rows(rng.standard_normal((B, Hk, dk)))
        v = rng.standard_normal((B, Hv, dv))
        g = -np.logaddexp(0.0, -rng.normal(2.0, 1.0, (B, Hv, dk)))
        beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, Hv))))
        toks.append((q, k, v, g, beta))
    return S0, slot, toks


# ----------------------------------------------------------------- exact rationals

def exact_kda_sequence(S0, toks):
    """Exact rational run of the per-key-gate delta rule with explicit loops.
    toks: (a [dk], beta, k, v, q). Column j of the state decays by a[j]."""
    dv, dk = len(S0), len(S0[0])
    S = [row[:] for row in S0]
    states, ys, us = [], [], []
    for a, b, k, v, q in toks:
        St = [[a[j] * S[i][j] for j in range(dk)] for i in range(dv)]
        u = [b * (v[i] - sum(St[i][j] * k[j] for j in range(dk))) for i in range(dv)]
        S = [[St[i][j] + u[i] * k[j] for j in range(dk)] for i in range(dv)]
        ys.append([sum(S[i][j] * q[j] for j in range(dk)) for i in range(dv)])
        us.append(u)
        states.append([row[:] for row in S])
    return states, ys, us


def exact_kda_closed_form(S_c, alphas, us, ks):
    """Per channel j: P[j] = prod_i a_i[j], w_t[j] = prod_{i>t} a_i[j],
    S = S_c Diag(P) + sum_t u_t (w_t o k_t)^T, in exact rationals."""
    dv, dk = len(S_c), len(S_c[0])
    h = len(alphas)
    S = []
    for i in range(dv):
        row = []
        for j in range(dk):
            P = Fr(1)
            for a in alphas:
                P *= a[j]
            x = P * S_c[i][j]
            for t in range(h):
                w = Fr(1)
                for r in range(t + 1, h):
                    w *= alphas[r][j]
                x += us[t][i] * w * ks[t][j]
            row.append(x)
        S.append(row)
    return S


def _rational_kda_case(seed, h=6, dv=2, dk=2):
    r = np.random.default_rng(seed)
    S0 = [[Fr(int(r.integers(-9, 10)), 10) for _ in range(dk)] for _ in range(dv)]
    toks = []
    for _ in range(h):
        a = [Fr(int(r.integers(3, 10)), 10) for _ in range(dk)]   # per channel
        b = Fr(int(r.integers(1, 10)), 10)
        c, s = PYTH[int(r.integers(len(PYTH)))]
        k = [c, s] if r.integers(2) else [-s, c]
        c2, s2 = PYTH[int(r.integers(len(PYTH)))]
        q = [c2 / 4, s2 / 4]
        v = [Fr(int(r.integers(-20, 21)), 8) for _ in range(dv)]
        toks.append((a, b, k, v, q))
    return S0, toks


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_kda_closed_form_equals_recurrence_exactly(seed):
    """The per-channel closed form (decay products on the keys) equals the
    per-key recurrence exactly at every h, including h = 0."""
    S0, toks = _rational_kda_case(seed)
    states, _, us = exact_kda_sequence(S0, toks)
    alphas = [t[0] for t in toks]
    ks = [t[2] for t in toks]
    assert exact_kda_closed_form(S0, [], [], []) == S0
    for h in range(1, len(toks) + 1):
        assert exact_kda_closed_form(S0, alphas[:h], us[:h], ks[:h]) == states[h - 1]


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_kda_step_matches_exact_rationals(seed):
    """O6 in fp64 agrees with the exact rational per-key recurrence to ~1e-12
    (state, output and correction), with distinct decays per channel."""
    S0, toks = _rational_kda_case(seed)
    states, ys, us = exact_kda_sequence(S0, toks)
    S = np.array([[float(x) for x in row] for row in S0])[None, None]
    slot = np.array([0], np.int32)
    for t, (a, b, k, v, q) in enumerate(toks):
        qa = np.array([[[float(x) for x in q]]])
        ka = np.array([[[float(x) for x in k]]])
        va = np.array([[[float(x) for x in v]]])
        ga = np.array([[[math.log(x) for x in a]]])
        o, u = kda_step(S, slot, qa, ka, va, ga, np.array([[float(b)]]), want_u=True)
        exact_S = np.array([[float(x) for x in row] for row in states[t]])
        assert np.max(np.abs(S[0, 0] - exact_S)) <= 1e-12 * max(1.0, np.max(np.abs(exact_S)))
        assert np.max(np.abs(o[0, 0] - np.array([float(x) for x in ys[t]]))) <= 1e-12
        assert np.max(np.abs(u[0, 0] - np.array([float(x) for x in us[t]]))) <= 1e-12


# ----------------------------------------------------------------- brute force / special cases

def test_kda_step_matches_transition_matrices():
    """Brute force: S_t = S_{t-1} Diag(a_t) (I - beta k k^T) + beta v k^T,
    composed as explicit matrices, y_t = S_t q_t, for every slot, head and
    GQA mapping h -> h // (Hv/Hk); untouched slots keep their bits."""
    rng = np.random.default_rng(21)
    S0, slot, toks = kda_problem(rng, B=3, N=4, Hv=6, Hk=3, dk=7, dv=5, steps=9)
    S = S0.copy()
    ref = S0.copy()
    for (q, k, v, g, beta) in toks:
        o = kda_step(S, slot, q, k, v, g, beta)
        for b, s in enumerate(slot):
            for h in range(6):
                kk, qq = k[b, h // 2], q[b, h // 2]
                D = np.diag(np.exp(g[b, h]))
                M = D @ (np.eye(7) - beta[b, h] * np.outer(kk, kk))
                ref[s, h] = ref[s, h] @ M + beta[b, h] * np.outer(v[b, h], kk)
                assert np.allclose(o[b, h], ref[s, h] @ qq, rtol=0, atol=1e-12)
    assert np.allclose(S, ref, rtol=0, atol=1e-12)
    for s in range(4):
        if s not in slot:
            assert np.array_equal(S[s], S0[s])


def test_kda_with_channel_constant_gates_is_the_scalar_gate_step_bitwise():
    """With a[c] the same for every channel, O6 is O1 operation for operation:
    identical bits for the state and the output."""
    rng = np.random.default_rng(22)
    S0, slot, toks = kda_problem(rng, B=2, N=3, steps=6)
    S1, S2 = S0.copy(), S0.copy()
    for (q, k, v, g, beta) in toks:
        gh = g[:, :, 0]
        o1 = gdn_step(S1, slot, q, k, v, gh, beta)
        o2 = kda_step(S2, slot, q, k, v, np.repeat(gh[:, :, None], S0.shape[3], axis=2), beta)
        assert np.array_equal(o1, o2)
        assert np.array_equal(S1, S2)


def test_kda_special_cases():
    """Closed forms from the mathematics of the per-key rule:
    - beta = 0: pure per-channel decay, S_t[:, c] = a[c] S[:, c];
    - k = e_m: only column m is written, S_t[:, m] = (1 - beta) a[m] S[:, m]
      + beta v, every other column is only decayed; reading with q = e_n
      returns column n;
    - a channel with a = 1 and a zero key component keeps its column."""
    rng = np.random.default_rng(23)
    dv, dk = 5, 6
    one = np.array([0], np.int32)
    S = rng.standard_normal((1, 1, dv, dk))
    prev = S.copy()
    g = rng.normal(-0.5, 0.3, (1, 1, dk))
    q = rng.standard_normal((1, 1, dk))
    k = unit_rows(rng.standard_normal((1, 1, dk)))
    v = rng.standard_normal((1, 1, dv))
    o = kda_step(S, one, q, k, v, g, np.zeros((1, 1)))
    a = np.exp(g[0, 0])
    for c in range(dk):
        assert np.allclose(S[0, 0][:, c], a[c] * prev[0, 0][:, c], rtol=0, atol=1e-15)
    assert np.allclose(o[0, 0], S[0, 0] @ q[0, 0], rtol=0, atol=1e-14)
    for m in range(dk):
        for n in (m, (m + 2) % dk):
            S = rng.standard_normal((1, 1, dv, dk))
            prev = S.copy()
            bt = 0.3 + 0.1 * m
            em = np.zeros((1, 1, dk))
            em[0, 0, m] = 1.0
            en = np.zeros((1, 1, dk))
            en[0, 0, n] = 1.0
            o = kda_step(S, one, en, em, v, g, np.full((1, 1), bt))
            for c in range(dk):
                want = ((1 - bt) * a[c] * prev[0, 0][:, c] + bt * v[0, 0]) if c == m \
                    else a[c] * prev[0, 0][:, c]
                assert np.allclose(S[0, 0][:, c], want, rtol=0, atol=1e-14)
            assert np.allclose(o[0, 0], S[0, 0][:, n], rtol=0, atol=1e-14)
    S = rng.standard_normal((1, 1, dv, dk))
    prev = S.copy()
    g2 = g.copy()
    g2[0, 0, 3] = 0.0
    k2 = k.copy()
    k2[0, 0, 3] = 0.0
    kda_step(S, one, q, k2, v, g2, np.full((1, 1), 0.7))
    assert np.array_equal(S[0, 0][:, 3], prev[0, 0][:, 3])


def test_kda_padding_rows_output_zero_and_touch_nothing():
    rng = np.random.default_rng(24)
    S0, _, toks = kda_problem(rng, B=3, N=3, steps=1)
    slot = np.array([2, -1, 0], np.int32)
    S = S0.copy()
    o = kda_step(S, slot, *toks[0])
    assert np.all(o[1] == 0.0)
    assert np.array_equal(S[1], S0[1])


# ----------------------------------------------------------------- O2 with a per-key gate

@pytest.mark.parametrize("L", [1, 2, 4, 5])
def test_kda_replay_model_matches_recurrence(L):
    """The per-key checkpoint + ring machine (closed form with the decay on
    the keys, readout with the decay on q and k) reproduces O6's outputs at
    every step and O6's state after every flush, with natural and forced
    flushes and a padding row. At L = 1 every step flushes."""
    rng = np.random.default_rng(200 + L)
    S0, _, toks = kda_problem(rng, B=3, N=4, steps=13)
    slot = np.array([3, -1, 1], np.int32)
    S = S0.copy()
    model = ReplayModel(S0, Hk=2, L=L, gate="key")
    assert model.ring_g.shape == (4, 4, L, 6)
    for t, (q, k, v, g, beta) in enumerate(toks):
        ff = np.array([t == 3, 0, t == 5], dtype=np.uint8)
        o_ref = kda_step(S, slot, q, k, v, g, beta)
        o, flush = model.decode(slot, q, k, v, g, beta, ff)
        assert rel_err(o, o_ref) <= 1e-12
        for b, s in enumerate(slot):
            if s >= 0 and flush[b]:
                assert rel_err(model.ckpt[s], S[s]) <= 1e-12
        model.advance(slot, flush)
        for s in slot[slot >= 0]:
            assert rel_err(model.state(s), S[s]) <= 1e-12
        if L == 1:
            assert np.all(flush[slot >= 0])


def test_kda_window_matches_closed_form_route_and_commit_fold():
    """A per-key verify window: the closed-form route equals the token-by-token
    reference (O4 over O6); commit + fold lands on the true state advanced by
    the accepted tokens."""
    rng = np.random.default_rng(31)
    B, T, Hk, Hv, dk, dv = 3, 4, 2, 4, 6, 5
    S0 = 0.1 * rng.standard_normal((3, Hv, dv, dk))
    slot = np.array([2, 0, 1], np.int32)
    q = unit_rows(rng.standard_normal((B, T, Hk, dk))) * dk ** -0.5
    k = unit_rows(rng.standard_normal((B, T, Hk, dk)))
    v = rng.standard_normal((B, T, Hv, dv))
    g = -np.logaddexp(0.0, -rng.normal(2.0, 1.0, (B, T, Hv, dk)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, Hv))))
    o_ref = window_ref(S0, slot, q, k, v, g, beta)
    m = ReplayModel(S0, Hk=Hk, L=8, gate="key")
    o = m.verify(slot, q, k, v, g, beta)
    assert rel_err(o, o_ref) <= 1e-12
    acc = np.array([0, 2, 4], np.int32)
    m.commit(slot, acc)
    S_true = S0.copy()
    for b, s in enumerate(slot):
        for t in range(acc[b]):
            kda_step(S_true, np.array([s], np.int32), q[b:b + 1, t], k[b:b + 1, t],
                     v[b:b + 1, t], g[b:b + 1, t], beta[b:b + 1, t])
    m.fold(slot)
    for s in slot:
        assert rel_err(m.ckpt[s], S_true[s]) <= 1e-12


# ----------------------------------------------------------------- O7

def _exact_fold_element_kda(x, ds, ks, gs):
    for d, k, g in zip(ds, ks, gs):
        a = rn32(Fr(math.exp(float(g))))
        t = rn32(Fr(a) * Fr(float(x)))
        x = rn32(Fr(float(d)) * Fr(float(k)) + Fr(t))
    return x


def _kda_ring(rng, N, Hv, Hk, dv, dk, L, f16=True):
    rd = rng.standard_normal((N, Hv, L, dv)).astype(np.float32)
    rk = unit_rows(rng.standard_normal((N, Hk, L, dk))).astype(np.float32)
    if f16:
        rd, rk = (x.astype(np.float16).astype(np.float32) for x in (rd, rk))
    rg = (-np.logaddexp(0.0, -rng.normal(2.0, 1.0, (N, Hv, L, dk)))).astype(np.float32)
    return rd, rk, rg


def test_kda_fold_matches_exact_rounding_model():
    """O7 bitwise equals an exact-rational model of t = RN(a x),
    x = RN(d k + t), a = RN(exp(g[c])), with the channel's own decay."""
    rng = np.random.default_rng(33)
    N, Hv, Hk, dv, dk, L = 2, 2, 1, 3, 4, 5
    ckpt = (0.1 * rng.standard_normal((N, Hv, dv, dk))).astype(np.float32)
    rd, rk, rg = _kda_ring(rng, N, Hv, Hk, dv, dk, L)
    wp = np.array([5, 3], np.int32)
    out, wpo = ckpt.copy(), wp.copy()
    fold_kda_f32(out, np.array([0, 1], np.int32), wpo, rd, rk, rg)
    assert np.all(wpo == 0)
    for s in range(N):
        p = wp[s]
        for h in range(Hv):
            for i in range(dv):
                for c in range(dk):
                    ref = _exact_fold_element_kda(ckpt[s, h, i, c], rd[s, h, :p, i],
                                                  rk[s, 0, :p, c], rg[s, h, :p, c])
                    assert np.float32(ref).tobytes() == out[s, h, i, c].tobytes()


def test_kda_fold_with_channel_constant_gates_is_the_scalar_fold_bitwise():
    rng = np.random.default_rng(34)
    N, Hv, Hk, dv, dk, L = 3, 4, 2, 8, 16, 6
    ckpt = (0.1 * rng.standard_normal((N, Hv, dv, dk))).astype(np.float32)
    rd, rk, rg = _kda_ring(rng, N, Hv, Hk, dv, dk, L)
    rg_head = np.ascontiguousarray(rg[..., 0])
    rg_key = np.ascontiguousarray(np.repeat(rg_head[..., None], dk, axis=3))
    wp = np.array([6, 2, 0], np.int32)
    slot = np.array([1, 0, 2], np.int32)
    a, b = ckpt.copy(), ckpt.copy()
    fold_f32(a, slot, wp.copy(), rd, rk, rg_head)
    fold_kda_f32(b, slot, wp.copy(), rd, rk, rg_key)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_kda_fold_agrees_with_fp64_model_and_edge_cases():
    rng = np.random.default_rng(35)
    N, Hv, Hk, dv, dk, L = 3, 2, 1, 8, 8, 4
    S0 = (0.1 * rng.standard_normal((N, Hv, dv, dk))).astype(np.float32)
    rd, rk, rg = _kda_ring(rng, N, Hv, Hk, dv, dk, L, f16=False)
    wp = np.array([4, 0, 2], np.int32)
    slot = np.array([0, 1, -1, 2], np.int32)
    out, wpo = S0.copy(), wp.copy()
    fold_kda_f32(out, slot, wpo, rd, rk, rg)
    m = ReplayModel(S0.astype(np.float64), Hk=Hk, L=L, gate="key")
    m.ring_u[:], m.ring_k[:], m.ring_g[:] = rd, rk, rg
    m.write_pos[:] = wp
    m.fold(slot)
    assert rel_err(out, m.ckpt) < 1e-5
    assert np.array_equal(out[1], S0[1])
    assert np.all(wpo == 0)
