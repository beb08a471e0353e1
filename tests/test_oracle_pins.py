"""Pins for the CPU oracle (runs without a GPU).

Each test checks the oracle against something that does not reuse its code:
the worked flush table printed on the ReplaySSM blog, exact rational
arithmetic, brute-force products of the transition matrices, closed-form
special cases, an exact-rounding re-implementation of the fold, and the
mathematical invariants the pages state (closed-form replay, output-only
readout, L = 1 degeneracy, causality of the verify window).
"""
import json
import math
import os
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle
from oracle import ReplayModel, fold_f32, gdn_step, next_cursor, rel_err, window_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


# ----------------------------------------------------------------- helpers

def unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def random_problem(rng, B=2, N=3, Hv=4, Hk=2, dk=6, dv=5, steps=7):
    S0 = 0.1 * rng.standard_normal((N, Hv, dv, dk))
    slot = rng.permutation(N)[:B].astype(np.int32)
    toks = []
    for _ in range(steps):
        q = unit_rows(rng.standard_normal((B, Hk, dk))) * dk ** -0.5
        k = unit_rows(rng.standard_normal((B, Hk, dk)))
        v = rng.standard_normal((B, Hv, dv))
        g = -np.logaddexp(0.0, -rng.normal(2.0, 1.0, (B, Hv)))
        beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, Hv))))
        toks.append((q, k, v, g, beta))
    return S0, slot, toks


PYTH = [(Fr(3, 5), Fr(4, 5)), (Fr(5, 13), Fr(12, 13)), (Fr(8, 17), Fr(15, 17)),
        (Fr(7, 25), Fr(24, 25)), (Fr(20, 29), Fr(21, 29)), (Fr(-4, 5), Fr(3, 5))]


def exact_sequence(S0, toks):
    """Exact rational run of the delta rule, written with explicit loops.
    toks: list of (alpha, beta, k, v, q). Returns the states after every token,
    the outputs y_t = S_t q_t and the corrections u_t."""
    dv, dk = len(S0), len(S0[0])
    S = [row[:] for row in S0]
    states, ys, us = [], [], []
    for a, b, k, v, q in toks:
        St = [[a * S[i][j] for j in range(dk)] for i in range(dv)]
        u = [b * (v[i] - sum(St[i][j] * k[j] for j in range(dk))) for i in range(dv)]
        S = [[St[i][j] + u[i] * k[j] for j in range(dk)] for i in range(dv)]
        ys.append([sum(S[i][j] * q[j] for j in range(dk)) for i in range(dv)])
        us.append(u)
        states.append([row[:] for row in S])
    return states, ys, us


def exact_closed_form(S_c, alphas, us, ks):
    """S_{c+h} = P_h S_c + sum_j w_{j,h} u_j k_j^T with exact rationals."""
    dv, dk = len(S_c), len(S_c[0])
    h = len(alphas)
    P = Fr(1)
    for a in alphas:
        P *= a
    S = [[P * S_c[i][j] for j in range(dk)] for i in range(dv)]
    for jj in range(h):
        w = Fr(1)
        for i in range(jj + 1, h):
            w *= alphas[i]
        for i in range(dv):
            for j in range(dk):
                S[i][j] += w * us[jj][i] * ks[jj][j]
    return S


def rn32(x: Fr) -> float:
    """Exact round-to-nearest-even of a rational to IEEE binary32 (with
    subnormals), returned as a Python float holding that binary32 value."""
    if x == 0:
        return 0.0
    neg = x < 0
    a = -x if neg else x
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fr(2) ** e > a:
        e -= 1
    elif Fr(2) ** (e + 1) <= a:
        e += 1
    qe = max(e - 23, -149)
    scaled = a / (Fr(2) ** qe)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fr(1, 2) or (rem == Fr(1, 2) and n % 2 == 1):
        n += 1
    val = float(n) * 2.0 ** qe
    if val >= 2.0 ** 128:
        val = math.inf
    return -val if neg else val


# ----------------------------------------------------------------- cursor table

def test_flush_table_L4_matches_blog():
    """The state machine reproduces the worked L = 4 table of the blog."""
    tab = json.load(open(os.path.join(GOLDEN, "flush_table_L4.json")))
    L = tab["L"]
    p = 0
    ckpt_tokens = 0
    ring_tokens = [None] * L
    for row in tab["rows"]:
        t = row["step"]
        assert ckpt_tokens == row["checkpoint_before"]
        assert ring_tokens[:p] == row["valid_before"]
        flush, nxt = next_cursor(p, L, force=False)
        assert ("flush" if flush else "append") == row["action"]
        if flush:
            ckpt_tokens = t
            assert ckpt_tokens == row["checkpoint_after"]
        else:
            ring_tokens[p] = t
        p = nxt


def test_flush_period_and_forced_flush():
    """Natural flushes land every L steps (40 steps at L = 4 give 10 flushes:
    steps 4, 8, ..., 40); a forced flush resets the cycle mid-buffer and the
    entries before it are the only ones valid at that step."""
    L, p, flushes = 4, 0, []
    for t in range(1, 41):
        f, p = next_cursor(p, L, False)
        if f:
            flushes.append(t)
    assert flushes == list(range(4, 41, 4))
    p = 0
    seq = []
    for t in range(1, 9):
        f, nxt = next_cursor(p, L, force=(t == 2))
        seq.append((p, f))
        p = nxt
    assert seq == [(0, False), (1, True), (0, False), (1, False), (2, False),
                   (3, True), (0, False), (1, False)]
    # L = 1: no entry is ever kept, each step flushes
    p = 0
    for _ in range(5):
        f, p = next_cursor(p, 1, False)
        assert f and p == 0


# ----------------------------------------------------------------- O1 exactness

def _rational_case(seed, h=6, dv=2, dk=2):
    r = np.random.default_rng(seed)
    S0 = [[Fr(int(r.integers(-9, 10)), 10) for _ in range(dk)] for _ in range(dv)]
    toks = []
    for t in range(h):
        a = Fr(int(r.integers(5, 10)), 10)         # alpha in [0.5, 0.9]
        b = Fr(int(r.integers(1, 10)), 10)         # beta in [0.1, 0.9]
        c, s = PYTH[int(r.integers(len(PYTH)))]
        k = [c, s] if r.integers(2) else [-s, c]
        c2, s2 = PYTH[int(r.integers(len(PYTH)))]
        q = [c2 / 4, s2 / 4]
        v = [Fr(int(r.integers(-20, 21)), 8) for _ in range(dv)]
        toks.append((a, b, k, v, q))
    return S0, toks


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_closed_form_equals_recurrence_exactly(seed):
    """Blog section 2.1: the closed-form replay equals the sequential
    recurrence, exactly, at every h (including h = 0: empty product = 1)."""
    S0, toks = _rational_case(seed)
    states, _, us = exact_sequence(S0, toks)
    alphas = [t[0] for t in toks]
    ks = [t[2] for t in toks]
    assert exact_closed_form(S0, [], [], []) == S0
    for h in range(1, len(toks) + 1):
        assert exact_closed_form(S0, alphas[:h], us[:h], ks[:h]) == states[h - 1]


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_oracle_step_matches_exact_rationals(seed):
    """O1 in fp64 agrees with the exact rational recurrence to ~1e-12."""
    S0, toks = _rational_case(seed)
    states, ys, us = exact_sequence(S0, toks)
    S = np.array([[float(x) for x in row] for row in S0])[None, None]
    slot = np.array([0], np.int32)
    for t, (a, b, k, v, q) in enumerate(toks):
        qa = np.array([[[float(x) for x in q]]])
        ka = np.array([[[float(x) for x in k]]])
        va = np.array([[[float(x) for x in v]]])
        o, u = gdn_step(S, slot, qa, ka, va, np.array([[math.log(a)]]),
                        np.array([[float(b)]]), want_u=True)
        exact_S = np.array([[float(x) for x in row] for row in states[t]])
        assert np.max(np.abs(S[0, 0] - exact_S)) <= 1e-12 * max(1.0, np.max(np.abs(exact_S)))
        assert np.max(np.abs(o[0, 0] - np.array([float(x) for x in ys[t]]))) <= 1e-12
        assert np.max(np.abs(u[0, 0] - np.array([float(x) for x in us[t]]))) <= 1e-12


def test_oracle_step_matches_transition_matrices():
    """Brute force: S_t = S_{t-1} M_t + beta v k^T with
    M_t = alpha (I - beta k k^T), composed as explicit matrices, and
    y_t = S_t q_t, for every slot, head and GQA mapping h -> h // (Hv/Hk)."""
    S0, slot, toks = random_problem(RNG, B=3, N=4, Hv=6, Hk=3, dk=7, dv=5, steps=9)
    S = S0.copy()
    ref = S0.copy()
    G = 2
    for (q, k, v, g, beta) in toks:
        o = gdn_step(S, slot, q, k, v, g, beta)
        for b, s in enumerate(slot):
            for h in range(6):
                kk, qq = k[b, h // G], q[b, h // G]
                a = math.exp(g[b, h])
                M = a * (np.eye(7) - beta[b, h] * np.outer(kk, kk))
                ref[s, h] = ref[s, h] @ M + beta[b, h] * np.outer(v[b, h], kk)
                assert np.allclose(o[b, h], ref[s, h] @ qq, rtol=0, atol=1e-12)
    assert np.allclose(S, ref, rtol=0, atol=1e-12)
    untouched = [s for s in range(4) if s not in slot]
    for s in untouched:
        assert np.array_equal(S[s], S0[s])


def test_oracle_special_cases():
    rng = np.random.default_rng(7)
    dk = dv = 8
    # beta = 0: pure decay, o = alpha S q and S <- alpha S
    S = rng.standard_normal((1, 1, dv, dk))
    S_prev = S.copy()
    q = rng.standard_normal((1, 1, dk))
    k = unit_rows(rng.standard_normal((1, 1, dk)))
    v = rng.standard_normal((1, 1, dv))
    g = np.array([[-0.3]])
    o = gdn_step(S, np.array([0], np.int32), q, k, v, g, np.zeros((1, 1)))
    a = math.exp(-0.3)
    assert np.allclose(S[0, 0], a * S_prev[0, 0], rtol=0, atol=1e-14)
    assert np.allclose(o[0, 0], a * S_prev[0, 0] @ q[0, 0], rtol=0, atol=1e-13)
    # beta = 1 and |k| = 1: S_t k = v for any prior state, so reading with q = k gives v
    S = rng.standard_normal((1, 1, dv, dk))
    o = gdn_step(S, np.array([0], np.int32), k, k, v, np.array([[-0.7]]), np.ones((1, 1)))
    assert np.allclose(o[0, 0], v[0, 0], rtol=0, atol=1e-12)
    # alpha = 1, S0 = 0, beta = 1, orthonormal keys: an exact associative memory
    Q, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    S = np.zeros((1, 1, dv, dk))
    vs = rng.standard_normal((dk, dv))
    for j in range(dk):
        gdn_step(S, np.array([0], np.int32), Q[:, j][None, None], Q[:, j][None, None],
                 vs[j][None, None], np.zeros((1, 1)), np.ones((1, 1)))
    for j in range(dk):
        assert np.allclose(S[0, 0] @ Q[:, j], vs[j], rtol=0, atol=1e-12)


def test_padding_rows_output_zero_and_touch_nothing():
    S0, slot, toks = random_problem(RNG, B=3, N=3, steps=1)
    slot = np.array([2, -1, 0], np.int32)
    S = S0.copy()
    q, k, v, g, beta = toks[0]
    o = gdn_step(S, slot, q, k, v, g, beta)
    assert np.all(o[1] == 0.0)
    assert np.array_equal(S[1], S0[1])


def test_output_only_identity():
    """SGLang PR #28451 (Modifications): alpha (S q) + d_cur (k^T q) equals the
    new state read with q, and d_cur = beta (v - alpha (S k)) equals the
    blog's u. Checked on O1's own step (S before vs after)."""
    S0, slot, toks = random_problem(RNG, B=2, N=2, steps=5)
    S = S0.copy()
    for (q, k, v, g, beta) in toks:
        prev = S.copy()
        o, u = gdn_step(S, slot, q, k, v, g, beta, want_u=True)
        for b, s in enumerate(slot):
            for h in range(prev.shape[1]):
                hk = h // 2
                a = math.exp(g[b, h])
                d = beta[b, h] * (v[b, h] - a * (prev[s, h] @ k[b, hk]))
                oo = a * (prev[s, h] @ q[b, hk]) + d * (k[b, hk] @ q[b, hk])
                assert np.allclose(d, u[b, h], rtol=0, atol=1e-13)
                assert np.allclose(oo, o[b, h], rtol=0, atol=1e-13)


# ----------------------------------------------------------------- O2

@pytest.mark.parametrize("L", [1, 2, 4, 5])
def test_replay_model_matches_recurrence(L):
    """The checkpoint + ring machine (closed-form route, output-only readout)
    reproduces O1's outputs at every step and O1's state after every flush,
    with natural and forced flushes and a padding row; only entries below
    write_pos are ever valid."""
    rng = np.random.default_rng(100 + L)
    S0, slot, toks = random_problem(rng, B=3, N=4, steps=13)
    slot = np.array([3, -1, 1], np.int32)
    S = S0.copy()
    model = ReplayModel(S0, Hk=2, L=L)
    for t, (q, k, v, g, beta) in enumerate(toks):
        ff = np.array([t == 3, 0, t == 5], dtype=np.uint8)
        p_before = model.write_pos.copy()
        o_ref = gdn_step(S, slot, q, k, v, g, beta)
        o, flush = model.decode(slot, q, k, v, g, beta, ff)
        assert rel_err(o, o_ref) <= 1e-12
        for b, s in enumerate(slot):
            if s < 0:
                continue
            assert flush[b] == ((p_before[s] == L - 1) or bool(ff[b]))
            if flush[b]:
                assert rel_err(model.ckpt[s], S[s]) <= 1e-12
        model.advance(slot, flush)
        for b, s in enumerate(slot):
            if s >= 0:
                assert 0 <= model.write_pos[s] <= L - 1
                assert rel_err(model.state(s), S[s]) <= 1e-12
        if L == 1:
            assert np.all(model.write_pos == 0)
    assert np.array_equal(model.ckpt[0], S0[0]) and np.array_equal(model.ckpt[2], S0[2])


def test_replay_model_stale_entries_are_not_read():
    """After a flush the ring bytes are left as they were; corrupting the
    stale entries (positions >= write_pos) must not change anything, while
    corrupting a valid entry must change the output."""
    rng = np.random.default_rng(5)
    S0, slot, toks = random_problem(rng, B=1, N=1, steps=6)
    slot = np.array([0], np.int32)
    m = ReplayModel(S0, Hk=2, L=4)
    for (q, k, v, g, beta) in toks[:5]:
        _, f = m.decode(slot, q, k, v, g, beta)
        m.advance(slot, f)
    assert m.write_pos[0] == 1          # flushed at step 4, one entry since
    m2 = ReplayModel(S0, Hk=2, L=4)
    m2.ckpt, m2.write_pos = m.ckpt.copy(), m.write_pos.copy()
    m2.ring_u, m2.ring_k, m2.ring_g = m.ring_u.copy(), m.ring_k.copy(), m.ring_g.copy()
    m2.ring_u[0, :, 1:] = 1e9
    m2.ring_k[0, :, 1:] = -1e9
    q, k, v, g, beta = toks[5]
    o1, _ = m.decode(slot, q, k, v, g, beta)
    o2, _ = m2.decode(slot, q, k, v, g, beta)
    assert np.array_equal(o1, o2)
    m3 = ReplayModel(S0, Hk=2, L=4)
    m3.ckpt, m3.write_pos = m.ckpt.copy(), np.array([1])
    m3.ring_u, m3.ring_k, m3.ring_g = m.ring_u.copy(), m.ring_k.copy(), m.ring_g.copy()
    m3.ring_k[0, 0, 0] = m3.ring_k[0, 0, 0][::-1]
    # m was advanced by the decode above; compare against a fresh evaluation
    o3, _ = m3.decode(slot, q, k, v, g, beta)
    assert not np.allclose(o3, o1)


# ----------------------------------------------------------------- O4 / windows

def test_window_is_causal_and_matches_closed_form_route():
    """Verify window (vLLM PR #49887): outputs of token t depend only on
    tokens <= t; the closed-form route (O2.verify) matches the token-by-token
    reference (O4); commit moves the cursor and the committed state equals the
    true state advanced by the accepted tokens only."""
    rng = np.random.default_rng(11)
    S0, slot, _ = random_problem(rng, B=3, N=3, steps=0)
    B, T, Hk, Hv, dk, dv = 3, 4, 2, 4, 6, 5
    q = unit_rows(rng.standard_normal((B, T, Hk, dk))) * dk ** -0.5
    k = unit_rows(rng.standard_normal((B, T, Hk, dk)))
    v = rng.standard_normal((B, T, Hv, dv))
    g = -np.logaddexp(0.0, -rng.normal(2.0, 1.0, (B, T, Hv)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, Hv))))
    o_ref = window_ref(S0, slot, q, k, v, g, beta)
    v2 = v.copy()
    v2[:, 2:] += 3.0
    o_ref2 = window_ref(S0, slot, q, k, v2, g, beta)
    assert np.array_equal(o_ref[:, :2], o_ref2[:, :2])
    assert not np.allclose(o_ref[:, 2:], o_ref2[:, 2:])
    m = ReplayModel(S0, Hk=Hk, L=8)
    m.write_pos[:] = 0
    o = m.verify(slot, q, k, v, g, beta)
    assert rel_err(o, o_ref) <= 1e-12
    acc = np.array([0, 2, 4], np.int32)
    m.commit(slot, acc)
    S_true = S0.copy()
    for b, s in enumerate(slot):
        for t in range(acc[b]):
            one = np.array([s], np.int32)
            gdn_step(S_true, one, q[b:b + 1, t], k[b:b + 1, t], v[b:b + 1, t],
                     g[b:b + 1, t], beta[b:b + 1, t])
    for b, s in enumerate(slot):
        assert m.write_pos[s] == acc[b]
        assert rel_err(m.state(s), S_true[s]) <= 1e-12
    m.fold(slot)
    assert np.all(m.write_pos == 0)
    for s in slot:
        assert rel_err(m.ckpt[s], S_true[s]) <= 1e-12
    # a window that would overrun the ring is rejected (zero output, no writes)
    m.write_pos[slot[0]] = 6
    o = m.verify(slot[:1], q[:1], k[:1], v[:1], g[:1], beta[:1])
    assert np.all(o == 0)


# ----------------------------------------------------------------- O3

def _exact_fold_element(x, ds, ks, gs):
    for d, k, g in zip(ds, ks, gs):
        a = rn32(Fr(math.exp(float(g))))
        t = rn32(Fr(a) * Fr(float(x)))
        x = rn32(Fr(float(d)) * Fr(float(k)) + Fr(t))
    return x


def test_fold_matches_exact_rounding_model():
    """O3 bitwise equals an independent exact-rational model of the two
    instructions t = RN(a*x), x = RN(d*k + t) with a = RN(exp(g))."""
    rng = np.random.default_rng(3)
    N, Hv, Hk, dv, dk, L = 2, 2, 1, 3, 4, 5
    ckpt = (0.1 * rng.standard_normal((N, Hv, dv, dk))).astype(np.float32)
    rd = rng.standard_normal((N, Hv, L, dv)).astype(np.float16).astype(np.float32)
    rk = unit_rows(rng.standard_normal((N, Hk, L, dk))).astype(np.float16).astype(np.float32)
    rg = (-np.logaddexp(0.0, -rng.normal(2.0, 1.0, (N, Hv, L)))).astype(np.float32)
    wp = np.array([5, 3], np.int32)
    slot = np.array([0, 1], np.int32)
    out = ckpt.copy()
    wpo = wp.copy()
    fold_f32(out, slot, wpo, rd, rk, rg)
    assert np.all(wpo == 0)
    for s in range(N):
        for h in range(Hv):
            for i in range(dv):
                for c in range(dk):
                    p = wp[s]
                    ref = _exact_fold_element(ckpt[s, h, i, c], rd[s, h, :p, i],
                                              rk[s, 0, :p, c], rg[s, h, :p])
                    assert np.float32(ref).tobytes() == out[s, h, i, c].tobytes()


def test_fold_control_detects_other_operation_order():
    """The bitwise check has teeth: the other association
    x = fma(a, x, RN(d*k)) (the naive single-expression form) differs in some
    elements, mirroring the 1-2 ULP drift case of SGLang PR #42388."""
    rng = np.random.default_rng(4)
    N, Hv, Hk, dv, dk, L = 2, 4, 2, 32, 32, 8
    ckpt = (0.1 * rng.standard_normal((N, Hv, dv, dk))).astype(np.float32)
    rd = rng.standard_normal((N, Hv, L, dv)).astype(np.float16).astype(np.float32)
    rk = unit_rows(rng.standard_normal((N, Hk, L, dk))).astype(np.float16).astype(np.float32)
    rg = (-np.logaddexp(0.0, -rng.normal(2.0, 1.0, (N, Hv, L)))).astype(np.float32)
    slot = np.arange(N, dtype=np.int32)
    a, b = ckpt.copy(), ckpt.copy()
    fold_f32(a, slot, np.full(N, L, np.int32), rd, rk, rg, order=0)
    fold_f32(b, slot, np.full(N, L, np.int32), rd, rk, rg, order=1)
    diff = np.count_nonzero(a.view(np.uint32) != b.view(np.uint32))
    assert diff > 0
    assert rel_err(a, b) < 1e-5          # but only by rounding


def test_fold_agrees_with_fp64_fold_and_edge_cases():
    rng = np.random.default_rng(6)
    N, Hv, Hk, dv, dk, L = 3, 2, 1, 8, 8, 4
    S0 = (0.1 * rng.standard_normal((N, Hv, dv, dk))).astype(np.float32)
    rd = rng.standard_normal((N, Hv, L, dv)).astype(np.float32)
    rk = unit_rows(rng.standard_normal((N, Hk, L, dk))).astype(np.float32)
    rg = (-np.logaddexp(0.0, -rng.normal(2.0, 1.0, (N, Hv, L)))).astype(np.float32)
    wp = np.array([4, 0, 2], np.int32)
    slot = np.array([0, 1, -1, 2], np.int32)
    out, wpo = S0.copy(), wp.copy()
    fold_f32(out, slot, wpo, rd, rk, rg)
    m = ReplayModel(S0.astype(np.float64), Hk=Hk, L=L)
    m.ring_u[:], m.ring_k[:], m.ring_g[:] = rd, rk, rg
    m.write_pos[:] = wp
    m.fold(slot)
    assert rel_err(out, m.ckpt) < 1e-5
    assert np.array_equal(out[1], S0[1])          # p = 0 leaves the bits alone
    assert np.all(wpo == 0)
    # a slot listed by no row keeps its cursor and checkpoint
    out2, wp2 = S0.copy(), wp.copy()
    fold_f32(out2, np.array([1], np.int32), wp2, rd, rk, rg)
    assert wp2[0] == 4 and np.array_equal(out2[0], S0[0])


def test_rn32_model_is_correct_rounding():
    """The exact rounding helper agrees with numpy's own fp32 rounding of
    doubles that are exactly representable midpoints and ordinary values."""
    rng = np.random.default_rng(0)
    for x in rng.standard_normal(2000) * 10.0 ** rng.integers(-40, 38, 2000):
        assert rn32(Fr(float(x))) == float(np.float32(x))
    # ties to even
    one = Fr(1)
    ulp = Fr(1, 2 ** 23)
    assert rn32(one + ulp / 2) == 1.0
    assert rn32(one + ulp + ulp / 2) == float(np.float32(1 + 2 * 2.0 ** -23))
    # subnormal
    assert rn32(Fr(3, 2 ** 150)) == float(np.float32(2.0 ** -148))


# ----------------------------------------------------------------- O5

def _f16_grid_samples(rng):
    """Values around binary16: random magnitudes (normal and subnormal range),
    exact midpoints between neighbours, points just off the midpoints, and the
    overflow threshold."""
    mags = np.ldexp(rng.uniform(0.5, 1.0, 4000), rng.integers(-30, 17, 4000))
    a = rng.standard_normal(2000).astype(np.float16)
    a = a[np.isfinite(a)]
    b = np.nextafter(a, np.float16(np.inf))
    mid = (a.astype(np.float64) + b.astype(np.float64)) / 2       # exact in float64
    off = np.concatenate([np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)])
    sub = np.ldexp(rng.integers(0, 2048, 500).astype(np.float64) + 0.5, -24)   # subnormal ties
    edge = np.array([65504.0, 65519.99, 65520.0, 65536.0, 2.0 ** -24, 2.0 ** -25,
                     1.5 * 2.0 ** -25, 2.0 ** -26, 0.0, -0.0, np.inf, -np.inf])
    x = np.concatenate([mags, -mags, mid, off, sub, -sub, edge])
    return x


def test_quantize_f16_matches_numpy_binary16():
    """O5 'f16' equals numpy's float64 -> float16 conversion (round to
    nearest, ties to even, with subnormals and overflow to infinity)."""
    x = _f16_grid_samples(np.random.default_rng(501))
    got = oracle.quantize(x, "f16")
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(got, ref, equal_nan=True)


def _bf16_bits(y: float) -> int:
    return int(np.array([y], np.float32).view(np.uint32)[0])


def _from_bits(u: int) -> float:
    return float(np.array([u], np.uint32).view(np.float32)[0])


def test_quantize_bf16_is_nearest_even():
    """O5 'bf16' against the definition of round-to-nearest-even on the
    bfloat16 grid, in exact rational arithmetic: the result is a bfloat16 value
    (a binary32 value whose low 16 bits are zero), no neighbouring bfloat16
    value is nearer, and a tie goes to the even significand."""
    rng = np.random.default_rng(502)
    mags = np.ldexp(rng.uniform(0.5, 1.0, 1500), rng.integers(-140, 60, 1500))
    grid = rng.integers(1, 0x7F7F, 600, dtype=np.int64) << 16      # bfloat16 bit patterns
    lo = np.array(grid, np.uint32).view(np.float32).astype(np.float64)
    hi = np.array(grid + 0x10000, np.uint32).view(np.float32).astype(np.float64)
    ties = (lo + hi) / 2
    x = np.concatenate([mags, ties, np.nextafter(ties, np.inf), np.nextafter(ties, -np.inf),
                        [0.0, 2.0 ** -133, 1.5 * 2.0 ** -133, 2.0 ** -134]])
    y = oracle.quantize(x, "bf16")
    assert np.array_equal(oracle.quantize(-x, "bf16"), -y)
    n_ties = 0
    for xi, yi in zip(x, y):
        u = _bf16_bits(yi)
        assert float(np.float32(yi)) == yi and (u & 0xFFFF) == 0
        X, Y = Fr(xi), Fr(yi)
        for nb in (u + 0x10000, u - 0x10000 if u >= 0x10000 else None):
            if nb is None or nb >= 0x7F800000:
                continue
            d_nb, d_y = abs(X - Fr(_from_bits(nb))), abs(X - Y)
            assert d_y <= d_nb, (xi, yi)
            if d_y == d_nb:
                n_ties += 1
                assert (u >> 16) & 1 == 0, (xi, yi)
    assert n_ties > 300


def test_quantize_bf16_matches_torch_on_binary32_inputs():
    """On binary32 inputs O5 'bf16' equals torch's float32 -> bfloat16
    conversion (an independent implementation)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(503)
    x32 = (rng.standard_normal(20000) * np.ldexp(1.0, rng.integers(-40, 40, 20000))).astype(np.float32)
    u = x32.view(np.uint32)
    x32 = np.concatenate([x32, ((u & 0xFFFF0000) | 0x8000).view(np.float32)])   # exact ties
    ref = torch.from_numpy(x32).to(torch.bfloat16).float().numpy().astype(np.float64)
    assert np.array_equal(oracle.quantize(x32.astype(np.float64), "bf16"), ref)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_replay_model_16bit_state_at_L1_equals_quantized_recurrence(fmt):
    """With a ring of one entry every step flushes, so the 16-bit checkpoint
    is written (and rounded) after every token: the replay machine must match
    the sequential recurrence that stores its state in the same format after
    every token, outputs and states."""
    rng = np.random.default_rng(510)
    S0, slot, toks = random_problem(rng, B=3, N=4, steps=9)
    S0 = oracle.quantize(S0, fmt)
    slot = np.array([3, -1, 1], np.int32)
    S = S0.copy()
    model = ReplayModel(S0, Hk=2, L=1, state_fmt=fmt)
    for q, k, v, g, beta in toks:
        o_ref = gdn_step(S, slot, q, k, v, g, beta, state_fmt=fmt)
        o, flush = model.decode(slot, q, k, v, g, beta)
        model.advance(slot, flush)
        assert flush[[0, 2]].all()
        assert rel_err(o, o_ref) <= 1e-9
        assert np.array_equal(model.ckpt, S)
    # the rounding is really applied: the unrounded run drifts away
    S_plain = S0.copy()
    for q, k, v, g, beta in toks:
        gdn_step(S_plain, slot, q, k, v, g, beta)
    assert rel_err(S, S_plain) > 1e-5


def test_replay_model_16bit_rounds_only_when_writing():
    """At L = 4 the 16-bit checkpoint changes only at flushes and folds, always
    holds values of the format, and the model stays within the format's
    rounding of the exact recurrence."""
    rng = np.random.default_rng(511)
    S0, slot, toks = random_problem(rng, B=2, N=3, steps=11)
    S0 = oracle.quantize(S0, "bf16")
    S = S0.copy()
    model = ReplayModel(S0, Hk=2, L=4, state_fmt="bf16")
    for q, k, v, g, beta in toks:
        before = model.ckpt.copy()
        o_ref = gdn_step(S, slot, q, k, v, g, beta)
        o, flush = model.decode(slot, q, k, v, g, beta)
        model.advance(slot, flush)
        for b, s in enumerate(slot):
            if not flush[b]:
                assert np.array_equal(model.ckpt[s], before[s])
        assert np.array_equal(oracle.quantize(model.ckpt, "bf16"), model.ckpt)
        assert rel_err(o, o_ref) <= 2e-2
    model.fold(slot)
    assert np.array_equal(oracle.quantize(model.ckpt, "bf16"), model.ckpt)
    assert rel_err(model.ckpt[slot], S[slot]) <= 2e-2
