"""GPU parity of the decode's front end: strided inputs read from the packed
mixed_qkv row, and q/k L2-normalisation with q scaling done in the kernel.

The ReplaySSM blog (section 3.1) describes the decode's input as one packed
row per token, [q (Hk*dk) | k (Hk*dk) | v (Hv*dv)]; SGLang PR #28451
(Modifications) hands the decode q and k L2-normalised and q scaled. Reading
q, k, v as views into the packed row must give the same bits as dense copies
of the same values. With qk_norm the kernels normalise themselves; the
oracle normalises the same raw values in fp64 (O8) and runs the recurrence
(O1, or O6 for the per-key gate).
"""
import dataclasses

import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gdn_harness import DEV, Pool, bits, dev_inputs, log, to_dev, to_f64, tol_o, tol_state
from oracle import l2norm_qk, rel_err, step, window_ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import linear_attention_ssm_amd as m
    return m


def mixed_views(xi, w):
    """q, k, v as views into one packed [B, T, 2*Hk*dk + Hv*dv] tensor holding
    the same values."""
    B, T = xi.q.shape[:2]
    nq, nv = w.Hk * w.dk, w.Hv * w.dv
    m = torch.empty((B, T, 2 * nq + nv), dtype=xi.q.dtype, device=DEV)
    m[..., :nq] = xi.q.reshape(B, T, nq)
    m[..., nq:2 * nq] = xi.k.reshape(B, T, nq)
    m[..., 2 * nq:] = xi.v.reshape(B, T, nv)
    q = m[..., :nq].view(B, T, w.Hk, w.dk)
    k = m[..., nq:2 * nq].view(B, T, w.Hk, w.dk)
    v = m[..., 2 * nq:].view(B, T, w.Hv, w.dv)
    assert not q.is_contiguous() and q.stride(0) == T * (2 * nq + nv)
    return m, q, k, v


@pytest.mark.parametrize("gate,qk_norm", [("head", False), ("key", False), ("head", True),
                                          ("key", True)])
def test_mixed_row_equals_dense_bitwise(gdn, gate, qk_norm):
    """Decode steps (with flushes), the fused advance, the packed decode and a
    verify window: the packed-row views and dense tensors give identical bits."""
    w = gi.scaled(gi.C2, name=f"mixed_{gate}_{int(qk_norm)}", B=12, N=14, L=4, steps=9,
                  n_pad=1, permute=True, gate=gate, qk_raw=qk_norm, seed=71)
    S0 = gi.initial_state(w)
    slots = gi.slot_map(w)
    slot_t = to_dev(slots)
    a, b = Pool(w, S0), Pool(w, S0)
    pa, pb = to_dev(S0), to_dev(S0)
    arrive = gdn.arrive_workspace(w.B, DEV)
    for t in range(w.steps):
        xi = dev_inputs(gi.step_inputs(w, t))
        m, q, k, v = mixed_views(xi, w)
        ff = to_dev(gi.force_flush_schedule(w, t, slots))
        oa = gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, a.ckpt, a.ring_d,
                                   a.ring_k, a.ring_g, a.write_pos, force_flush=ff,
                                   qk_norm=qk_norm)
        gdn.gdn_replay_advance(slot_t, a.write_pos, w.L, force_flush=ff)
        ob = gdn.gdn_replay_decode_advance(q, k, v, xi.g, xi.beta, slot_t, b.ckpt, b.ring_d,
                                           b.ring_k, b.ring_g, b.write_pos, arrive,
                                           force_flush=ff, qk_norm=qk_norm)
        assert torch.equal(bits(oa), bits(ob)), f"step {t}: replay outputs differ"
        for x, y in zip((a.ckpt, a.ring_d, a.ring_k, a.ring_g, a.write_pos),
                        (b.ckpt, b.ring_d, b.ring_k, b.ring_g, b.write_pos)):
            assert torch.equal(bits(x) if x.is_floating_point() else x,
                               bits(y) if y.is_floating_point() else y), f"step {t}"
        o1 = gdn.gdn_packed_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, pa, qk_norm=qk_norm)
        o2 = gdn.gdn_packed_decode(q, k, v, xi.g, xi.beta, slot_t, pb, qk_norm=qk_norm)
        assert torch.equal(bits(o1), bits(o2)) and torch.equal(bits(pa), bits(pb))
    # a 3-token verify window from the same pools
    wv = dataclasses.replace(w, T=3)
    xi = dev_inputs(gi.step_inputs(wv, 50))
    m, q, k, v = mixed_views(xi, wv)
    a.write_pos.zero_()
    b.write_pos.zero_()
    oa = gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, a.ckpt, a.ring_d,
                               a.ring_k, a.ring_g, a.write_pos, window=True, qk_norm=qk_norm)
    ob = gdn.gdn_replay_decode(q, k, v, xi.g, xi.beta, slot_t, b.ckpt, b.ring_d, b.ring_k,
                               b.ring_g, b.write_pos, window=True, qk_norm=qk_norm)
    assert torch.equal(bits(oa), bits(ob)) and torch.equal(bits(a.ring_k), bits(b.ring_k))


@pytest.mark.parametrize("gate", ["head", "key"])
def test_qk_norm_decode_vs_oracle(gdn, gate):
    """Raw q, k ~ N(0, 1) (bf16): the kernel normalises them; the oracle
    normalises the same values in fp64 (O8) and runs the recurrence. Replay
    decode (read from the packed row) and packed decode, outputs every step,
    checkpoints after flushes; the ring holds the normalised keys."""
    w = gi.scaled(gi.C2, name=f"qknorm_{gate}", B=16, N=16, L=8, steps=20, gate=gate,
                  qk_raw=True, seed=72)
    S0 = gi.initial_state(w)
    slots = gi.slot_map(w)
    slot_t = to_dev(slots)
    pool = Pool(w, S0)
    packed = to_dev(S0)
    S_true = S0.astype(np.float64)
    S_pk = S0.astype(np.float64)
    wp = np.zeros(w.N, np.int64)
    worst = [0.0, 0.0, 0.0]
    for t in range(w.steps):
        x = gi.step_inputs(w, t)
        xi = dev_inputs(x)
        m, q, k, v = mixed_views(xi, w)
        ff = gi.force_flush_schedule(w, t, slots)
        o = gdn.gdn_replay_decode(q, k, v, xi.g, xi.beta, slot_t, pool.ckpt, pool.ring_d,
                                  pool.ring_k, pool.ring_g, pool.write_pos,
                                  force_flush=to_dev(ff), qk_norm=True)
        gdn.gdn_replay_advance(slot_t, pool.write_pos, w.L, force_flush=to_dev(ff))
        op = gdn.gdn_packed_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, packed,
                                   qk_norm=True)
        q64, k64, v64, g64, b64 = (a[:, 0] for a in x.f64())
        qn, kn = l2norm_qk(q64, k64)
        o_ref = step(S_true, slots, qn, kn, v64, g64, b64)
        step(S_pk, slots, qn, kn, v64, g64, b64)
        e = rel_err(to_f64(o[:, 0]), o_ref)
        ep = rel_err(to_f64(op[:, 0]), o_ref)
        worst[0], worst[1] = max(worst[0], e), max(worst[1], ep)
        assert e <= tol_o(w) and ep <= tol_o(w), f"step {t}: {e:.3e} {ep:.3e}"
        for bi, s in enumerate(slots):
            fl = wp[s] == w.L - 1 or ff[bi]
            if not fl:
                # the appended key is the normalised one
                rk = to_f64(pool.ring_k[s, :, wp[s]])
                assert rel_err(rk, kn[bi]) <= 1e-2
            else:
                es = rel_err(to_f64(pool.ckpt[s]), S_true[s])
                worst[2] = max(worst[2], es)
                assert es <= tol_state(w)
            wp[s] = 0 if fl else wp[s] + 1
    assert rel_err(to_f64(packed), S_pk) <= 1e-4
    log(f"[{w.name}] o {worst[0]:.2e} packed o {worst[1]:.2e} ckpt {worst[2]:.2e}")


def test_qk_norm_L1_replay_equals_packed_bitwise(gdn):
    w = gi.scaled(gi.c4(1), name="qknorm_L1", B=10, N=10, steps=4, qk_raw=True, seed=73)
    S0 = gi.initial_state(w)
    slots = gi.slot_map(w)
    slot_t = to_dev(slots)
    a = Pool(w, S0)
    state = to_dev(S0)
    for t in range(w.steps):
        xi = dev_inputs(gi.step_inputs(w, t))
        o1 = gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, a.ckpt, a.ring_d,
                                   a.ring_k, a.ring_g, a.write_pos, qk_norm=True)
        gdn.gdn_replay_advance(slot_t, a.write_pos, w.L)
        o2 = gdn.gdn_packed_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, state, qk_norm=True)
        assert torch.equal(bits(o1), bits(o2)) and torch.equal(bits(a.ckpt), bits(state))


def test_qk_norm_window_vs_oracle(gdn):
    """A 5-token verify window read from the packed row with qk_norm."""
    w = gi.scaled(gi.C5, name="qknorm_window", B=8, N=8, steps=1, qk_raw=True, seed=74)
    S0 = gi.initial_state(w)
    slots = gi.slot_map(w)
    pool = Pool(w, S0)
    x = gi.step_inputs(w, 0)
    xi = dev_inputs(x)
    m, q, k, v = mixed_views(xi, w)
    o = gdn.gdn_replay_decode(q, k, v, xi.g, xi.beta, to_dev(slots), pool.ckpt, pool.ring_d,
                              pool.ring_k, pool.ring_g, pool.write_pos, window=True,
                              qk_norm=True)
    q64, k64, v64, g64, b64 = x.f64()
    qn, kn = l2norm_qk(q64, k64)
    o_ref = window_ref(S0.astype(np.float64), slots, qn, kn, v64, g64, b64)
    e = rel_err(to_f64(o), o_ref)
    assert e <= tol_o(w), f"window rel err {e:.3e}"
