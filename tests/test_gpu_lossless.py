"""Lossless verify (SGLang PR #42388, "The idea" and Commit).

A verify window read from an exact checkpoint (no ring entries) stores fp32
(d, k, g) tuples; committing the accepted prefix and folding it replays the
tuples with the verify kernel's own rounding. The result must be
bit-identical to decoding the accepted tokens one at a time with the packed
read-update-write step: the output of every accepted position, the output of
the first rejected position (the verified token), and the state. Both sides
of that comparison run on the GPU, so every round is also checked against the
oracle's fp64 recurrence within tolerance.
"""
import dataclasses

import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gdn_harness import Pool, bits, dev_inputs, log, to_dev, to_f64, tol_o, tol_state
from oracle import rel_err, step, window_ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import linear_attention_ssm_amd as m
    return m


def _tok(x, t):
    return x[:, t:t + 1].contiguous()


@pytest.mark.parametrize("fmt,gate", [("f32", "head"), ("bf16", "head"), ("f16", "head"),
                                      ("f32", "key"), ("bf16", "key")])
def test_lossless_rounds_bitwise_equal_packed(gdn, fmt, gate):
    """fp32 state, and 16-bit state pools with step_rounding (the window
    rounds its state after each token, the fold after each entry); per-head
    and per-key (KDA) gates."""
    w = dataclasses.replace(gi.C6, state=fmt, gate=gate)
    T, L = w.T, w.L
    stepr = fmt != "f32"
    sfmt = fmt if stepr else None
    S0s = gi.stored_state(w)
    S0 = gi.as_f64(S0s, w.state).astype(np.float32)
    slots = gi.slot_map(w)
    live = slots >= 0
    pool = Pool(w, S0, garbage=True)
    pool.ckpt = to_dev(S0s, w.state)
    state = to_dev(S0s, w.state)            # the packed decode's state
    S_true = gi.as_f64(S0s, w.state)
    slot_t = to_dev(slots)
    err = torch.zeros(1, dtype=torch.int32, device=state.device)
    worst_o = worst_s = 0.0
    n_out = 0
    for r in range(w.steps):
        x = gi.step_inputs(w, 3000 + r)
        xi = dev_inputs(x)
        o_win = gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, pool.ckpt,
                                      pool.ring_d, pool.ring_k, pool.ring_g, pool.write_pos,
                                      err_flags=err, window=True, step_rounding=stepr)
        x64 = x.f64()
        o_ref = window_ref(S_true, slots, *x64, state_fmt=sfmt)
        worst_o = max(worst_o, rel_err(to_f64(o_win), o_ref))
        acc = gi.accepted_counts(w, r)
        for t in range(T):
            args = [_tok(a, t) for a in (xi.q, xi.k, xi.v, xi.g, xi.beta)]
            nxt = live & (acc == t)         # the verified token after an accepted prefix
            if nxt.any():
                scratch = state.clone()
                o_n = gdn.gdn_packed_decode(*args, to_dev(np.where(nxt, slots, -1).astype(np.int32)),
                                            scratch, err_flags=err)
                rows = torch.from_numpy(np.nonzero(nxt)[0]).to(state.device)
                assert torch.equal(bits(o_win[rows, t]), bits(o_n[rows, 0])), \
                    f"round {r} token {t}: verified-token output differs from packed decode"
                n_out += int(nxt.sum())
            take = live & (acc > t)
            if take.any():
                o_t = gdn.gdn_packed_decode(*args, to_dev(np.where(take, slots, -1).astype(np.int32)),
                                            state, err_flags=err)
                rows = torch.from_numpy(np.nonzero(take)[0]).to(state.device)
                assert torch.equal(bits(o_win[rows, t]), bits(o_t[rows, 0])), \
                    f"round {r} token {t}: accepted-token output differs from packed decode"
                n_out += int(take.sum())
        gdn.gdn_replay_commit(slot_t, to_dev(acc), pool.write_pos, L, T, err_flags=err)
        gdn.gdn_replay_fold(slot_t, pool.ckpt, pool.ring_d, pool.ring_k, pool.ring_g,
                            pool.write_pos, err_flags=err, step_rounding=stepr)
        gdn.gdn_replay_reset(slot_t, pool.write_pos, err_flags=err)
        mism = int((bits(pool.ckpt) != bits(state)).sum().item())
        assert mism == 0, f"round {r}: {mism} checkpoint elements differ from packed decode"
        assert int(pool.write_pos.abs().sum().item()) == 0
        for b, s in enumerate(slots):
            if s >= 0:
                one = np.array([s], np.int32)
                for t in range(int(acc[b])):
                    step(S_true, one, *(a[b:b + 1, t] for a in x64), state_fmt=sfmt)
        worst_s = max(worst_s, rel_err(to_f64(pool.ckpt), S_true))
    assert int(err.item()) == 0
    assert worst_o <= tol_o(w), f"window outputs vs oracle: {worst_o:.3e}"
    assert worst_s <= (tol_state(w) if not stepr else 2e-2), f"state vs oracle: {worst_s:.3e}"
    log(f"[{w.name}/{fmt}/{gate}] {w.steps} rounds: state and {n_out} outputs bit-identical to packed "
        f"decode; vs oracle o {worst_o:.2e}, state {worst_s:.2e}")


def test_16bit_state_without_step_rounding_is_not_lossless(gdn):
    """Control: with a bf16 state and the default rounding (once, at the fold)
    a verify round does not reproduce the per-token rounding of the packed
    decode, so the step_rounding flag is what makes the previous test pass."""
    w = dataclasses.replace(gi.C6, state="bf16", steps=1)
    S0s = gi.stored_state(w)
    slots = gi.slot_map(w)
    live = slots >= 0
    pool = Pool(w, gi.as_f64(S0s, w.state).astype(np.float32))
    pool.ckpt = to_dev(S0s, w.state)
    state = to_dev(S0s, w.state)
    slot_t = to_dev(slots)
    x = gi.step_inputs(w, 3000)
    xi = dev_inputs(x)
    gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, pool.ckpt, pool.ring_d,
                          pool.ring_k, pool.ring_g, pool.write_pos, window=True)
    acc = np.full(w.B, w.T, np.int32)
    for t in range(w.T):
        args = [_tok(a, t) for a in (xi.q, xi.k, xi.v, xi.g, xi.beta)]
        gdn.gdn_packed_decode(*args, slot_t, state)
    gdn.gdn_replay_commit(slot_t, to_dev(acc), pool.write_pos, w.L, w.T)
    gdn.gdn_replay_fold(slot_t, pool.ckpt, pool.ring_d, pool.ring_k, pool.ring_g, pool.write_pos)
    rows = torch.from_numpy(slots[live]).to(state.device)
    mism = int((bits(pool.ckpt[rows]) != bits(state[rows])).sum().item())
    log(f"[lossless control] bf16 state, rounding once: {mism} elements differ")
    assert mism > 0
