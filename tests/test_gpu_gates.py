"""GPU parity of the gate activations in front of a per-key-gate decode
(gdn_kda_gates) against the oracle's O10, and of gates -> KDA replay decode
against O10 -> O6.

SGLang PR #36821 (Technical principle) forms g = l * sigma(e^A (a + b_dt)) per
key channel and beta = sigma(b). Tolerance from the arithmetic: exp, the
product, the sum and the division in fp32 each add at most a few ulps, so
|g - g_ref| <= 1e-6 |l| and |beta - beta_ref| <= 1e-6 per element.
"""
import dataclasses

import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gdn_harness import DEV, Pool, log, to_dev, to_f64, tol_o, tol_state
from oracle import kda_gates, quantize, rel_err, step

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import linear_attention_ssm_amd as m
    return m


def gate_inputs(seed, B, T, Hv, dk):
    r = np.random.default_rng(seed)
    a = (2.0 * r.standard_normal((B, T, Hv, dk))).astype(np.float32)
    b = r.standard_normal((B, T, Hv)).astype(np.float32)
    A = r.normal(-0.5, 1.0, Hv).astype(np.float32)
    dt = r.standard_normal((Hv, dk)).astype(np.float32)
    return a, b, A, dt


@pytest.mark.parametrize("B,T,Hv,dk", [(3, 1, 5, 32), (2, 5, 32, 128), (1, 2, 3, 256), (64, 1, 32, 128)])
def test_gates_vs_oracle(gdn, B, T, Hv, dk):
    a, b, A, dt = gate_inputs(B * 131 + dk, B, T, Hv, dk)
    lb = -5.0
    g, beta = gdn.gdn_kda_gates(to_dev(a), to_dev(b), to_dev(A), to_dev(dt), lb)
    g_ref, b_ref = kda_gates(a, b, A, dt, lb)
    eg = np.max(np.abs(to_f64(g) - g_ref))
    eb = np.max(np.abs(to_f64(beta) - b_ref))
    assert eg <= 1e-6 * abs(lb) and eb <= 1e-6, f"g {eg:.3e} beta {eb:.3e}"
    assert np.all(to_f64(g) <= 0) and np.all(to_f64(g) >= lb)     # fp32 may reach either end
    log(f"[gates {B}x{T}x{Hv}x{dk}] g {eg:.2e} beta {eb:.2e}")


def test_gates_then_kda_decode(gdn):
    """The per-key-gate decode fed by the kernel's gates against the oracle:
    O10, g and beta rounded to fp32 as the device stores them (O5), then the
    per-key-gate recurrence (O6). Replay decode steps with flushes."""
    w = gi.scaled(gi.C7, name="gates_kda", B=8, N=10, L=4, steps=8, n_pad=1, permute=True,
                  seed=950)
    S0 = gi.initial_state(w)
    slots = gi.slot_map(w)
    slot_t = to_dev(slots)
    pool = Pool(w, S0)
    S_true = S0.astype(np.float64)
    wp = np.zeros(w.N, np.int64)
    worst = 0.0
    for t in range(w.steps):
        x = gi.step_inputs(w, t)
        a, b, A, dt = gate_inputs(7000 + t, w.B, 1, w.Hv, w.dk)
        g, beta = gdn.gdn_kda_gates(to_dev(a), to_dev(b), to_dev(A), to_dev(dt), -5.0)
        xi = [to_dev(arr, x.dtype) for arr in (x.q, x.k, x.v)]
        ff = gi.force_flush_schedule(w, t, slots)
        o = gdn.gdn_replay_decode(*xi, g, beta, slot_t, pool.ckpt, pool.ring_d, pool.ring_k,
                                  pool.ring_g, pool.write_pos, force_flush=to_dev(ff))
        gdn.gdn_replay_advance(slot_t, pool.write_pos, w.L, force_flush=to_dev(ff))
        g_ref, b_ref = kda_gates(a, b, A, dt, -5.0)
        q64, k64, v64, _, _ = x.f64()
        o_ref = step(S_true, slots, q64[:, 0], k64[:, 0], v64[:, 0],
                     quantize(g_ref[:, 0], "f32"), quantize(b_ref[:, 0], "f32"))
        e = rel_err(to_f64(o[:, 0]), o_ref)
        worst = max(worst, e)
        assert e <= tol_o(w), f"step {t}: o rel err {e:.3e}"
        for bi, s in enumerate(slots):
            if s < 0:
                continue
            if wp[s] == w.L - 1 or ff[bi]:
                assert rel_err(to_f64(pool.ckpt[s]), S_true[s]) <= tol_state(w)
                wp[s] = 0
            else:
                wp[s] += 1
    log(f"[gates -> kda decode] o {worst:.2e}")


def test_gates_then_kda_verify_window(gdn):
    """A 5-token verify window of the per-key-gate decode fed by the kernel's
    gates, against O10 -> O5 -> O4 (the window token by token through O6)."""
    from oracle import window_ref
    w = gi.scaled(gi.C7, name="gates_window", B=6, N=6, L=8, T=5, steps=1, seed=951)
    S0 = gi.initial_state(w)
    slots = gi.slot_map(w)
    pool = Pool(w, S0)
    x = gi.step_inputs(w, 0)
    a, b, A, dt = gate_inputs(7100, w.B, w.T, w.Hv, w.dk)
    g, beta = gdn.gdn_kda_gates(to_dev(a), to_dev(b), to_dev(A), to_dev(dt), -5.0)
    xi = [to_dev(arr, x.dtype) for arr in (x.q, x.k, x.v)]
    o = gdn.gdn_replay_decode(*xi, g, beta, to_dev(slots), pool.ckpt, pool.ring_d, pool.ring_k,
                              pool.ring_g, pool.write_pos, window=True)
    g_ref, b_ref = kda_gates(a, b, A, dt, -5.0)
    q64, k64, v64, _, _ = x.f64()
    o_ref = window_ref(S0.astype(np.float64), slots, q64, k64, v64, quantize(g_ref, "f32"),
                       quantize(b_ref, "f32"))
    e = rel_err(to_f64(o), o_ref)
    assert e <= tol_o(w), f"window rel err {e:.3e}"
