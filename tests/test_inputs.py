"""The seeded input generator (no GPU): determinism, dtype rounding, the
workload structure, and an end-to-end oracle self-check on the tiny fp32
workload (the sequential recurrence against the checkpoint + ring machine
over all 40 steps and 10 flushes)."""
import numpy as np
import torch

import gdn_inputs as gi
from oracle import ReplayModel, gdn_step, rel_err


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000)).astype(np.float32)
    x[:4] = [0.0, -0.0, np.inf, -np.inf]
    ours = gi.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = gi.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generator_is_deterministic_and_well_formed():
    w = gi.C2
    a, b = gi.step_inputs(w, 3), gi.step_inputs(w, 3)
    for x, y in zip((a.q, a.k, a.v, a.g, a.beta), (b.q, b.k, b.v, b.g, b.beta)):
        assert np.array_equal(x, y)
    c = gi.step_inputs(w, 4)
    assert not np.array_equal(a.q, c.q)
    q, k, v, g, beta = a.f64()
    assert q.shape == (64, 1, 16, 128) and v.shape == (64, 1, 32, 128)
    assert np.all(g < 0) and np.all((beta > 0) & (beta < 1))
    assert np.allclose(np.linalg.norm(k, axis=-1), 1.0, atol=1e-2)
    assert np.allclose(np.linalg.norm(q, axis=-1), 128 ** -0.5, atol=1e-3)
    S0 = gi.initial_state(gi.C1)
    assert S0.shape == (2, 2, 32, 32) and S0.dtype == np.float32
    assert 0.05 < S0.std() < 0.2


def test_large_pool_slot_map():
    s = gi.slot_map(gi.C3)
    assert s.shape == (256,) and np.count_nonzero(s < 0) == 8
    live = s[s >= 0]
    assert len(np.unique(live)) == 248 and live.max() < 512


def test_stagger_spreads_flush_phases():
    w = gi.C2
    slots = gi.slot_map(w)
    forced = np.zeros(w.N, int)
    for t in range(w.steps):
        forced[slots] += gi.force_flush_schedule(w, t, slots)
    assert np.all(forced == 1)


def test_tiny_workload_oracle_self_consistency():
    """c1 end to end on the oracle: the sequential recurrence and the replay
    state machine agree on every output and (after each flush) on the
    checkpoint, and the flushes land on steps 4, 8, ..., 40."""
    w = gi.C1
    S0 = gi.initial_state(w).astype(np.float64)
    slots = gi.slot_map(w)
    S = S0.copy()
    m = ReplayModel(S0, Hk=w.Hk, L=w.L)
    flush_steps = []
    for t in range(w.steps):
        x = gi.step_inputs(w, t)
        q, k, v, g, beta = (a[:, 0] for a in x.f64())
        o_ref = gdn_step(S, slots, q, k, v, g, beta)
        o, fl = m.decode(slots, q, k, v, g, beta, gi.force_flush_schedule(w, t, slots))
        assert rel_err(o, o_ref) < 1e-12
        if fl[0]:
            flush_steps.append(t + 1)
            assert rel_err(m.ckpt, S) < 1e-12
        m.advance(slots, fl)
    assert flush_steps == list(range(4, 41, 4))
