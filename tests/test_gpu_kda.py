"""GPU parity of the per-key-gate (KDA) path against the CPU oracle.

SGLang PR #28451 (Modifications, item 7) runs KDA through the same decode
kernels with the decay taken per key channel: g and the ring's g carry one
log-decay per key channel, the replay's decay products fold onto the stored
keys and the token's own decay into q and k. These tests drive the library
with gate = GDN_GATE_KEY through the C-ABI and compare with the oracle's
per-key recurrence (O6), per-key replay model (O2) and per-key fold (O7):
outputs and states within the workload tolerance, cursors and flush
positions exactly, the fold and the L = 1 identity bit for bit.
"""
import dataclasses

import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gdn_harness import (DEV, Pool, bits, dev_inputs, log, run_decode, to_dev, to_f64, tol_o,
                         tol_state)
from oracle import fold_kda_f32, kda_step, quantize, rel_err, window_ref
from test_gpu_state16 import run_packed16, run_replay16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import linear_attention_ssm_amd as m
    return m


def test_kda_tiny_fp32_replay(gdn):
    rep = run_decode(gi.C7_TINY, "replay", garbage=True, recon_every=1)
    assert rep.flushes == 2 * 10


def test_kda_tiny_fp32_packed(gdn):
    run_decode(gi.C7_TINY, "packed")


def test_kda_standard_replay(gdn):
    run_decode(gi.C7, "replay", garbage=True, recon_every=16)


def test_kda_standard_packed(gdn):
    run_decode(gi.C7, "packed")


@pytest.mark.parametrize("L", [1, 4, 32])
def test_kda_ring_depth(gdn, L):
    w = dataclasses.replace(gi.C7, name=f"c7_kda_L{L}", L=L, steps=40, seed=810 + L)
    run_decode(w, "replay", recon_every=20 if L > 1 else 0)


def test_kda_fp32_ring(gdn):
    w = dataclasses.replace(gi.C7, name="c7_kda_f32ring", ring="f32", qkv="f32",
                            bf16_values=True, steps=40, seed=850)
    run_decode(w, "replay", recon_every=16)


@pytest.mark.parametrize("ring", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("dims", [(64, 48, 6, 2), (32, 16, 3, 3), (256, 128, 4, 1)])
def test_kda_ragged_shapes(gdn, ring, dims):
    """Several key tiles, odd value blocks, GQA groups of 1..3, padding rows,
    permuted slots, garbage-filled rings."""
    dk, dv, Hv, Hk = dims
    qkv = "f32" if ring == "f32" else "bf16"
    w = gi.Workload(f"kda_ragged_{dk}_{dv}_{Hv}_{Hk}_{ring}", B=5, N=7, Hv=Hv, Hk=Hk, dk=dk,
                    dv=dv, L=5, steps=13, qkv=qkv, ring=ring, n_pad=1, permute=True,
                    bf16_values=(ring == "f32"), gate="key", seed=960 + dk + dv + Hv)
    run_decode(w, "replay", garbage=True, recon_every=4, check_untouched=True)
    run_decode(w, "packed")


@pytest.mark.parametrize("fmt", ["f32", "bf16"])
def test_kda_L1_replay_equals_packed_bitwise(gdn, fmt):
    """At L = 1 every step flushes and the replay decode reproduces the
    packed decode bit for bit, also with the per-key gate."""
    w = dataclasses.replace(gi.C7, name="kda_L1", L=1, steps=5, n_pad=2, permute=True, N=80,
                            state=fmt)
    S0s = gi.stored_state(w)
    slots = gi.slot_map(w)
    a = Pool(w, gi.initial_state(w))
    a.ckpt = to_dev(S0s, w.state)
    state = to_dev(S0s, w.state)
    slot_t = to_dev(slots)
    for t in range(w.steps):
        xi = dev_inputs(gi.step_inputs(w, t))
        o1 = gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, a.ckpt, a.ring_d,
                                   a.ring_k, a.ring_g, a.write_pos, err_flags=a.err)
        gdn.gdn_replay_advance(slot_t, a.write_pos, w.L, err_flags=a.err)
        o2 = gdn.gdn_packed_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, state)
        assert torch.equal(bits(o1), bits(o2)), f"step {t}: outputs differ"
        assert torch.equal(bits(a.ckpt), bits(state)), f"step {t}: states differ"
    assert int(a.err.item()) == 0


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_kda_state16(gdn, fmt):
    w = dataclasses.replace(gi.C7, name=f"c7_kda_{fmt}", state=fmt, B=16, N=16, steps=34,
                            seed=870)
    run_packed16(gdn, w)
    assert run_replay16(gdn, w) > 0


@pytest.mark.parametrize("ring", ["f16", "f32"])
def test_kda_verify_commit_fold(gdn, ring):
    """Verify windows from the checkpoint with the per-key gate: outputs and
    stored corrections against the token-by-token oracle, commit by cursor
    move, fold of the committed entries against the true per-key state."""
    w = dataclasses.replace(gi.C5, name=f"kda_window_{ring}", gate="key", ring=ring,
                            qkv="f32" if ring == "f32" else "bf16",
                            bf16_values=(ring == "f32"), B=8, N=8, steps=8, seed=880)
    T, L = w.T, w.L
    S0 = gi.initial_state(w)
    slots = gi.slot_map(w)
    pool = Pool(w, S0, garbage=True)
    S_true = S0.astype(np.float64)
    wp = np.zeros(w.N, dtype=np.int64)
    slot_t = to_dev(slots)
    worst = {"win": 0.0, "d": 0.0, "fold": 0.0}
    for r in range(w.steps):
        x = gi.step_inputs(w, 2000 + r)
        xi = dev_inputs(x)
        p_before = wp.copy()
        o = gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, pool.ckpt,
                                  pool.ring_d, pool.ring_k, pool.ring_g, pool.write_pos,
                                  err_flags=pool.err, window=True)
        x64 = x.f64()
        o_ref, u_ref = window_ref(S_true, slots, *x64, want_u=True)
        e = rel_err(to_f64(o), o_ref)
        worst["win"] = max(worst["win"], e)
        assert e <= tol_o(w), f"round {r}: window output rel err {e:.3e}"
        # only the written entries are converted (the rest hold a garbage template)
        d_gpu = np.stack([to_f64(pool.ring_d[s, :, p_before[s]:p_before[s] + T]).transpose(1, 0, 2)
                          for s in slots])
        ed = rel_err(d_gpu, u_ref)
        worst["d"] = max(worst["d"], ed)
        assert ed <= tol_state(w)
        # the stored g entries are the window's per-key gates, bit for bit
        rg = pool.ring_g.cpu().numpy()
        for b, s in enumerate(slots):
            assert np.array_equal(rg[s, :, p_before[s]:p_before[s] + T],
                                  x.g[b].transpose(1, 0, 2))
        acc = gi.accepted_counts(w, r)
        gdn.gdn_replay_commit(slot_t, to_dev(acc), pool.write_pos, L, T, err_flags=pool.err)
        q, k, v, g, beta = x64
        for b, s in enumerate(slots):
            for t in range(int(acc[b])):
                kda_step(S_true, np.array([s], np.int32), q[b:b + 1, t], k[b:b + 1, t],
                         v[b:b + 1, t], g[b:b + 1, t], beta[b:b + 1, t])
        wp[slots] += acc
        assert np.array_equal(pool.write_pos.cpu().numpy(), wp)
        need = wp[slots] + T > L          # fold the rows whose ring cannot take another window
        if need.any() or r == w.steps - 1:
            sel = need if r < w.steps - 1 else np.ones_like(need)
            sl = np.where(sel, slots, -1).astype(np.int32)
            gdn.gdn_replay_fold(to_dev(sl), pool.ckpt, pool.ring_d, pool.ring_k, pool.ring_g,
                                pool.write_pos, err_flags=pool.err)
            gdn.gdn_replay_reset(to_dev(sl), pool.write_pos, err_flags=pool.err)
            wp[slots[sel]] = 0
            idx = torch.from_numpy(slots[sel]).to(DEV)
            ef = rel_err(to_f64(pool.ckpt[idx]), S_true[slots[sel]])
            worst["fold"] = max(worst["fold"], ef)
            assert ef <= tol_state(w), f"round {r}: folded checkpoint rel err {ef:.3e}"
    assert int(pool.write_pos.abs().sum().item()) == 0
    assert int(pool.err.item()) == 0
    log(f"[{w.name}] " + "  ".join(f"{k} {v:.2e}" for k, v in worst.items()))


@pytest.mark.parametrize("ring", ["f16", "bf16", "f32"])
def test_kda_fold_bitwise_against_oracle(gdn, ring):
    """gdn_replay_fold with the per-key gate is bit-identical to the oracle's
    pinned per-key fold (O7) over every element of every slot."""
    w = dataclasses.replace(gi.C5, gate="key", ring=ring, N=40, B=36, n_pad=3, permute=True)
    rc = gi.random_ring(w, seed_tag={"f16": 11, "bf16": 12, "f32": 13}[ring])
    assert rc.g.shape == (w.N, w.Hv, w.L, w.dk)
    slots = gi.slot_map(w)
    wp = rc.write_pos.copy()
    live = slots[slots >= 0]
    wp[live[0]] = w.L
    wp[live[1]] = 0
    ckpt = to_dev(rc.ckpt)
    rd, rk = to_dev(rc.d, ring), to_dev(rc.k, ring)
    rg = to_dev(rc.g)
    wpt = to_dev(wp.astype(np.int32))
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    gdn.gdn_replay_fold(to_dev(slots), ckpt, rd, rk, rg, wpt, err_flags=err)
    ref = rc.ckpt.copy()
    wref = wp.astype(np.int32).copy()
    fold_kda_f32(ref, slots, wref, gi.as_f64(rc.d, ring).astype(np.float32),
                 gi.as_f64(rc.k, ring).astype(np.float32), rc.g)
    got = ckpt.cpu().numpy()
    mism = np.count_nonzero(got.view(np.uint32) != ref.view(np.uint32))
    assert mism == 0, f"{mism} elements differ from the oracle's per-key fold"
    assert int(err.item()) == 0
    log(f"[kda fold/{ring}] bit-exact over {got.size} elements")


def test_kda_fold_state16_rounds_once(gdn):
    """A bf16 checkpoint folds in fp32 and is rounded once at the end: the
    oracle's per-key fold on the widened values, then the O5 rounding."""
    w = dataclasses.replace(gi.C5, gate="key", state="bf16", N=12, B=12)
    rc = gi.random_ring(w, seed_tag=21)
    slots = gi.slot_map(w)
    st = gi.cast(rc.ckpt, "bf16")
    ckpt = to_dev(st, "bf16")
    rd, rk, rg = to_dev(rc.d, w.ring), to_dev(rc.k, w.ring), to_dev(rc.g)
    wpt = to_dev(rc.write_pos)
    gdn.gdn_replay_fold(to_dev(slots), ckpt, rd, rk, rg, wpt)
    ref = gi.as_f64(st, "bf16").astype(np.float32)
    fold_kda_f32(ref, slots, rc.write_pos.copy(), gi.as_f64(rc.d, w.ring).astype(np.float32),
                 gi.as_f64(rc.k, w.ring).astype(np.float32), rc.g)
    want = quantize(ref.astype(np.float64), "bf16")
    assert np.array_equal(to_f64(ckpt), want)


def test_kda_shape_checks(gdn):
    """A per-key g needs a per-key ring_g and the reverse; a misaligned
    per-key g is rejected."""
    w = dataclasses.replace(gi.C7_TINY, B=2, N=2)
    S0 = gi.initial_state(w)
    pool = Pool(w, S0)
    xi = dev_inputs(gi.step_inputs(w, 0))
    slot_t = to_dev(gi.slot_map(w))
    g_head = xi.g[..., 0].contiguous()
    with pytest.raises(ValueError):
        gdn.gdn_replay_decode(xi.q, xi.k, xi.v, g_head, xi.beta, slot_t, pool.ckpt, pool.ring_d,
                              pool.ring_k, pool.ring_g, pool.write_pos)
    with pytest.raises(ValueError):
        gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, pool.ckpt, pool.ring_d,
                              pool.ring_k, pool.ring_g[..., 0].contiguous(), pool.write_pos)
    buf = torch.zeros(xi.g.numel() + 1, dtype=torch.float32, device=DEV)
    g_mis = buf[1:].view(xi.g.shape)
    with pytest.raises(gdn.GdnError):
        gdn.gdn_packed_decode(xi.q, xi.k, xi.v, g_mis, xi.beta, slot_t, pool.ckpt)
