"""GPU parity of the verify window, the commit and the fold.

The c5 protocol: a T = 1 history that never flushes, then rounds of
verify (T = 5) -> accept a ~ U{0..5} -> commit -> fold when the ring cannot
hold another window, then a final fold. Outputs, stored corrections and
folded checkpoints are checked against the oracle's true recurrence within
the 16-bit-ring tolerance; cursors bit for bit. The fold itself is checked
bit for bit against the oracle's pinned-rounding fold on seeded rings.
"""
import dataclasses

import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gdn_harness import (DEV, TORCH_DT, CanaryTensor, Pool, bits, dev_inputs, log, to_dev,
                         to_f64, tol_o, tol_state)
from oracle import fold_f32, gdn_step, rel_err, step, window_ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import linear_attention_ssm_amd as m
    return m


def _advance_true(S, slots, x64, counts):
    """Advance the oracle's true states by the first counts[b] tokens of each row."""
    q, k, v, g, beta = x64
    for b, s in enumerate(slots):
        if s < 0:
            continue
        one = np.array([s], np.int32)
        for t in range(int(counts[b])):
            step(S, one, q[b:b + 1, t], k[b:b + 1, t], v[b:b + 1, t], g[b:b + 1, t],
                     beta[b:b + 1, t])


@pytest.mark.parametrize("ring", ["f16", "f32"])
def test_c5_verify_commit_fold_protocol(gdn, ring):
    w = gi.C5 if ring == "f16" else dataclasses.replace(gi.C5, name="c5_f32ring", ring="f32",
                                                       qkv="f32", bf16_values=True)
    T, L = w.T, w.L
    S0 = gi.initial_state(w)
    slots = gi.slot_map(w)
    hist = gi.history_lengths(w)
    pool = Pool(w, S0, garbage=True, canary=True)
    o_win = CanaryTensor((w.B, T, w.Hv, w.dv), w.qkv)
    S_true = S0.astype(np.float64)
    wp = np.zeros(w.N, dtype=np.int64)
    tol_o_, tol_s_ = tol_o(w), tol_state(w)
    errs = {"hist": [], "win": [], "d": [], "fold": []}
    # -- history of single-token steps (never reaching a flush)
    for i in range(int(hist.max())):
        act = np.array([hist[s] > i for s in slots])
        sl = np.where(act, slots, -1).astype(np.int32)
        x = gi.step_inputs(w, 1000 + i, T=1)
        xi = dev_inputs(x)
        slt = to_dev(sl)
        o = gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slt, pool.ckpt, pool.ring_d,
                                  pool.ring_k, pool.ring_g, pool.write_pos, err_flags=pool.err)
        gdn.gdn_replay_advance(slt, pool.write_pos, L, err_flags=pool.err)
        q, k, v, g, beta = (a[:, 0] for a in x.f64())
        o_ref = gdn_step(S_true, sl, q, k, v, g, beta)
        e = rel_err(to_f64(o[:, 0]), o_ref)
        errs["hist"].append(e)
        assert e <= tol_o_
        wp[sl[sl >= 0]] += 1
    assert np.array_equal(pool.write_pos.cpu().numpy(), wp)
    assert np.array_equal(wp, hist)
    slot_t = to_dev(slots)
    for r in range(w.steps):
        x = gi.step_inputs(w, 2000 + r)
        xi = dev_inputs(x)
        p_before = wp.copy()
        assert np.all(p_before[slots] + T <= L)
        o = gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, pool.ckpt,
                                  pool.ring_d, pool.ring_k, pool.ring_g, pool.write_pos,
                                  o=o_win.t, err_flags=pool.err, window=True)
        o_win.check(f"round {r}: window o")
        pool.check_canaries(f"round {r}: window")
        x64 = x.f64()
        o_ref, u_ref = window_ref(S_true, slots, *x64, want_u=True)
        e = rel_err(to_f64(o), o_ref)
        errs["win"].append(e)
        assert e <= tol_o_, f"round {r}: window output rel err {e:.3e}"
        # the window's corrections were written at p .. p+T-1
        # only the written entries are converted (the rest hold a garbage template)
        d_gpu = np.stack([to_f64(pool.ring_d[s, :, p_before[s]:p_before[s] + T]).transpose(1, 0, 2)
                          for s in slots])                              # [B, T, Hv, dv]
        ed = rel_err(d_gpu, u_ref)
        errs["d"].append(ed)
        assert ed <= tol_s_, f"round {r}: stored corrections rel err {ed:.3e}"
        assert np.array_equal(pool.write_pos.cpu().numpy(), wp), "verify moved a cursor"
        acc = gi.accepted_counts(w, r)
        gdn.gdn_replay_commit(slot_t, to_dev(acc), pool.write_pos, L, T, err_flags=pool.err)
        _advance_true(S_true, slots, x64, acc)
        wp[slots] += acc
        assert np.array_equal(pool.write_pos.cpu().numpy(), wp)
        need = wp[slots] + T > L
        if need.any():
            sl = np.where(need, slots, -1).astype(np.int32)
            gdn.gdn_replay_fold(to_dev(sl), pool.ckpt, pool.ring_d, pool.ring_k, pool.ring_g,
                                pool.write_pos, err_flags=pool.err)
            pool.check_canaries(f"round {r}: fold")
            assert np.array_equal(pool.write_pos.cpu().numpy(), wp), "the fold moved a cursor"
            gdn.gdn_replay_reset(to_dev(sl), pool.write_pos, err_flags=pool.err)
            wp[slots[need]] = 0
            ef = rel_err(to_f64(pool.ckpt[to_dev(slots[need]).long()]), S_true[slots[need]])
            errs["fold"].append(ef)
            assert ef <= tol_s_, f"round {r}: folded checkpoint rel err {ef:.3e}"
            assert np.array_equal(pool.write_pos.cpu().numpy(), wp)
    gdn.gdn_replay_fold(slot_t, pool.ckpt, pool.ring_d, pool.ring_k, pool.ring_g,
                        pool.write_pos, err_flags=pool.err)
    gdn.gdn_replay_reset(slot_t, pool.write_pos, err_flags=pool.err)
    pool.check_canaries("final fold and reset")
    ef = rel_err(to_f64(pool.ckpt), S_true)
    errs["fold"].append(ef)
    assert ef <= tol_s_
    assert int(pool.write_pos.abs().sum().item()) == 0
    assert int(pool.err.item()) == 0
    log(f"[{w.name}] " + "  ".join(f"{k} {max(v):.2e}" for k, v in errs.items() if v))


def test_window_equals_token_by_token_windows(gdn):
    """A T-token window and T single-token windows (each committed with
    accepted = 1) give the same outputs within tolerance, and both match the
    oracle (vLLM PR #49887, Tests: window vs one token at a time)."""
    w = gi.scaled(gi.C5, name="win_vs_tok", B=8, N=8, steps=1, seed=606)
    S0 = gi.initial_state(w)
    slots = gi.slot_map(w)
    a, b = Pool(w, S0), Pool(w, S0)
    slot_t = to_dev(slots)
    x = gi.step_inputs(w, 0)
    xi = dev_inputs(x)
    oa = gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, a.ckpt, a.ring_d,
                               a.ring_k, a.ring_g, a.write_pos, window=True)
    ob = []
    one = torch.ones(w.B, dtype=torch.int32, device=DEV)
    for t in range(w.T):
        sl = lambda z: z[:, t:t + 1].contiguous()
        ob.append(gdn.gdn_replay_decode(sl(xi.q), sl(xi.k), sl(xi.v), sl(xi.g), sl(xi.beta),
                                        slot_t, b.ckpt, b.ring_d, b.ring_k, b.ring_g,
                                        b.write_pos, window=True))
        gdn.gdn_replay_commit(slot_t, one, b.write_pos, w.L, 1)
    ob = torch.cat(ob, dim=1)
    o_ref = window_ref(S0.astype(np.float64), slots, *x.f64())
    assert rel_err(to_f64(oa), o_ref) <= tol_o(w)
    assert rel_err(to_f64(ob), o_ref) <= tol_o(w)
    assert rel_err(to_f64(oa), to_f64(ob)) <= tol_o(w)


@pytest.mark.parametrize("dk,dv,L", [(128, 96, 16), (64, 48, 16), (128, 16, 16), (128, 128, 64)])
def test_fold_bitwise_smaller_row_blocks(gdn, dk, dv, L):
    """The fold's workgroups cover 32 or 16 value rows when dv is not a
    multiple of 64 (two rows or one per thread), and a ring of 64 entries
    holds more d and key pieces than the workgroup has threads (staged in
    more than one pass): bit-identical to the oracle's pinned-rounding fold
    there too, with full, empty and partial rings."""
    w = dataclasses.replace(gi.C5, dk=dk, dv=dv, L=L, Hv=8, Hk=2, N=20, B=16, n_pad=2,
                            permute=True, seed=830 + dv + L)
    rc = gi.random_ring(w, seed_tag=7)
    slots = gi.slot_map(w)
    wp = rc.write_pos.copy()
    live = slots[slots >= 0]
    wp[live[0]] = w.L
    wp[live[1]] = 0
    ckpt = to_dev(rc.ckpt)
    rd, rk = to_dev(rc.d, w.ring), to_dev(rc.k, w.ring)
    rg = to_dev(rc.g)
    wpt = to_dev(wp.astype(np.int32))
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    gdn.gdn_replay_fold(to_dev(slots), ckpt, rd, rk, rg, wpt, err_flags=err)
    assert int(err.item()) == 0
    ref = rc.ckpt.copy()
    fold_f32(ref, slots, wp.astype(np.int32).copy(), gi.as_f64(rc.d, w.ring).astype(np.float32),
             gi.as_f64(rc.k, w.ring).astype(np.float32), rc.g)
    got = ckpt.cpu().numpy()
    mism = np.count_nonzero(got.view(np.uint32) != ref.view(np.uint32))
    assert mism == 0, f"{mism} elements differ from the oracle's fold"


@pytest.mark.parametrize("ring", ["f16", "bf16", "f32"])
def test_fold_bitwise_against_oracle(gdn, ring):
    """gdn_replay_fold is bit-identical to the oracle's pinned-rounding fold
    (every element of every slot, listed or not) and leaves the cursors alone;
    gdn_replay_reset then clears the listed ones."""
    w = dataclasses.replace(gi.C5, ring=ring, N=40, B=36, n_pad=3, permute=True)
    rc = gi.random_ring(w, seed_tag={"f16": 1, "bf16": 2, "f32": 3}[ring])
    slots = gi.slot_map(w)
    wp = rc.write_pos.copy()
    live = slots[slots >= 0]
    wp[live[0]] = w.L          # a full ring
    wp[live[1]] = 0            # an empty one
    ck_guard = CanaryTensor(rc.ckpt.shape, "f32", init=to_dev(rc.ckpt))
    ckpt = ck_guard.t
    rd, rk = to_dev(rc.d, ring), to_dev(rc.k, ring)
    rg = to_dev(rc.g)
    wpt = to_dev(wp.astype(np.int32))
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    gdn.gdn_replay_fold(to_dev(slots), ckpt, rd, rk, rg, wpt, err_flags=err)
    ck_guard.check("fold: ckpt")
    assert np.array_equal(wpt.cpu().numpy(), wp.astype(np.int32))
    gdn.gdn_replay_reset(to_dev(slots), wpt, err_flags=err)
    ref = rc.ckpt.copy()
    wref = wp.astype(np.int32).copy()
    fold_f32(ref, slots, wref, gi.as_f64(rc.d, ring).astype(np.float32),
             gi.as_f64(rc.k, ring).astype(np.float32), rc.g)
    got = ckpt.cpu().numpy()
    mism = np.count_nonzero(got.view(np.uint32) != ref.view(np.uint32))
    assert mism == 0, f"{mism} elements differ from the oracle's fold"
    assert np.array_equal(wpt.cpu().numpy(), wref)
    assert int(err.item()) == 0
    log(f"[fold/{ring}] bit-exact over {got.size} elements, "
        f"{int(wp[live].sum())} entries folded")


@pytest.mark.parametrize("n_layers,ring,state,gate", [
    (3, "f16", "f32", "head"), (17, "bf16", "f32", "head"), (2, "f32", "bf16", "head"),
    (2, "f16", "f32", "key")])
def test_fold_layers_bitwise(gdn, n_layers, ring, state, gate):
    """gdn_replay_fold_layers folds each layer's own ring into its own
    checkpoint under one cursor array, bit-identical to gdn_replay_fold on
    that layer and, with an fp32 state and the per-head gate, to the oracle's
    pinned-rounding fold; 17 layers take two launches (16 + 1). Canaries
    around every checkpoint stay untouched."""
    w = dataclasses.replace(gi.C5, ring=ring, state=state, gate=gate, Hv=4, Hk=2, N=10, B=8,
                            n_pad=1, permute=True, seed=870 + n_layers)
    rcs = [gi.random_ring(w, seed_tag=20 + i) for i in range(n_layers)]
    slots = gi.slot_map(w)
    slot_t = to_dev(slots)
    wp = rcs[0].write_pos.copy()
    live = slots[slots >= 0]
    wp[live[0]] = w.L
    wp[live[1]] = 0
    wpt = to_dev(wp.astype(np.int32))
    sdt = TORCH_DT[state]
    guards, ones, rings = [], [], []
    for rc in rcs:
        init = to_dev(rc.ckpt).to(sdt)
        guards.append(CanaryTensor(rc.ckpt.shape, state, init=init))
        ones.append(init.clone())
        rings.append((to_dev(rc.d, ring), to_dev(rc.k, ring), to_dev(rc.g)))
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    gdn.gdn_replay_fold_layers(slot_t, [g.t for g in guards], [r[0] for r in rings],
                               [r[1] for r in rings], [r[2] for r in rings], wpt, err_flags=err)
    for ck, r in zip(ones, rings):
        gdn.gdn_replay_fold(slot_t, ck, r[0], r[1], r[2], wpt, err_flags=err)
    assert int(err.item()) == 0
    assert np.array_equal(wpt.cpu().numpy(), wp.astype(np.int32))
    for i, (g, ck, rc) in enumerate(zip(guards, ones, rcs)):
        g.check(f"fold_layers: layer {i}")
        assert torch.equal(bits(g.t), bits(ck)), f"layer {i} differs from its own fold"
        if state == "f32" and gate == "head":
            ref = rc.ckpt.copy()
            fold_f32(ref, slots, wp.astype(np.int32).copy(),
                     gi.as_f64(rc.d, ring).astype(np.float32),
                     gi.as_f64(rc.k, ring).astype(np.float32), rc.g)
            got = g.t.cpu().numpy()
            mism = np.count_nonzero(got.view(np.uint32) != ref.view(np.uint32))
            assert mism == 0, f"layer {i}: {mism} elements differ from the oracle's fold"
    log(f"[fold_layers/{n_layers}/{ring}/{state}/{gate}] every layer bit-identical, "
        f"{int(wp[live].sum())} entries per layer")


def test_fold_layers_full_size_eight_layers(gdn):
    """The launch the benchmark times: the speculative workload's 8 layers
    (B = 32, Hv = 32, dk = dv = 128, fp16 ring) in one gdn_replay_fold_layers
    call, with cursors from 0 to L over the slots. Every layer's checkpoint is
    bit-identical to gdn_replay_fold on that layer, whose own parity with the
    oracle's fold at these shapes test_fold_bitwise_against_oracle checks;
    layer 0 is also checked against the oracle's fold directly."""
    w = dataclasses.replace(gi.C5, seed=890)
    n = 8
    rcs = [gi.random_ring(w, seed_tag=40 + i) for i in range(n)]
    slots = gi.slot_map(w)
    slot_t = to_dev(slots)
    wp = rcs[0].write_pos.copy()
    wp[slots[0]] = w.L
    wp[slots[1]] = 0
    wpt = to_dev(wp.astype(np.int32))
    many = [to_dev(rc.ckpt) for rc in rcs]
    one = [c.clone() for c in many]
    rings = [(to_dev(rc.d, w.ring), to_dev(rc.k, w.ring), to_dev(rc.g)) for rc in rcs]
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    gdn.gdn_replay_fold_layers(slot_t, many, [r[0] for r in rings], [r[1] for r in rings],
                               [r[2] for r in rings], wpt, err_flags=err)
    for c, r in zip(one, rings):
        gdn.gdn_replay_fold(slot_t, c, r[0], r[1], r[2], wpt, err_flags=err)
    assert int(err.item()) == 0
    for i in range(n):
        assert torch.equal(bits(many[i]), bits(one[i])), f"layer {i} differs from its own fold"
    ref = rcs[0].ckpt.copy()
    fold_f32(ref, slots, wp.astype(np.int32).copy(), gi.as_f64(rcs[0].d, w.ring).astype(np.float32),
             gi.as_f64(rcs[0].k, w.ring).astype(np.float32), rcs[0].g)
    got = many[0].cpu().numpy()
    mism = np.count_nonzero(got.view(np.uint32) != ref.view(np.uint32))
    assert mism == 0, f"layer 0: {mism} elements differ from the oracle's fold"
    log(f"[fold_layers/full] 8 layers bit-identical, {int(wp[slots].sum())} entries per layer")


def test_fold_layers_rejects_mismatched_layers(gdn):
    """The binding refuses layers whose counts, dtypes, shapes or ring depths
    differ from layer 0's, and the library refuses a checkpoint passed twice;
    all before any launch, so the checkpoints stay as they were."""
    w = dataclasses.replace(gi.C5, Hv=4, Hk=2, N=6, B=4, seed=880)
    rc = gi.random_ring(w, seed_tag=1)
    slot_t = to_dev(gi.slot_map(w))
    wpt = to_dev(rc.write_pos.astype(np.int32))
    mk = lambda: (to_dev(rc.ckpt), to_dev(rc.d, w.ring), to_dev(rc.k, w.ring), to_dev(rc.g))
    (c0, d0, k0, g0), (c1, d1, k1, g1) = mk(), mk()
    before = [bits(c0).clone(), bits(c1).clone()]
    with pytest.raises(ValueError):       # one ring_d short
        gdn.gdn_replay_fold_layers(slot_t, [c0, c1], [d0], [k0, k1], [g0, g1], wpt)
    with pytest.raises(ValueError):       # layer 1's checkpoint in another dtype
        gdn.gdn_replay_fold_layers(slot_t, [c0, c1.to(torch.bfloat16)], [d0, d1], [k0, k1],
                                   [g0, g1], wpt)
    with pytest.raises(ValueError):       # layer 1's ring one entry shorter
        gdn.gdn_replay_fold_layers(slot_t, [c0, c1], [d0, d1[:, :, :-1].contiguous()],
                                   [k0, k1[:, :, :-1].contiguous()], [g0, g1[:, :, :-1].contiguous()],
                                   wpt)
    with pytest.raises(gdn.GdnError):     # the same checkpoint twice
        gdn.gdn_replay_fold_layers(slot_t, [c0, c0], [d0, d1], [k0, k1], [g0, g1], wpt)
    torch.cuda.synchronize()
    assert torch.equal(bits(c0), before[0]) and torch.equal(bits(c1), before[1])


@pytest.mark.parametrize("T", [1, 2, 4, 6, 8])
def test_window_length_sweep_verify_commit_verify(gdn, T):
    """Windows of T in {1, 2, 4, 6, 8} tokens (vLLM PR #49887, Tests) at B = 16:
    a single-token history, a verify window, a commit of a ~ U{0..T}, then a
    second window that reads the committed entries; both windows against the
    oracle, the cursors exact."""
    w = gi.scaled(gi.C5, name=f"win_T{T}", B=16, N=16, T=T, steps=2, seed=640 + T)
    _verify_commit_verify(gdn, w)


@pytest.mark.parametrize("gate", ["head", "key"])
def test_window_wide_group_long_window(gdn, gate):
    """Eight value heads per key head and a 16-token window: every (head,
    token) pair of a workgroup needs its own staged decay and beta, more pairs
    than one wavefront has lanes when the workgroup holds many heads. Both
    windows against the oracle, the cursors exact."""
    w = gi.scaled(gi.C5, name=f"win_G8_T16_{gate}", B=6, N=6, Hv=16, Hk=2, dk=64, dv=64,
                  L=48, T=16, steps=2, gate=gate, seed=652)
    _verify_commit_verify(gdn, w)


def _verify_commit_verify(gdn, w):
    T, L = w.T, w.L
    S0 = gi.initial_state(w)
    slots = gi.slot_map(w)
    slot_t = to_dev(slots)
    pool = Pool(w, S0, garbage=True)
    S_true = S0.astype(np.float64)
    # history: h_s single-token steps, never reaching a flush, p + 2T <= L after it
    hist = np.random.default_rng(w.seed).integers(0, L - 2 * T + 1, size=w.N)
    for i in range(int(hist.max())):
        sl = np.array([s if hist[s] > i else -1 for s in slots], np.int32)
        x = gi.step_inputs(w, 100 + i, T=1)
        xi = dev_inputs(x)
        gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, to_dev(sl), pool.ckpt,
                              pool.ring_d, pool.ring_k, pool.ring_g, pool.write_pos,
                              err_flags=pool.err)
        gdn.gdn_replay_advance(to_dev(sl), pool.write_pos, L, err_flags=pool.err)
        q, k, v, g, beta = (a[:, 0] for a in x.f64())
        step(S_true, sl, q, k, v, g, beta)
    wp = hist[slots].astype(np.int64)
    assert np.array_equal(pool.write_pos.cpu().numpy()[slots], wp)
    for r in range(w.steps):
        x = gi.step_inputs(w, 200 + r)
        xi = dev_inputs(x)
        o = gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, pool.ckpt,
                                  pool.ring_d, pool.ring_k, pool.ring_g, pool.write_pos,
                                  err_flags=pool.err, window=True)
        x64 = x.f64()
        e = rel_err(to_f64(o), window_ref(S_true, slots, *x64))
        assert e <= tol_o(w), f"{w.name} round {r}: window rel err {e:.3e}"
        acc = gi.accepted_counts(w, r)
        gdn.gdn_replay_commit(slot_t, to_dev(acc), pool.write_pos, L, T, err_flags=pool.err)
        _advance_true(S_true, slots, x64, acc)
        wp += acc
        assert np.array_equal(pool.write_pos.cpu().numpy()[slots], wp)
    assert int(pool.err.item()) == 0


@pytest.mark.parametrize("gate", ["head", "key"])
def test_one_token_window_at_the_last_ring_entry(gdn, gate):
    """Every cursor at L - 1: a one-token verify window appends entry L - 1
    and, unlike a decode step at that cursor, does not flush (checkpoint
    untouched, cursor unmoved). Committing it fills the ring (p = L); the fold
    then writes the true state and the reset clears the cursors."""
    w = gi.scaled(gi.C5, name=f"win1_last_{gate}", B=8, N=8, T=1, L=4, steps=1, gate=gate,
                  seed=661)
    L = w.L
    S0 = gi.initial_state(w)
    slots = gi.slot_map(w)
    slot_t = to_dev(slots)
    pool = Pool(w, S0, garbage=True, canary=True)
    S_true = S0.astype(np.float64)
    for i in range(L - 1):                      # history: L - 1 steps, no flush
        x = gi.step_inputs(w, 300 + i)
        xi = dev_inputs(x)
        gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, pool.ckpt, pool.ring_d,
                              pool.ring_k, pool.ring_g, pool.write_pos, err_flags=pool.err)
        gdn.gdn_replay_advance(slot_t, pool.write_pos, L, err_flags=pool.err)
        step(S_true, slots, *(a[:, 0] for a in x.f64()))
    assert pool.write_pos.cpu().numpy()[slots].tolist() == [L - 1] * w.B
    ck0 = bits(pool.ckpt).clone()
    x = gi.step_inputs(w, 400)
    xi = dev_inputs(x)
    o = gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, pool.ckpt, pool.ring_d,
                              pool.ring_k, pool.ring_g, pool.write_pos, err_flags=pool.err,
                              window=True)
    x64 = x.f64()
    e = rel_err(to_f64(o), window_ref(S_true, slots, *x64))
    assert e <= tol_o(w), f"one-token window rel err {e:.3e}"
    assert torch.equal(bits(pool.ckpt), ck0), "a window flushed"
    assert pool.write_pos.cpu().numpy()[slots].tolist() == [L - 1] * w.B
    gdn.gdn_replay_commit(slot_t, to_dev(np.ones(w.B, np.int32)), pool.write_pos, L, 1,
                          err_flags=pool.err)
    _advance_true(S_true, slots, x64, np.ones(w.B, np.int64))
    assert pool.write_pos.cpu().numpy()[slots].tolist() == [L] * w.B
    gdn.gdn_replay_fold(slot_t, pool.ckpt, pool.ring_d, pool.ring_k, pool.ring_g,
                        pool.write_pos, err_flags=pool.err)
    gdn.gdn_replay_reset(slot_t, pool.write_pos, err_flags=pool.err)
    torch.cuda.synchronize()
    es = rel_err(to_f64(pool.ckpt)[slots], S_true[slots])
    assert es <= tol_state(w), f"folded state rel err {es:.3e}"
    assert pool.write_pos.cpu().numpy()[slots].tolist() == [0] * w.B
    assert int(pool.err.item()) == 0
    pool.check_canaries("one-token window")
    log(f"[win1/{gate}] window at p = L-1: no flush; commit, fold (rel err {es:.2e}), reset")
