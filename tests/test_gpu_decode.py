"""GPU parity of the single-token decode (packed and ReplaySSM) against the
CPU oracle, at the five workloads' sizes, plus the edge cases: padding rows,
forced mid-buffer flushes, the L = 1 degeneracy (bitwise against the packed
decode), ragged shapes, a corrupted ring key, stale-entry garbage, and the
device-side error flags."""
import dataclasses

import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gdn_harness import DEV, Pool, bits, dev_inputs, log, run_decode, to_dev, to_f64
from oracle import gdn_step, rel_err, step

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import linear_attention_ssm_amd as m
    return m


def test_c1_tiny_fp32_replay(gdn):
    rep = run_decode(gi.C1, "replay", garbage=True, recon_every=1)
    assert rep.flushes == 2 * 10          # 2 slots x flushes at steps 4, 8, ..., 40


def test_c1_tiny_fp32_packed(gdn):
    run_decode(gi.C1, "packed")


def test_c2_standard_replay(gdn):
    run_decode(gi.C2, "replay", garbage=True, recon_every=16)


def test_c2_standard_packed(gdn):
    run_decode(gi.C2, "packed")


@pytest.mark.parametrize("kind", ["replay", "packed"])
def test_c2_long_run_does_not_drift(gdn, kind):
    """192 steps at the standard shapes: 12 flush cycles per slot, every
    output and every flushed checkpoint (replay) or the whole state (packed)
    against the fp64 recurrence. Every head decays (alpha < 1), so the
    rounding a flush leaves in a checkpoint is damped by later steps and the
    error settles instead of growing: the largest state error over the last
    64 steps stays within 1.5x of the middle 64 steps' (and under the same
    tolerance as the short runs)."""
    rep = run_decode(gi.scaled(gi.C2, name=f"c2_long_{kind}", steps=192), kind,
                     recon_every=64 if kind == "replay" else 0)
    mid, last = rep.state_max(64, 128), rep.state_max(128, 192)
    log(f"[long {kind}] {rep.summary()}  state max mid {mid:.2e} last {last:.2e}")
    assert last <= 1.5 * mid, f"state error grows: {mid:.2e} -> {last:.2e}"
    if kind == "replay":
        assert rep.flushes >= 64 * 11


def test_c3_large_pool_with_padding(gdn):
    run_decode(gi.C3, "replay", check_untouched=True)


@pytest.mark.parametrize("L", [1, 4, 16, 32])
def test_c4_ring_depth(gdn, L):
    run_decode(gi.c4(L), "replay", recon_every=32 if L > 1 else 0)


def test_c4_fp32_ring(gdn):
    run_decode(gi.c4(16, "f32"), "replay", recon_every=16)


@pytest.mark.parametrize("ring", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("dims", [(64, 48, 6, 2), (32, 16, 3, 3), (256, 128, 4, 1)])
def test_ragged_shapes(gdn, ring, dims):
    """Several key tiles, value blocks that are not a power of two, GQA
    groups of 1..3, a row count that fills no tile evenly."""
    dk, dv, Hv, Hk = dims
    qkv = "f32" if ring == "f32" else "bf16"
    w = gi.Workload(f"ragged_{dk}_{dv}_{Hv}_{Hk}_{ring}", B=5, N=7, Hv=Hv, Hk=Hk, dk=dk, dv=dv,
                    L=5, steps=13, qkv=qkv, ring=ring, n_pad=1, permute=True,
                    bf16_values=(ring == "f32"), seed=900 + dk + dv + Hv)
    run_decode(w, "replay", garbage=True, recon_every=4, check_untouched=True)
    run_decode(w, "packed")


def test_L1_replay_equals_packed_bitwise(gdn):
    """At L = 1 no entry is ever kept (each step flushes), so the replay
    decode must reproduce the packed decode bit for bit (SGLang PR #28451,
    Design 1: the L = 1 kernel reduces to the packed decode)."""
    w = dataclasses.replace(gi.c4(1), steps=6, n_pad=2, permute=True, N=80)
    S0 = gi.initial_state(w)
    slots = gi.slot_map(w)
    a = Pool(w, S0)
    state = to_dev(S0)
    slot_t = to_dev(slots)
    for t in range(w.steps):
        xi = dev_inputs(gi.step_inputs(w, t))
        o1 = gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, a.ckpt, a.ring_d,
                                   a.ring_k, a.ring_g, a.write_pos, err_flags=a.err)
        gdn.gdn_replay_advance(slot_t, a.write_pos, w.L, err_flags=a.err)
        o2 = gdn.gdn_packed_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, state)
        assert torch.equal(bits(o1), bits(o2)), f"step {t}: outputs differ"
        assert torch.equal(bits(a.ckpt), bits(state)), f"step {t}: states differ"
        assert int(a.write_pos.abs().sum().item()) == 0
    assert int(a.err.item()) == 0


@pytest.mark.parametrize("p,Hv,Hk", [(1, 4, 2), (7, 4, 2), (16, 4, 2), (9, 2, 2), (12, 8, 2)])
def test_split_readout_matches_reconstruction(gdn, p, Hv, Hk):
    """A single-token row that does not flush is read out without forming its
    state, S x = A (S0 x) + sum_j (w_j d_j)(k_j . x); a forced flush of the
    same step forms S = A S0 + sum_j w_j d_j k_j^T first (fp32 checkpoint,
    dk = 128, fp16 ring, 1..16 valid entries). With fp32 q/k/v/o the two
    outputs differ only by where each rounds to the ring's 16-bit format:
    the split form rounds q and k (the ring products' operand), the
    reconstruction rounds w_j d_j (the MFMA's operand), 2^-11 relative
    each. So per output element
      |o_split - o_flush| <= alpha (E_q + |k.q| beta E_k) + fp32 slack,
      E_x = 2^-10 sum_j |w_j d_j| |k_j| |x|,
    where a dropped or misplaced ring entry would cost |w_j d_j (k_j . q)|,
    many times that bound. Value heads per key head 1, 2 and 4: one head of
    64 rows, two of 32 or four of 16 per workgroup."""
    w = gi.scaled(gi.C2, name=f"split_{p}_{Hv}_{Hk}", B=8, N=8, Hv=Hv, Hk=Hk, L=32, steps=p,
                  qkv="f32", stagger=False, seed=720 + p + 100 * Hv)
    S0 = gi.initial_state(w)
    slots = gi.slot_map(w)
    pool = Pool(w, S0)
    slot_t = to_dev(slots)
    for t in range(p):
        xi = dev_inputs(gi.step_inputs(w, t))
        gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, pool.ckpt, pool.ring_d,
                              pool.ring_k, pool.ring_g, pool.write_pos, err_flags=pool.err)
        gdn.gdn_replay_advance(slot_t, pool.write_pos, w.L, err_flags=pool.err)
    assert pool.write_pos.cpu().tolist() == [p] * w.N
    x = gi.step_inputs(w, p)
    xi = dev_inputs(x)
    outs = []
    for ff in (np.zeros(w.B, np.int32), np.ones(w.B, np.int32)):
        c = [t.clone() for t in (pool.ckpt, pool.ring_d, pool.ring_k, pool.ring_g)]
        outs.append(to_f64(gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, *c,
                                                 pool.write_pos, force_flush=to_dev(ff),
                                                 err_flags=pool.err)))
    assert int(pool.err.item()) == 0
    o_split, o_flush = (o[:, 0] for o in outs)                 # [B, Hv, dv]
    q, k, v, g, beta = (a[:, 0] for a in x.f64())
    G = w.Hv // w.Hk
    rd, rk, rg = (to_f64(t) for t in (pool.ring_d, pool.ring_k, pool.ring_g))
    bound = np.zeros_like(o_flush)
    for b, s in enumerate(slots):
        for h in range(w.Hv):
            hk = h // G
            gs = rg[s, h, :p]
            wj = np.exp(np.array([gs[j + 1:].sum() for j in range(p)]))
            wd = np.abs(wj[:, None] * rd[s, h, :p])                       # [p, dv]
            kn = np.linalg.norm(rk[s, hk, :p], axis=1)                     # [p]
            qn, knt = np.linalg.norm(q[b, hk]), np.linalg.norm(k[b, hk])
            alpha, kq = np.exp(g[b, h]), abs(q[b, hk] @ k[b, hk])
            e_q = 2.0 ** -10 * (wd * kn[:, None]).sum(0) * qn
            e_k = 2.0 ** -10 * (wd * kn[:, None]).sum(0) * knt
            bound[b, h] = alpha * (e_q + kq * beta[b, h] * e_k)
    bound += 1e-5 * np.abs(o_flush).max()
    diff = np.abs(o_split - o_flush)
    log(f"[split p={p} Hv={Hv} Hk={Hk}] max diff {diff.max():.3e}, max bound {bound.max():.3e}, "
        f"worst diff/bound {(diff / bound).max():.3f}")
    assert (diff <= bound).all(), f"split readout off by {(diff / bound).max():.2f}x its bound"
    assert diff.max() > 0, "the two paths should round differently"


def test_corrupted_ring_key_changes_output(gdn):
    """Negative test (vLLM PR #49887, Tests): corrupting one valid cached key
    must change the output of the heads that read it, and only those."""
    w = gi.scaled(gi.C2, name="corrupt", B=4, N=4, L=8, steps=5, stagger=False, seed=31)
    S0 = gi.initial_state(w)
    slots = gi.slot_map(w)
    pool = Pool(w, S0)
    slot_t = to_dev(slots)
    for t in range(w.steps):
        xi = dev_inputs(gi.step_inputs(w, t))
        gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, pool.ckpt, pool.ring_d,
                              pool.ring_k, pool.ring_g, pool.write_pos)
        gdn.gdn_replay_advance(slot_t, pool.write_pos, w.L)
    assert pool.write_pos.cpu().tolist() == [5, 5, 5, 5]
    xi = dev_inputs(gi.step_inputs(w, 99))
    saved = [x.clone() for x in (pool.ckpt, pool.ring_d, pool.ring_k, pool.ring_g)]
    o1 = gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, *saved[:1],
                               saved[1].clone(), saved[2].clone(), saved[3].clone(),
                               pool.write_pos)
    rk = saved[2].clone()
    rk[slots[1], 3, 2] = -rk[slots[1], 3, 2]          # slot of row 1, k-head 3, entry 2
    o2 = gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, saved[0].clone(),
                               saved[1].clone(), rk, saved[3].clone(), pool.write_pos)
    G = w.Hv // w.Hk
    diff = (bits(o1) != bits(o2)).any(dim=-1)[:, 0]    # [B, Hv]
    expect = torch.zeros_like(diff)
    expect[1, 3 * G:3 * G + G] = True
    assert torch.equal(diff, expect)
    e = rel_err(to_f64(o2[1, 0, 3 * G]), to_f64(o1[1, 0, 3 * G]))
    assert e > 1e-2


def test_forced_flush_mid_buffer_reads_only_valid_entries(gdn):
    """A forced flush in the middle of the ring (SGLang PR #28451, Design 5)
    folds only the entries below write_pos; garbage beyond them is never
    read. Covered by the staggered workloads too; here every slot is forced
    at a different depth and the rings start as a garbage template."""
    w = gi.scaled(gi.C2, name="midflush", B=8, N=8, L=8, steps=20, seed=41)
    run_decode(w, "replay", garbage=True, recon_every=5)


def test_device_error_flags(gdn):
    w = gi.scaled(gi.C2, name="errors", B=4, N=4, L=4, steps=1, stagger=False, seed=51)
    S0 = gi.initial_state(w)
    pool = Pool(w, S0)
    xi = dev_inputs(gi.step_inputs(w, 0))
    # slot index beyond the pool: EF_SLOT_RANGE, zero output, nothing written
    slots = to_dev(np.array([0, 9, 2, -1], np.int32))
    ck0 = pool.ckpt.clone()
    o = gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slots, pool.ckpt, pool.ring_d,
                              pool.ring_k, pool.ring_g, pool.write_pos, err_flags=pool.err)
    assert int(pool.err.item()) == gdn.EF_SLOT_RANGE
    assert torch.count_nonzero(o[1]).item() == 0 and torch.count_nonzero(o[3]).item() == 0
    assert torch.count_nonzero(o[0]).item() > 0
    # cursor out of range: EF_CURSOR_RANGE, row treated as padding
    pool.err.zero_()
    pool.write_pos.copy_(to_dev(np.array([0, 4, 0, 0], np.int32)))
    slots = to_dev(np.array([0, 1, 2, 3], np.int32))
    o = gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slots, pool.ckpt, pool.ring_d,
                              pool.ring_k, pool.ring_g, pool.write_pos, err_flags=pool.err)
    assert int(pool.err.item()) == gdn.EF_CURSOR_RANGE
    assert torch.count_nonzero(o[1]).item() == 0
    assert torch.equal(bits(pool.ckpt[1]), bits(ck0[1]))
    gdn.gdn_replay_advance(slots, pool.write_pos, w.L, err_flags=pool.err)
    assert pool.write_pos.cpu().tolist() == [1, 4, 1, 1]
    # verify window that does not fit: EF_WINDOW
    pool.err.zero_()
    wv = gi.scaled(w, T=3)
    xv = dev_inputs(gi.step_inputs(wv, 0))
    o = gdn.gdn_replay_decode(xv.q, xv.k, xv.v, xv.g, xv.beta, slots, pool.ckpt, pool.ring_d,
                              pool.ring_k, pool.ring_g, pool.write_pos, err_flags=pool.err,
                              window=True)
    # row 1 (p = 4, T = 3, L = 4) overflows the ring: exactly GDN_EF_WINDOW
    assert int(pool.err.item()) == gdn.EF_WINDOW
    assert torch.count_nonzero(o[1]).item() == 0 and torch.count_nonzero(o[0]).item() > 0
    # commit beyond the window: EF_ACCEPTED, cursor unchanged
    pool.err.zero_()
    acc = to_dev(np.array([4, 0, 1, 2], np.int32))
    gdn.gdn_replay_commit(slots, acc, pool.write_pos, w.L, 3, err_flags=pool.err)
    assert int(pool.err.item()) == gdn.EF_ACCEPTED
    assert pool.write_pos.cpu().tolist() == [1, 4, 2, 3]
    # fold with a cursor beyond the ring: EF_CURSOR_RANGE, checkpoint untouched
    pool.err.zero_()
    pool.write_pos.copy_(to_dev(np.array([1, 5, 0, 3], np.int32)))
    ck0 = pool.ckpt.clone()
    gdn.gdn_replay_fold(slots, pool.ckpt, pool.ring_d, pool.ring_k, pool.ring_g,
                        pool.write_pos, err_flags=pool.err)
    assert int(pool.err.item()) == gdn.EF_CURSOR_RANGE
    assert torch.equal(bits(pool.ckpt[1]), bits(ck0[1]))
    assert torch.equal(bits(pool.ckpt[2]), bits(ck0[2]))      # p = 0: nothing to fold
    assert pool.write_pos.cpu().tolist() == [1, 5, 0, 3]      # the fold only reads cursors
    # reset: every listed slot, out of range or not; a slot beyond the pool is flagged
    pool.err.zero_()
    gdn.gdn_replay_reset(to_dev(np.array([0, -1, 9, 1], np.int32)), pool.write_pos,
                         err_flags=pool.err)
    assert int(pool.err.item()) == gdn.EF_SLOT_RANGE
    assert pool.write_pos.cpu().tolist() == [0, 0, 0, 3]


@pytest.mark.parametrize("gate", ["head", "key"])
def test_decode_advance_equals_decode_then_advance(gdn, gate):
    """gdn_replay_decode_advance (the cursor advance fused into the last
    layer's decode) leaves outputs, checkpoints, rings and cursors bit for bit
    as gdn_replay_decode followed by gdn_replay_advance, with forced flushes,
    padding rows, a permuted pool and a row whose cursor is out of range; the
    arrive workspace is back to zero after every call."""
    w = gi.scaled(gi.C2, name=f"fused_adv_{gate}", B=16, N=20, L=4, steps=12, n_pad=2,
                  permute=True, gate=gate, seed=61)
    S0 = gi.initial_state(w)
    slots = gi.slot_map(w)
    a, b = Pool(w, S0), Pool(w, S0)
    slot_t = to_dev(slots)
    arrive = gdn.arrive_workspace(w.B, DEV)
    live = slots[slots >= 0]
    bad = int(live[3])
    for t in range(w.steps):
        if t == 5:                       # one slot's cursor out of range for one step
            for p in (a, b):
                p.write_pos[bad] = w.L
        if t == 6:
            for p in (a, b):
                p.write_pos[bad] = 0
        xi = dev_inputs(gi.step_inputs(w, t))
        ff = to_dev(gi.force_flush_schedule(w, t, slots))
        oa = gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, a.ckpt, a.ring_d,
                                   a.ring_k, a.ring_g, a.write_pos, force_flush=ff,
                                   err_flags=a.err)
        gdn.gdn_replay_advance(slot_t, a.write_pos, w.L, force_flush=ff, err_flags=a.err)
        ob = gdn.gdn_replay_decode_advance(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, b.ckpt,
                                           b.ring_d, b.ring_k, b.ring_g, b.write_pos, arrive,
                                           force_flush=ff, err_flags=b.err)
        assert torch.equal(bits(oa), bits(ob)), f"step {t}: outputs differ"
        assert torch.equal(a.write_pos, b.write_pos), f"step {t}: cursors differ"
        for x, y, name in zip((a.ckpt, a.ring_d, a.ring_k, a.ring_g),
                              (b.ckpt, b.ring_d, b.ring_k, b.ring_g), ("ckpt", "d", "k", "g")):
            assert torch.equal(bits(x), bits(y)), f"step {t}: {name} differs"
        assert int(arrive.abs().sum().item()) == 0, f"step {t}: arrive not cleared"
        assert int(a.err.item()) == int(b.err.item())
    assert int(b.err.item()) == gdn.EF_CURSOR_RANGE


@pytest.mark.parametrize("ring,gate", [("f16", "head"), ("f32", "head"), ("f16", "key")])
def test_maximum_sizes(gdn, ring, gate):
    """The largest supported sizes: dk = 256, dv = 512, L = 64 (70 decode steps,
    crossing the natural flush at step 64), then a T = 16 verify window and its
    fold; against the oracle."""
    qkv = "f32" if ring == "f32" else "bf16"
    w = gi.Workload(f"max_{ring}_{gate}", B=3, N=4, Hv=2, Hk=1, dk=256, dv=512, L=64,
                    steps=70, qkv=qkv, ring=ring, n_pad=1, permute=True, stagger=False,
                    bf16_values=(ring == "f32"), gate=gate, seed=990)
    TW = 16
    rep = run_decode(w, "replay", garbage=True, recon_every=35)
    assert rep.flushes == 2                         # two live rows, one natural flush each
    run_decode(dataclasses.replace(w, steps=3), "packed")
    wv = dataclasses.replace(w, T=TW, steps=1)
    S0 = gi.initial_state(wv)
    slots = gi.slot_map(wv)
    pool = Pool(wv, S0)
    x = gi.step_inputs(wv, 7)
    xi = dev_inputs(x)
    o = gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, to_dev(slots), pool.ckpt,
                              pool.ring_d, pool.ring_k, pool.ring_g, pool.write_pos,
                              err_flags=pool.err, window=True)
    from oracle import window_ref
    o_ref = window_ref(S0.astype(np.float64), slots, *x.f64())
    tol = 1e-4 if ring == "f32" else 2e-2
    assert rel_err(to_f64(o), o_ref) <= tol
    acc = to_dev(np.full(wv.B, TW, np.int32))
    gdn.gdn_replay_commit(to_dev(slots), acc, pool.write_pos, wv.L, TW, err_flags=pool.err)
    gdn.gdn_replay_fold(to_dev(slots), pool.ckpt, pool.ring_d, pool.ring_k, pool.ring_g,
                        pool.write_pos, err_flags=pool.err)
    S_true = S0.astype(np.float64)
    q, k, v, g, beta = x.f64()
    for t in range(TW):
        step(S_true, slots, q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t])
    live = slots[slots >= 0]
    assert rel_err(to_f64(pool.ckpt[torch.from_numpy(live).to(DEV)]), S_true[live]) <= tol
    assert int(pool.err.item()) == 0


@pytest.mark.parametrize("gate", ["head", "key"])
def test_batch_of_padding_rows_only(gdn, gate):
    """A batch whose every row is padding (slot -1): each entry point runs,
    returns zero outputs, writes no checkpoint, ring or cursor byte (checked
    bit for bit, with canary guards around the pool) and sets no error bit:
    the replay decode (step and window), the fused advance, the packed decode,
    the cursor calls and the fold."""
    w = gi.scaled(gi.C2, name=f"all_pad_{gate}", B=6, N=8, L=4, steps=1, gate=gate, seed=77)
    S0 = gi.initial_state(w)
    pool = Pool(w, S0, garbage=True, canary=True)
    # a nonzero phase, so that a stray advance or fold would change something
    pool.write_pos.copy_(to_dev(np.array([1, 2, 3, 0, 1, 2, 3, 0], np.int32)))
    snap = [bits(t).clone() for t in (pool.ckpt, pool.ring_d, pool.ring_k, pool.ring_g,
                                      pool.write_pos)]
    slots = to_dev(np.full(w.B, -1, np.int32))
    xi = dev_inputs(gi.step_inputs(w, 0))
    ff = to_dev(np.ones(w.B, np.int32))                 # forced flushes, ignored on padding
    o = gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slots, pool.ckpt, pool.ring_d,
                              pool.ring_k, pool.ring_g, pool.write_pos, force_flush=ff,
                              err_flags=pool.err)
    assert torch.count_nonzero(o).item() == 0
    arrive = gdn.arrive_workspace(w.B, DEV)
    o = gdn.gdn_replay_decode_advance(xi.q, xi.k, xi.v, xi.g, xi.beta, slots, pool.ckpt,
                                      pool.ring_d, pool.ring_k, pool.ring_g, pool.write_pos,
                                      arrive, force_flush=ff, err_flags=pool.err)
    assert torch.count_nonzero(o).item() == 0
    assert torch.count_nonzero(arrive).item() == 0      # the workspace is left zero
    xw = dev_inputs(gi.step_inputs(gi.scaled(w, T=3), 0))
    o = gdn.gdn_replay_decode(xw.q, xw.k, xw.v, xw.g, xw.beta, slots, pool.ckpt, pool.ring_d,
                              pool.ring_k, pool.ring_g, pool.write_pos, err_flags=pool.err,
                              window=True)
    assert torch.count_nonzero(o).item() == 0
    gdn.gdn_replay_advance(slots, pool.write_pos, w.L, force_flush=ff, err_flags=pool.err)
    gdn.gdn_replay_commit(slots, to_dev(np.full(w.B, 2, np.int32)), pool.write_pos, w.L, 3,
                          err_flags=pool.err)
    gdn.gdn_replay_fold(slots, pool.ckpt, pool.ring_d, pool.ring_k, pool.ring_g,
                        pool.write_pos, err_flags=pool.err)
    gdn.gdn_replay_reset(slots, pool.write_pos, err_flags=pool.err)
    torch.cuda.synchronize()
    for now, before, name in zip((pool.ckpt, pool.ring_d, pool.ring_k, pool.ring_g,
                                  pool.write_pos), snap, ("ckpt", "ring d", "ring k", "ring g",
                                                          "cursors")):
        assert torch.equal(bits(now), before), f"{name} changed"
    assert int(pool.err.item()) == 0
    pool.check_canaries("padding-only batch")
    state = pool.ckpt.clone()
    o = gdn.gdn_packed_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slots, state, err_flags=pool.err)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o).item() == 0
    assert torch.equal(bits(state), bits(pool.ckpt)) and int(pool.err.item()) == 0
    log(f"[padding-only/{gate}] every entry point: zero outputs, nothing written")
