"""GPU parity of the 16-bit (bf16 / fp16) state against the CPU oracle.

The state is stored in 16 bits and every kernel computes in fp32 from the
exactly widened values. The packed decode rounds the state after every token
(the per-step quantized recurrence, oracle gdn_step with state_fmt); the
ReplaySSM decode rounds the checkpoint only when it writes it, at a flush
(oracle ReplayModel with state_fmt, the reading of vLLM PR #49887's review
thread); the fold rounds once, after the exact fp32 fold (oracle fold_f32,
then the O5 rounding). Expected values come from the oracle only.

Tolerance (max |x - ref| <= tol * max |ref|): 2e-2 for outputs and states.
The GPU rounds fp32 results and the oracle fp64 results to the same 16-bit
format, so a stored element may differ by one unit in its last place (2^-8
relative for bf16, 2^-11 for fp16); the decay alpha < 1 attenuates such
differences from step to step. Cursors and flush positions are exact; the
fold and the L = 1 identity are bitwise.
"""
import dataclasses

import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gdn_harness import DEV, Pool, bits, dev_inputs, log, to_dev, to_f64
from oracle import ReplayModel, fold_f32, gdn_step, next_cursor, quantize, rel_err, step

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module")
def gdn():
    import linear_attention_ssm_amd as m
    return m


def state_tensor(w):
    """The initial state pool on the device in the state dtype, and its exact
    fp64 values."""
    st = gi.stored_state(w)
    return to_dev(st, w.state), gi.as_f64(st, w.state)


def make_pool(w):
    pool = Pool(w, gi.initial_state(w))
    pool.ckpt, S0 = state_tensor(w)
    return pool, S0


def run_packed16(gdn, w):
    slots = gi.slot_map(w)
    state, S0 = state_tensor(w)
    rows = np.where(slots >= 0)[0]
    S_ref = S0[slots[rows]].copy()
    sub = np.arange(len(rows), dtype=np.int32)
    slot_t = to_dev(slots)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    worst_o = worst_s = 0.0
    for t in range(w.steps):
        x = gi.step_inputs(w, t)
        xi = dev_inputs(x)
        o = gdn.gdn_packed_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, state, err_flags=err)
        q, k, v, g, beta = (a[rows, 0] for a in x.f64())
        o_ref = step(S_ref, sub, q, k, v, g, beta, state_fmt=w.state)
        eo = rel_err(to_f64(o[rows, 0]), o_ref)
        es = rel_err(to_f64(state[torch.from_numpy(slots[rows].astype(np.int64)).to(DEV)]), S_ref)
        worst_o, worst_s = max(worst_o, eo), max(worst_s, es)
        assert eo <= TOL, f"{w.name} step {t}: o rel err {eo:.3e}"
        assert es <= TOL, f"{w.name} step {t}: state rel err {es:.3e}"
    assert int(err.item()) == 0
    log(f"[{w.name}/packed16] o {worst_o:.2e} state {worst_s:.2e}")


def run_replay16(gdn, w, check_untouched=False):
    slots = gi.slot_map(w)
    pool, S0 = make_pool(w)
    model = ReplayModel(S0, w.Hk, w.L, state_fmt=w.state, gate=w.gate)
    live = np.where(slots >= 0)[0]
    rows = live
    slot_t = to_dev(slots)
    ck0 = pool.ckpt.clone()
    worst_o = worst_s = 0.0
    flushes = 0
    for t in range(w.steps):
        x = gi.step_inputs(w, t)
        xi = dev_inputs(x)
        ff = gi.force_flush_schedule(w, t, slots)
        ff_t = to_dev(ff)
        ck_before = pool.ckpt.clone()
        o = gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, pool.ckpt, pool.ring_d,
                                  pool.ring_k, pool.ring_g, pool.write_pos, force_flush=ff_t,
                                  err_flags=pool.err)
        gdn.gdn_replay_advance(slot_t, pool.write_pos, w.L, force_flush=ff_t, err_flags=pool.err)
        q, k, v, g, beta = (a[:, 0] for a in x.f64())
        o_ref, flush = model.decode(slots, q, k, v, g, beta, force_flush=ff)
        model.advance(slots, flush)
        eo = rel_err(to_f64(o[rows, 0]), o_ref[rows])
        worst_o = max(worst_o, eo)
        assert eo <= TOL, f"{w.name} step {t}: o rel err {eo:.3e}"
        assert np.array_equal(pool.write_pos.cpu().numpy(), model.write_pos), \
            f"{w.name} step {t}: cursor mismatch"
        changed = (bits(pool.ckpt) != bits(ck_before)).flatten(1).any(dim=1).cpu().numpy()
        exp = np.zeros(w.N, dtype=bool)
        exp[slots[live]] = flush[live]
        assert np.array_equal(changed[slots[live]], exp[slots[live]]), \
            f"{w.name} step {t}: flush positions differ"
        for r in rows:
            if flush[r]:
                s = slots[r]
                ck = to_f64(pool.ckpt[s])
                # the written checkpoint holds values of the state format
                assert np.array_equal(quantize(ck, w.state), ck)
                es = rel_err(ck, model.ckpt[s])
                worst_s = max(worst_s, es)
                flushes += 1
                assert es <= TOL, f"{w.name} step {t}: checkpoint rel err {es:.3e}"
    assert int(pool.err.item()) == 0
    if check_untouched:
        idle = np.setdiff1d(np.arange(w.N), slots[live])
        it = torch.from_numpy(idle).to(DEV)
        assert torch.equal(bits(pool.ckpt[it]), bits(ck0[it])), "an unused slot changed"
    log(f"[{w.name}/replay16] o {worst_o:.2e} ckpt {worst_s:.2e} flushes checked {flushes}")
    return flushes


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_packed_state16_small(gdn, fmt):
    w = gi.scaled(gi.C2, name=f"packed16_{fmt}", B=6, N=9, Hv=4, Hk=2, steps=24, n_pad=1,
                  permute=True, state=fmt, seed=1600)
    run_packed16(gdn, w)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_replay_state16_small(gdn, fmt):
    """Staggered cursors (one forced flush per slot in the first L steps),
    then natural flushes every L steps."""
    w = gi.scaled(gi.C2, name=f"replay16_{fmt}", B=6, N=9, Hv=4, Hk=2, L=8, steps=30, n_pad=1,
                  permute=True, state=fmt, seed=1610)
    assert run_replay16(gdn, w, check_untouched=True) > 0


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_c2_standard_state16(gdn, fmt):
    """The standard workload's sizes (B = 64, Hv = 32, Hk = 16, dk = dv = 128,
    L = 16) with a 16-bit checkpoint, every live row checked every step."""
    w = dataclasses.replace(gi.C2, name=f"c2_state16_{fmt}", steps=24, state=fmt)
    run_replay16(gdn, w)
    run_packed16(gdn, dataclasses.replace(w, steps=8))


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("dims", [(64, 48, 6, 2), (32, 16, 3, 3), (256, 128, 4, 1)])
def test_state16_ragged_shapes(gdn, fmt, dims):
    dk, dv, Hv, Hk = dims
    w = gi.Workload(f"ragged16_{dk}_{dv}_{Hv}_{Hk}_{fmt}", B=5, N=7, Hv=Hv, Hk=Hk, dk=dk, dv=dv,
                    L=5, steps=13, n_pad=1, permute=True, state=fmt, seed=1700 + dk + dv + Hv)
    run_replay16(gdn, w)
    run_packed16(gdn, w)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_L1_replay_equals_packed_state16_bitwise(gdn, fmt):
    """At L = 1 every replay step flushes from an empty ring: the replay and
    packed decodes read the same 16-bit state, compute the same fp32 values
    and round them once, so they agree bit for bit."""
    w = dataclasses.replace(gi.c4(1), steps=6, n_pad=2, permute=True, N=80, state=fmt)
    slots = gi.slot_map(w)
    a, _ = make_pool(w)
    state, _ = state_tensor(w)
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
@pytest.mark.parametrize("ring", ["f16", "bf16", "f32"])
def test_fold_state16_bitexact(gdn, fmt, ring):
    """The fold runs the pinned fp32 recurrence from the widened checkpoint
    and rounds once: bit for bit the oracle's fold_f32 followed by the O5
    rounding to the state format."""
    w = gi.Workload(f"fold16_{fmt}_{ring}", B=6, N=8, Hv=4, Hk=2, dk=128, dv=64, L=16, steps=1,
                    ring=ring, n_pad=1, permute=True, state=fmt, seed=1800)
    rc = gi.random_ring(w, seed_tag=3)
    ck16 = gi.cast(rc.ckpt, fmt)
    slots = gi.slot_map(w)
    ckpt = to_dev(ck16, fmt)
    rd, rk = to_dev(rc.d, ring), to_dev(rc.k, ring)
    rg, wp = to_dev(rc.g), to_dev(rc.write_pos)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    gdn.gdn_replay_fold(to_dev(slots), ckpt, rd, rk, rg, wp, err_flags=err)
    ref32 = gi.as_f64(ck16, fmt).astype(np.float32)
    fold_f32(ref32, slots, rc.write_pos, gi.as_f64(rc.d, ring).astype(np.float32),
             gi.as_f64(rc.k, ring).astype(np.float32), rc.g)
    ref = gi.cast(quantize(ref32.astype(np.float64), fmt).astype(np.float32), fmt)
    got = ckpt.cpu()
    got = got.view(torch.int16).numpy().view(np.uint16) if fmt == "bf16" else got.numpy()
    same = np.array_equal(np.asarray(got).view(np.uint16), np.asarray(ref).view(np.uint16))
    assert same, f"{int((np.asarray(got).view(np.uint16) != np.asarray(ref).view(np.uint16)).sum())} elements differ"
    assert int(err.item()) == 0
