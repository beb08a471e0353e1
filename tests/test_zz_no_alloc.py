"""gdn_replay_decode_advance_noalloc (the cursor advance fused into a decode
step, counting in the library's static device scratch instead of a caller's
workspace) against gdn_replay_decode_advance: outputs, checkpoints, rings,
cursors and error bits bit for bit, call after call, with the batch shrinking
from one call to the next (the scratch keeps what the previous call left)."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gdn_harness import DEV, Pool, bits, dev_inputs, log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import linear_attention_ssm_amd as m
    return m


@pytest.mark.parametrize("gate", ["head", "key"])
def test_noalloc_equals_workspace_variant(gdn, gate):
    # the standard sizes (Hv = 32, Hk = 16, dk = dv = 128, L = 16) over a pool
    # of 64 slots; calls alternate between all 64 rows and a smaller batch of
    # 24 rows (8 of them padding) over a permuted subset of the slots
    w = gi.scaled(gi.C2, name=f"noalloc_{gate}", B=64, N=64, steps=20, gate=gate, seed=4242)
    S0 = gi.initial_state(w)
    big = gi.slot_map(w)
    r = np.random.default_rng(w.seed)
    small = r.permutation(w.N)[:24].astype(np.int32)
    small[r.choice(24, size=8, replace=False)] = -1
    a, b = Pool(w, S0, canary=True), Pool(w, S0, canary=True)
    for t in range(w.steps):
        slots = big if t % 2 == 0 else small
        B = len(slots)
        ws = gi.scaled(w, B=B)
        xi = dev_inputs(gi.step_inputs(ws, t))
        slot_t = to_dev(slots)
        ff = to_dev(gi.force_flush_schedule(ws, t, slots) if t < w.L else
                    np.zeros(B, np.int32))
        arrive = gdn.arrive_workspace(B, DEV)
        oa = gdn.gdn_replay_decode_advance(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, a.ckpt,
                                           a.ring_d, a.ring_k, a.ring_g, a.write_pos, arrive,
                                           force_flush=ff, err_flags=a.err)
        ob = torch.empty_like(oa)
        gdn.gdn_replay_decode_advance_noalloc(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, b.ckpt,
                                              b.ring_d, b.ring_k, b.ring_g, b.write_pos, ob,
                                              force_flush=ff, err_flags=b.err)
        torch.cuda.synchronize()
        assert torch.equal(bits(oa), bits(ob)), f"step {t} (B={B}): outputs differ"
        assert torch.equal(a.write_pos, b.write_pos), f"step {t}: cursors differ"
        for x, y, name in zip((a.ckpt, a.ring_d, a.ring_k, a.ring_g),
                              (b.ckpt, b.ring_d, b.ring_k, b.ring_g), ("ckpt", "d", "k", "g")):
            assert torch.equal(bits(x), bits(y)), f"step {t}: {name} differs"
        assert int(a.err.item()) == int(b.err.item()) == 0
        b.check_canaries(f"step {t}")
    live = big[big >= 0]
    assert int(b.write_pos[to_dev(live).long()].abs().sum().item()) > 0   # cursors moved
    log(f"[noalloc/{gate}] {w.steps} calls equal to the workspace variant")


def test_noalloc_at_its_row_limit(gdn):
    """GDN_SCRATCH_MAX_ROWS rows in one call (every arrival counter of the
    static scratch in use), then a call of 100 rows, then the limit again,
    each equal to the workspace variant bit for bit. Small heads (Hv = 2,
    Hk = 1, dk = dv = 32, L = 4, bf16 inputs, fp16 ring) keep the pool at
    about 34 MB."""
    B = gdn.SCRATCH_MAX_ROWS
    w = gi.scaled(gi.C1, name="noalloc_limit", B=B, N=B, Hv=2, Hk=1, qkv="bf16", ring="f16",
                  stagger=True, steps=3, seed=4343)
    S0 = gi.initial_state(w)
    full = gi.slot_map(w)
    few = np.random.default_rng(w.seed).permutation(w.N)[:100].astype(np.int32)
    a, b = Pool(w, S0, canary=True), Pool(w, S0, canary=True)
    for t, slots in enumerate((full, few, full)):
        n = len(slots)
        ws = gi.scaled(w, B=n)
        xi = dev_inputs(gi.step_inputs(ws, t))
        slot_t = to_dev(slots)
        ff = to_dev(gi.force_flush_schedule(ws, t, slots))
        arrive = gdn.arrive_workspace(n, DEV)
        oa = gdn.gdn_replay_decode_advance(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, a.ckpt,
                                           a.ring_d, a.ring_k, a.ring_g, a.write_pos, arrive,
                                           force_flush=ff, err_flags=a.err)
        ob = torch.empty_like(oa)
        gdn.gdn_replay_decode_advance_noalloc(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, b.ckpt,
                                              b.ring_d, b.ring_k, b.ring_g, b.write_pos, ob,
                                              force_flush=ff, err_flags=b.err)
        torch.cuda.synchronize()
        assert torch.equal(bits(oa), bits(ob)), f"call {t} ({n} rows): outputs differ"
        assert torch.equal(a.write_pos, b.write_pos), f"call {t}: cursors differ"
        for x, y, name in zip((a.ckpt, a.ring_d, a.ring_k, a.ring_g),
                              (b.ckpt, b.ring_d, b.ring_k, b.ring_g), ("ckpt", "d", "k", "g")):
            assert torch.equal(bits(x), bits(y)), f"call {t}: {name} differs"
        assert int(a.err.item()) == int(b.err.item()) == 0
        b.check_canaries(f"call {t}")
    assert int((b.write_pos != 0).sum().item()) > 0                       # cursors moved
    log(f"[noalloc/limit] {B} rows, 100 rows, {B} rows: equal to the workspace variant")
