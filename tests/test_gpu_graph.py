"""The decode path under HIP-graph capture and through prepared calls.

A forward (two layers' replay decodes plus the cursor advance) is captured
once and replayed several times; after every replay (with eager work and a
synchronisation in between) its outputs, checkpoints, rings and cursors must
equal, bit for bit, those of the same forward run eagerly on a twin pool. The
kernels are deterministic (fixed reduction order, no atomics on data), so
equality is exact. The prepared-call path must match the plain call the same
way."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gdn_harness import DEV, Pool, bits, dev_inputs, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import linear_attention_ssm_amd as m
    return m


def _state(p):
    return [bits(t).clone() for t in (p.ckpt, p.ring_d, p.ring_k, p.ring_g)] + [p.write_pos.clone()]


@pytest.mark.parametrize("fused,gate", [(False, "head"), (True, "head"), (True, "key")])
def test_graph_replays_match_eager(gdn, fused, gate):
    """fused: the second layer's call is gdn_replay_decode_advance (its
    arrival counters must come back to zero after every replay)."""
    w = gi.scaled(gi.C2, name="graph", B=8, N=12, L=4, steps=1, stagger=False, permute=True,
                  n_pad=1, gate=gate, seed=71)
    S0 = gi.initial_state(w)
    slots = to_dev(gi.slot_map(w))
    eager = [Pool(w, S0), Pool(w, S0)]           # two layers sharing one cursor array
    graphd = [Pool(w, S0), Pool(w, S0)]
    wp_e = torch.zeros(w.N, dtype=torch.int32, device=DEV)
    wp_g = torch.zeros(w.N, dtype=torch.int32, device=DEV)
    xi = dev_inputs(gi.step_inputs(w, 0))
    o_e = torch.empty((w.B, 1, w.Hv, w.dv), dtype=torch.bfloat16, device=DEV)
    o_g = torch.empty_like(o_e)

    arrive_e = gdn.arrive_workspace(w.B, DEV)
    arrive_g = gdn.arrive_workspace(w.B, DEV)

    def forward(pools, wp, o, arrive):
        for i, p in enumerate(pools):
            if fused and i == len(pools) - 1:
                gdn.gdn_replay_decode_advance(xi.q, xi.k, xi.v, xi.g, xi.beta, slots, p.ckpt,
                                              p.ring_d, p.ring_k, p.ring_g, wp, arrive, o=o)
            else:
                gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slots, p.ckpt, p.ring_d,
                                      p.ring_k, p.ring_g, wp, o=o)
        if not fused:
            gdn.gdn_replay_advance(slots, wp, w.L)

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        forward(graphd, wp_g, o_g, arrive_g)
    torch.cuda.synchronize()
    for step in range(6):                          # crosses a natural flush (L = 4)
        forward(eager, wp_e, o_e, arrive_e)
        g.replay()
        torch.cuda.synchronize()
        _ = (o_e.float() * 2).sum().item()         # unrelated eager work between replays
        assert torch.equal(bits(o_e), bits(o_g)), f"replay {step}: outputs differ"
        for a, b in zip(_state(eager[0]) + _state(eager[1]), _state(graphd[0]) + _state(graphd[1])):
            assert torch.equal(a, b), f"replay {step}: state differs"
        assert torch.equal(wp_e, wp_g)
        assert int(arrive_g.abs().sum().item()) == 0 and int(arrive_e.abs().sum().item()) == 0
    assert int(wp_e.max().item()) < w.L


def test_graph_verify_round_matches_eager(gdn):
    """A speculative round captured once and replayed: two layers' verify
    windows from their checkpoints, the commit of the accepted prefix, both
    layers' folds in one gdn_replay_fold_layers call and the cursor reset.
    After every replay (eager work and a synchronisation in between) the
    outputs, checkpoints, rings and cursors equal, bit for bit, those of the
    same round run eagerly on a twin pool."""
    w = gi.scaled(gi.C5, name="graph_round", B=8, N=12, T=3, steps=1, permute=True, n_pad=1,
                  seed=73)
    S0 = gi.initial_state(w)
    slots = to_dev(gi.slot_map(w))
    eager = [Pool(w, S0), Pool(w, S0)]
    graphd = [Pool(w, S0), Pool(w, S0)]
    wp_e = torch.zeros(w.N, dtype=torch.int32, device=DEV)
    wp_g = torch.zeros(w.N, dtype=torch.int32, device=DEV)
    xi = dev_inputs(gi.step_inputs(w, 0))
    acc = to_dev(gi.accepted_counts(w, 0))
    assert int(acc.max().item()) > 0
    o_e = torch.empty((w.B, w.T, w.Hv, w.dv), dtype=torch.bfloat16, device=DEV)
    o_g = torch.empty_like(o_e)

    def round_(pools, wp, o):
        for p in pools:
            gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slots, p.ckpt, p.ring_d,
                                  p.ring_k, p.ring_g, wp, o=o, window=True)
        gdn.gdn_replay_commit(slots, acc, wp, w.L, w.T)
        gdn.gdn_replay_fold_layers(slots, [p.ckpt for p in pools], [p.ring_d for p in pools],
                                   [p.ring_k for p in pools], [p.ring_g for p in pools], wp)
        gdn.gdn_replay_reset(slots, wp)

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        round_(graphd, wp_g, o_g)
    torch.cuda.synchronize()
    for step in range(4):
        round_(eager, wp_e, o_e)
        g.replay()
        torch.cuda.synchronize()
        _ = (o_e.float() * 2).sum().item()         # unrelated eager work between replays
        assert torch.equal(bits(o_e), bits(o_g)), f"replay {step}: outputs differ"
        for a, b in zip(_state(eager[0]) + _state(eager[1]), _state(graphd[0]) + _state(graphd[1])):
            assert torch.equal(a, b), f"replay {step}: state differs"
        assert torch.equal(wp_e, wp_g)
        assert int(wp_e.abs().sum().item()) == 0


def test_prepared_call_matches_plain_call(gdn):
    w = gi.scaled(gi.C2, name="prepared", B=6, N=6, L=8, steps=1, stagger=False, seed=72)
    S0 = gi.initial_state(w)
    slots = to_dev(gi.slot_map(w))
    a, b = Pool(w, S0), Pool(w, S0)
    xi = dev_inputs(gi.step_inputs(w, 0))
    call, o_b = gdn.prepare_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slots, b.ckpt,
                                          b.ring_d, b.ring_k, b.ring_g, b.write_pos)
    for step in range(3):
        o_a = gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slots, a.ckpt, a.ring_d,
                                    a.ring_k, a.ring_g, a.write_pos)
        gdn.gdn_replay_advance(slots, a.write_pos, w.L)
        call()
        gdn.gdn_replay_advance(slots, b.write_pos, w.L)
        torch.cuda.synchronize()
        assert torch.equal(bits(o_a), bits(o_b))
        for x, y in zip(_state(a), _state(b)):
            assert torch.equal(x, y)
    pa = Pool(w, S0)
    pcall, o_p = gdn.prepare_packed_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slots, pa.ckpt)
    pcall()
    st = to_dev(S0)
    o_q = gdn.gdn_packed_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slots, st)
    torch.cuda.synchronize()
    assert torch.equal(bits(o_p), bits(o_q)) and torch.equal(bits(pa.ckpt), bits(st))


def test_graph_conv_front_end_matches_eager(gdn):
    """The front end with the convolution under capture: per layer
    gdn_conv_update on a raw packed row, then the replay decode reading the
    convolved row with q/k normalised in the kernel; the last layer advances
    the cursors. Every replay (eager work between) equals the eager run on
    twin buffers bit for bit, conv windows included."""
    w = gi.scaled(gi.C2, name="graph_conv", B=8, N=12, L=4, steps=6, stagger=False,
                  permute=True, n_pad=1, qk_raw=True, seed=73)
    S0 = gi.initial_state(w)
    slots = to_dev(gi.slot_map(w))
    ci = gi.conv_inputs(w, w.steps, W=4)
    taps = to_dev(ci.w, "bf16")
    nq = w.Hk * w.dk
    xi = dev_inputs(gi.step_inputs(w, 0))             # g and beta
    xs = to_dev(ci.x[0], "bf16")

    def twin():
        return dict(pools=[Pool(w, S0), Pool(w, S0)],
                    cst=[to_dev(ci.state, "bf16"), to_dev(ci.state, "bf16")],
                    y=[torch.empty_like(xs), torch.empty_like(xs)],
                    o=torch.empty((w.B, 1, w.Hv, w.dv), dtype=torch.bfloat16, device=DEV),
                    wp=torch.zeros(w.N, dtype=torch.int32, device=DEV),
                    arrive=gdn.arrive_workspace(w.B, DEV))

    def forward(t):
        for i, p in enumerate(t["pools"]):
            y = gdn.gdn_conv_update(xs, taps, t["cst"][i], slots, y=t["y"][i])
            q = y[:, :nq].view(w.B, 1, w.Hk, w.dk)
            k = y[:, nq:2 * nq].view(w.B, 1, w.Hk, w.dk)
            v = y[:, 2 * nq:].view(w.B, 1, w.Hv, w.dv)
            if i == len(t["pools"]) - 1:
                gdn.gdn_replay_decode_advance(q, k, v, xi.g, xi.beta, slots, p.ckpt, p.ring_d,
                                              p.ring_k, p.ring_g, t["wp"], t["arrive"],
                                              o=t["o"], qk_norm=True)
            else:
                gdn.gdn_replay_decode(q, k, v, xi.g, xi.beta, slots, p.ckpt, p.ring_d,
                                      p.ring_k, p.ring_g, t["wp"], o=t["o"], qk_norm=True)

    e, gd = twin(), twin()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        forward(gd)
    torch.cuda.synchronize()
    for step in range(w.steps):                    # crosses a natural flush (L = 4)
        forward(e)
        g.replay()
        torch.cuda.synchronize()
        _ = (e["o"].float() * 2).sum().item()      # unrelated eager work between replays
        assert torch.equal(bits(e["o"]), bits(gd["o"])), f"replay {step}: outputs differ"
        for i in range(2):
            assert torch.equal(bits(e["cst"][i]), bits(gd["cst"][i])), f"replay {step}: window"
            assert torch.equal(bits(e["y"][i]), bits(gd["y"][i]))
            for a, b in zip(_state(e["pools"][i]), _state(gd["pools"][i])):
                assert torch.equal(a, b), f"replay {step}: state differs"
        assert torch.equal(e["wp"], gd["wp"])
