"""GPU parity of the causal convolution step in front of the decode
(gdn_conv_update) against the oracle's O9, and of the whole front end
(convolution, then the replay decode reading the convolved packed row with
q/k normalised in the kernel) against O9 -> O8 -> O1.

The ReplaySSM blog (section 3.1) has the decode path update the causal
convolution before handing the packed row to the decode; SGLang PR #36821
(Technical principle) writes the step as x_hat_t = SiLU(w * x_{t-3:t}).

Tolerances, per element, from the arithmetic: the kernel sums the taps in
fp32 (absolute error below 2^-23 * sum_i |w_i z_i|) and evaluates SiLU in
fp32 (a few ulp), then rounds to the I/O type: bf16 adds at most half an ulp
(2^-9 relative). So |y - y_ref| <= rel * |y_ref| + abs * sum_i |w_i z_i| with
rel = 2^-8 (bf16) or 1e-6 (fp32) and abs = 1e-6. The window moves by copies
of inputs as given, so the state is compared bit for bit.
"""
import dataclasses

import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gdn_harness import DEV, Pool, log, to_dev, to_f64, tol_o, tol_state
from oracle import conv_update, l2norm_qk, quantize, rel_err, step

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import linear_attention_ssm_amd as m
    return m


def check_y(y, y_ref, w64, window, dtype, what):
    rel = 2.0 ** -8 if dtype == "bf16" else 1e-6
    mag = np.einsum("cw,bwc->bc", np.abs(w64), np.abs(window))
    err = np.abs(y - y_ref)
    bound = rel * np.abs(y_ref) + 1e-6 * mag
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} elements out of bound, worst " \
                          f"{np.max(err - bound):.3e}"
    return float(np.max(err / (np.abs(y_ref) + 1e-30)))


def run_conv(gdn, w, W, steps, C=None, strided=False, seed_tag=0):
    ci = gi.conv_inputs(w, steps, W=W, C=C, seed_tag=seed_tag)
    x64, w64, st64 = ci.f64()
    C = x64.shape[-1]
    slots = gi.slot_map(w)
    slot_t = to_dev(slots)
    dt = ci.dtype
    taps = to_dev(ci.w, dt)
    state = to_dev(ci.state, dt)
    ref_state = st64.copy()
    worst = 0.0
    for t in range(steps):
        if strided:
            # x and y as the first C columns of wider rows
            xb = torch.zeros((w.B, C + 12), dtype=taps.dtype, device=DEV)
            xb[:, :C] = to_dev(ci.x[t], dt)
            x = xb[:, :C]
            yb = torch.full((w.B, C + 20), 7.0, dtype=taps.dtype, device=DEV)
            y = gdn.gdn_conv_update(x, taps, state, slot_t, y=yb[:, :C])
            assert torch.all(yb[:, C:] == 7.0), "y written past its rows"
        else:
            y = gdn.gdn_conv_update(to_dev(ci.x[t], dt), taps, state, slot_t)
        windows = np.stack([np.concatenate([ref_state[s], x64[t][b][None]], 0)
                            if 0 <= s < w.N else np.zeros((W, C))
                            for b, s in enumerate(slots)])
        y_ref = conv_update(x64[t], w64, ref_state, slots)
        worst = max(worst, check_y(to_f64(y), y_ref, w64, windows, dt, f"{w.name} step {t}"))
        assert np.array_equal(to_f64(state), ref_state), f"{w.name} step {t}: window differs"
    return worst


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("W", [2, 3, 4])
def test_conv_tiny_vs_oracle(gdn, dtype, W):
    """The tiny workload's packed row (C = 192), permuted slots, a padding row."""
    w = gi.scaled(gi.C1, name=f"conv_tiny_{dtype}_{W}", B=5, N=7, qkv=dtype, n_pad=1,
                  permute=True, seed=900 + W)
    e = run_conv(gdn, w, W, steps=6)
    log(f"[conv tiny {dtype} W={W}] worst rel {e:.2e}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv_ragged_and_strided(gdn, dtype):
    """C = 148 (a partial workgroup of channel groups) with x and y as views
    into wider rows."""
    w = gi.scaled(gi.C1, name=f"conv_ragged_{dtype}", B=6, N=9, qkv=dtype, n_pad=2,
                  permute=True, seed=910)
    run_conv(gdn, w, 4, steps=4, C=148, strided=True)


def test_conv_standard_row(gdn):
    """The standard workload's packed row: B = 64, C = 8192, bf16, width 4."""
    run_conv(gdn, gi.C2, 4, steps=3, seed_tag=1)


def test_conv_slot_out_of_pool(gdn):
    w = gi.scaled(gi.C1, name="conv_oob", B=3, N=2, qkv="f32", seed=920)
    ci = gi.conv_inputs(w, 1, W=4)
    state = to_dev(ci.state)
    before = state.clone()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    slots = to_dev(np.array([1, 5, -1], np.int32))
    y = gdn.gdn_conv_update(to_dev(ci.x[0]), to_dev(ci.w), state, slots, err_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) == gdn.EF_SLOT_RANGE
    assert torch.all(y[1:] == 0)
    assert torch.equal(state[0], before[0]) and not torch.equal(state[1], before[1])


def test_front_end_conv_then_replay_decode(gdn):
    """The whole front end: the raw packed row goes through the convolution,
    the replay decode reads q, k, v as views into the convolved row and
    normalises q and k in the kernel. The oracle runs O9, rounds the row to
    bf16 as the device stores it (O5), splits it, normalises (O8) and steps
    the recurrence (O1). bf16 row, decode steps with staggered forced
    flushes."""
    w = gi.scaled(gi.C2, name="front_end_conv", B=8, N=10, L=4, steps=10, qk_raw=True,
                  n_pad=1, permute=True, seed=930)
    ci = gi.conv_inputs(w, w.steps, W=4)
    x64, w64, st64 = ci.f64()
    S0 = gi.initial_state(w)
    slots = gi.slot_map(w)
    slot_t = to_dev(slots)
    pool = Pool(w, S0)
    taps = to_dev(ci.w, "bf16")
    cstate = to_dev(ci.state, "bf16")
    ref_cstate = st64.copy()
    S_true = S0.astype(np.float64)
    nq, nv = w.Hk * w.dk, w.Hv * w.dv
    wp = np.zeros(w.N, np.int64)
    worst_o = worst_s = 0.0
    for t in range(w.steps):
        x = gi.step_inputs(w, t)                    # g and beta of the step
        y = gdn.gdn_conv_update(to_dev(ci.x[t], "bf16"), taps, cstate, slot_t)
        B = w.B
        q = y[:, :nq].view(B, 1, w.Hk, w.dk)
        k = y[:, nq:2 * nq].view(B, 1, w.Hk, w.dk)
        v = y[:, 2 * nq:].view(B, 1, w.Hv, w.dv)
        g = torch.from_numpy(x.g).to(DEV)
        beta = torch.from_numpy(x.beta).to(DEV)
        ff = gi.force_flush_schedule(w, t, slots)
        o = gdn.gdn_replay_decode(q, k, v, g, beta, slot_t, pool.ckpt, pool.ring_d,
                                  pool.ring_k, pool.ring_g, pool.write_pos,
                                  force_flush=to_dev(ff), qk_norm=True)
        gdn.gdn_replay_advance(slot_t, pool.write_pos, w.L, force_flush=to_dev(ff))
        # oracle: O9, the row stored in the I/O type (O5 rounds it to bf16),
        # split into q, k, v, then O8 and O1
        y_ref = quantize(conv_update(x64[t], w64, ref_cstate, slots), "bf16")
        assert rel_err(to_f64(y), y_ref) <= 2.0 ** -7
        q64 = y_ref[:, :nq].reshape(B, w.Hk, w.dk)
        k64 = y_ref[:, nq:2 * nq].reshape(B, w.Hk, w.dk)
        v64 = y_ref[:, 2 * nq:].reshape(B, w.Hv, w.dv)
        qn, kn = l2norm_qk(q64, k64)
        o_ref = step(S_true, slots, qn, kn, v64, x.g[:, 0].astype(np.float64),
                     x.beta[:, 0].astype(np.float64))
        e = rel_err(to_f64(o[:, 0]), o_ref)
        worst_o = max(worst_o, e)
        assert e <= tol_o(w), f"step {t}: o rel err {e:.3e}"
        for bi, s in enumerate(slots):
            if s < 0:
                continue
            if wp[s] == w.L - 1 or ff[bi]:
                es = rel_err(to_f64(pool.ckpt[s]), S_true[s])
                worst_s = max(worst_s, es)
                assert es <= tol_state(w)
                wp[s] = 0
            else:
                wp[s] += 1
        assert np.array_equal(to_f64(cstate), ref_cstate), f"step {t}: conv window differs"
    log(f"[front end conv] o {worst_o:.2e} ckpt {worst_s:.2e}")
