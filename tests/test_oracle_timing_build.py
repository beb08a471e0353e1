"""The CPU baseline's builds of the oracle: the fp32 instance of O1 and the
threaded -O3 timing library agree with the fp64 parity build (they are only
timed, never used to judge parity)."""
import numpy as np

import gdn_inputs as gi
import oracle


def _case():
    w = gi.scaled(gi.C2, name="timing_pin", B=6, N=8, Hv=4, Hk=2, steps=3, n_pad=1, permute=True,
                  seed=2024)
    return w, gi.initial_state(w).astype(np.float64), gi.slot_map(w)


def test_fp32_instance_tracks_the_fp64_recurrence():
    w, S, slots = _case()
    S32 = S.astype(np.float32)
    for t in range(w.steps):
        q, k, v, g, beta = (a[:, 0] for a in gi.step_inputs(w, t).f64())
        o64 = oracle.gdn_step(S, slots, q, k, v, g, beta)
        o32 = oracle.gdn_step_f32(S32, slots, q, k, v, g, beta)
        assert oracle.rel_err(o32, o64) < 1e-5
        assert oracle.rel_err(S32, S) < 1e-5
    assert np.all(o32[slots < 0] == 0)


def test_threaded_timing_build_equals_the_parity_build(tmp_path):
    L, flags = oracle.timing_library(str(tmp_path))
    assert "-fopenmp" in flags
    assert L.oracle_threads(4) >= 1
    w, S, slots = _case()
    S2 = S.copy()
    for t in range(w.steps):
        q, k, v, g, beta = (np.ascontiguousarray(a[:, 0]) for a in gi.step_inputs(w, t).f64())
        o_ref = oracle.gdn_step(S, slots, q, k, v, g, beta)
        o = np.empty_like(o_ref)
        L.oracle_gdn_step_f64(w.B, w.N, w.Hv, w.Hk, w.dk, w.dv, oracle._p(slots.astype(np.int32)),
                              oracle._p(S2), oracle._p(q), oracle._p(k), oracle._p(v),
                              oracle._p(g), oracle._p(beta), oracle._p(o), None)
        # the same operations per (row, head); -O3 may contract multiply-adds
        assert oracle.rel_err(o, o_ref) < 1e-12
    assert oracle.rel_err(S2, S) < 1e-12
