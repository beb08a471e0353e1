"""Benchmark of the ReplaySSM GDN decode step on one MI355X.

One step = one decode forward of the standard workload (B = 64 rows, Hv = 32,
Hk = 16, dk = dv = 128, ring L = 16, fp32 checkpoint, bf16 q/k/v/o, fp16 d/k
ring, staggered cursors) through R = 8 GDN layers: one gdn_replay_decode call
per layer, each on its own checkpoint + ring set; the last layer's call is
gdn_replay_decode_advance, which also advances the cursors (they are shared
by the layers and advance once per forward). The 8 layer sets (~1.1 GiB)
exceed the 256 MB Infinity Cache, so the checkpoint is streamed from HBM as in
a real multi-layer model.

Printed: one JSON line with head-steps/s (value), the HBM roofline of the
replay decode kernel (per-launch HIP events on the launch stream, against the
8 TB/s specification and against the read bandwidth measured on the same GPU
with the library's read probe; the read + write kernels against its copy
probe), the packed read-update-write decode built
alongside it, the no-flush ("best") mode, the large-pool and ring-depth
workloads, the 16-bit-state, per-key-gate and front-end variants, the verify
window + fold of the speculative workload (the fold one layer per launch and
all layers in one gdn_replay_fold_layers launch), lossless verify, the pages' own
context figures, and the CPU oracle baseline on the host's cores.

Modes for profiling runs (same kernels, fewer steps, no CPU baseline):
  --profile-pass   warmup + a few timed steps of each kernel
  --copy-probe     one plain 1 GiB device copy (counter calibration)
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gdn_inputs as gi  # noqa: E402

HBM_PEAK_GBS = 8000.0
METRIC = "GDN decode head-steps/sec and achieved HBM GB/s (% of peak) at B=64, L=16"
PROFILES = os.path.join(ROOT, "profiles")
# every source that decides what the timed kernels do: the kernels, the
# launch geometry and dispatch
KERNEL_SOURCES = ["linear_attention_ssm_amd/csrc/gdn_kernels.h",
                  "linear_attention_ssm_amd/csrc/gdn_device.h",
                  "linear_attention_ssm_amd/csrc/gdn_api.hip",
                  "linear_attention_ssm_amd/csrc/gdn_launch_impl.h"]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------ byte model

def bytes_decode_head_step(w: gi.Workload, p: int, flush: bool, kind: str) -> float:
    """Algorithmic HBM bytes of one (row, value head) decode step.
    State fp32; ring entries and I/O in the workload dtypes; the key side
    (q, k and the key ring) is counted once per key head, i.e. 1/G per value
    head."""
    es = 2 if w.qkv != "f32" else 4
    rs = 2 if w.ring != "f32" else 4
    ss = 2 if w.state != "f32" else 4
    G = w.Hv // w.Hk
    gb = 4 * w.dk if w.gate == "key" else 4            # g per value head (per key channel: KDA)
    state = ss * w.dv * w.dk
    io = 2 * es * w.dk / G + 2 * es * w.dv + gb + 4     # q, k (per k-head), v, o, g, beta
    if kind == "packed":
        return 2 * state + io
    b = state + io
    b += p * (rs * w.dv + rs * w.dk / G + gb)            # valid ring entries read
    if flush:
        b += state                                       # checkpoint written from registers
    else:
        b += rs * w.dv + rs * w.dk / G + gb              # ring append
    return b


def cursor_sequence(w: gi.Workload, slots: np.ndarray, steps: int):
    """Per step: list of (p, flush) per live row, from the cursor rule
    (flush when p == L-1 or forced; next = 0 on flush, else p+1)."""
    wp = np.zeros(w.N, dtype=np.int64)
    seq = []
    for t in range(steps):
        ff = gi.force_flush_schedule(w, t, slots)
        cur = []
        for b, s in enumerate(slots):
            if s < 0:
                continue
            fl = (wp[s] == w.L - 1) or bool(ff[b])
            cur.append((int(wp[s]), bool(fl)))
            wp[s] = 0 if fl else wp[s] + 1
        seq.append(cur)
    return seq


# ------------------------------------------------------------------ helpers

def dev_tensor(x, dt, dev):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dt == "bf16":
        t = t.view(torch.bfloat16)
    return t.to(dev)


class LayerSet:
    """One layer's checkpoint (or packed state) and rings. The state is drawn
    on the device, S0 ~ N(0, 0.1^2) from a seeded generator, and rounded to
    the state dtype (the workload's distribution; the timing does not depend
    on the values). Rings start empty (zeros)."""

    def __init__(self, w, seed, dev, with_ring=True):
        import torch
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed)
        sdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[w.state]
        self.state = (0.1 * torch.randn((w.N, w.Hv, w.dv, w.dk), generator=gen, device=dev)).to(sdt)
        if with_ring:
            rdt = torch.float16 if w.ring == "f16" else (
                torch.bfloat16 if w.ring == "bf16" else torch.float32)
            self.ring_d = torch.zeros((w.N, w.Hv, w.L, w.dv), dtype=rdt, device=dev)
            self.ring_k = torch.zeros((w.N, w.Hk, w.L, w.dk), dtype=rdt, device=dev)
            gshape = (w.N, w.Hv, w.L, w.dk) if w.gate == "key" else (w.N, w.Hv, w.L)
            self.ring_g = torch.zeros(gshape, dtype=torch.float32, device=dev)


def input_sets(w, n, dev, T=None, mixed=False):
    """n seeded input sets on the device. mixed: q, k, v as views into one
    packed [B, T, 2*Hk*dk + Hv*dv] row per token (the mixed_qkv layout)."""
    import torch
    out = []
    for i in range(n):
        x = gi.step_inputs(w, 10_000 + i, T=T)
        q, k, v, g, beta = (dev_tensor(a, x.dtype if j < 3 else None, dev)
                            for j, a in enumerate((x.q, x.k, x.v, x.g, x.beta)))
        if mixed:
            B, TT = q.shape[:2]
            nq, nv = w.Hk * w.dk, w.Hv * w.dv
            m = torch.cat([q.reshape(B, TT, nq), k.reshape(B, TT, nq), v.reshape(B, TT, nv)], -1)
            q = m[..., :nq].view(B, TT, w.Hk, w.dk)
            k = m[..., nq:2 * nq].view(B, TT, w.Hk, w.dk)
            v = m[..., 2 * nq:].view(B, TT, w.Hv, w.dv)
        out.append((q, k, v, g, beta))
    return out


def graph_of(fn):
    """Capture fn's launches (all enqueued on torch's current stream, which is
    the capture stream during capture) into a HIP graph."""
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                   # one eager run on the capture stream first
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_graph(g, reps, samples=False):
    """Mean milliseconds per replay, HIP events on the replay stream (one pair
    around all replays). samples=True also records an event between replays
    and returns (mean, per-replay list)."""
    import torch
    g.replay()
    torch.cuda.synchronize()
    if not samples:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        g.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]
    return ev[0].elapsed_time(ev[reps]) / reps, per


def pct(xs, q):
    return float(np.percentile(np.asarray(xs, np.float64), q))


def load_traffic(name: str):
    """HBM bytes per launch from a committed rocprofv3 summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"kernel_sources_sha256_16:\s*(\w+)", txt)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m or not t or m.group(1) != kernel_hash():
        return None
    return float(t.group(1))


# ------------------------------------------------------------------ benches

def bench_replay(w, R, steps, warmup, dev, log, front_end=False, conv=False, best=False):
    """front_end: q, k, v read from the packed mixed_qkv row and normalised in
    the kernel (the workload draws raw q, k). conv: each layer first runs the
    causal convolution (width 4) on a raw packed row and the decode reads the
    convolved row; the figures then cover both launches of a layer."""
    import torch
    import linear_attention_ssm_amd as gdn
    slots = gi.slot_map(w)
    slot_t = dev_tensor(slots, None, dev)
    layers = [LayerSet(w, w.seed + 17 * i, dev) for i in range(R)]
    wp = torch.zeros(w.N, dtype=torch.int32, device=dev)
    ins = input_sets(w, 4, dev, mixed=front_end)
    fe = dict(qk_norm=True) if front_end else {}
    if conv:
        nq = w.Hk * w.dk
        ci = [gi.conv_inputs(w, 1, W=4, seed_tag=i) for i in range(R)]
        taps = [dev_tensor(c.w, c.dtype, dev) for c in ci]
        cstate = [dev_tensor(c.state, c.dtype, dev) for c in ci]
        xraw = [dev_tensor(c.x[0], c.dtype, dev) for c in ci]
        ybuf = [torch.empty_like(x) for x in xraw]

        def qkv_of(i):
            gdn.gdn_conv_update(xraw[i], taps[i], cstate[i], slot_t, y=ybuf[i])
            y = ybuf[i]
            _, _, _, g, beta = ins[i % len(ins)]
            return (y[:, :nq].view(w.B, 1, w.Hk, w.dk), y[:, nq:2 * nq].view(w.B, 1, w.Hk, w.dk),
                    y[:, 2 * nq:].view(w.B, 1, w.Hv, w.dv), g, beta)
    else:
        def qkv_of(i):
            return ins[i % len(ins)]
    ff_sched = [dev_tensor(gi.force_flush_schedule(w, t, slots), None, dev) for t in range(w.L)]
    no_ff = torch.zeros(w.B, dtype=torch.int32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    odt = torch.float32 if w.qkv == "f32" else torch.bfloat16
    o = torch.empty((w.B, 1, w.Hv, w.dv), dtype=odt, device=dev)

    def decodes(ff):
        for i, ls in enumerate(layers):
            q, k, v, g, beta = qkv_of(i)
            gdn.gdn_replay_decode(q, k, v, g, beta, slot_t, ls.state, ls.ring_d, ls.ring_k,
                                  ls.ring_g, wp, force_flush=ff, o=o, err_flags=err, **fe)

    arrive = gdn.arrive_workspace(w.B, dev)

    def forward(ff):
        # the last layer's decode advances the cursors (fused advance)
        for i, ls in enumerate(layers):
            q, k, v, g, beta = qkv_of(i)
            if i < len(layers) - 1:
                gdn.gdn_replay_decode(q, k, v, g, beta, slot_t, ls.state, ls.ring_d, ls.ring_k,
                                      ls.ring_g, wp, force_flush=ff, o=o, err_flags=err, **fe)
            else:
                gdn.gdn_replay_decode_advance(q, k, v, g, beta, slot_t, ls.state, ls.ring_d,
                                              ls.ring_k, ls.ring_g, wp, arrive, force_flush=ff,
                                              o=o, err_flags=err, **fe)

    # eager warm-up: the staggered forced flushes of the first L steps spread
    # the slots' flush phases evenly over the ring cycle
    warmup = max(warmup, w.L)
    for t in range(warmup):
        forward(ff_sched[t] if t < w.L else no_ff)
    torch.cuda.synchronize()
    n_fwd = warmup                                    # forwards applied so far
    g_fwd = graph_of(lambda: forward(no_ff))          # runs one forward eagerly, then captures
    n_fwd += 1
    g_dec = graph_of(lambda: decodes(no_ff))          # one decode-only run, then captures
    # pass 1: whole-job throughput (R decodes, the last one advancing the cursors)
    ms_step = time_graph(g_fwd, steps)
    n_fwd += steps + 1                                # time_graph replays once before timing
    # pass 2: the R decode kernels alone, back to back in one graph (cursors
    # frozen at this phase; the decodes do not move them). HIP events on the
    # replay stream bracket the timed replays; per-kernel figure = total / R
    # (it includes the short gap between two kernels of a graph). An event
    # between replays gives the spread: p10 / p50 / p90 of the per-launch mean
    # of each replay.
    ms_dec, per = time_graph(g_dec, steps, samples=True)
    ms_dec /= R
    per = [x / R for x in per]
    assert int(err.item()) == 0, f"device error flags {int(err.item())}"
    seq = cursor_sequence(w, slots, n_fwd + 1)
    cur = seq[n_fwd]                                   # the phase the frozen decodes see
    bytes_launch = sum(bytes_decode_head_step(w, p, fl, "replay") for p, fl in cur) * w.Hv
    live = int(np.count_nonzero(slots >= 0))
    mean_p = float(np.mean([p for p, _ in cur]))
    flush_frac = float(np.mean([fl for _, fl in cur]))
    fe_tag = ", conv + front end" if conv else (", front end" if front_end else "")
    log(f"replay [{w.name}: {w.state} state, {w.gate} gate, {w.ring} ring, L={w.L}{fe_tag}]: "
        f"{ms_step * 1e3:.1f} us/step ({R} layers, fused advance), decode kernel "
        f"{ms_dec * 1e3:.2f} us (p10 {pct(per, 10) * 1e3:.2f}, p90 {pct(per, 90) * 1e3:.2f}), "
        f"{bytes_launch / 1e6:.2f} MB/launch, mean p {mean_p:.2f}, flush frac {flush_frac:.4f}")
    out = dict(ms_per_step=ms_step, head_steps_per_s=live * w.Hv * R / (ms_step / 1e3),
               kernel_ms=ms_dec, kernel_us_p10=pct(per, 10) * 1e3,
               kernel_us_p50=pct(per, 50) * 1e3, kernel_us_p90=pct(per, 90) * 1e3,
               bytes_per_launch=bytes_launch, head_steps_per_launch=live * w.Hv,
               mean_p=mean_p, flush_frac=flush_frac)
    if best and w.L > 1:
        # "best" mode: every row on a step that does not flush (the cursor of
        # every slot set to pb = (L - 1) // 2, so each reads pb entries and
        # appends one); the same decode graph, now reading these cursors
        pb = (w.L - 1) // 2
        wp.fill_(pb)
        ms_b, per_b = time_graph(g_dec, steps, samples=True)
        ms_b /= R
        assert int(err.item()) == 0, f"device error flags {int(err.item())}"
        b_best = live * w.Hv * bytes_decode_head_step(w, pb, False, "replay")
        log(f"replay best mode (no flush, p = {pb}): decode kernel {ms_b * 1e3:.2f} us, "
            f"{b_best / 1e6:.2f} MB/launch ({b_best / ms_b / 1e6:.0f} GB/s)")
        out["best"] = dict(kernel_us=ms_b * 1e3, valid_entries=pb,
                           kernel_us_p10=pct(per_b, 10) / R * 1e3,
                           kernel_us_p90=pct(per_b, 90) / R * 1e3,
                           bytes_per_launch=b_best, achieved_gbs=b_best / ms_b / 1e6,
                           frac=b_best / ms_b / 1e6 / HBM_PEAK_GBS,
                           head_steps_per_s=live * w.Hv / (ms_b / 1e3))
    return out


def bench_conv(w, R, steps, dev, log):
    """The causal convolution alone (width 4) on the packed mixed_qkv row of
    the workload: R launches (one per layer) in a graph, per-launch time."""
    import torch
    import linear_attention_ssm_amd as gdn
    slot_t = dev_tensor(gi.slot_map(w), None, dev)
    ci = [gi.conv_inputs(w, 1, W=4, seed_tag=i) for i in range(R)]
    taps = [dev_tensor(c.w, c.dtype, dev) for c in ci]
    cstate = [dev_tensor(c.state, c.dtype, dev) for c in ci]
    xraw = [dev_tensor(c.x[0], c.dtype, dev) for c in ci]
    ybuf = [torch.empty_like(x) for x in xraw]

    def run():
        for i in range(R):
            gdn.gdn_conv_update(xraw[i], taps[i], cstate[i], slot_t, y=ybuf[i])

    g = graph_of(run)
    ms = time_graph(g, steps) / R
    C, es = gi.conv_channels(w), (4 if w.qkv == "f32" else 2)
    live = int(np.count_nonzero(gi.slot_map(w) >= 0))
    # x, three window rows read, three written, y; the taps once
    nbytes = live * C * es * 8 + C * 4 * es
    log(f"conv update (W=4, C={C}, B={w.B}): {ms * 1e3:.2f} us/launch, "
        f"{nbytes / 1e6:.2f} MB/launch ({nbytes / (ms / 1e3) / 1e9:.0f} GB/s)")
    return dict(kernel_ms=ms, bytes_per_launch=nbytes)


def bench_gates(w, R, steps, dev, log):
    """The per-key gate and beta activations (gdn_kda_gates) for one decode
    step of the workload: R launches (one per layer) in a graph."""
    import torch
    import linear_attention_ssm_amd as gdn
    r = np.random.default_rng(w.seed)
    mk = lambda *shape: torch.from_numpy(r.standard_normal(shape).astype(np.float32)).to(dev)
    ins = [(mk(w.B, 1, w.Hv, w.dk), mk(w.B, 1, w.Hv), mk(w.Hv), mk(w.Hv, w.dk)) for _ in range(R)]
    outs = [(torch.empty_like(a), torch.empty_like(b)) for a, b, _, _ in ins]

    def run():
        for (a, b, A, dt), (g, beta) in zip(ins, outs):
            gdn.gdn_kda_gates(a, b, A, dt, -5.0, g=g, beta=beta)

    ms = time_graph(graph_of(run), steps) / R
    nbytes = w.B * w.Hv * (w.dk * 8 + 8) + w.Hv * (w.dk + 1) * 4
    log(f"kda gates (B={w.B}, Hv={w.Hv}, dk={w.dk}): {ms * 1e3:.2f} us/launch, "
        f"{nbytes / 1e6:.2f} MB/launch")
    return dict(kernel_ms=ms, bytes_per_launch=nbytes)


def bench_packed(w, R, steps, dev, log):
    import torch
    import linear_attention_ssm_amd as gdn
    slots = gi.slot_map(w)
    slot_t = dev_tensor(slots, None, dev)
    layers = [LayerSet(w, w.seed + 17 * i, dev, with_ring=False) for i in range(R)]
    ins = input_sets(w, 4, dev)
    odt = torch.float32 if w.qkv == "f32" else torch.bfloat16
    o = torch.empty((w.B, 1, w.Hv, w.dv), dtype=odt, device=dev)

    def forward():
        for i, ls in enumerate(layers):
            q, k, v, g, beta = ins[i % len(ins)]
            gdn.gdn_packed_decode(q, k, v, g, beta, slot_t, ls.state, o=o)

    g = graph_of(forward)
    ms_step, per = time_graph(g, steps, samples=True)
    ms_k = ms_step / R
    live = int(np.count_nonzero(slots >= 0))
    bytes_launch = live * w.Hv * bytes_decode_head_step(w, 0, False, "packed")
    log(f"packed [{w.name}: {w.state} state, {w.gate} gate]: {ms_step * 1e3:.1f} us/step ({R} layers), "
        f"kernel {ms_k * 1e3:.2f} us (p10 {pct(per, 10) / R * 1e3:.2f}, p90 {pct(per, 90) / R * 1e3:.2f}), "
        f"{bytes_launch / 1e6:.2f} MB/launch")
    return dict(ms_per_step=ms_step, head_steps_per_s=live * w.Hv * R / (ms_step / 1e3),
                kernel_ms=ms_k, kernel_us_p10=pct(per, 10) / R * 1e3,
                kernel_us_p90=pct(per, 90) / R * 1e3, bytes_per_launch=bytes_launch)


def bench_window_fold(w, R, steps, dev, log):
    """Kernel figures at the speculative workload's shapes (B = 32, T = 5,
    L = 16): a verify window read from checkpoint + ring with a fixed
    p0 = L - T - 1 valid entries, and the fold of a ring holding p0 + T
    entries, R layer sets each. (The verify-commit-fold protocol itself, with
    its random acceptance, is exercised by the tests.)"""
    import torch
    import linear_attention_ssm_amd as gdn
    slots = gi.slot_map(w)
    slot_t = dev_tensor(slots, None, dev)
    layers = [LayerSet(w, w.seed + 17 * i, dev) for i in range(R)]
    ins = input_sets(w, 2, dev)
    p0 = w.L - w.T - 1
    pf = p0 + w.T
    wps = [torch.full((w.N,), p0, dtype=torch.int32, device=dev) for _ in range(R)]
    wpf = torch.full((w.N,), pf, dtype=torch.int32, device=dev)    # shared by the layers
    o = torch.empty((w.B, w.T, w.Hv, w.dv), dtype=torch.bfloat16, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)

    def verify():
        for i, ls in enumerate(layers):
            q, k, v, g, beta = ins[i % 2]
            gdn.gdn_replay_decode(q, k, v, g, beta, slot_t, ls.state, ls.ring_d, ls.ring_k,
                                  ls.ring_g, wps[i], o=o, err_flags=err, window=True)

    def fold():
        for ls in layers:
            gdn.gdn_replay_fold(slot_t, ls.state, ls.ring_d, ls.ring_k, ls.ring_g, wpf,
                                err_flags=err)

    def fold_all():
        gdn.gdn_replay_fold_layers(slot_t, [ls.state for ls in layers],
                                   [ls.ring_d for ls in layers], [ls.ring_k for ls in layers],
                                   [ls.ring_g for ls in layers], wpf, err_flags=err)

    mv = time_graph(graph_of(verify), steps) / R
    mf = time_graph(graph_of(fold), steps) / R
    mfl = time_graph(graph_of(fold_all), steps) / R
    assert int(err.item()) == 0
    G = w.Hv // w.Hk
    live = int(np.count_nonzero(slots >= 0))
    rs, es = 2, 2
    ent = rs * w.dv + rs * w.dk / G + 4
    vb = live * w.Hv * (4 * w.dv * w.dk + p0 * ent + w.T * ent
                        + w.T * (2 * es * w.dk / G + 2 * es * w.dv + 8))
    fb = live * w.Hv * (8 * w.dv * w.dk + pf * ent)
    log(f"verify T={w.T}: {mv * 1e3:.2f} us/launch ({vb / mv / 1e6:.0f} GB/s); "
        f"fold p={pf}: {mf * 1e3:.2f} us/launch ({fb / mf / 1e6:.0f} GB/s); "
        f"{R} layers in one fold call: {mfl * 1e3:.2f} us per layer ({fb / mfl / 1e6:.0f} GB/s)")
    return dict(verify_kernel_us=mv * 1e3, verify_gbs=vb / mv / 1e6,
                verify_head_tokens_per_s=live * w.Hv * w.T / (mv / 1e3),
                fold_kernel_us=mf * 1e3, fold_gbs=fb / mf / 1e6, window_p=p0, fold_p=pf,
                fold_layers_us_per_layer=mfl * 1e3, fold_layers_gbs=fb / mfl / 1e6,
                fold_layers_n=R)


def bench_lossless(w, R, steps, dev, log):
    """Lossless verify rounds (SGLang PR #42388): per round, every layer
    verifies a T-token window from its exact checkpoint (empty ring, fp32
    tuples), the accepted prefix is committed once, every layer folds it, and
    the cursors are reset once. Seeded accepted counts a ~ U{0..T}."""
    import torch
    import linear_attention_ssm_amd as gdn
    slots = gi.slot_map(w)
    slot_t = dev_tensor(slots, None, dev)
    layers = [LayerSet(w, w.seed + 17 * i, dev) for i in range(R)]
    ins = input_sets(w, 2, dev)
    acc_np = gi.accepted_counts(w, 0)
    acc = dev_tensor(acc_np, None, dev)
    wp = torch.zeros((w.N,), dtype=torch.int32, device=dev)
    o = torch.empty((w.B, w.T, w.Hv, w.dv), dtype=torch.bfloat16, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)

    def verify():
        for i, ls in enumerate(layers):
            q, k, v, g, beta = ins[i % 2]
            gdn.gdn_replay_decode(q, k, v, g, beta, slot_t, ls.state, ls.ring_d, ls.ring_k,
                                  ls.ring_g, wp, o=o, err_flags=err, window=True)

    def fold():
        for ls in layers:
            gdn.gdn_replay_fold(slot_t, ls.state, ls.ring_d, ls.ring_k, ls.ring_g, wp,
                                err_flags=err)

    def fold_all():
        gdn.gdn_replay_fold_layers(slot_t, [ls.state for ls in layers],
                                   [ls.ring_d for ls in layers], [ls.ring_k for ls in layers],
                                   [ls.ring_g for ls in layers], wp, err_flags=err)

    def round_():
        verify()
        gdn.gdn_replay_commit(slot_t, acc, wp, w.L, w.T, err_flags=err)
        fold()
        gdn.gdn_replay_reset(slot_t, wp, err_flags=err)

    def round_layers():
        verify()
        gdn.gdn_replay_commit(slot_t, acc, wp, w.L, w.T, err_flags=err)
        fold_all()
        gdn.gdn_replay_reset(slot_t, wp, err_flags=err)

    m_round = time_graph(graph_of(round_), steps)
    m_round_l = time_graph(graph_of(round_layers), steps)
    m_verify = time_graph(graph_of(verify), steps) / R
    wpn = np.zeros(w.N, np.int32)                    # the cursors a commit leaves
    wpn[slots[slots >= 0]] = acc_np[slots >= 0]
    wp.copy_(dev_tensor(wpn, None, dev))
    m_fold = time_graph(graph_of(fold), steps) / R
    m_fold_l = time_graph(graph_of(fold_all), steps) / R
    assert int(err.item()) == 0
    G = w.Hv // w.Hk
    live = slots >= 0
    nh = int(np.count_nonzero(live)) * w.Hv
    ent = 4 * w.dv + 4 * w.dk / G + 4
    es = 2
    vb = nh * (4 * w.dv * w.dk + w.T * ent + w.T * (2 * es * w.dk / G + 2 * es * w.dv + 8))
    a_sum = float(acc_np[live].sum()) * w.Hv
    n_fold = int(np.count_nonzero(acc_np[live] > 0)) * w.Hv     # heads with entries to fold
    fb = n_fold * 8 * w.dv * w.dk + a_sum * ent
    log(f"lossless verify T={w.T}: round {m_round * 1e3:.1f} us ({R} layers: verify, commit, "
        f"fold, reset); verify {m_verify * 1e3:.2f} us/launch ({vb / m_verify / 1e6:.0f} GB/s), "
        f"fold {m_fold * 1e3:.2f} us/launch ({fb / m_fold / 1e6:.0f} GB/s); with the {R} "
        f"layers folded in one call: round {m_round_l * 1e3:.1f} us, fold "
        f"{m_fold_l * 1e3:.2f} us per layer ({fb / m_fold_l / 1e6:.0f} GB/s)")
    return dict(round_us=m_round * 1e3, layers=R,
                accepted_tokens_per_s=float(acc_np[live].sum()) / (m_round / 1e3),
                verify_kernel_us=m_verify * 1e3, verify_gbs=vb / m_verify / 1e6,
                fold_kernel_us=m_fold * 1e3, fold_gbs=fb / m_fold / 1e6,
                mean_accepted=float(acc_np[live].mean()),
                round_us_fold_layers=m_round_l * 1e3,
                accepted_tokens_per_s_fold_layers=float(acc_np[live].sum()) / (m_round_l / 1e3),
                fold_layers_us_per_layer=m_fold_l * 1e3, fold_layers_gbs=fb / m_fold_l / 1e6)


def read_probe(R, reps, dev, log):
    """The library's read probe over R buffers of 128 MiB (the decode's layer
    rotation): the read bandwidth this GPU reaches for the checkpoint's access
    pattern. HIP events around `reps` rounds of R launches."""
    import torch
    import linear_attention_ssm_amd as gdn
    nb = 128 << 20
    bufs = [torch.zeros(nb // 4, dtype=torch.float32, device=dev) for _ in range(R)]
    sink = torch.zeros(1, dtype=torch.float32, device=dev)

    def run():
        for b in bufs:
            gdn.gdn_hbm_read_probe(b, sink)

    ms = time_graph(graph_of(run), reps) / R
    gbs = nb / (ms / 1e3) / 1e9
    log(f"read probe: 128 MiB in {ms * 1e3:.2f} us ({gbs:.0f} GB/s)")
    del bufs
    return dict(bytes=nb, us=ms * 1e3, gbs=gbs)


def rw_probe(R, reps, dev, log):
    """The library's copy probe over R buffers of 128 MiB, each copied onto
    itself (a checkpoint block read and written back, with the decode's load
    and store policies): the read + write bandwidth this GPU reaches for that
    pattern. HIP events around `reps` rounds of R launches."""
    import torch
    import linear_attention_ssm_amd as gdn
    nb = 128 << 20
    bufs = [torch.zeros(nb // 4, dtype=torch.float32, device=dev) for _ in range(R)]

    def run():
        for b in bufs:
            gdn.gdn_hbm_copy_probe(b, b)

    ms = time_graph(graph_of(run), reps) / R
    gbs = 2 * nb / (ms / 1e3) / 1e9
    log(f"copy probe: 128 MiB read and written back in {ms * 1e3:.2f} us ({gbs:.0f} GB/s)")
    del bufs
    return dict(bytes=2 * nb, us=ms * 1e3, gbs=gbs)


def copy_probe_timed(reps, dev, log):
    """A plain device copy of 1 GiB (torch's copy kernel): read + write."""
    import torch
    n = 1 << 28
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    ms = time_graph(graph_of(lambda: b.copy_(a)), reps)
    gbs = 2 * 4 * n / (ms / 1e3) / 1e9
    log(f"copy probe: 1 GiB copied in {ms * 1e3:.1f} us ({gbs:.0f} GB/s read + write)")
    del a, b
    return dict(bytes=2 * 4 * n, us=ms * 1e3, gbs=gbs)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s, log):
    """The CPU oracle's sequential decode recurrence (O1), fp64 and its fp32
    instance, on a bounded sample of the standard workload: its 64-row batch
    stepped for about budget_s / 4 seconds per configuration, on one thread
    and on all the host cores this process may use (the OpenMP loop over
    (row, value head) of a -O3 build of the same C source for this host)."""
    import tempfile
    import oracle
    L, flags = oracle.timing_library(tempfile.mkdtemp(prefix="gdn_oracle_"))
    avail = len(os.sched_getaffinity(0))
    n_all = min(avail, int(os.environ.get("OMP_NUM_THREADS", avail)))
    slots = gi.slot_map(w)
    live = int(np.count_nonzero(slots >= 0))
    xs = [gi.step_inputs(w, i) for i in range(4)]
    x64 = [tuple(np.ascontiguousarray(a[:, 0]) for a in x.f64()) for x in xs]
    x32 = [tuple(a.astype(np.float32) for a in x) for x in x64]
    per = budget_s / 4
    res = {}
    for prec in ("f64", "f32"):
        for nt in (1, n_all):
            used = L.oracle_threads(nt)
            S = gi.initial_state(w).astype(np.float64 if prec == "f64" else np.float32)
            n, t0 = 0, time.perf_counter()
            while True:
                if prec == "f64":
                    _oracle_step(L, S, slots, x64[n % 4], np.float64)
                else:
                    _oracle_step(L, S, slots, x32[n % 4], np.float32)
                n += 1
                el = time.perf_counter() - t0
                if el >= per:
                    break
            hs = live * w.Hv * n / el
            res[(prec, nt)] = dict(head_steps_per_s=hs, threads=used, steps=n, seconds=el,
                                   gbs=hs * 8 * w.dv * w.dk * (2 if prec == "f64" else 1) / 1e9)
            log(f"cpu oracle {prec}, {used} thread(s): {n} steps of {live}x{w.Hv} head-steps in "
                f"{el:.1f} s -> {hs:.0f} head-steps/s")
    top = res[("f64", n_all)]
    return dict(value=top["head_steps_per_s"], unit="head-steps/s", cores=top["threads"],
                kind="oracle",
                sample=(f"{top['steps']} decode steps of the B={live} x Hv={w.Hv} (dk=dv={w.dk}) "
                        f"batch through the fp64 sequential recurrence on {top['threads']} threads, "
                        f"{top['seconds']:.1f} s (the whole CPU leg, fp64 and fp32 on 1 and "
                        f"{top['threads']} threads: {sum(v['seconds'] for v in res.values()):.1f} s)"),
                cpu_model=cpu_model(), host_cpus_available=avail, build_flags=flags,
                fp64_1_thread=res[("f64", 1)]["head_steps_per_s"],
                fp32_1_thread=res[("f32", 1)]["head_steps_per_s"],
                fp32_all_threads=res[("f32", n_all)]["head_steps_per_s"],
                fp64_all_threads=top["head_steps_per_s"])


def _oracle_step(L, S, slots, x, dt):
    """One decode step of the timing library's fp64 or fp32 recurrence."""
    import oracle
    q, k, v, g, beta = x
    B, Hk, dk = q.shape
    N, Hv, dv, _ = S.shape
    o = np.empty((B, Hv, dv), dt)
    sl = oracle._p(slots.astype(np.int32))
    if dt == np.float64:
        L.oracle_gdn_step_f64(B, N, Hv, Hk, dk, dv, sl, oracle._p(S), oracle._p(q), oracle._p(k),
                              oracle._p(v), oracle._p(g), oracle._p(beta), oracle._p(o), None)
    else:
        L.oracle_gdn_step_f32(B, N, Hv, Hk, dk, dv, sl, oracle._p(S), oracle._p(q), oracle._p(k),
                              oracle._p(v), oracle._p(g), oracle._p(beta), oracle._p(o))
    return o


def copy_probe(dev, log):
    import torch
    n = 1 << 28                                     # 1 GiB of fp32
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy probe: 3 copies of {n * 4} bytes")


def summary(r, pk=None, w=None):
    """The usual figures of one replay bench (and its packed counterpart)."""
    gbs = r["bytes_per_launch"] / (r["kernel_ms"] / 1e3) / 1e9
    d = dict(replay_kernel_us=r["kernel_ms"] * 1e3, replay_kernel_us_p10=r["kernel_us_p10"],
             replay_kernel_us_p90=r["kernel_us_p90"], replay_gbs=gbs, replay_frac=gbs / HBM_PEAK_GBS,
             replay_bytes_per_launch=r["bytes_per_launch"],
             replay_head_steps_per_s=r["head_steps_per_s"], mean_valid_entries=r["mean_p"],
             flush_fraction=r["flush_frac"])
    if pk is not None:
        pg = pk["bytes_per_launch"] / (pk["kernel_ms"] / 1e3) / 1e9
        d.update(packed_kernel_us=pk["kernel_ms"] * 1e3, packed_gbs=pg, packed_frac=pg / HBM_PEAK_GBS,
                 packed_bytes_per_launch=pk["bytes_per_launch"],
                 packed_head_steps_per_s=pk["head_steps_per_s"],
                 replay_vs_packed_kernel=pk["kernel_ms"] / r["kernel_ms"],
                 replay_vs_packed=r["head_steps_per_s"] / pk["head_steps_per_s"])
    return d


# The pages' own figures for this path, with the hardware they were taken on
# (context, not targets; the pages publish no absolute head-steps/s or GB/s).
PAGES_CONTEXT = {
    "packed_decode_hbm_bound": ("the packed (read-update-write) GDN decode is 70-79% bound by HBM "
                                "bandwidth at batch >= 64 on H20-3e, fp32 state (SGLang PR #28451, "
                                "Motivation)"),
    "state_bytes_per_head_step": ("about 8*dv*dk bytes of state per head-step for the packed decode "
                                  "(read + write) against about 4*dv*dk for the replay decode "
                                  "(read only), fp32 state (SGLang PR #28451, Motivation; "
                                  "ReplaySSM blog, section 5.1)"),
    "replay_vs_packed_kernel_h20": ("1.2-1.5x at batch >= 16 with L = 8, slightly slower at batch 1, "
                                    "on H20-3e (SGLang PR #28451, Performance)"),
}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--cpu-budget", type=float, default=16.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--profile-pass", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    args = ap.parse_args()
    log = lambda m: print(f"[bench] {m}", file=sys.stderr, flush=True)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library runs on a single MI355X and has "
              "no multi-GPU path (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    import linear_attention_ssm_amd  # noqa: F401  (fails loudly if the library is missing)
    if args.copy_probe:
        copy_probe(dev, log)
        return
    w = gi.C2
    R = args.layers
    steps, warmup = args.steps, args.warmup
    if args.profile_pass:
        steps, warmup = 4, 16
    small = max(4, steps // 4)
    # the packed baseline first (it also brings the GPU to its working clocks)
    pk = bench_packed(w, R, steps, dev, log)
    rep = bench_replay(w, R, steps, warmup, dev, log, best=True)
    rp = read_probe(R, small, dev, log)
    rw = rw_probe(R, small, dev, log)
    cp = copy_probe_timed(small, dev, log)
    w16 = dataclasses.replace(w, state="bf16")
    rep16 = bench_replay(w16, R, steps, warmup, dev, log, best=True)
    pk16 = bench_packed(w16, R, steps, dev, log)
    repk = bench_replay(gi.C7, R, steps, warmup, dev, log)
    pkk = bench_packed(gi.C7, R, steps, dev, log)
    gts = bench_gates(gi.C7, R, steps, dev, log)
    w_fe = dataclasses.replace(w, qk_raw=True)
    repf = bench_replay(w_fe, R, steps, warmup, dev, log, front_end=True)
    repc = bench_replay(w_fe, R, steps, warmup, dev, log, front_end=True, conv=True)
    cv = bench_conv(w_fe, R, steps, dev, log)
    # the large pool: 256 rows (8 of them padding) over 512 slots, 4 layer sets
    rep3 = bench_replay(gi.C3, 4, small, warmup, dev, log)
    pk3 = bench_packed(gi.C3, 4, small, dev, log)
    # ring depth
    depth = {}
    for L in (1, 4, 32):
        depth[f"L{L}"] = summary(bench_replay(gi.c4(L), R, small, warmup, dev, log))
    depth["L16"] = summary(rep)
    rep_f32r = bench_replay(gi.c4(16, "f32"), R, small, warmup, dev, log)
    wf = bench_window_fold(gi.C5, R, max(4, steps // 8), dev, log)
    ll = bench_lossless(gi.C6, R, max(4, steps // 8), dev, log)
    if args.profile_pass:
        return
    achieved = rep["bytes_per_launch"] / (rep["kernel_ms"] / 1e3) / 1e9
    traffic = load_traffic("replay_decode_c2_hbm_traffic.txt")
    pk_gbs = pk["bytes_per_launch"] / (pk["kernel_ms"] / 1e3) / 1e9
    out = {
        "metric": METRIC,
        "value": rep["head_steps_per_s"],
        "unit": "head-steps/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": rep["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"ReplaySSM GDN single-token decode, B={w.B} rows, Hv={w.Hv}, Hk={w.Hk}, "
                         f"dk=dv={w.dk}, ring L={w.L}, fp32 checkpoint, bf16 q/k/v/o, fp16 d/k "
                         f"ring (fp16 MFMA operands), staggered cursors; one step = {R} layers: "
                         f"{R - 1} x gdn_replay_decode + 1 x gdn_replay_decode_advance (the "
                         f"last layer advances the cursors)"),
            "global_batch": w.B, "layers_per_step": R, "ring_L": w.L,
            "head_steps_per_launch": rep["head_steps_per_launch"],
            "mean_valid_entries": round(rep["mean_p"], 3),
            "flush_fraction": round(rep["flush_frac"], 4),
        },
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
            "kernel": "replay_decode_kernel<128, bf16, f16, f32>",
            "kernel_us": rep["kernel_ms"] * 1e3,
            "kernel_us_p10": rep["kernel_us_p10"], "kernel_us_p50": rep["kernel_us_p50"],
            "kernel_us_p90": rep["kernel_us_p90"],
            "algorithmic_bytes_per_launch": rep["bytes_per_launch"],
            "measured_read_peak_gbs": rp["gbs"],
            "frac_of_measured_read_peak": achieved / rp["gbs"],
            "measured_copy_peak_gbs": rw["gbs"],
        },
        "packed_baseline": {
            "head_steps_per_s": pk["head_steps_per_s"], "ms_per_step": pk["ms_per_step"],
            "kernel_us": pk["kernel_ms"] * 1e3, "kernel_us_p10": pk["kernel_us_p10"],
            "kernel_us_p90": pk["kernel_us_p90"],
            "achieved_gbs": pk_gbs, "frac": pk_gbs / HBM_PEAK_GBS,
            "frac_of_measured_copy_peak": pk_gbs / rw["gbs"],
            "algorithmic_bytes_per_launch": pk["bytes_per_launch"],
        },
        "replay_vs_packed": rep["head_steps_per_s"] / pk["head_steps_per_s"],
        "replay_vs_packed_kernel": pk["kernel_ms"] / rep["kernel_ms"],
        "best_mode_c2": rep["best"],
        "probes": {"read_128MiB": rp, "copy_128MiB_in_place": rw, "torch_copy_1GiB": cp,
                   "note": ("read: the library's gdn_hbm_read_probe over 8 buffers of 128 MiB in "
                            "the checkpoint's access pattern; copy_128MiB_in_place: the "
                            "library's gdn_hbm_copy_probe writing each of them back onto itself "
                            "(the measured read + write peak); torch_copy_1GiB: torch's plain "
                            "device copy, for context")},
        "state_bf16": {
            "note": "the standard workload with a bf16 checkpoint / packed state (fp32 math)",
            **summary(rep16, pk16),
            "best_mode": rep16.get("best"),
            "replay_vs_fp32_replay": rep["kernel_ms"] / rep16["kernel_ms"],
        },
        "kda_c7": {
            "note": ("the standard workload with a per-key gate (KDA): g [B, Hv, dk] and "
                     "ring_g [N, Hv, L, dk]; replay vs the packed decode with the same gate"),
            **summary(repk, pkk),
            "gates_kernel_us": gts["kernel_ms"] * 1e3,
            "gates_bytes_per_launch": gts["bytes_per_launch"],
        },
        "front_end_c2": {
            "note": ("the standard workload with q, k, v read from the packed mixed_qkv row "
                     "and q/k L2-normalised (q scaled) in the kernel"),
            **summary(repf),
            "vs_plain_replay_kernel": rep["kernel_ms"] / repf["kernel_ms"],
        },
        "front_end_conv_c2": {
            "note": ("the front end with the causal convolution: per layer, the convolution "
                     "(width 4, SiLU) of a raw packed mixed_qkv row, then the replay decode "
                     "reading the convolved row with q/k normalised in the kernel"),
            "step_us": repc["ms_per_step"] * 1e3,
            "head_steps_per_s": repc["head_steps_per_s"],
            "conv_plus_decode_us_per_layer": repc["kernel_ms"] * 1e3,
            "conv_kernel_us": cv["kernel_ms"] * 1e3,
            "conv_bytes_per_launch": cv["bytes_per_launch"],
            "conv_gbs": cv["bytes_per_launch"] / (cv["kernel_ms"] / 1e3) / 1e9,
            "vs_plain_replay_step": rep["ms_per_step"] / repc["ms_per_step"],
        },
        "large_pool_c3": {
            "note": ("B=256 rows (8 padding) over a pool of N=512 slots, a seeded slot "
                     "permutation, standard shapes and dtypes; 4 layer sets (4 GiB of checkpoints)"),
            **summary(rep3, pk3),
        },
        "ring_depth_c4": {
            "note": ("the standard workload at ring depths L = 1, 4, 16, 32 (L16 is the headline "
                     "run); L = 1 flushes every step, i.e. the packed decode's traffic"),
            **depth,
            "L16_fp32_ring": {"note": "fp32 ring (fp32 MFMA reconstruction), fp32 q/k/v/o",
                              **summary(rep_f32r)},
        },
        "verify_window_c5_shapes": {
            **wf, "fold_frac_of_measured_copy_peak": wf["fold_gbs"] / rw["gbs"],
            "fold_layers_frac": wf["fold_layers_gbs"] / 8000.0,
            "fold_layers_frac_of_measured_copy_peak": wf["fold_layers_gbs"] / rw["gbs"],
            "fold_layers_note": ("fold_layers_*: the same folds with every layer set in one "
                                 "gdn_replay_fold_layers call (one launch), per layer")},
        "lossless_verify_c6": {
            **ll, "fold_frac_of_measured_copy_peak": ll["fold_gbs"] / rw["gbs"],
            "fold_layers_frac_of_measured_copy_peak": ll["fold_layers_gbs"] / rw["gbs"]},
        "pages_context": PAGES_CONTEXT,
        "cpu_baseline": None,
        "kernel_sources_sha256_16": kernel_hash(),
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_budget, log)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
