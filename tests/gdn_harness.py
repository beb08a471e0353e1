"""Shared machinery of the GPU parity tests.

Runs a workload's decode protocol through the C-ABI (via the Python binding)
and, on the same seeded inputs, through the CPU oracle; compares outputs and
states within the tolerance of the workload and cursors / flush positions
bit for bit. Expected values only ever come from the oracle.

Tolerance (max |x - ref| <= tol * max |ref|, per tensor and step):
  1e-4 when the ring and the outputs are fp32, 2e-2 when the ring is fp16 /
  bf16 or the outputs are bf16. The packed decode has no ring: its fp32
  state is held to 1e-4 and its outputs to the output dtype's bar.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

import gdn_inputs as gi
from oracle import ReplayModel, next_cursor, rel_err, step

DEV = torch.device("cuda:0")
TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def log(msg: str) -> None:
    print(msg, flush=True)


def to_dev(x: np.ndarray, dt: Optional[str] = None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dt == "bf16":
        t = t.view(torch.bfloat16)
    return t.to(DEV)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits(t: torch.Tensor) -> torch.Tensor:
    """Integer view of a tensor's bit patterns (NaN-safe comparisons)."""
    return t.view(torch.int32) if t.element_size() == 4 else t.view(torch.int16)


def tol_o(w: gi.Workload) -> float:
    return 1e-4 if (w.qkv == "f32" and w.ring == "f32") else 2e-2


def tol_state(w: gi.Workload) -> float:
    return 1e-4 if w.ring == "f32" else 2e-2


def tol_packed_o(w: gi.Workload) -> float:
    return 1e-4 if w.qkv == "f32" else 2e-2


@dataclass
class DevInputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor


def dev_inputs(x: gi.StepInputs) -> DevInputs:
    return DevInputs(to_dev(x.q, x.dtype), to_dev(x.k, x.dtype), to_dev(x.v, x.dtype),
                     to_dev(x.g), to_dev(x.beta))


CANARY_BYTES = 4096         # guard bytes on each side of a canary tensor


class CanaryTensor:
    """A device tensor placed inside a larger buffer whose CANARY_BYTES before
    and after it hold a fixed byte pattern (a garbage template around the
    buffer, SGLang PR #36821, Tests): check() asserts that no kernel wrote
    outside the tensor. The tensor is 256-byte aligned, like torch's own
    allocations."""

    PATTERN = 0xA5

    def __init__(self, shape, dt, init: Optional[torch.Tensor] = None):
        dtype = TORCH_DT[dt] if isinstance(dt, str) else dt
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.buf = torch.full((CANARY_BYTES + n + CANARY_BYTES,), self.PATTERN,
                              dtype=torch.uint8, device=DEV)
        self.n = n
        self.t = self.buf[CANARY_BYTES:CANARY_BYTES + n].view(dtype).view(shape)
        if init is not None:
            self.t.copy_(init)
        else:
            self.t.zero_()

    def check(self, what: str) -> None:
        head = self.buf[:CANARY_BYTES]
        tail = self.buf[CANARY_BYTES + self.n:]
        assert bool((head == self.PATTERN).all()), f"{what}: bytes before the tensor changed"
        assert bool((tail == self.PATTERN).all()), f"{what}: bytes after the tensor changed"


class Pool:
    """Device buffers of one layer: checkpoint, rings, cursors, error word.
    canary: each of them sits inside a guarded buffer (CanaryTensor)."""

    def __init__(self, w: gi.Workload, S0: np.ndarray, garbage: bool = False,
                 canary: bool = False):
        self.w = w
        rdt = TORCH_DT[w.ring]
        gshape = (w.N, w.Hv, w.L, w.dk) if w.gate == "key" else (w.N, w.Hv, w.L)
        dshape, kshape = (w.N, w.Hv, w.L, w.dv), (w.N, w.Hk, w.L, w.dk)
        if garbage:
            init = (to_dev(S0), to_dev(gi.garbage_like(dshape, w.ring, 1), w.ring),
                    to_dev(gi.garbage_like(kshape, w.ring, 2), w.ring),
                    to_dev(gi.garbage_like(gshape, "f32", 3)))
        else:
            init = (to_dev(S0), torch.zeros(dshape, dtype=rdt, device=DEV),
                    torch.zeros(kshape, dtype=rdt, device=DEV),
                    torch.zeros(gshape, dtype=torch.float32, device=DEV))
        self.guards = []
        if canary:
            for x in init:
                self.guards.append(CanaryTensor(tuple(x.shape), x.dtype, init=x))
            self.guards.append(CanaryTensor((w.N,), torch.int32))
            self.ckpt, self.ring_d, self.ring_k, self.ring_g, self.write_pos = \
                (c.t for c in self.guards)
        else:
            self.ckpt, self.ring_d, self.ring_k, self.ring_g = init
            self.write_pos = torch.zeros(w.N, dtype=torch.int32, device=DEV)
        self.err = torch.zeros(1, dtype=torch.int32, device=DEV)

    def check_canaries(self, what: str) -> None:
        for c, name in zip(self.guards, ("ckpt", "ring_d", "ring_k", "ring_g", "write_pos")):
            c.check(f"{what}: {name}")

    def ring_bits(self):
        return bits(self.ring_d).clone(), bits(self.ring_k).clone(), bits(self.ring_g).clone()


def reconstruct(pool: Pool, s: int, p: int) -> np.ndarray:
    """The state a slot's (checkpoint, valid ring entries) represent, decoded
    in fp64 with the closed-form replay. Used to check non-flush steps."""
    w = pool.w
    ck = to_f64(pool.ckpt[s])
    rd = to_f64(pool.ring_d[s, :, :p])
    rk = to_f64(pool.ring_k[s, :, :p])
    rg = to_f64(pool.ring_g[s, :, :p])
    G = w.Hv // w.Hk
    return np.stack([ReplayModel.replay(ck[h], rd[h], rk[h // G], rg[h]) for h in range(w.Hv)])


@dataclass
class Report:
    o_err: List[float] = field(default_factory=list)
    state_err: List[float] = field(default_factory=list)
    recon_err: List[float] = field(default_factory=list)
    state_t: List[int] = field(default_factory=list)   # step of each state_err entry
    flushes: int = 0

    def state_max(self, t0: int, t1: int) -> float:
        """Largest checkpoint / state error recorded at steps t0 <= t < t1."""
        return max(e for e, t in zip(self.state_err, self.state_t) if t0 <= t < t1)

    def summary(self) -> str:
        f = lambda x: f"{max(x):.2e}" if x else "-"
        return (f"o {f(self.o_err)}  state {f(self.state_err)}  recon {f(self.recon_err)}  "
                f"flushes {self.flushes}")


def run_decode(w: gi.Workload, kind: str = "replay", steps: Optional[int] = None,
               garbage: bool = False, recon_every: int = 0,
               check_untouched: bool = False, canary: bool = True) -> Report:
    """Drive `steps` single-token forwards of workload w through the library
    (kind 'replay': decode + advance; kind 'packed': packed decode) and the
    oracle, asserting parity at every step, on every live row: the outputs of
    every row and head, every flushed checkpoint (replay) or the whole state
    (packed) against the fp64 recurrence, cursors and flush positions bit for
    bit. recon_every: every so many steps, the state each live slot's
    checkpoint and valid ring entries represent is decoded in fp64 and
    compared too. canary: o, the checkpoint pool and the rings are views into
    larger buffers whose tails hold a fixed pattern, checked unchanged after
    every step."""
    import linear_attention_ssm_amd as gdn

    steps = w.steps if steps is None else steps
    S0 = gi.initial_state(w)
    slots = gi.slot_map(w)
    rows = np.where(slots >= 0)[0]
    sub = np.arange(len(rows), dtype=np.int32)
    S_true = S0[slots[rows]].astype(np.float64)
    pool = Pool(w, S0, garbage=garbage, canary=canary)
    o_buf = CanaryTensor((w.B, 1, w.Hv, w.dv), w.qkv) if canary else None
    slot_t = to_dev(slots)
    wp_model = np.zeros(w.N, dtype=np.int64)
    written = np.zeros((w.N, w.L), dtype=bool)        # ring positions written so far
    ring0 = pool.ring_bits() if garbage else None
    ck0 = pool.ckpt.clone() if check_untouched else None
    pad = torch.from_numpy(np.where(slots < 0)[0]).to(DEV)
    rep = Report()
    tol_o_ = tol_packed_o(w) if kind == "packed" else tol_o(w)
    tol_s_ = 1e-4 if kind == "packed" else tol_state(w)
    for t in range(steps):
        x = gi.step_inputs(w, t)
        xi = dev_inputs(x)
        ff = gi.force_flush_schedule(w, t, slots)
        ff_t = to_dev(ff)
        ck_before = pool.ckpt.clone() if kind == "replay" else None
        o_arg = o_buf.t if o_buf is not None else None
        if kind == "replay":
            o = gdn.gdn_replay_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, pool.ckpt,
                                      pool.ring_d, pool.ring_k, pool.ring_g, pool.write_pos,
                                      force_flush=ff_t, o=o_arg, err_flags=pool.err)
            gdn.gdn_replay_advance(slot_t, pool.write_pos, w.L, force_flush=ff_t,
                                   err_flags=pool.err)
        else:
            o = gdn.gdn_packed_decode(xi.q, xi.k, xi.v, xi.g, xi.beta, slot_t, pool.ckpt,
                                      o=o_arg, err_flags=pool.err)
        if o_buf is not None:
            o_buf.check(f"{w.name} step {t}: o")
            pool.check_canaries(f"{w.name} step {t}")
        # expected cursors / flushes (integer state machine)
        exp_flush = np.zeros(w.N, dtype=bool)
        for b, s in enumerate(slots):
            if s < 0:
                continue
            fl, nxt = next_cursor(int(wp_model[s]), w.L, bool(ff[b]))
            exp_flush[s] = fl
            if not fl:
                written[s, wp_model[s]] = True
            wp_model[s] = nxt
        # oracle values on every live row
        q, k, v, g, beta = (a[rows, 0] for a in x.f64())
        o_ref = step(S_true, sub, q, k, v, g, beta)
        o_gpu = to_f64(o[rows, 0])
        e = rel_err(o_gpu, o_ref)
        rep.o_err.append(e)
        assert e <= tol_o_, f"{w.name} step {t}: o rel err {e:.3e} > {tol_o_}"
        if len(pad):
            assert torch.count_nonzero(o[pad]).item() == 0, "padding row output not zero"
        if kind == "replay":
            wp_gpu = pool.write_pos.cpu().numpy()
            assert np.array_equal(wp_gpu, wp_model), f"{w.name} step {t}: cursor mismatch"
            changed = (bits(pool.ckpt) != bits(ck_before)).flatten(1).any(dim=1).cpu().numpy()
            live = slots[slots >= 0]
            assert np.array_equal(changed[live], exp_flush[live]), \
                f"{w.name} step {t}: flush positions differ"
            rep.flushes += int(exp_flush.sum())
            fl_i = np.array([i for i, r in enumerate(rows) if exp_flush[slots[r]]], np.int64)
            if len(fl_i):
                # every flushed checkpoint, each slot against its own true state
                ck = to_f64(pool.ckpt[torch.from_numpy(slots[rows[fl_i]].astype(np.int64)).to(DEV)])
                for j, i in enumerate(fl_i):
                    es = rel_err(ck[j], S_true[i])
                    rep.state_err.append(es)
                    rep.state_t.append(t)
                    assert es <= tol_s_, \
                        f"{w.name} step {t}: row {rows[i]} ckpt rel err {es:.3e}"
            if recon_every and (t % recon_every == recon_every - 1 or t == steps - 1):
                for i, r in enumerate(rows):
                    s = slots[r]
                    er = rel_err(reconstruct(pool, s, int(wp_model[s])), S_true[i])
                    rep.recon_err.append(er)
                    assert er <= tol_s_, \
                        f"{w.name} step {t}: row {r} reconstructed state {er:.3e}"
        else:
            ck = to_f64(pool.ckpt[torch.from_numpy(slots[rows].astype(np.int64)).to(DEV)])
            es = rel_err(ck, S_true)
            rep.state_err.append(es)
            rep.state_t.append(t)
            assert es <= tol_s_, f"{w.name} step {t}: packed state rel err {es:.3e}"
    assert int(pool.err.item()) == 0, f"unexpected error flags {int(pool.err.item())}"
    if ring0 is not None and kind == "replay":
        # every changed ring entry must be one the state machine says was written
        wm = torch.from_numpy(written).to(DEV).unsqueeze(1)
        for before, after, name in zip(ring0, pool.ring_bits(), ("d", "k", "g")):
            moved = before != after
            if moved.dim() == 4:
                moved = moved.any(dim=-1)
            assert not bool((moved & ~wm).any()), f"ring_{name} written outside its entries"
    if ck0 is not None:
        used = np.zeros(w.N, dtype=bool)
        used[slots[slots >= 0]] = True
        idle = torch.from_numpy(np.where(~used)[0]).to(DEV)
        assert torch.equal(bits(pool.ckpt[idle]), bits(ck0[idle])), "an unused slot changed"
    log(f"[{w.name}/{kind}] {rep.summary()}")
    return rep
