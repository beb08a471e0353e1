"""Seeded synthetic inputs for the GDN decode workloads.

This module is shared by the oracle-side tests and by the GPU tests and the
benchmark. It holds the workload shapes and the random draws only: none of the
decode's own arithmetic lives here. Everything it returns is a numpy array on
the host; callers copy to the device themselves.

Draws (per row, token and head), as the workloads specify:
  S0   ~ N(0, 0.1^2)                                  checkpoint / initial state
  q, k ~ N(0, 1), L2-normalised in fp32, q scaled by dk**-0.5
  v    ~ N(0, 1)
  g    = logsigmoid(N(2, 1))                          log-decay, per v-head
                                                      (per v-head and key channel
                                                      for a per-key gate, KDA)
  beta = sigmoid(N(0, 1))                             delta-rule strength
  conv front end: raw packed row x ~ N(0, 1), taps ~ N(0, 1/W), first
  window ~ N(0, 1)
The draws are cast to the workload's I/O dtype; consumers that need the exact
values the device sees should use `as_f64`, which upcasts the rounded values.

Normalising q/k and forming g/beta from their pre-activations is the caller's
job in the serving stack (the decode kernel takes q, k, g, beta as given), so it
belongs to the workload recipe, not to the method.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

# ---------------------------------------------------------------- dtypes

try:  # numpy has no bfloat16; emulate it as uint16 bit patterns
    import ml_dtypes  # type: ignore  # noqa: F401
except Exception:  # pragma: no cover
    ml_dtypes = None

DTYPES = ("f32", "bf16", "f16")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (round-to-nearest-even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def cast(x: np.ndarray, dtype: str) -> np.ndarray:
    """Cast fp32 values to a storage dtype: f32 -> float32, f16 -> float16,
    bf16 -> uint16 bit patterns."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return np.ascontiguousarray(x)
    if dtype == "f16":
        return np.ascontiguousarray(x.astype(np.float16))
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a stored array (bf16 given as uint16 bits)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x).astype(np.float64)


# ---------------------------------------------------------------- workloads

@dataclass(frozen=True)
class Workload:
    name: str
    B: int            # rows per call
    N: int            # slots in the pool
    Hv: int
    Hk: int
    dk: int
    dv: int
    L: int            # ring capacity
    steps: int        # decode steps (forwards)
    qkv: str = "bf16"   # q, k, v (and o) storage dtype
    ring: str = "f16"   # d / k ring dtype (g ring is always fp32)
    T: int = 1          # tokens per row per call (verify window when > 1)
    n_pad: int = 0      # rows whose slot index is -1
    permute: bool = False  # rows map to slots by a seeded injection into [0, N)
    stagger: bool = True   # one forced flush per slot during the first L steps
    bf16_values: bool = False  # fp32 tensors carrying bf16-representable values
    state: str = "f32"  # storage dtype of the checkpoint / packed state
    gate: str = "head"  # "head": one log-decay per v-head (GDN); "key": one per
                        # v-head and key channel (KDA)
    qk_raw: bool = False  # q, k as drawn (N(0,1)), for a decode that normalises
                          # them itself
    seed: int = 0

    @property
    def G(self) -> int:
        return self.Hv // self.Hk


# The five workloads (sizes and dtypes as stated for this decode path).
C1 = Workload("c1_tiny_f32", B=2, N=2, Hv=2, Hk=2, dk=32, dv=32, L=4, steps=40,
              qkv="f32", ring="f32", stagger=False, seed=101)
C2 = Workload("c2_standard", B=64, N=64, Hv=32, Hk=16, dk=128, dv=128, L=16,
              steps=64, seed=202)
C3 = Workload("c3_large_pool", B=256, N=512, Hv=32, Hk=16, dk=128, dv=128, L=16,
              steps=64, n_pad=8, permute=True, seed=303)


def c4(L: int, ring: str = "f16") -> Workload:
    """Ring-depth sweep at the standard shapes. The fp32-ring variant carries
    bf16-representable values in fp32 q/k/v/o tensors so that the output dtype
    does not mask the fp32 reconstruction."""
    qkv = "f32" if ring == "f32" else "bf16"
    return replace(C2, name=f"c4_L{L}_{ring}", L=L, ring=ring, qkv=qkv,
                   bf16_values=(ring == "f32"),
                   seed=400 + L + (1000 if ring == "f32" else 0))


C5 = Workload("c5_verify_window", B=32, N=32, Hv=32, Hk=16, dk=128, dv=128,
              L=16, steps=8, T=5, stagger=False, seed=505)

# Lossless verify: every round starts from an exact checkpoint (empty ring),
# stores fp32 tuples for a T-token window, commits the accepted prefix and
# folds it (SGLang PR #42388: MTP-style drafts of 4 plus the verified token).
C6 = Workload("c6_lossless_verify", B=32, N=40, Hv=32, Hk=16, dk=128, dv=128,
              L=8, steps=8, ring="f32", T=5, n_pad=2, permute=True, stagger=False,
              seed=707)

# Per-key gate (KDA, SGLang PR #28451 Modifications item 7) at the shapes the
# pages benchmark it on (Hv=32, Hk=16, dk=dv=128, bf16, L=16), plus a tiny
# fp32 case.
C7 = replace(C2, name="c7_kda", gate="key", seed=808)
C7_TINY = replace(C1, name="c7_kda_tiny", gate="key", seed=809)

WORKLOADS = {w.name: w for w in (C1, C2, C3, c4(1), c4(4), c4(16), c4(32),
                                 c4(16, "f32"), C5, C6, C7, C7_TINY)}


def gate_shape(w: Workload, *lead: int) -> tuple:
    """Shape of a gate tensor with leading dims `lead`: [..., Hv] for the
    per-head gate, [..., Hv, dk] for the per-key gate."""
    return (*lead, w.Hv) + ((w.dk,) if w.gate == "key" else ())


def scaled(w: Workload, **kw) -> Workload:
    """A smaller (or otherwise edited) copy of a workload."""
    return replace(w, **kw)


# ---------------------------------------------------------------- draws

def _rng(seed: int, *tags: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([seed, *tags]))


def _logsigmoid(x: np.ndarray) -> np.ndarray:
    return -np.logaddexp(0.0, -x)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _unit_rows(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float32)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def initial_state(w: Workload) -> np.ndarray:
    """fp32 checkpoint pool [N, Hv, dv, dk], S0 ~ N(0, 0.1^2)."""
    r = _rng(w.seed, 0)
    return (0.1 * r.standard_normal((w.N, w.Hv, w.dv, w.dk), dtype=np.float32)).astype(np.float32)


def stored_state(w: Workload) -> np.ndarray:
    """The initial state pool in the workload's state storage dtype (S0 as
    drawn, rounded to nearest even for a 16-bit format; bf16 as uint16 bits)."""
    return cast(initial_state(w), w.state)


def slot_map(w: Workload) -> np.ndarray:
    """Row -> slot indices [B] int32; -1 marks a padding row."""
    r = _rng(w.seed, 1)
    if w.permute:
        slots = r.permutation(w.N)[: w.B].astype(np.int32)
    else:
        slots = np.arange(w.B, dtype=np.int32) % max(w.N, 1)
    if w.n_pad:
        pad = r.choice(w.B, size=w.n_pad, replace=False)
        slots[pad] = -1
    return slots


@dataclass
class StepInputs:
    """One call's inputs in storage dtypes (bf16 as uint16 bits)."""
    q: np.ndarray      # [B, T, Hk, dk]
    k: np.ndarray      # [B, T, Hk, dk]
    v: np.ndarray      # [B, T, Hv, dv]
    g: np.ndarray      # [B, T, Hv] fp32 ([B, T, Hv, dk] with a per-key gate)
    beta: np.ndarray   # [B, T, Hv] fp32
    dtype: str

    def f64(self):
        """Exact float64 values of (q, k, v, g, beta)."""
        return (as_f64(self.q, self.dtype), as_f64(self.k, self.dtype),
                as_f64(self.v, self.dtype), self.g.astype(np.float64),
                self.beta.astype(np.float64))


def step_inputs(w: Workload, step: int, B: Optional[int] = None,
                T: Optional[int] = None) -> StepInputs:
    B = w.B if B is None else B
    T = w.T if T is None else T
    r = _rng(w.seed, 2, step)
    q = r.standard_normal((B, T, w.Hk, w.dk), dtype=np.float32)
    k = r.standard_normal((B, T, w.Hk, w.dk), dtype=np.float32)
    if not w.qk_raw:
        q = (_unit_rows(q) * np.float32(w.dk ** -0.5)).astype(np.float32)
        k = _unit_rows(k)
    v = r.standard_normal((B, T, w.Hv, w.dv), dtype=np.float32)
    g = _logsigmoid(r.normal(2.0, 1.0, gate_shape(w, B, T))).astype(np.float32)
    beta = _sigmoid(r.standard_normal((B, T, w.Hv))).astype(np.float32)
    if w.bf16_values:
        q, k, v = (bf16_bits_to_f32(f32_to_bf16_bits(a)) for a in (q, k, v))
    return StepInputs(cast(q, w.qkv), cast(k, w.qkv), cast(v, w.qkv), g, beta, w.qkv)


def force_flush_schedule(w: Workload, step: int, slots: np.ndarray) -> np.ndarray:
    """[B] int32 flags. With stagger on, slot s is forced to flush at step s mod L
    during the first L steps, which spreads the flush phases of the slots
    evenly over the ring cycle; afterwards no row is forced."""
    ff = np.zeros(slots.shape[0], dtype=np.int32)
    if w.stagger and step < w.L:
        ff[(slots >= 0) & ((slots % w.L) == step)] = 1
    return ff


def accepted_counts(w: Workload, rnd: int) -> np.ndarray:
    """Accepted prefix length per row of a verify round, a ~ U{0..T}."""
    r = _rng(w.seed, 3, rnd)
    return r.integers(0, w.T + 1, size=w.B).astype(np.int32)


def history_lengths(w: Workload) -> np.ndarray:
    """Per-slot number of single-token steps run before the verify rounds,
    h ~ U{0..L-T}, so that no history step reaches a flush."""
    r = _rng(w.seed, 4)
    return r.integers(0, max(w.L - w.T, 0) + 1, size=w.N).astype(np.int32)


# ---------------------------------------------------------------- ring contents

@dataclass
class RingContents:
    """A filled ring pool (storage dtypes) plus its per-slot cursors."""
    ckpt: np.ndarray     # [N, Hv, dv, dk] fp32
    d: np.ndarray        # [N, Hv, L, dv] ring dtype (bf16 as bits)
    k: np.ndarray        # [N, Hk, L, dk]
    g: np.ndarray        # [N, Hv, L] fp32 ([N, Hv, L, dk] with a per-key gate)
    write_pos: np.ndarray  # [N] int32
    dtype: str


def random_ring(w: Workload, seed_tag: int = 0, full: bool = False) -> RingContents:
    """Random ring pool: d ~ N(0, 1) (the magnitude of beta*(v - ...)), unit keys,
    g as above, cursors p ~ U{0..L} (or p = L when `full`)."""
    r = _rng(w.seed, 5, seed_tag)
    ckpt = (0.1 * r.standard_normal((w.N, w.Hv, w.dv, w.dk), dtype=np.float32)).astype(np.float32)
    d = r.standard_normal((w.N, w.Hv, w.L, w.dv), dtype=np.float32)
    k = _unit_rows(r.standard_normal((w.N, w.Hk, w.L, w.dk), dtype=np.float32))
    if w.gate == "key":
        g = _logsigmoid(r.normal(2.0, 1.0, (w.N, w.Hv, w.L, w.dk))).astype(np.float32)
    else:
        g = _logsigmoid(r.normal(2.0, 1.0, (w.N, w.Hv, w.L))).astype(np.float32)
    if full:
        wp = np.full(w.N, w.L, dtype=np.int32)
    else:
        wp = r.integers(0, w.L + 1, size=w.N).astype(np.int32)
    return RingContents(ckpt, cast(d, w.ring), cast(k, w.ring), g, wp, w.ring)


# ---------------------------------------------------------------- conv front end

@dataclass
class ConvInputs:
    """Raw mixed_qkv rows, taps and a first window for the causal convolution
    in front of the decode (storage dtypes, bf16 as bits)."""
    x: np.ndarray      # [steps, B, C]
    w: np.ndarray      # [C, W]
    state: np.ndarray  # [N, W-1, C]
    dtype: str

    def f64(self):
        return (as_f64(self.x, self.dtype), as_f64(self.w, self.dtype),
                as_f64(self.state, self.dtype))


def conv_channels(w: Workload) -> int:
    """Channels of the packed mixed_qkv row, 2*Hk*dk + Hv*dv."""
    return 2 * w.Hk * w.dk + w.Hv * w.dv


def conv_inputs(w: Workload, steps: int, W: int = 4, C: Optional[int] = None,
                seed_tag: int = 0) -> ConvInputs:
    """x ~ N(0, 1) per channel (raw projection outputs), taps ~ N(0, 1/W) (a
    filter that keeps the input's scale), first window ~ N(0, 1)."""
    C = conv_channels(w) if C is None else C
    r = _rng(w.seed, 6, seed_tag)
    x = r.standard_normal((steps, w.B, C), dtype=np.float32)
    taps = (r.standard_normal((C, W), dtype=np.float32) / np.float32(np.sqrt(W))).astype(np.float32)
    st = r.standard_normal((w.N, W - 1, C), dtype=np.float32)
    return ConvInputs(cast(x, w.qkv), cast(taps, w.qkv), cast(st, w.qkv), w.qkv)


def garbage_like(shape, dtype: str, seed: int = 7) -> np.ndarray:
    """A recognisable garbage template (including NaN/Inf bit patterns) used to
    pre-fill buffers so that writes outside the intended entries show up."""
    r = _rng(seed, 9)
    if dtype == "f32":
        bits = r.integers(0, 2**32, size=shape, dtype=np.uint64).astype(np.uint32)
        return bits.view(np.float32)
    if dtype == "f16":
        return r.integers(0, 2**16, size=shape, dtype=np.uint64).astype(np.uint16).view(np.float16)
    if dtype == "bf16":
        return r.integers(0, 2**16, size=shape, dtype=np.uint64).astype(np.uint16)
    raise ValueError(dtype)
