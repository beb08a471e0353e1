"""CPU oracle for the ReplaySSM Gated DeltaNet decode path.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg import this package. The product library neither imports,
links nor calls anything here, and nothing here imports the product.

Parts:
  O1  gdn_step          plain sequential fp64 recurrence (C, liboracle.so);
                        gdn_step_f32, the same in fp32 (the CPU baseline)
  O2  ReplayModel       the checkpoint + ring + cursor state machine, run
                        exactly on the integers and in fp64 on the values,
                        producing outputs through the closed-form replay
  O3  fold_f32          the pinned-rounding fp32 fold (C, liboracle.so)
  O4  window_ref        a verify window evaluated token by token with O1
  O5  quantize          exact rounding to a 16-bit state format (binary16 or
                        bfloat16), for the 16-bit checkpoint variant
  O6  kda_step          the per-key-gate (KDA) recurrence in fp64 (C)
  O7  fold_kda_f32      the pinned-rounding fold with a per-key gate (C)
  O8  l2norm_qk         the decode's front end: q/k L2-normalised, q scaled
  O9  conv_update       the causal convolution (width W, SiLU) and its state
                        in front of the decode
  O10 kda_gates         the per-key gate and beta activations in front of a
                        per-key-gate (KDA) decode
  O2, O4 take the per-key gate as well (ReplayModel(gate="key"), window_ref
  with g [B, T, Hv, dk]).

Every function states the passage it follows. The pages cited are: SGLang
PR #28451 (ReplaySSM decode port), the ReplaySSM blog on llm.rainlin.net,
vLLM PR #49887 (GDN speculative decode), SGLang PR #36821 (KDA fused verify
with a ring) and SGLang PR #42388 (lossless verify).

Parity pins: every function here is checked in tests/test_oracle_pins.py
against exact rational arithmetic, brute-force matrix products, the worked
flush table, closed forms and special cases (none of which reuse this code).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (no contraction, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _bind(L):
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    L.oracle_gdn_step_f64.argtypes = [i32] * 6 + [P] * 9
    L.oracle_gdn_step_f64.restype = None
    L.oracle_gdn_step_f32.argtypes = [i32] * 6 + [P] * 8
    L.oracle_gdn_step_f32.restype = None
    L.oracle_threads.argtypes = [i32]
    L.oracle_threads.restype = i32
    L.oracle_fold_f32.argtypes = [i32] * 7 + [P] * 6 + [i32]
    L.oracle_fold_f32.restype = None
    L.oracle_kda_step_f64.argtypes = [i32] * 6 + [P] * 9
    L.oracle_kda_step_f64.restype = None
    L.oracle_fold_kda_f32.argtypes = [i32] * 7 + [P] * 6
    L.oracle_fold_kda_f32.restype = None
    L.oracle_version.restype = i32
    assert L.oracle_version() == 2
    return L


def timing_library(out_dir: str):
    """A separate build of the same gdn_oracle.c for timing the CPU baseline
    on the machine that runs it: -O3 for that host's instruction set, with the
    OpenMP loop over (row, value head) enabled. Never used for parity (the
    parity build above is -O2 without contraction). Returns (library, flags)."""
    os.makedirs(out_dir, exist_ok=True)
    path = os.path.join(out_dir, "liboracle_timing.so")
    base = ["-std=c11", "-O3", "-fopenmp", "-fPIC", "-shared"]
    for arch in (["-march=native"], []):
        r = subprocess.run(["gcc", *base, *arch, "-o", path, _SRC, "-lm"], capture_output=True)
        if r.returncode == 0:
            return _bind(ctypes.CDLL(path)), " ".join(base + arch)
    raise RuntimeError("could not build the oracle's timing library: " + r.stderr.decode())


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------ O5

# (significant bits, exponent of the smallest normal, largest finite value)
_FORMATS = {"f16": (11, -14, 65504.0),
            "bf16": (8, -126, float(np.ldexp(2.0 - 2.0 ** -7, 127)))}


def quantize(x, fmt: str) -> np.ndarray:
    """O5: round float64 values to the nearest value of a storage format,
    ties to even, returned as float64.

    The pages note that the decode code also handles fp16 and bf16 state
    (vLLM PR #49887, Out of scope: low-precision state); a 16-bit checkpoint
    holds values of these formats. 'f16' is IEEE binary16: 11 significant
    bits, smallest normal 2^-14, subnormal spacing 2^-24, largest finite 65504.
    'bf16' is bfloat16: 8 significant bits and the exponent range of binary32
    (smallest normal 2^-126, subnormal spacing 2^-133). 'f32' rounds to
    binary32. Values beyond the largest finite one round to infinity.
    """
    x = np.asarray(x, np.float64)
    if fmt == "f32":
        return x.astype(np.float32).astype(np.float64)
    p, emin, vmax = _FORMATS[fmt]
    _, e = np.frexp(x)                       # |x| in [2^(e-1), 2^e)
    qexp = np.maximum(e - p, emin - p + 1)   # exponent of the spacing at x
    with np.errstate(over="ignore", invalid="ignore"):
        y = np.ldexp(np.rint(np.ldexp(x, -qexp)), qexp)
        y = np.where(np.abs(y) > vmax, np.copysign(np.inf, x), y)
    return np.where(np.isfinite(x), y, x)


# ------------------------------------------------------------------ O1

def gdn_step(S: np.ndarray, slot: np.ndarray, q, k, v, g, beta,
             want_u: bool = False, state_fmt: Optional[str] = None):
    """O1: one decode token of the gated delta rule, fp64, in place on S.

    Follows the ReplaySSM blog (section 1): S~ = alpha S, u = beta (v - S~ k),
    S_t = S~ + u k^T, y = S_t q, alpha = exp(g).
    S [N,Hv,dv,dk] float64 (modified), slot [B], q,k [B,Hk,dk], v [B,Hv,dv],
    g,beta [B,Hv]. Returns o [B,Hv,dv] (and u when want_u).
    state_fmt ('f16' / 'bf16'): the state is stored in that format after every
    token (O5), as a read-update-write decode with a 16-bit state does.
    """
    assert S.dtype == np.float64 and S.flags.c_contiguous
    N, Hv, dv, dk = S.shape
    B = slot.shape[0]
    Hk = q.shape[1]
    slot = _c(slot, np.int32)
    q, k, v, g, beta = (_c(x, np.float64) for x in (q, k, v, g, beta))
    assert q.shape == (B, Hk, dk) and k.shape == (B, Hk, dk)
    assert v.shape == (B, Hv, dv) and g.shape == (B, Hv) and beta.shape == (B, Hv)
    o = np.empty((B, Hv, dv), np.float64)
    u = np.empty((B, Hv, dv), np.float64) if want_u else None
    lib().oracle_gdn_step_f64(B, N, Hv, Hk, dk, dv, _p(slot), _p(S), _p(q), _p(k),
                              _p(v), _p(g), _p(beta), _p(o), _p(u))
    if state_fmt is not None:
        for s in slot:
            if 0 <= s < N:
                S[s] = quantize(S[s], state_fmt)
    return (o, u) if want_u else o


def gdn_step_f32(S: np.ndarray, slot: np.ndarray, q, k, v, g, beta, library=None):
    """O1's fp32 instance (the same recurrence in float32), in place on S
    [N,Hv,dv,dk] float32; the CPU baseline's decode step. Returns o."""
    assert S.dtype == np.float32 and S.flags.c_contiguous
    N, Hv, dv, dk = S.shape
    B = slot.shape[0]
    Hk = q.shape[1]
    slot = _c(slot, np.int32)
    q, k, v, g, beta = (_c(x, np.float32) for x in (q, k, v, g, beta))
    o = np.empty((B, Hv, dv), np.float32)
    (library or lib()).oracle_gdn_step_f32(B, N, Hv, Hk, dk, dv, _p(slot), _p(S), _p(q), _p(k),
                                           _p(v), _p(g), _p(beta), _p(o))
    return o


# ------------------------------------------------------------------ O6

def kda_step(S: np.ndarray, slot: np.ndarray, q, k, v, g, beta,
             want_u: bool = False, state_fmt: Optional[str] = None):
    """O6: one decode token of the delta rule with a per-key gate (KDA),
    fp64, in place on S.

    Follows SGLang PR #28451 (Modifications, item 7): the same delta rule as
    O1 with the decay per key channel, S~ = S Diag(a), a = exp(g) over the dk
    channels; u = beta (v - S~ k), S_t = S~ + u k^T, y = S_t q.
    g [B, Hv, dk]; every other argument as gdn_step.
    """
    assert S.dtype == np.float64 and S.flags.c_contiguous
    N, Hv, dv, dk = S.shape
    B = slot.shape[0]
    Hk = q.shape[1]
    slot = _c(slot, np.int32)
    q, k, v, g, beta = (_c(x, np.float64) for x in (q, k, v, g, beta))
    assert q.shape == (B, Hk, dk) and k.shape == (B, Hk, dk)
    assert v.shape == (B, Hv, dv) and g.shape == (B, Hv, dk) and beta.shape == (B, Hv)
    o = np.empty((B, Hv, dv), np.float64)
    u = np.empty((B, Hv, dv), np.float64) if want_u else None
    lib().oracle_kda_step_f64(B, N, Hv, Hk, dk, dv, _p(slot), _p(S), _p(q), _p(k),
                              _p(v), _p(g), _p(beta), _p(o), _p(u))
    if state_fmt is not None:
        for s in slot:
            if 0 <= s < N:
                S[s] = quantize(S[s], state_fmt)
    return (o, u) if want_u else o


def step(S: np.ndarray, slot: np.ndarray, q, k, v, g, beta, want_u: bool = False,
         state_fmt: Optional[str] = None):
    """O1 or O6, by the gate's shape: g [B, Hv] (per head) or [B, Hv, dk]
    (per key channel)."""
    f = kda_step if np.ndim(g) == 3 else gdn_step
    return f(S, slot, q, k, v, g, beta, want_u=want_u, state_fmt=state_fmt)


# ------------------------------------------------------------------ O8

QK_NORM_EPS = 1e-6


def l2norm_qk(q, k):
    """O8: the front end the pages put before the decode (SGLang PR #28451,
    Modifications: q arrives L2-normalised and scaled): over the last axis
    (dk), q <- q / sqrt(sum q^2 + eps) * dk^-1/2 and k <- k / sqrt(sum k^2 +
    eps), eps = 1e-6, in fp64. Returns (q, k)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    dk = q.shape[-1]
    nq = np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + QK_NORM_EPS)
    nk = np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + QK_NORM_EPS)
    return q / nq * dk ** -0.5, k / nk


# ------------------------------------------------------------------ O9

def conv_update(x, w, conv_state: np.ndarray, slot) -> np.ndarray:
    """O9: the causal convolution step in front of the decode (ReplaySSM
    blog, section 3.1: the decode path updates the causal convolution first;
    SGLang PR #36821, Technical principle: x_hat_t = SiLU(w * x_{t-3:t})).
    Per channel, the window holds the W-1 previous inputs (conv_state[s],
    [W-1, C], oldest first) and the current one; the output is SiLU of the
    tap-weighted sum (tap W-1 on the current input), in fp64; the window then
    moves by one input. Rows with a slot outside [0, N) are padding: zero
    output, no state change. x [B, C], w [C, W]; conv_state [N, W-1, C] is
    updated in place (fp64). Returns y [B, C] (fp64)."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    B, C = x.shape
    N = conv_state.shape[0]
    y = np.zeros((B, C))
    for b in range(B):
        s = int(slot[b])
        if s < 0 or s >= N:
            continue
        window = np.concatenate([conv_state[s], x[b][None, :]], axis=0)   # [W, C]
        acc = np.einsum("cw,wc->c", w, window)
        y[b] = acc / (1.0 + np.exp(-acc))
        conv_state[s] = window[1:]
    return y


# ------------------------------------------------------------------ O10

def kda_gates(a, b, A, dt_bias, lower_bound: float):
    """O10: the gate activations in front of a per-key-gate (KDA) decode
    (SGLang PR #36821, Technical principle): per key channel the log-decay
    g = lower_bound * sigmoid(exp(A_h) * (a + dt_bias_{h,c})), and per head
    beta = sigmoid(b), in fp64. a [B, T, Hv, dk], b [B, T, Hv], A [Hv],
    dt_bias [Hv, dk], lower_bound < 0 a scalar. Returns (g, beta)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    A = np.asarray(A, np.float64)
    dt = np.asarray(dt_bias, np.float64)
    z = np.exp(A)[:, None] * (a + dt)
    g = lower_bound / (1.0 + np.exp(-z))
    beta = 1.0 / (1.0 + np.exp(-b))
    return g, beta


# ------------------------------------------------------------------ O3

def fold_f32(ckpt: np.ndarray, slot: np.ndarray, write_pos: np.ndarray,
             ring_d: np.ndarray, ring_k: np.ndarray, ring_g: np.ndarray,
             order: int = 0) -> None:
    """O3: fold each listed slot's valid ring entries into its fp32 checkpoint
    with pinned rounding, x <- fma(d_j[v], k_j[k], RN(RN(exp(g_j)) * x)),
    then reset the slot's write_pos to 0 (in place on ckpt and write_pos).

    Follows SGLang PR #42388 ("The idea": a separately rounded decayed state,
    then one FMA for the update) applied to the checkpoint fold of SGLang PR
    #36821 ("Technical principle"). ring_d/ring_k are the ring values upcast
    exactly to fp32. order=1 selects a deliberately different association and
    exists only for the control test.
    """
    assert ckpt.dtype == np.float32 and ckpt.flags.c_contiguous
    assert write_pos.dtype == np.int32 and write_pos.flags.c_contiguous
    N, Hv, dv, dk = ckpt.shape
    Hk, L = ring_k.shape[1], ring_k.shape[2]
    slot = _c(slot, np.int32)
    ring_d, ring_k, ring_g = (_c(x, np.float32) for x in (ring_d, ring_k, ring_g))
    assert ring_d.shape == (N, Hv, L, dv) and ring_k.shape == (N, Hk, L, dk)
    assert ring_g.shape == (N, Hv, L)
    lib().oracle_fold_f32(slot.shape[0], N, Hv, Hk, dk, dv, L, _p(slot), _p(write_pos),
                          _p(ckpt), _p(ring_d), _p(ring_k), _p(ring_g), order)


def fold_kda_f32(ckpt: np.ndarray, slot: np.ndarray, write_pos: np.ndarray,
                 ring_d: np.ndarray, ring_k: np.ndarray, ring_g: np.ndarray) -> None:
    """O7: the fold of O3 with a per-key gate: per element and entry,
    x <- fma(d_j[v], k_j[c], RN(RN(exp(g_j[c])) * x)), then write_pos <- 0.

    The KDA update S Diag(a) + d k^T (SGLang PR #28451, Modifications item 7)
    in the two-instruction rounding of SGLang PR #42388 ("The idea").
    ring_g [N, Hv, L, dk]; everything else as fold_f32.
    """
    assert ckpt.dtype == np.float32 and ckpt.flags.c_contiguous
    assert write_pos.dtype == np.int32 and write_pos.flags.c_contiguous
    N, Hv, dv, dk = ckpt.shape
    Hk, L = ring_k.shape[1], ring_k.shape[2]
    slot = _c(slot, np.int32)
    ring_d, ring_k, ring_g = (_c(x, np.float32) for x in (ring_d, ring_k, ring_g))
    assert ring_d.shape == (N, Hv, L, dv) and ring_k.shape == (N, Hk, L, dk)
    assert ring_g.shape == (N, Hv, L, dk)
    lib().oracle_fold_kda_f32(slot.shape[0], N, Hv, Hk, dk, dv, L, _p(slot), _p(write_pos),
                              _p(ckpt), _p(ring_d), _p(ring_k), _p(ring_g))


# ------------------------------------------------------------------ O2

def next_cursor(p: int, L: int, force: bool) -> Tuple[bool, int]:
    """Flush decision and next cursor of one slot for a single-token step.

    SGLang PR #28451, Design 3 and 5: a step flushes when write_pos == L-1 or
    when force_flush is set; the cursor then becomes 0, otherwise write_pos+1.
    """
    flush = (p == L - 1) or bool(force)
    return flush, (0 if flush else p + 1)


class ReplayModel:
    """O2: the ReplaySSM per-slot state machine, exact on the integers and fp64
    on the values.

    State per slot (ReplaySSM blog, section 2.2 cache layout): a checkpoint
    [Hv, dv, dk], a ring of (u, k, g) entries with capacity L (u per v-head,
    k per k-head, g per v-head) and write_pos, the number of valid entries.

    Values are produced by the method's own route, not by the sequential
    recurrence: the pre-token state is rebuilt with the closed-form replay of
    the blog's section 2.1,
        S_{c+h} = P_h S_c + sum_j w_{j,h} u_j k_j^T,
        P_h = prod_{i=1..h} alpha_i,  w_{j,h} = prod_{i=j+1..h} alpha_i,
    (empty products are 1), and the token is read out with the output-only
    form of SGLang PR #28451 (Modifications):
        d_cur = beta (v - alpha (S k)),  o = alpha (S q) + d_cur (k^T q).
    A non-flush step appends (d_cur, k, g) at position write_pos; a flush step
    writes alpha S + d_cur k^T into the checkpoint and leaves the ring bytes as
    they are (blog section 3.3); only entries below write_pos are ever read
    (SGLang PR #28451, Design 5).

    state_fmt ('f16' / 'bf16'): the checkpoint is stored in that format. It is
    rounded (O5) only when it is written, at a flush and at the end of a fold;
    between writes the state lives in the ring and the replay.

    gate ('head' / 'key'): 'key' is the per-key gate of KDA (SGLang PR #28451,
    Modifications item 7): the ring keeps one log-decay per key channel
    (ring_g [N, Hv, L, dk]), the products above run channel by channel,
        S_{c+h} = S_c Diag(P_h) + sum_j u_j (w_{j,h} o k_j)^T,
    with the decay folded onto the stored keys, and the token's own decay
    a = exp(g) folds into q and k:
        d_cur = beta (v - S (a o k)),  o = S (a o q) + d_cur (k^T q),
    and a flush writes S Diag(a) + d_cur k^T.
    """

    def __init__(self, S0: np.ndarray, Hk: int, L: int, state_fmt: Optional[str] = None,
                 gate: str = "head"):
        assert L >= 1 and gate in ("head", "key")
        self.gate = gate
        self.state_fmt = state_fmt
        self.N, self.Hv, self.dv, self.dk = S0.shape
        self.Hk, self.L = Hk, L
        self.G = self.Hv // Hk
        self.ckpt = np.array(S0, dtype=np.float64, copy=True)
        if state_fmt is not None:
            assert np.array_equal(quantize(self.ckpt, state_fmt), self.ckpt), \
                "the initial checkpoint must hold values of the state format"
        self.ring_u = np.zeros((self.N, self.Hv, L, self.dv))
        self.ring_k = np.zeros((self.N, Hk, L, self.dk))
        self.ring_g = np.zeros((self.N, self.Hv, L) + ((self.dk,) if gate == "key" else ()))
        self.write_pos = np.zeros(self.N, dtype=np.int64)

    def _store(self, X: np.ndarray) -> np.ndarray:
        """A checkpoint write: rounded to the state format, if any."""
        return X if self.state_fmt is None else quantize(X, self.state_fmt)

    # -- closed form -------------------------------------------------------
    @staticmethod
    def replay(S_c: np.ndarray, us, ks, gs) -> np.ndarray:
        """Closed-form state after h entries (blog section 2.1) for one head.
        S_c [dv,dk], us [h,dv], ks [h,dk], gs [h] (or [h,dk]: per-key gate)."""
        h = len(gs)
        if h and np.ndim(gs[0]) == 1:
            return ReplayModel._replay_per_key(S_c, us, ks, gs)
        alpha = [float(np.exp(x)) for x in gs]
        P = 1.0
        for a in alpha:
            P *= a
        S = P * S_c
        for j in range(h):
            w = 1.0
            for i in range(j + 1, h):
                w *= alpha[i]
            S = S + w * np.outer(us[j], ks[j])
        return S

    @staticmethod
    def _replay_per_key(S_c: np.ndarray, us, ks, gs) -> np.ndarray:
        """The closed form with a per-key gate: per channel c,
        P[c] = prod_i exp(g_i[c]), w_j[c] = prod_{i>j} exp(g_i[c]),
        S = S_c Diag(P) + sum_j u_j (w_j o k_j)^T."""
        h = len(gs)
        alpha = [np.exp(np.asarray(x, np.float64)) for x in gs]
        P = np.ones(S_c.shape[1])
        for a in alpha:
            P = P * a
        S = S_c * P[None, :]
        for j in range(h):
            w = np.ones(S_c.shape[1])
            for i in range(j + 1, h):
                w = w * alpha[i]
            S = S + np.outer(us[j], w * np.asarray(ks[j]))
        return S

    def _readout(self, S, qv, kv, vv, gv, bt):
        """(d_cur, o, decayed state) of one token for one head."""
        if self.gate == "key":
            a = np.exp(np.asarray(gv, np.float64))
            d = bt * (vv - S @ (a * kv))
            o = S @ (a * qv) + d * float(kv @ qv)
            return d, o, S * a[None, :]
        alpha = float(np.exp(gv))
        d = bt * (vv - alpha * (S @ kv))
        o = alpha * (S @ qv) + d * float(kv @ qv)
        return d, o, alpha * S

    def head_state(self, s: int, h: int) -> np.ndarray:
        p = int(self.write_pos[s])
        hk = h // self.G
        return self.replay(self.ckpt[s, h], self.ring_u[s, h, :p],
                           self.ring_k[s, hk, :p], self.ring_g[s, h, :p])

    def state(self, s: int) -> np.ndarray:
        return np.stack([self.head_state(s, h) for h in range(self.Hv)])

    # -- single-token decode ---------------------------------------------
    def decode(self, slot, q, k, v, g, beta, force_flush=None):
        """One single-token decode over a batch (T = 1). q,k [B,Hk,dk],
        v [B,Hv,dv], g,beta [B,Hv] (float64). Returns (o [B,Hv,dv], flush [B]).
        The cursors are not moved here; call advance() once per forward."""
        B = len(slot)
        o = np.zeros((B, self.Hv, self.dv))
        flush = np.zeros(B, dtype=bool)
        for b in range(B):
            s = int(slot[b])
            if s < 0:
                continue
            p = int(self.write_pos[s])
            ff = bool(force_flush[b]) if force_flush is not None else False
            flush[b], _ = next_cursor(p, self.L, ff)
            for h in range(self.Hv):
                hk = h // self.G
                S = self.head_state(s, h)
                d, o[b, h], Sd = self._readout(S, q[b, hk], k[b, hk], v[b, h], g[b, h],
                                               beta[b, h])
                if flush[b]:
                    self.ckpt[s, h] = self._store(Sd + np.outer(d, k[b, hk]))
                else:
                    self.ring_u[s, h, p] = d
                    self.ring_g[s, h, p] = g[b, h]
                    self.ring_k[s, hk, p] = k[b, hk]
        return o, flush

    def advance(self, slot, flush) -> None:
        """Cursor advance, once per forward (SGLang PR #28451, Design 3)."""
        for b in range(len(slot)):
            s = int(slot[b])
            if s < 0:
                continue
            self.write_pos[s] = 0 if flush[b] else self.write_pos[s] + 1

    # -- verify window -------------------------------------------------------
    def verify(self, slot, q, k, v, g, beta):
        """A T-token verify window read from the checkpoint and ring (vLLM PR
        #49887, Core concept): every window output comes from the same
        checkpoint plus ring, token t sees tokens < t of the window; the
        window's entries are written at positions p .. p+T-1 and the cursor
        does not move. q,k [B,T,Hk,dk], v [B,T,Hv,dv], g,beta [B,T,Hv].
        Returns o [B,T,Hv,dv]. Rows with p + T > L are invalid: they get zero
        outputs and no writes."""
        B, T = q.shape[0], q.shape[1]
        o = np.zeros((B, T, self.Hv, self.dv))
        for b in range(B):
            s = int(slot[b])
            if s < 0:
                continue
            p = int(self.write_pos[s])
            if p + T > self.L:
                continue
            for h in range(self.Hv):
                hk = h // self.G
                us = list(self.ring_u[s, h, :p])
                ks = list(self.ring_k[s, hk, :p])
                gs = list(self.ring_g[s, h, :p])
                for t in range(T):
                    S = self.replay(self.ckpt[s, h], us, ks, gs)
                    d, o[b, t, h], _ = self._readout(S, q[b, t, hk], k[b, t, hk], v[b, t, h],
                                                     g[b, t, h], beta[b, t, h])
                    us.append(d)
                    ks.append(k[b, t, hk])
                    gs.append(g[b, t, h])
                    self.ring_u[s, h, p + t] = d
                    self.ring_g[s, h, p + t] = g[b, t, h]
                    self.ring_k[s, hk, p + t] = k[b, t, hk]
        return o

    def commit(self, slot, accepted) -> None:
        """Keep the first `accepted` window entries: write_pos += a (vLLM PR
        #49887: rollback is a cursor move)."""
        for b in range(len(slot)):
            s = int(slot[b])
            if s < 0:
                continue
            self.write_pos[s] += int(accepted[b])

    def fold(self, slot) -> None:
        """Fold the valid entries into the checkpoint (fp64, sequential
        S <- alpha S + u k^T per entry) and reset write_pos to 0."""
        for b in range(len(slot)):
            s = int(slot[b])
            if s < 0:
                continue
            p = int(self.write_pos[s])
            for h in range(self.Hv):
                hk = h // self.G
                X = self.ckpt[s, h]
                for j in range(p):
                    a = np.exp(self.ring_g[s, h, j])
                    X = (X * a[None, :] if self.gate == "key" else a * X) + np.outer(
                        self.ring_u[s, h, j], self.ring_k[s, hk, j])
                self.ckpt[s, h] = self._store(X)
            self.write_pos[s] = 0


# ------------------------------------------------------------------ O4

def window_ref(S: np.ndarray, slot, q, k, v, g, beta, want_u: bool = False,
               state_fmt: Optional[str] = None):
    """O4: the outputs of a T-token window, computed by running O1 token by
    token on a copy of the true state (vLLM PR #49887, Tests: the reference
    is the packed decode run on a clone through the window). S is not changed.
    q,k [B,T,Hk,dk], v [B,T,Hv,dv], g,beta [B,T,Hv] (g [B,T,Hv,dk] for the
    per-key gate, which runs O6 instead of O1). Returns o [B,T,Hv,dv]
    (and u [B,T,Hv,dv]). state_fmt: the state is stored in that 16-bit format
    after every token (O5), as the packed decode with a 16-bit state does."""
    Sc = np.array(S, dtype=np.float64, copy=True)
    T = q.shape[1]
    outs, us = [], []
    for t in range(T):
        o, u = step(Sc, slot, q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], want_u=True,
                    state_fmt=state_fmt)
        outs.append(o)
        us.append(u)
    o = np.stack(outs, axis=1)
    return (o, np.stack(us, axis=1)) if want_u else o


def rel_err(x: np.ndarray, ref: np.ndarray) -> float:
    """max |x - ref| / max |ref| (the tolerance measure used throughout)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(x - ref))) if ref.size else 0.0
    if den == 0.0:
        return num
    return num / den
