"""Python binding of libgdn_replay.so (the MI355X ReplaySSM GDN decode library).

Argument marshalling only: every function checks the tensors it is given,
derives the sizes, and calls the C entry point of the same name on the
current HIP stream. All arithmetic runs in the library's gfx950 kernels. There
is no fallback: if the library is missing, importing this package raises.

PyTorch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn_replay.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "gdn_replay.h")

GDN_OK, GDN_ERR_INVALID_ARG, GDN_ERR_UNSUPPORTED, GDN_ERR_HIP, GDN_ERR_SCRATCH_LIMIT = 0, 1, 2, 3, 4
GDN_F32, GDN_BF16, GDN_F16 = 0, 1, 2
GDN_GATE_HEAD, GDN_GATE_KEY = 0, 1
ARRIVE_STRIDE = 32          # int32 per row in the arrive workspace (GDN_ARRIVE_STRIDE)
SCRATCH_MAX_ROWS = 4096     # rows of gdn_replay_decode_advance_noalloc (GDN_SCRATCH_MAX_ROWS)
EF_SLOT_RANGE, EF_CURSOR_RANGE, EF_WINDOW, EF_ACCEPTED = 1, 2, 4, 8

_DT = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16, torch.float16: GDN_F16}
STATE_DTYPES = (torch.float32, torch.bfloat16, torch.float16)


class gdn_shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "T", "N", "Hv", "Hk", "dk", "dv", "L", "qkv_dtype", "ring_dtype", "window",
                 "state_dtype", "step_rounding", "gate", "qk_row_stride", "v_row_stride",
                 "qk_norm")]


class gdn_conv_shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "N", "C", "W", "dtype", "x_row_stride", "y_row_stride")]


class gdn_gate_shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("Hv", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("lower_bound", ctypes.c_float)]


class GdnError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {lib().gdn_status_string(status).decode()} (status {status})")
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run __graft_entry__.build() "
        "(or python linear_attention_ssm_amd/build.py) first")

_lib = ctypes.CDLL(LIB_PATH)
_P = ctypes.c_void_p
_S = ctypes.POINTER(gdn_shape)
_lib.gdn_packed_decode.argtypes = [_S] + [_P] * 10
_lib.gdn_replay_decode.argtypes = [_S] + [_P] * 15
_lib.gdn_replay_decode_advance.argtypes = [_S] + [_P] * 16
_lib.gdn_replay_decode_advance_noalloc.argtypes = [_S] + [_P] * 15
_lib.gdn_replay_advance.argtypes = [_S] + [_P] * 5
_lib.gdn_replay_commit.argtypes = [_S] + [_P] * 5
_lib.gdn_replay_fold.argtypes = [_S] + [_P] * 8
_lib.gdn_replay_fold_layers.argtypes = [_S, ctypes.c_int32] + [_P] * 8
_lib.gdn_replay_reset.argtypes = [_S] + [_P] * 4
_lib.gdn_conv_update.argtypes = [ctypes.POINTER(gdn_conv_shape)] + [_P] * 7
_lib.gdn_kda_gates.argtypes = [ctypes.POINTER(gdn_gate_shape)] + [_P] * 7
for _f in ("gdn_packed_decode", "gdn_replay_decode", "gdn_replay_decode_advance",
           "gdn_replay_decode_advance_noalloc", "gdn_replay_advance",
           "gdn_replay_commit", "gdn_replay_fold", "gdn_replay_fold_layers",
           "gdn_replay_reset", "gdn_conv_update",
           "gdn_kda_gates"):
    getattr(_lib, _f).restype = ctypes.c_int
_lib.gdn_hbm_read_probe.argtypes = [_P, ctypes.c_size_t, _P, _P]
_lib.gdn_hbm_read_probe.restype = ctypes.c_int
_lib.gdn_hbm_copy_probe.argtypes = [_P, _P, ctypes.c_size_t, _P]
_lib.gdn_hbm_copy_probe.restype = ctypes.c_int
_lib.gdn_status_string.argtypes = [ctypes.c_int]
_lib.gdn_status_string.restype = ctypes.c_char_p
_lib.gdn_abi_version.restype = ctypes.c_int32
ABI_VERSION = 12
if _lib.gdn_abi_version() != ABI_VERSION:
    raise ImportError("libgdn_replay.so ABI version mismatch; rebuild it")


def lib():
    return _lib


def declared_symbols() -> list:
    """Function names declared in include/gdn_replay.h."""
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"^\S[^;(]*?\b(gdn_\w+)\s*\(", text, flags=re.M)))


# ------------------------------------------------------------------ helpers

def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(t: torch.Tensor, name: str, dtype=None, ndim=None, dev=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def _raise(status: int, what: str):
    if status != GDN_OK:
        raise GdnError(status, what)


def _row_stride(t: torch.Tensor, name: str) -> int:
    """Elements between consecutive (b, t) rows of a [B, T, H, d] input whose
    [H, d] part is dense: q, k and v may be views into one packed mixed_qkv
    row (the C ABI's qk_row_stride / v_row_stride)."""
    B, T, H, d = t.shape
    s0, s1, s2, s3 = t.stride()
    if s3 != 1 or s2 != d:
        raise ValueError(f"{name}: each row's [heads, d] block must be dense, got strides "
                         f"{t.stride()} for shape {tuple(t.shape)}")
    if T > 1:
        rs = s1
        if B > 1 and s0 != T * s1:
            raise ValueError(f"{name}: rows must be evenly spaced over (b, t)")
    else:
        rs = s0 if B > 1 else H * d
    if rs < H * d:
        raise ValueError(f"{name}: rows overlap (row stride {rs} < {H * d})")
    return int(rs)


def _check_rows(t, name, dtype, dev):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda or t.device != dev:
        raise ValueError(f"{name} must be a device tensor on {dev}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.dim() != 4:
        raise ValueError(f"{name} must have 4 dims, got {tuple(t.shape)}")


def _io_shape(q, k, v, g, beta, slot_idx):
    """Sizes of a call; the gate is per head when g is [B,T,Hv] and per key
    channel (KDA) when g is [B,T,Hv,dk]. q, k, v may be strided views (rows of
    [heads, d] dense), e.g. into a packed mixed_qkv tensor."""
    if not isinstance(q, torch.Tensor):
        raise TypeError("q must be a torch.Tensor")
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"q has dtype {q.dtype}")
    dev = q.device
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _check_rows(t, name, q.dtype, dev)
    _check(g, "g", torch.float32, None, dev)
    _check(beta, "beta", torch.float32, 3, dev)
    _check(slot_idx, "slot_idx", torch.int32, 1, dev)
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    gate = GDN_GATE_KEY if g.dim() == 4 else GDN_GATE_HEAD
    g_shape = (B, T, Hv, dk) if gate == GDN_GATE_KEY else (B, T, Hv)
    if k.shape != q.shape or v.shape[:2] != (B, T) or tuple(g.shape) != g_shape \
            or beta.shape != (B, T, Hv) or slot_idx.shape != (B,):
        raise ValueError("inconsistent q/k/v/g/beta/slot_idx shapes")
    qs, ks, vs = _row_stride(q, "q"), _row_stride(k, "k"), _row_stride(v, "v")
    if ks != qs:
        raise ValueError("q and k must have the same row stride")
    return B, T, Hk, dk, Hv, dv, dev, gate, qs, vs


def _row_flags(t, name, B, dev):
    """An optional int32 [B] per-row array (force_flush, accepted)."""
    if t is not None:
        _check(t, name, torch.int32, 1, dev)
        if tuple(t.shape) != (B,):
            raise ValueError(f"{name} must be [B] = [{B}], got {tuple(t.shape)}")


def _err_word(err_flags, dev):
    if err_flags is not None:
        _check(err_flags, "err_flags", torch.int32, None, dev)
        if err_flags.numel() < 1:
            raise ValueError("err_flags must hold at least one int32")


def _state_of(state, Hv, dv, dk, dev):
    _check(state, "state", STATE_DTYPES, 4, dev)
    if tuple(state.shape[1:]) != (Hv, dv, dk):
        raise ValueError("state must be [N, Hv, dv, dk]")


def _out(o, B, T, Hv, dv, dtype, dev):
    if o is None:
        return torch.empty((B, T, Hv, dv), dtype=dtype, device=dev)
    _check(o, "o", dtype, 4, dev)
    if tuple(o.shape) != (B, T, Hv, dv):
        raise ValueError("o has the wrong shape")
    return o


# ------------------------------------------------------------------ entry points

def _shape(B, T, N, Hv, Hk, dk, dv, L, qkv, ring, window, state, stepr, gate, qs, vs, qk_norm):
    """The gdn_shape of a decode call (dense strides passed as 0)."""
    return gdn_shape(B, T, N, Hv, Hk, dk, dv, L, qkv, ring, int(bool(window)), state,
                     int(bool(stepr)), gate, 0 if qs == Hk * dk else qs,
                     0 if vs == Hv * dv else vs, int(bool(qk_norm)))


def gdn_packed_decode(q, k, v, g, beta, slot_idx, state, o=None, err_flags=None, stream=None,
                      qk_norm=False):
    """Plain read-update-write decode step; see gdn_packed_decode in gdn_replay.h.
    q,k [B,1,Hk,dk]; v [B,1,Hv,dv]; g,beta [B,1,Hv] fp32 (g [B,1,Hv,dk] for the
    per-key gate); slot_idx [B] int32; state [N,Hv,dv,dk] fp32, bf16 or fp16
    (updated in place). q, k, v may be strided views (e.g. into a packed
    mixed_qkv row); qk_norm L2-normalises q and k in the kernel and scales q.
    Returns o [B,1,Hv,dv]."""
    B, T, Hk, dk, Hv, dv, dev, gate, qs, vs = _io_shape(q, k, v, g, beta, slot_idx)
    _state_of(state, Hv, dv, dk, dev)
    _err_word(err_flags, dev)
    o = _out(o, B, T, Hv, dv, q.dtype, dev)
    sh = _shape(B, T, state.shape[0], Hv, Hk, dk, dv, 1, _DT[q.dtype], GDN_F32, 0,
                _DT[state.dtype], 0, gate, qs, vs, qk_norm)
    _raise(_lib.gdn_packed_decode(ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                  _ptr(slot_idx), _ptr(state), _ptr(o), _ptr(err_flags),
                                  _stream(stream)), "gdn_packed_decode")
    return o


def _ring_shape(ckpt, ring_d, ring_k, ring_g, write_pos, Hv, Hk, dk, dv, dev, gate):
    _check(ckpt, "ckpt", STATE_DTYPES, 4, dev)
    _check(ring_d, "ring_d", (torch.float32, torch.float16, torch.bfloat16), 4, dev)
    _check(ring_k, "ring_k", ring_d.dtype, 4, dev)
    _check(ring_g, "ring_g", torch.float32, 4 if gate == GDN_GATE_KEY else 3, dev)
    _check(write_pos, "write_pos", torch.int32, 1, dev)
    N = ckpt.shape[0]
    L = ring_d.shape[2]
    g_shape = (N, Hv, L, dk) if gate == GDN_GATE_KEY else (N, Hv, L)
    if tuple(ckpt.shape) != (N, Hv, dv, dk) or tuple(ring_d.shape) != (N, Hv, L, dv) \
            or tuple(ring_k.shape) != (N, Hk, L, dk) or tuple(ring_g.shape) != g_shape \
            or tuple(write_pos.shape) != (N,):
        raise ValueError("inconsistent checkpoint / ring / write_pos shapes")
    return N, L


def gdn_replay_decode(q, k, v, g, beta, slot_idx, ckpt, ring_d, ring_k, ring_g, write_pos,
                      force_flush=None, o=None, err_flags=None, window=False, stream=None,
                      step_rounding=False, qk_norm=False):
    """ReplaySSM decode step (window=False, T=1) or verify window (window=True);
    see gdn_replay_decode in gdn_replay.h. step_rounding (windows only) rounds
    a 16-bit state after every token. Returns o [B,T,Hv,dv]."""
    B, T, Hk, dk, Hv, dv, dev, gate, qs, vs = _io_shape(q, k, v, g, beta, slot_idx)
    N, L = _ring_shape(ckpt, ring_d, ring_k, ring_g, write_pos, Hv, Hk, dk, dv, dev, gate)
    _row_flags(force_flush, "force_flush", B, dev)
    _err_word(err_flags, dev)
    o = _out(o, B, T, Hv, dv, q.dtype, dev)
    sh = _shape(B, T, N, Hv, Hk, dk, dv, L, _DT[q.dtype], _DT[ring_d.dtype], window,
                _DT[ckpt.dtype], step_rounding, gate, qs, vs, qk_norm)
    _raise(_lib.gdn_replay_decode(ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                  _ptr(slot_idx), _ptr(ckpt), _ptr(ring_d), _ptr(ring_k),
                                  _ptr(ring_g), _ptr(write_pos), _ptr(force_flush), _ptr(o),
                                  _ptr(err_flags), _stream(stream)), "gdn_replay_decode")
    return o


def arrive_workspace(B: int, device) -> torch.Tensor:
    """A zeroed arrive workspace for gdn_replay_decode_advance with B rows
    (torch's allocations are 256-byte aligned)."""
    return torch.zeros(B * ARRIVE_STRIDE, dtype=torch.int32, device=device)


def gdn_replay_decode_advance(q, k, v, g, beta, slot_idx, ckpt, ring_d, ring_k, ring_g,
                              write_pos, arrive, force_flush=None, o=None, err_flags=None,
                              stream=None, qk_norm=False):
    """A decode step with the cursor advance fused in (the forward's last
    layer); see gdn_replay_decode_advance in gdn_replay.h. arrive: int32
    [B * ARRIVE_STRIDE] workspace, all zero (the call leaves it zero); see
    arrive_workspace(). Returns o [B,1,Hv,dv]."""
    B, T, Hk, dk, Hv, dv, dev, gate, qs, vs = _io_shape(q, k, v, g, beta, slot_idx)
    N, L = _ring_shape(ckpt, ring_d, ring_k, ring_g, write_pos, Hv, Hk, dk, dv, dev, gate)
    _check(arrive, "arrive", torch.int32, 1, dev)
    if arrive.shape != (B * ARRIVE_STRIDE,):
        raise ValueError("arrive must be [B * ARRIVE_STRIDE]")
    _row_flags(force_flush, "force_flush", B, dev)
    _err_word(err_flags, dev)
    o = _out(o, B, T, Hv, dv, q.dtype, dev)
    sh = _shape(B, T, N, Hv, Hk, dk, dv, L, _DT[q.dtype], _DT[ring_d.dtype], 0,
                _DT[ckpt.dtype], 0, gate, qs, vs, qk_norm)
    _raise(_lib.gdn_replay_decode_advance(
        ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(slot_idx),
        _ptr(ckpt), _ptr(ring_d), _ptr(ring_k), _ptr(ring_g), _ptr(write_pos), _ptr(force_flush),
        _ptr(o), _ptr(arrive), _ptr(err_flags), _stream(stream)), "gdn_replay_decode_advance")
    return o


def gdn_replay_decode_advance_noalloc(q, k, v, g, beta, slot_idx, ckpt, ring_d, ring_k, ring_g,
                                      write_pos, o, force_flush=None, err_flags=None,
                                      stream=None, qk_norm=False):
    """gdn_replay_decode_advance without the arrive workspace, for callers that
    cannot allocate: the library counts in its own static device scratch (at
    most SCRATCH_MAX_ROWS rows); see gdn_replay_decode_advance_noalloc in
    gdn_replay.h. o [B,1,Hv,dv] must be given (nothing is allocated here
    either). Returns o."""
    B, T, Hk, dk, Hv, dv, dev, gate, qs, vs = _io_shape(q, k, v, g, beta, slot_idx)
    N, L = _ring_shape(ckpt, ring_d, ring_k, ring_g, write_pos, Hv, Hk, dk, dv, dev, gate)
    _row_flags(force_flush, "force_flush", B, dev)
    _err_word(err_flags, dev)
    if o is None:
        raise ValueError("o must be given: this call allocates nothing")
    o = _out(o, B, T, Hv, dv, q.dtype, dev)
    sh = _shape(B, T, N, Hv, Hk, dk, dv, L, _DT[q.dtype], _DT[ring_d.dtype], 0,
                _DT[ckpt.dtype], 0, gate, qs, vs, qk_norm)
    _raise(_lib.gdn_replay_decode_advance_noalloc(
        ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(slot_idx),
        _ptr(ckpt), _ptr(ring_d), _ptr(ring_k), _ptr(ring_g), _ptr(write_pos), _ptr(force_flush),
        _ptr(o), _ptr(err_flags), _stream(stream)), "gdn_replay_decode_advance_noalloc")
    return o


def gdn_replay_advance(slot_idx, write_pos, L, force_flush=None, err_flags=None, stream=None):
    """Cursor advance once per forward; see gdn_replay_advance in gdn_replay.h."""
    _check(slot_idx, "slot_idx", torch.int32, 1)
    _check(write_pos, "write_pos", torch.int32, 1, slot_idx.device)
    _row_flags(force_flush, "force_flush", slot_idx.shape[0], slot_idx.device)
    _err_word(err_flags, slot_idx.device)
    sh = gdn_shape(slot_idx.shape[0], 1, write_pos.shape[0], 1, 1, 32, 16, int(L), 0, 0, 0, 0)
    _raise(_lib.gdn_replay_advance(ctypes.byref(sh), _ptr(slot_idx), _ptr(write_pos),
                                   _ptr(force_flush), _ptr(err_flags), _stream(stream)),
           "gdn_replay_advance")


def gdn_replay_commit(slot_idx, accepted, write_pos, L, T, err_flags=None, stream=None):
    """write_pos[slot] += accepted; see gdn_replay_commit in gdn_replay.h."""
    _check(slot_idx, "slot_idx", torch.int32, 1)
    _check(accepted, "accepted", torch.int32, 1, slot_idx.device)
    _row_flags(accepted, "accepted", slot_idx.shape[0], slot_idx.device)
    _check(write_pos, "write_pos", torch.int32, 1, slot_idx.device)
    _err_word(err_flags, slot_idx.device)
    sh = gdn_shape(slot_idx.shape[0], int(T), write_pos.shape[0], 1, 1, 32, 16, int(L), 0, 0, 0,
                   0)
    _raise(_lib.gdn_replay_commit(ctypes.byref(sh), _ptr(slot_idx), _ptr(accepted),
                                  _ptr(write_pos), _ptr(err_flags), _stream(stream)),
           "gdn_replay_commit")


def gdn_replay_fold(slot_idx, ckpt, ring_d, ring_k, ring_g, write_pos, err_flags=None,
                    stream=None, step_rounding=False):
    """Exact fold of one layer's valid ring entries into its checkpoint
    (write_pos is only read); see gdn_replay_fold in gdn_replay.h.
    step_rounding rounds a 16-bit state after every entry."""
    _check(slot_idx, "slot_idx", torch.int32, 1)
    dev = slot_idx.device
    _check(ckpt, "ckpt", STATE_DTYPES, 4, dev)
    N, Hv, dv, dk = ckpt.shape
    Hk = ring_k.shape[1]
    gate = GDN_GATE_KEY if ring_g.dim() == 4 else GDN_GATE_HEAD
    _, L = _ring_shape(ckpt, ring_d, ring_k, ring_g, write_pos, Hv, Hk, dk, dv, dev, gate)
    _err_word(err_flags, dev)
    sh = gdn_shape(slot_idx.shape[0], 1, N, Hv, Hk, dk, dv, L, GDN_F32, _DT[ring_d.dtype], 0,
                   _DT[ckpt.dtype], int(bool(step_rounding)), gate)
    _raise(_lib.gdn_replay_fold(ctypes.byref(sh), _ptr(slot_idx), _ptr(ckpt), _ptr(ring_d),
                                _ptr(ring_k), _ptr(ring_g), _ptr(write_pos), _ptr(err_flags),
                                _stream(stream)), "gdn_replay_fold")


def gdn_replay_fold_layers(slot_idx, ckpts, ring_ds, ring_ks, ring_gs, write_pos,
                           err_flags=None, stream=None, step_rounding=False):
    """gdn_replay_fold of several layers of equal shapes and dtypes in as few
    launches as possible (ckpts[l] folds ring_ds[l], ring_ks[l], ring_gs[l]);
    see gdn_replay_fold_layers in gdn_replay.h."""
    n = len(ckpts)
    if n < 1 or not (len(ring_ds) == len(ring_ks) == len(ring_gs) == n):
        raise ValueError("one checkpoint, ring_d, ring_k and ring_g per layer")
    _check(slot_idx, "slot_idx", torch.int32, 1)
    dev = slot_idx.device
    _check(ckpts[0], "ckpt", STATE_DTYPES, 4, dev)
    N, Hv, dv, dk = ckpts[0].shape
    Hk = ring_ks[0].shape[1]
    gate = GDN_GATE_KEY if ring_gs[0].dim() == 4 else GDN_GATE_HEAD
    L = None
    for c, rd, rk, rg in zip(ckpts, ring_ds, ring_ks, ring_gs):
        if c.dtype != ckpts[0].dtype or rd.dtype != ring_ds[0].dtype or rg.dim() != ring_gs[0].dim():
            raise ValueError("every layer needs the dtypes of layer 0")
        if c.shape != ckpts[0].shape:
            raise ValueError("every layer needs the checkpoint shape of layer 0")
        _, Ll = _ring_shape(c, rd, rk, rg, write_pos, Hv, Hk, dk, dv, dev, gate)
        if L is not None and Ll != L:
            raise ValueError("every layer needs the ring depth of layer 0")
        L = Ll
    _err_word(err_flags, dev)
    sh = gdn_shape(slot_idx.shape[0], 1, N, Hv, Hk, dk, dv, L, GDN_F32, _DT[ring_ds[0].dtype], 0,
                   _DT[ckpts[0].dtype], int(bool(step_rounding)), gate)
    arr = lambda ts: (ctypes.c_void_p * n)(*[t.data_ptr() for t in ts])
    _raise(_lib.gdn_replay_fold_layers(ctypes.byref(sh), n, _ptr(slot_idx), arr(ckpts),
                                       arr(ring_ds), arr(ring_ks), arr(ring_gs), _ptr(write_pos),
                                       _ptr(err_flags), _stream(stream)),
           "gdn_replay_fold_layers")


def gdn_replay_reset(slot_idx, write_pos, err_flags=None, stream=None):
    """write_pos[slot] = 0 after every layer has folded; see gdn_replay_reset
    in gdn_replay.h."""
    _check(slot_idx, "slot_idx", torch.int32, 1)
    _check(write_pos, "write_pos", torch.int32, 1, slot_idx.device)
    _err_word(err_flags, slot_idx.device)
    sh = gdn_shape(slot_idx.shape[0], 1, write_pos.shape[0], 1, 1, 32, 16, 1, 0, 0, 0, 0)
    _raise(_lib.gdn_replay_reset(ctypes.byref(sh), _ptr(slot_idx), _ptr(write_pos),
                                 _ptr(err_flags), _stream(stream)), "gdn_replay_reset")


def gdn_hbm_read_probe(src: torch.Tensor, sink: torch.Tensor, stream=None):
    """Stream `src` (a device tensor, its byte size a multiple of 32 KiB) once
    in the decode's checkpoint read pattern; see gdn_hbm_read_probe in
    gdn_replay.h. A measurement aid (the measured read peak)."""
    _check(src, "src", None, None)
    _check(sink, "sink", torch.float32, None, src.device)
    nbytes = src.numel() * src.element_size()
    _raise(_lib.gdn_hbm_read_probe(_ptr(src), ctypes.c_size_t(nbytes), _ptr(sink), _stream(stream)),
           "gdn_hbm_read_probe")


def gdn_hbm_copy_probe(src: torch.Tensor, dst: torch.Tensor, stream=None):
    """Copy `src` into `dst` (device tensors of the same byte size, a multiple
    of 32 KiB; `dst` may be `src`) in the pattern of a checkpoint read and
    written back; see gdn_hbm_copy_probe in gdn_replay.h. A measurement aid
    (the measured read + write peak)."""
    _check(src, "src", None, None)
    _check(dst, "dst", None, None, src.device)
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must have the same byte size")
    _raise(_lib.gdn_hbm_copy_probe(_ptr(src), _ptr(dst), ctypes.c_size_t(nbytes), _stream(stream)),
           "gdn_hbm_copy_probe")


# ------------------------------------------------------------------ prepared calls

def gdn_conv_update(x, w, conv_state, slot_idx, y=None, err_flags=None, stream=None):
    """Causal convolution step in front of the decode; see gdn_conv_update in
    gdn_replay.h. x [B, C] fp32 or bf16 (rows may be strided, channels dense);
    w [C, W] and conv_state [N, W-1, C] (updated in place) of x's dtype;
    slot_idx [B] int32. Returns y [B, C] (SiLU of the tap sum), the convolved
    mixed_qkv row for the decode."""
    if not isinstance(x, torch.Tensor):
        raise TypeError("x must be a torch.Tensor")
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"x has dtype {x.dtype}")
    dev = x.device
    if not x.is_cuda or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a [B, C] device tensor with dense channels")
    B, C = x.shape
    xs = int(x.stride(0)) if B > 1 else C
    _check(w, "w", x.dtype, 2, dev)
    _check(conv_state, "conv_state", x.dtype, 3, dev)
    _check(slot_idx, "slot_idx", torch.int32, 1, dev)
    W = w.shape[1]
    if w.shape[0] != C or tuple(conv_state.shape[1:]) != (W - 1, C) or slot_idx.shape != (B,):
        raise ValueError("inconsistent x / w / conv_state / slot_idx shapes")
    if y is None:
        y = torch.empty((B, C), dtype=x.dtype, device=dev)
    else:
        if not isinstance(y, torch.Tensor) or y.dtype != x.dtype or y.device != dev \
                or tuple(y.shape) != (B, C) or y.stride(1) != 1:
            raise ValueError("y must be a [B, C] device tensor of x's dtype with dense channels")
    ys = int(y.stride(0)) if B > 1 else C
    sh = gdn_conv_shape(B, conv_state.shape[0], C, W, _DT[x.dtype], 0 if xs == C else xs,
                        0 if ys == C else ys)
    _raise(_lib.gdn_conv_update(ctypes.byref(sh), _ptr(x), _ptr(w), _ptr(conv_state),
                                _ptr(slot_idx), _ptr(y), _ptr(err_flags), _stream(stream)),
           "gdn_conv_update")
    return y


def gdn_kda_gates(a, b, A, dt_bias, lower_bound: float, g=None, beta=None, stream=None):
    """Gate activations in front of a per-key-gate decode; see gdn_kda_gates in
    gdn_replay.h. a [B, T, Hv, dk], b [B, T, Hv], A [Hv], dt_bias [Hv, dk], all
    fp32. Returns (g [B, T, Hv, dk], beta [B, T, Hv])."""
    _check(a, "a", torch.float32, 4)
    dev = a.device
    B, T, Hv, dk = a.shape
    _check(b, "b", torch.float32, 3, dev)
    _check(A, "A", torch.float32, 1, dev)
    _check(dt_bias, "dt_bias", torch.float32, 2, dev)
    if tuple(b.shape) != (B, T, Hv) or tuple(A.shape) != (Hv,) or tuple(dt_bias.shape) != (Hv, dk):
        raise ValueError("inconsistent a / b / A / dt_bias shapes")
    g = torch.empty_like(a) if g is None else g
    beta = torch.empty_like(b) if beta is None else beta
    _check(g, "g", torch.float32, 4, dev)
    _check(beta, "beta", torch.float32, 3, dev)
    if g.shape != a.shape or beta.shape != b.shape:
        raise ValueError("g and beta must have the shapes of a and b")
    sh = gdn_gate_shape(B, T, Hv, dk, float(lower_bound))
    _raise(_lib.gdn_kda_gates(ctypes.byref(sh), _ptr(a), _ptr(b), _ptr(A), _ptr(dt_bias), _ptr(g),
                              _ptr(beta), _stream(stream)), "gdn_kda_gates")
    return g, beta


class Prepared:
    """A library call with its arguments checked and marshalled once, for
    loops that issue the same call many times (a decode step per layer).
    Calling it enqueues the kernels again on the stream it was prepared for;
    the tensors must stay alive and keep their shapes."""

    __slots__ = ("_fn", "_args", "_keep", "_name")

    def __init__(self, fn, args, keep, name):
        self._fn, self._args, self._keep, self._name = fn, args, keep, name

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != GDN_OK:
            raise GdnError(st, self._name)


def prepare_replay_decode(q, k, v, g, beta, slot_idx, ckpt, ring_d, ring_k, ring_g, write_pos,
                          force_flush=None, o=None, err_flags=None, window=False, stream=None,
                          qk_norm=False):
    """gdn_replay_decode with the same arguments, prepared for repeated calls.
    Returns (call, o)."""
    B, T, Hk, dk, Hv, dv, dev, gate, qs, vs = _io_shape(q, k, v, g, beta, slot_idx)
    N, L = _ring_shape(ckpt, ring_d, ring_k, ring_g, write_pos, Hv, Hk, dk, dv, dev, gate)
    _row_flags(force_flush, "force_flush", B, dev)
    _err_word(err_flags, dev)
    o = _out(o, B, T, Hv, dv, q.dtype, dev)
    sh = _shape(B, T, N, Hv, Hk, dk, dv, L, _DT[q.dtype], _DT[ring_d.dtype], window,
                _DT[ckpt.dtype], 0, gate, qs, vs, qk_norm)
    args = (ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(slot_idx),
            _ptr(ckpt), _ptr(ring_d), _ptr(ring_k), _ptr(ring_g), _ptr(write_pos),
            _ptr(force_flush), _ptr(o), _ptr(err_flags), _stream(stream))
    keep = (sh, q, k, v, g, beta, slot_idx, ckpt, ring_d, ring_k, ring_g, write_pos,
            force_flush, o, err_flags)
    return Prepared(_lib.gdn_replay_decode, args, keep, "gdn_replay_decode"), o


def prepare_packed_decode(q, k, v, g, beta, slot_idx, state, o=None, err_flags=None,
                          stream=None, qk_norm=False):
    """gdn_packed_decode prepared for repeated calls. Returns (call, o)."""
    B, T, Hk, dk, Hv, dv, dev, gate, qs, vs = _io_shape(q, k, v, g, beta, slot_idx)
    _state_of(state, Hv, dv, dk, dev)
    _err_word(err_flags, dev)
    o = _out(o, B, T, Hv, dv, q.dtype, dev)
    sh = _shape(B, T, state.shape[0], Hv, Hk, dk, dv, 1, _DT[q.dtype], GDN_F32, 0,
                _DT[state.dtype], 0, gate, qs, vs, qk_norm)
    args = (ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(slot_idx),
            _ptr(state), _ptr(o), _ptr(err_flags), _stream(stream))
    keep = (sh, q, k, v, g, beta, slot_idx, state, o, err_flags)
    return Prepared(_lib.gdn_packed_decode, args, keep, "gdn_packed_decode"), o
