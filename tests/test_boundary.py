"""The C-ABI library without a GPU: it loads, exports every entry point the
header declares, and rejects invalid arguments on the host before any HIP
call (no kernel is launched by these tests)."""
import ctypes

import pytest

import linear_attention_ssm_amd as gdn
from linear_attention_ssm_amd import gdn_shape

EXPECTED = ["gdn_abi_version", "gdn_conv_update", "gdn_hbm_copy_probe", "gdn_hbm_read_probe",
            "gdn_kda_gates",
            "gdn_packed_decode",
            "gdn_replay_advance", "gdn_replay_commit",
            "gdn_replay_decode", "gdn_replay_decode_advance",
            "gdn_replay_decode_advance_noalloc", "gdn_replay_fold", "gdn_replay_fold_layers",
            "gdn_replay_reset", "gdn_status_string"]

# Fake, 256-byte aligned, non-null device addresses: never dereferenced, since
# every call below must fail validation (or return early for B = 0) first.
FAKE = [ctypes.c_void_p(0x100000 + 0x1000 * i) for i in range(16)]


def shape(**kw):
    d = dict(B=2, T=1, N=4, Hv=4, Hk=2, dk=128, dv=128, L=16, qkv_dtype=gdn.GDN_BF16,
             ring_dtype=gdn.GDN_F16, window=0)
    d.update(kw)
    return gdn_shape(**d)


def test_header_declares_exactly_the_exported_symbols():
    assert gdn.declared_symbols() == EXPECTED
    lib = gdn.lib()
    for name in EXPECTED:
        assert hasattr(lib, name), name
    assert lib.gdn_abi_version() == 12
    for st in range(5):
        assert lib.gdn_status_string(st)
    assert lib.gdn_status_string(99) == b"unknown status"


def replay(sh, ptrs=None, ff=None):
    p = list(ptrs or FAKE[:12])
    # q k v g beta slot ckpt ring_d ring_k ring_g write_pos | force_flush o err stream
    return gdn.lib().gdn_replay_decode(ctypes.byref(sh), *p[:11], ff, p[11], None, None)


def packed(sh, ptrs=None):
    p = list(ptrs or FAKE[:8])
    return gdn.lib().gdn_packed_decode(ctypes.byref(sh), *p, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(L=0), gdn.GDN_ERR_INVALID_ARG),
    (dict(L=65), gdn.GDN_ERR_INVALID_ARG),
    (dict(Hv=3, Hk=2), gdn.GDN_ERR_INVALID_ARG),
    (dict(Hv=34, Hk=2), gdn.GDN_ERR_INVALID_ARG),       # G = 17 > 16
    (dict(dk=96), gdn.GDN_ERR_UNSUPPORTED),
    (dict(dv=40), gdn.GDN_ERR_UNSUPPORTED),
    (dict(qkv_dtype=gdn.GDN_F16), gdn.GDN_ERR_UNSUPPORTED),
    (dict(ring_dtype=7), gdn.GDN_ERR_UNSUPPORTED),
    (dict(state_dtype=3), gdn.GDN_ERR_UNSUPPORTED),
    (dict(step_rounding=1), gdn.GDN_ERR_INVALID_ARG),   # decode step: windows only
    (dict(T=2, window=1, step_rounding=2), gdn.GDN_ERR_INVALID_ARG),
    (dict(state_dtype=-1), gdn.GDN_ERR_UNSUPPORTED),
    (dict(gate=2), gdn.GDN_ERR_INVALID_ARG),
    (dict(qk_norm=2), gdn.GDN_ERR_INVALID_ARG),
    (dict(qk_row_stride=100), gdn.GDN_ERR_INVALID_ARG),     # < Hk * dk: rows overlap
    (dict(qk_row_stride=260), gdn.GDN_ERR_INVALID_ARG),     # rows not 16-byte aligned
    (dict(v_row_stride=200), gdn.GDN_ERR_INVALID_ARG),      # < Hv * dv
    (dict(gate=-1), gdn.GDN_ERR_INVALID_ARG),
    # per-key gate, 16-token windows at dk = 256, L = 64 with an fp32 ring: the
    # staged gates and weighted keys exceed LDS
    (dict(gate=1, T=16, window=1, dk=256, L=64, ring_dtype=gdn.GDN_F32), gdn.GDN_ERR_UNSUPPORTED),
    (dict(T=2), gdn.GDN_ERR_INVALID_ARG),               # decode mode needs T = 1
    (dict(T=2, window=1, L=1), gdn.GDN_ERR_INVALID_ARG),  # window longer than the ring
    (dict(window=2), gdn.GDN_ERR_INVALID_ARG),
    (dict(B=-1), gdn.GDN_ERR_INVALID_ARG),
    (dict(N=0), gdn.GDN_ERR_INVALID_ARG),
])
def test_replay_decode_rejects_bad_shapes(kw, status):
    assert replay(shape(**kw)) == status


def test_replay_decode_rejects_bad_pointers():
    assert gdn.lib().gdn_replay_decode(None, *FAKE[:11], None, FAKE[11], None, None) \
        == gdn.GDN_ERR_INVALID_ARG
    for i in range(12):
        p = list(FAKE[:12])
        p[i] = None
        assert replay(shape(), p) == gdn.GDN_ERR_INVALID_ARG, i
    p = list(FAKE[:12])
    p[6] = ctypes.c_void_p(FAKE[6].value + 4)            # checkpoint not 16-byte aligned
    assert replay(shape(), p) == gdn.GDN_ERR_INVALID_ARG
    p = list(FAKE[:12])
    p[0] = ctypes.c_void_p(FAKE[0].value + 2)            # q not 16-byte aligned
    assert replay(shape(), p) == gdn.GDN_ERR_INVALID_ARG
    # force_flush is not allowed with a verify window
    assert replay(shape(T=2, window=1), ff=FAKE[13]) == gdn.GDN_ERR_INVALID_ARG
    # a per-key gate reads g and ring_g in 16-byte pieces
    for i in (3, 9):
        p = list(FAKE[:12])
        p[i] = ctypes.c_void_p(FAKE[i].value + 4)
        assert replay(shape(gate=gdn.GDN_GATE_KEY), p) == gdn.GDN_ERR_INVALID_ARG, i
    p = list(FAKE[:8])
    p[3] = ctypes.c_void_p(FAKE[3].value + 4)
    assert packed(shape(gate=gdn.GDN_GATE_KEY), p) == gdn.GDN_ERR_INVALID_ARG


def test_decode_advance_validates():
    lib = gdn.lib()

    def call(sh, arrive):
        p = list(FAKE[:12])
        return lib.gdn_replay_decode_advance(ctypes.byref(sh), *p[:11], None, p[11], arrive,
                                             None, None)
    assert call(shape(), None) == gdn.GDN_ERR_INVALID_ARG               # no workspace
    assert call(shape(), ctypes.c_void_p(FAKE[14].value + 64)) == gdn.GDN_ERR_INVALID_ARG
    assert call(shape(T=2, window=1), FAKE[14]) == gdn.GDN_ERR_INVALID_ARG   # windows: no
    assert call(shape(dk=96), FAKE[14]) == gdn.GDN_ERR_UNSUPPORTED
    assert call(shape(B=0), FAKE[14]) == gdn.GDN_OK


def test_read_probe_validates():
    lib = gdn.lib()
    probe = lambda src, n, sink: lib.gdn_hbm_read_probe(src, ctypes.c_size_t(n), sink, None)
    assert probe(None, 32768, FAKE[1]) == gdn.GDN_ERR_INVALID_ARG
    assert probe(FAKE[0], 32768, None) == gdn.GDN_ERR_INVALID_ARG
    assert probe(FAKE[0], 0, FAKE[1]) == gdn.GDN_ERR_INVALID_ARG
    assert probe(FAKE[0], 32768 + 16, FAKE[1]) == gdn.GDN_ERR_INVALID_ARG
    assert probe(ctypes.c_void_p(FAKE[0].value + 4), 32768, FAKE[1]) == gdn.GDN_ERR_INVALID_ARG


def test_copy_probe_validates():
    """Null pointers, sizes that are not a positive multiple of 32 KiB,
    misaligned buffers and buffers that overlap without being the same are
    rejected before any launch."""
    lib = gdn.lib()
    probe = lambda src, dst, n: lib.gdn_hbm_copy_probe(src, dst, ctypes.c_size_t(n), None)
    a, b = FAKE[0].value, 0x40000000
    P = ctypes.c_void_p
    assert probe(None, P(b), 32768) == gdn.GDN_ERR_INVALID_ARG
    assert probe(P(a), None, 32768) == gdn.GDN_ERR_INVALID_ARG
    assert probe(P(a), P(b), 0) == gdn.GDN_ERR_INVALID_ARG
    assert probe(P(a), P(b), 32768 + 16) == gdn.GDN_ERR_INVALID_ARG
    assert probe(P(a + 4), P(b), 32768) == gdn.GDN_ERR_INVALID_ARG
    assert probe(P(a), P(b + 8), 32768) == gdn.GDN_ERR_INVALID_ARG
    # overlapping, not the same: dst starts inside src, or src inside dst
    assert probe(P(a), P(a + 16384), 32768) == gdn.GDN_ERR_INVALID_ARG
    assert probe(P(a + 16384), P(a), 32768) == gdn.GDN_ERR_INVALID_ARG


def test_fold_layers_validates():
    """The multi-layer fold checks its layer count, every layer's pointers and
    alignment, and that no two checkpoints overlap, before any launch; with
    valid arguments and B = 0 it returns at once."""
    lib = gdn.lib()
    P = ctypes.c_void_p
    mib = 1 << 20            # one checkpoint of shape(): 4 x 4 x 128 x 128 fp32
    base = 0x10000000

    def arr(xs):
        return (P * len(xs))(*[P(x) if x is not None else None for x in xs])

    def call(n, ck, rd=None, rk=None, rg=None, B=2):
        rd = rd if rd is not None else [0x40000000 + 0x10000 * i for i in range(len(ck))]
        rk = rk if rk is not None else [0x50000000 + 0x10000 * i for i in range(len(ck))]
        rg = rg if rg is not None else [0x60000000 + 0x10000 * i for i in range(len(ck))]
        sh = shape(B=B)
        return lib.gdn_replay_fold_layers(ctypes.byref(sh), n, FAKE[0], arr(ck), arr(rd), arr(rk),
                                          arr(rg), FAKE[1], None, None)
    ok = [base + i * mib for i in range(3)]
    assert call(3, ok, B=0) == gdn.GDN_OK
    assert call(0, ok) == gdn.GDN_ERR_INVALID_ARG
    assert call(1025, ok) == gdn.GDN_ERR_INVALID_ARG
    sh = shape()
    assert lib.gdn_replay_fold_layers(ctypes.byref(sh), 1, FAKE[0], None, arr(ok), arr(ok),
                                      arr(ok), FAKE[1], None, None) == gdn.GDN_ERR_INVALID_ARG
    assert call(3, [ok[0], None, ok[2]]) == gdn.GDN_ERR_INVALID_ARG
    assert call(3, [ok[0], ok[1] + 8, ok[2]]) == gdn.GDN_ERR_INVALID_ARG          # misaligned
    assert call(2, ok[:2], rk=[0x50000000, 0x50000004]) == gdn.GDN_ERR_INVALID_ARG
    assert call(3, [ok[0], ok[1], ok[0]]) == gdn.GDN_ERR_INVALID_ARG              # same twice
    assert call(2, [ok[1], ok[0] + mib // 2]) == gdn.GDN_ERR_INVALID_ARG         # overlapping
    # shared rings are allowed (they are only read)
    assert call(2, ok[:2], rd=[0x40000000] * 2, rk=[0x50000000] * 2, rg=[0x60000000] * 2,
                B=0) == gdn.GDN_OK


def test_decode_advance_noalloc_validates():
    """The no-allocation variant rejects more rows than its static scratch
    holds with its own status, and otherwise validates like the workspace
    variant (all before any HIP call)."""
    lib = gdn.lib()

    def call(sh):
        p = list(FAKE[:12])
        return lib.gdn_replay_decode_advance_noalloc(ctypes.byref(sh), *p[:11], None, p[11],
                                                     None, None)
    assert call(shape(B=gdn.SCRATCH_MAX_ROWS + 1, N=8192)) == gdn.GDN_ERR_SCRATCH_LIMIT
    assert call(shape(T=2, window=1)) == gdn.GDN_ERR_INVALID_ARG     # windows: no
    assert call(shape(dk=96)) == gdn.GDN_ERR_UNSUPPORTED
    p = list(FAKE[:12])
    p[0] = ctypes.c_void_p(FAKE[0].value + 4)                        # misaligned q
    assert lib.gdn_replay_decode_advance_noalloc(ctypes.byref(shape()), *p[:11], None, p[11],
                                                 None, None) == gdn.GDN_ERR_INVALID_ARG
    assert call(shape(B=0)) == gdn.GDN_OK
    assert lib.gdn_status_string(gdn.GDN_ERR_SCRATCH_LIMIT).startswith(b"more rows")


def test_empty_batch_is_a_no_op():
    assert replay(shape(B=0)) == gdn.GDN_OK
    assert packed(shape(B=0)) == gdn.GDN_OK
    lib = gdn.lib()
    sh = shape(B=0)
    assert lib.gdn_replay_fold(ctypes.byref(sh), *FAKE[:6], None, None) == gdn.GDN_OK
    assert lib.gdn_replay_advance(ctypes.byref(sh), FAKE[0], FAKE[1], None, None, None) == gdn.GDN_OK
    assert lib.gdn_replay_commit(ctypes.byref(sh), FAKE[0], FAKE[1], FAKE[2], None, None) == gdn.GDN_OK
    assert lib.gdn_replay_reset(ctypes.byref(sh), FAKE[0], FAKE[1], None, None) == gdn.GDN_OK


def test_packed_and_cursor_entry_points_validate():
    assert packed(shape(T=2)) == gdn.GDN_ERR_INVALID_ARG
    assert packed(shape(dk=48)) == gdn.GDN_ERR_UNSUPPORTED
    assert packed(shape(state_dtype=5)) == gdn.GDN_ERR_UNSUPPORTED
    assert packed(shape(gate=3)) == gdn.GDN_ERR_INVALID_ARG
    assert gdn.lib().gdn_replay_fold(ctypes.byref(shape(gate=3)), *FAKE[:6], None, None) \
        == gdn.GDN_ERR_INVALID_ARG
    p = list(FAKE[:6])
    p[4] = ctypes.c_void_p(FAKE[4].value + 4)            # per-key ring_g misaligned
    assert gdn.lib().gdn_replay_fold(ctypes.byref(shape(gate=1)), *p, None, None) \
        == gdn.GDN_ERR_INVALID_ARG
    assert gdn.lib().gdn_replay_fold(ctypes.byref(shape(state_dtype=5)), *FAKE[:6], None, None) \
        == gdn.GDN_ERR_UNSUPPORTED
    p = list(FAKE[:8])
    p[6] = None
    assert packed(shape(), p) == gdn.GDN_ERR_INVALID_ARG
    lib = gdn.lib()
    sh = shape(L=0)
    assert lib.gdn_replay_advance(ctypes.byref(sh), FAKE[0], FAKE[1], None, None, None) \
        == gdn.GDN_ERR_INVALID_ARG
    assert lib.gdn_replay_advance(ctypes.byref(shape()), None, FAKE[1], None, None, None) \
        == gdn.GDN_ERR_INVALID_ARG
    assert lib.gdn_replay_commit(ctypes.byref(shape(T=0)), FAKE[0], FAKE[1], FAKE[2], None, None) \
        == gdn.GDN_ERR_INVALID_ARG
    assert lib.gdn_replay_commit(ctypes.byref(shape()), FAKE[0], None, FAKE[2], None, None) \
        == gdn.GDN_ERR_INVALID_ARG
    assert lib.gdn_replay_fold(ctypes.byref(shape(dv=8)), *FAKE[:6], None, None) \
        == gdn.GDN_ERR_UNSUPPORTED
    p = list(FAKE[:6])
    p[1] = ctypes.c_void_p(FAKE[1].value + 8)            # checkpoint misaligned
    assert lib.gdn_replay_fold(ctypes.byref(shape()), *p, None, None) == gdn.GDN_ERR_INVALID_ARG
    assert lib.gdn_replay_reset(ctypes.byref(shape()), None, FAKE[1], None, None) \
        == gdn.GDN_ERR_INVALID_ARG
    assert lib.gdn_replay_reset(ctypes.byref(shape(N=0)), FAKE[0], FAKE[1], None, None) \
        == gdn.GDN_ERR_INVALID_ARG


def test_python_binding_checks_tensors_before_calling():
    import torch
    q = torch.zeros(2, 1, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        gdn.gdn_packed_decode(q, q, q, torch.zeros(2, 1, 4), torch.zeros(2, 1, 4),
                              torch.zeros(2, dtype=torch.int32), torch.zeros(4, 4, 128, 128))


def test_binding_reads_row_strides_off_views():
    """q, k, v as views into a packed [B, T, 2*Hk*dk + Hv*dv] row: the
    binding derives the row strides the C ABI takes (0 for dense tensors)."""
    import torch
    from linear_attention_ssm_amd import _row_stride, _shape
    B, T, Hk, dk, Hv, dv = 3, 2, 2, 32, 4, 16
    rw = 2 * Hk * dk + Hv * dv
    m = torch.zeros(B, T, rw)
    q = m[..., :Hk * dk].view(B, T, Hk, dk)
    v = m[..., 2 * Hk * dk:].view(B, T, Hv, dv)
    assert _row_stride(q, "q") == rw and _row_stride(v, "v") == rw
    dense = torch.zeros(B, T, Hk, dk)
    assert _row_stride(dense, "q") == Hk * dk
    one = torch.zeros(B, 1, rw)[..., :Hk * dk].view(B, 1, Hk, dk)     # T = 1: stride of b
    assert _row_stride(one, "q") == rw
    sh = _shape(B, T, 8, Hv, Hk, dk, dv, 4, 1, 2, 0, 0, 0, 0, rw, Hv * dv, 1)
    assert (sh.qk_row_stride, sh.v_row_stride, sh.qk_norm) == (rw, 0, 1)
    with pytest.raises(ValueError):
        _row_stride(torch.zeros(B, T, dk, Hk).transpose(2, 3), "q")     # [H, d] not dense
    with pytest.raises(ValueError):
        _row_stride(torch.zeros(T, B, Hk, dk).transpose(0, 1), "q")     # rows not in (b, t) order


def test_conv_update_validates():
    """gdn_conv_update's host checks (sizes, dtype, strides, alignment,
    overlap), all before any launch."""
    lib = gdn.lib()

    def call(p=None, **kw):
        d = dict(B=2, N=3, C=64, W=4, dtype=gdn.GDN_BF16, x_row_stride=0, y_row_stride=0)
        d.update(kw)
        sh = gdn.gdn_conv_shape(**d)
        p = list(FAKE[:5]) if p is None else p
        return lib.gdn_conv_update(ctypes.byref(sh), *p, None, None)
    assert call(C=62) == gdn.GDN_ERR_UNSUPPORTED                 # not a multiple of 4
    assert call(C=0) == gdn.GDN_ERR_UNSUPPORTED
    assert call(W=1) == gdn.GDN_ERR_UNSUPPORTED
    assert call(W=5) == gdn.GDN_ERR_UNSUPPORTED
    assert call(dtype=gdn.GDN_F16) == gdn.GDN_ERR_UNSUPPORTED
    assert call(B=-1) == gdn.GDN_ERR_INVALID_ARG
    assert call(N=0) == gdn.GDN_ERR_INVALID_ARG
    assert call(x_row_stride=60) == gdn.GDN_ERR_INVALID_ARG     # rows overlap
    assert call(y_row_stride=66) == gdn.GDN_ERR_INVALID_ARG     # rows not 8-byte aligned
    assert call(dtype=gdn.GDN_F32, x_row_stride=70) == gdn.GDN_ERR_INVALID_ARG
    assert call(B=0) == gdn.GDN_OK
    for i in range(5):
        p = list(FAKE[:5])
        p[i] = None
        assert call(p) == gdn.GDN_ERR_INVALID_ARG, i
    p = list(FAKE[:5])
    p[0] = ctypes.c_void_p(FAKE[0].value + 4)                   # x not 8-byte aligned
    assert call(p) == gdn.GDN_ERR_INVALID_ARG
    p = list(FAKE[:5])
    p[4] = ctypes.c_void_p(FAKE[0].value + 64)                  # y overlaps x
    assert call(p) == gdn.GDN_ERR_INVALID_ARG
    p = list(FAKE[:5])
    p[4] = FAKE[2]                                              # y is the state
    assert call(p) == gdn.GDN_ERR_INVALID_ARG
    p = list(FAKE[:5])
    p[0] = ctypes.c_void_p(FAKE[2].value + 256)                 # x inside the state
    assert call(p) == gdn.GDN_ERR_INVALID_ARG


def test_kda_gates_validates():
    lib = gdn.lib()

    def call(p=None, **kw):
        d = dict(B=2, T=1, Hv=4, dk=128, lower_bound=-5.0)
        d.update(kw)
        sh = gdn.gdn_gate_shape(**d)
        p = list(FAKE[:6]) if p is None else p
        return lib.gdn_kda_gates(ctypes.byref(sh), *p, None)
    assert call(dk=6) == gdn.GDN_ERR_UNSUPPORTED
    assert call(dk=2048) == gdn.GDN_ERR_UNSUPPORTED
    assert call(lower_bound=0.0) == gdn.GDN_ERR_INVALID_ARG
    assert call(lower_bound=float("nan")) == gdn.GDN_ERR_INVALID_ARG
    assert call(T=0) == gdn.GDN_ERR_INVALID_ARG
    assert call(B=0) == gdn.GDN_OK
    for i in range(6):
        p = list(FAKE[:6])
        p[i] = None
        assert call(p) == gdn.GDN_ERR_INVALID_ARG, i
    p = list(FAKE[:6])
    p[0] = ctypes.c_void_p(FAKE[0].value + 8)           # a not 16-byte aligned
    assert call(p) == gdn.GDN_ERR_INVALID_ARG
