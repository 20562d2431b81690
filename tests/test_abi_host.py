"""The C-ABI library on the host (no GPU needed): it loads, exports every
symbol include/moe.h declares, and rejects every invalid request with the
documented status code before making any HIP call."""

import ctypes
import os
import re

import pytest

import quantized_routed_moe_amd as qm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

A16 = 0x10000          # fake, 16-byte aligned "device" addresses (never dereferenced)


def _declared_symbols():
    syms = set()
    for name in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if name.endswith(".h"):
            text = open(os.path.join(ROOT, "include", name)).read()
            syms |= set(re.findall(r"^(?:size_t|int|double|const char\s*\*)\s+(moe_\w+)\s*\(", text, re.M))
    return sorted(syms)


def test_library_exports_every_declared_symbol():
    syms = _declared_symbols()
    assert len(syms) >= 24
    assert sorted(qm.EXPORTS) == syms
    L = ctypes.CDLL(qm.LIB_PATH)
    for s in syms:
        assert hasattr(L, s), s


def test_status_strings():
    codes = [qm.MOE_OK, qm.MOE_ERR_NULL, qm.MOE_ERR_SHAPE, qm.MOE_ERR_FORMAT, qm.MOE_ERR_ALIGN,
             qm.MOE_ERR_WORKSPACE, qm.MOE_ERR_UNSUPPORTED, qm.MOE_ERR_HIP, qm.MOE_ERR_DEVICE]
    names = [qm.status_str(c) for c in codes]
    assert len(set(names)) == len(codes)
    for c, n in zip(codes, names):
        assert n.startswith("MOE_")
    assert "unknown" in qm.status_str(-99)


def _shape(T=4, d=256, E=8, k=2, f=128):
    return qm.moe_shape(T, d, E, k, f)


@pytest.mark.parametrize("bad", [
    dict(k=0), dict(k=9), dict(E=65, k=2), dict(E=0), dict(d=48), dict(f=100), dict(d=0),
    dict(T=-1), dict(T=1 << 20, d=4096, k=8),
])
def test_shape_validation(bad):
    s = _shape(**bad)
    assert qm.lib().moe_workspace_bytes(ctypes.byref(s)) == 0
    assert qm.lib().moe_layer_workspace_bytes(ctypes.byref(s)) == 0
    rc = qm.lib().moe_combine(ctypes.byref(s), A16, A16, A16, A16, None)
    assert rc == qm.MOE_ERR_SHAPE


def test_workspace_sizes():
    s = _shape(T=5, d=4096, E=64, k=2, f=2048)
    al = lambda v: (v + 255) // 256 * 256
    # 256-byte header + bf16 act[T*k][f] + 8-byte ready flags, one per
    # (m-tile, 256 rows of f) for ceil(T*k / 128) + min(E, T*k) m-tiles,
    # each part rounded up to 256
    mtiles = -(-10 // 128) + min(64, 10)
    ffn = 256 + al(5 * 2 * 2048 * 2) + al(mtiles * (2048 // 256) * 8)
    assert qm.lib().moe_workspace_bytes(ctypes.byref(s)) == ffn
    lw = qm.lib().moe_layer_workspace_bytes(ctypes.byref(s))
    assert lw == ffn + al(65 * 4) + 2 * al(10 * 4) + al(10 * 4096 * 4)
    # no flags when f is not a multiple of 256 (no single-launch grouped FFN)
    s2 = _shape(T=5, d=4096, E=64, k=2, f=224)
    assert qm.lib().moe_workspace_bytes(ctypes.byref(s2)) == 256 + al(5 * 2 * 224 * 2)


def test_null_shape_and_zero_tokens():
    assert qm.lib().moe_combine(None, A16, A16, A16, A16, None) == qm.MOE_ERR_NULL
    # T == 0 is valid and enqueues nothing, whatever the pointers
    s = _shape(T=0)
    assert qm.lib().moe_combine(ctypes.byref(s), None, None, None, None, None) == qm.MOE_OK
    assert qm.lib().moe_layer(ctypes.byref(s), *([None] * 9), 0, None) == qm.MOE_OK


TILES, ROWS = qm.MOE_LAYOUT_TILES, qm.MOE_LAYOUT_ROWS


def _experts(fmt=qm.MOE_FMT_MXFP4, mins=None, slots=8, soe=None, layout=TILES, **over):
    q = lambda: qm.moe_qmat(fmt, layout, A16, A16, mins)
    e = qm.moe_experts(q(), q(), q(), soe, slots)
    for k, v in over.items():
        setattr(e, k, v)
    return e


def _ffn(s, ex, x=A16, offsets=A16, perm=A16, y=A16, ws=A16, ws_bytes=1 << 30):
    return qm.lib().moe_expert_ffn(ctypes.byref(s), x, ctypes.byref(ex) if ex is not None else None,
                                   offsets, perm, y, ws, ws_bytes, None)


def test_ffn_validation():
    s = _shape()
    assert _ffn(s, None) == qm.MOE_ERR_NULL
    assert _ffn(s, _experts(), x=None) == qm.MOE_ERR_NULL
    assert _ffn(s, _experts(), y=None) == qm.MOE_ERR_NULL
    assert _ffn(s, _experts(fmt=7)) == qm.MOE_ERR_FORMAT
    mixed = _experts()
    mixed.down = qm.moe_qmat(qm.MOE_FMT_Q2G32, TILES, A16, A16, None)
    assert _ffn(s, mixed) == qm.MOE_ERR_FORMAT
    # the kernels read the tile layout only; its Q2 mins live in scales
    assert _ffn(s, _experts(layout=ROWS)) == qm.MOE_ERR_FORMAT
    assert _ffn(s, _experts(fmt=qm.MOE_FMT_Q2G32, mins=A16)) == qm.MOE_ERR_FORMAT
    assert _ffn(s, _experts(fmt=qm.MOE_FMT_Q2G32, mins=None), ws=None) == qm.MOE_ERR_NULL
    assert _ffn(s, _experts(slots=7)) == qm.MOE_ERR_SHAPE            # identity map needs E slots
    assert _ffn(s, _experts(slots=0, soe=A16)) == qm.MOE_ERR_SHAPE
    assert _ffn(s, _experts(), x=A16 + 8) == qm.MOE_ERR_ALIGN
    assert _ffn(s, _experts(), y=A16 + 4) == qm.MOE_ERR_ALIGN
    bad = _experts()
    bad.up = qm.moe_qmat(qm.MOE_FMT_MXFP4, TILES, A16 + 2, A16, None)
    assert _ffn(s, bad) == qm.MOE_ERR_ALIGN
    bad.up = qm.moe_qmat(qm.MOE_FMT_MXFP4, TILES, A16, A16 + 8, None)
    assert _ffn(s, bad) == qm.MOE_ERR_ALIGN
    assert _ffn(s, _experts(soe=A16 + 2, slots=4)) == qm.MOE_ERR_ALIGN
    need = qm.lib().moe_workspace_bytes(ctypes.byref(s))
    assert _ffn(s, _experts(), ws_bytes=need - 1) == qm.MOE_ERR_WORKSPACE
    assert _ffn(s, _experts(), ws=None) == qm.MOE_ERR_NULL


def test_route_dispatch_combine_validation():
    s = _shape()
    L = qm.lib()
    # given logits (no router) cannot take a bias
    assert L.moe_route_topk(ctypes.byref(s), A16, None, A16, A16, A16, A16, None) == qm.MOE_ERR_UNSUPPORTED
    assert L.moe_route_topk(ctypes.byref(s), None, A16, None, A16, A16, A16, None) == qm.MOE_ERR_NULL
    assert L.moe_route_topk(ctypes.byref(s), A16, A16, None, None, A16, A16, None) == qm.MOE_ERR_NULL
    assert L.moe_route_topk(ctypes.byref(s), A16 + 2, A16, None, A16, A16, A16, None) == qm.MOE_ERR_ALIGN
    assert L.moe_route_topk(ctypes.byref(s), A16, A16, None, A16, A16 + 2, A16, None) == qm.MOE_ERR_ALIGN
    assert L.moe_dispatch(ctypes.byref(s), None, A16, A16, A16, A16, 1 << 20, None) == qm.MOE_ERR_NULL
    assert L.moe_dispatch(ctypes.byref(s), A16, A16, A16 + 1, A16, A16, 1 << 20, None) == qm.MOE_ERR_ALIGN
    assert L.moe_dispatch(ctypes.byref(s), A16, A16, A16, A16, A16, 100, None) == qm.MOE_ERR_WORKSPACE
    assert L.moe_combine(ctypes.byref(s), A16, A16, None, A16, None) == qm.MOE_ERR_NULL
    assert L.moe_combine(ctypes.byref(s), A16, A16, A16, A16 + 4, None) == qm.MOE_ERR_ALIGN
    assert L.moe_workspace_init(None, 256, None) == qm.MOE_ERR_NULL
    assert L.moe_workspace_init(A16, 100, None) == qm.MOE_ERR_WORKSPACE
    assert L.moe_read_device_status(None, None) == qm.MOE_ERR_NULL
    assert L.moe_read_device_status_bits(None, None, None) == qm.MOE_ERR_NULL
    assert L.moe_read_device_status(A16 + 8, None) == qm.MOE_ERR_ALIGN


def test_layer_validation():
    s = _shape()
    L = qm.lib()
    ex = _experts()
    need = L.moe_layer_workspace_bytes(ctypes.byref(s))
    args = lambda **o: [ctypes.byref(s), o.get("x", A16), o.get("wr", A16), o.get("bias", None),
                        o.get("logits", A16), ctypes.byref(o.get("ex", ex)), o.get("ids", A16),
                        o.get("w", A16), o.get("out", A16), o.get("ws", A16), o.get("wsb", need), None]
    assert L.moe_layer(*args(ws=None)) == qm.MOE_ERR_NULL
    assert L.moe_layer(*args(out=None)) == qm.MOE_ERR_NULL
    assert L.moe_layer(*args(wsb=need - 1)) == qm.MOE_ERR_WORKSPACE
    assert L.moe_layer(*args(x=None)) == qm.MOE_ERR_NULL
    assert L.moe_layer(*args(ex=_experts(fmt=7))) == qm.MOE_ERR_FORMAT
    assert L.moe_layer(*args(wr=None, bias=A16)) == qm.MOE_ERR_UNSUPPORTED


def _qbytes(fmt, layout, slots, n, K):
    c, sc, m = ctypes.c_size_t(7), ctypes.c_size_t(7), ctypes.c_size_t(7)
    tot = qm.lib().moe_qmat_bytes(fmt, layout, slots, n, K, ctypes.byref(c), ctypes.byref(sc), ctypes.byref(m))
    return tot, c.value, sc.value, m.value


def test_qmat_bytes():
    MX, Q2 = qm.MOE_FMT_MXFP4, qm.MOE_FMT_Q2G32
    # row layout: the packed data itself
    assert _qbytes(MX, ROWS, 64, 2048, 4096) == (64 * 2048 * (2048 + 128),) + (64 * 2048 * 2048, 64 * 2048 * 128, 0)
    assert _qbytes(Q2, ROWS, 3, 16, 96)[1:] == (3 * 16 * 24, 3 * 16 * 3 * 2, 3 * 16 * 3 * 2)
    # tile layout: (slots * n/16 * ceil(K/128)) blocks of 64 pieces; no padding when 128 | K
    assert _qbytes(MX, TILES, 64, 2048, 4096)[1:] == (64 * 2048 * 2048, 64 * 2048 * 128, 0)
    assert _qbytes(MX, TILES, 2, 32, 160)[1:] == (2 * 2 * 2 * 64 * 16, 2 * 2 * 2 * 64, 0)
    assert _qbytes(Q2, TILES, 3, 16, 96)[1:] == (3 * 1 * 1 * 64 * 8, 3 * 1 * 1 * 64 * 4, 0)
    Q4 = qm.MOE_FMT_Q4G32
    assert _qbytes(Q4, ROWS, 3, 16, 96)[1:] == (3 * 16 * 48, 3 * 16 * 3 * 2, 3 * 16 * 3 * 2)
    assert _qbytes(Q4, TILES, 3, 16, 96)[1:] == (3 * 1 * 1 * 64 * 16, 3 * 1 * 1 * 64 * 4, 0)
    assert _qbytes(Q4, TILES, 64, 2048, 4096)[1:] == (64 * 2048 * 2048, 64 * 2048 * 128 * 4, 0)
    for bad in [(5, TILES, 1, 16, 32), (MX, 2, 1, 16, 32), (MX, TILES, 0, 16, 32), (MX, TILES, 1, 24, 32),
                (MX, TILES, 1, 16, 48), (MX, ROWS, 1, 0, 32), (Q2, TILES, 1, 16, 0)]:
        assert _qbytes(*bad) == (0, 0, 0, 0), bad


def test_pack_validation():
    L = qm.lib()
    MX, Q2 = qm.MOE_FMT_MXFP4, qm.MOE_FMT_Q2G32
    pk = lambda src, dst, n=32, K=128, slots=2: L.moe_pack_qmat(
        None if src is None else ctypes.byref(src), None if dst is None else ctypes.byref(dst), slots, n, K, None)
    rows = lambda fmt=MX, c=A16, sc=A16, mn=None: qm.moe_qmat(fmt, ROWS, c, sc, mn)
    tiles = lambda fmt=MX, c=A16, sc=A16, mn=None: qm.moe_qmat(fmt, TILES, c, sc, mn)
    assert pk(None, tiles()) == qm.MOE_ERR_NULL
    assert pk(rows(), None) == qm.MOE_ERR_NULL
    assert pk(tiles(), tiles()) == qm.MOE_ERR_FORMAT            # source must be the row layout
    assert pk(rows(), rows()) == qm.MOE_ERR_FORMAT              # destination must be the tile layout
    assert pk(rows(MX), tiles(Q2)) == qm.MOE_ERR_FORMAT         # same format on both sides
    assert pk(rows(9), tiles(9)) == qm.MOE_ERR_FORMAT
    assert pk(rows(), tiles(), n=24) == qm.MOE_ERR_SHAPE
    assert pk(rows(), tiles(), K=48) == qm.MOE_ERR_SHAPE
    assert pk(rows(), tiles(), slots=0) == qm.MOE_ERR_SHAPE
    assert pk(rows(Q2), tiles(Q2)) == qm.MOE_ERR_NULL           # Q2 rows need mins
    assert pk(rows(MX, mn=A16), tiles()) == qm.MOE_ERR_FORMAT
    assert pk(rows(Q2, mn=A16), tiles(Q2, mn=A16)) == qm.MOE_ERR_FORMAT
    assert pk(rows(c=A16 + 4), tiles()) == qm.MOE_ERR_ALIGN
    assert pk(rows(), tiles(sc=A16 + 2)) == qm.MOE_ERR_ALIGN
    assert pk(rows(Q2, mn=A16 + 2), tiles(Q2)) == qm.MOE_ERR_ALIGN
    Q4 = qm.MOE_FMT_Q4G32
    assert pk(rows(Q4), tiles(Q4)) == qm.MOE_ERR_NULL           # Q4 rows need mins
    assert pk(rows(Q4, mn=A16), tiles(Q2)) == qm.MOE_ERR_FORMAT
    assert pk(rows(Q4, mn=A16), tiles(Q4, mn=A16)) == qm.MOE_ERR_FORMAT
    assert pk(rows(Q4, mn=A16 + 2), tiles(Q4)) == qm.MOE_ERR_ALIGN


def test_layer_shared_validation():
    """moe_layer_shared rejects bad shared packs and workspaces on the host."""
    L = qm.lib()
    s = _shape(T=4, d=256, E=8, k=2, f=128)
    need = L.moe_layer_shared_workspace_bytes(ctypes.byref(s))
    assert need > L.moe_layer_workspace_bytes(ctypes.byref(s))        # T more rows of act, perm and y
    assert L.moe_layer_shared_workspace_bytes(ctypes.byref(_shape(k=0))) == 0

    def mat(fmt=qm.MOE_FMT_MXFP4, layout=qm.MOE_LAYOUT_TILES, mins=None):
        return qm.moe_qmat(fmt, layout, A16, A16, mins)

    ex = qm.moe_experts(mat(), mat(), mat(), None, 8)

    def call(shared, ws_bytes=need, ws=A16):
        return L.moe_layer_shared(ctypes.byref(s), A16, A16, None, A16, ctypes.byref(ex),
                                  None if shared is None else ctypes.byref(shared), A16, A16, A16, ws, ws_bytes,
                                  None)

    assert call(None) == qm.MOE_ERR_NULL
    assert call(qm.moe_experts(mat(qm.MOE_FMT_Q2G32), mat(), mat(), None, 1)) == qm.MOE_ERR_FORMAT
    assert call(qm.moe_experts(mat(), mat(layout=qm.MOE_LAYOUT_ROWS), mat(), None, 1)) == qm.MOE_ERR_FORMAT
    assert call(qm.moe_experts(mat(), mat(), mat(), None, 0)) == qm.MOE_ERR_SHAPE
    assert call(qm.moe_experts(mat(), mat(), mat(), None, 1), ws_bytes=need - 256) == qm.MOE_ERR_WORKSPACE
    assert call(qm.moe_experts(mat(), mat(), mat(), None, 1), ws=A16 + 8) == qm.MOE_ERR_ALIGN


@pytest.mark.parametrize("bits", [8, 4])
def test_mx_validation(bits):
    """The MXFP8- and MXFP4-activation entry points reject what they cannot
    run before any HIP call: other formats or shapes the grouped FFN does
    not take, short workspaces, invalid shapes."""
    L = qm.lib()
    ws_fn = getattr(L, f"moe_workspace_bytes_mx{bits}")
    s = _shape(T=64, d=512, E=8, k=2, f=256)
    need = ws_fn(ctypes.byref(s))
    R = 64 * 2
    assert need >= 256 + R * (256 + 512) * bits // 8             # header, act and token codes at least
    assert getattr(L, f"moe_layer_mx{bits}_workspace_bytes")(ctypes.byref(s)) > need
    assert ws_fn(ctypes.byref(_shape(k=0))) == 0
    if bits == 4:                                               # half the code bytes of MXFP8
        assert need < L.moe_workspace_bytes_mx8(ctypes.byref(s))

    def mat(fmt=qm.MOE_FMT_MXFP4):
        return qm.moe_qmat(fmt, qm.MOE_LAYOUT_TILES, A16, A16, None)

    def ffn(shape, fmt=qm.MOE_FMT_MXFP4, ws_bytes=need):
        ex = qm.moe_experts(mat(fmt), mat(fmt), mat(fmt), None, 8)
        return getattr(L, f"moe_expert_ffn_mx{bits}")(ctypes.byref(shape), A16, ctypes.byref(ex), A16, A16, A16,
                                                        A16, ws_bytes, None)

    assert ffn(s, qm.MOE_FMT_Q2G32) == qm.MOE_ERR_UNSUPPORTED
    assert ffn(s, qm.MOE_FMT_Q4G32) == qm.MOE_ERR_UNSUPPORTED
    s2 = _shape(T=64, d=256, E=8, k=2, f=256)                    # d not a multiple of 512
    assert ffn(s2, ws_bytes=ws_fn(ctypes.byref(s2))) == qm.MOE_ERR_UNSUPPORTED
    assert ffn(s, ws_bytes=need - 256) == qm.MOE_ERR_WORKSPACE
    assert ffn(_shape(T=64, d=512, E=8, k=9, f=256)) == qm.MOE_ERR_SHAPE
    assert ffn(_shape(T=0, d=512, E=8, k=2, f=256)) == qm.MOE_OK


def test_peak_kernels_validation():
    """The roofline measurement kernels (include/moe_peak.h) reject invalid
    requests before any HIP call."""
    L = qm.lib()
    assert L.moe_peak_stream(None, 1024, 0, A16, None) == qm.MOE_ERR_NULL
    assert L.moe_peak_stream(A16, 1024, 0, None, None) == qm.MOE_ERR_NULL
    assert L.moe_peak_stream(A16, 0, 0, A16, None) == qm.MOE_ERR_SHAPE
    assert L.moe_peak_stream(A16, 1000, 0, A16, None) == qm.MOE_ERR_SHAPE
    assert L.moe_peak_stream(A16, 1024, -1, A16, None) == qm.MOE_ERR_SHAPE
    assert L.moe_peak_stream(A16 + 8, 1024, 0, A16, None) == qm.MOE_ERR_ALIGN
    assert L.moe_peak_mfma(0, 10, 0, None, None) == qm.MOE_ERR_NULL
    assert L.moe_peak_mfma(3, 10, 0, A16, None) == qm.MOE_ERR_SHAPE
    assert L.moe_peak_mfma(0, 0, 0, A16, None) == qm.MOE_ERR_SHAPE
    assert L.moe_peak_mfma(1, 10, 0, A16 + 2, None) == qm.MOE_ERR_ALIGN
    assert L.moe_peak_hold(0, None) == qm.MOE_ERR_SHAPE
    assert L.moe_peak_hold(1000001, None) == qm.MOE_ERR_SHAPE
