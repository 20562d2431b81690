"""Python binding of the routed MoE layer's C ABI (``include/moe.h``, and the
roofline measurement kernels of ``include/moe_peak.h``).

Argument marshalling only: every step of the layer runs in the HIP kernels of
``libqrmoe.so``.  torch supplies device memory (tensors) and the stream
(``torch.cuda.current_stream()``).  There is no fallback: if the library is
missing or a call fails, an exception is raised.

The functions keep the C names.  Outputs are caller-allocated tensors, as in
the C ABI; ``layer()`` is a convenience wrapper that allocates them.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqrmoe.so")

MOE_OK = 0
MOE_ERR_NULL = -1
MOE_ERR_SHAPE = -2
MOE_ERR_FORMAT = -3
MOE_ERR_ALIGN = -4
MOE_ERR_WORKSPACE = -5
MOE_ERR_UNSUPPORTED = -6
MOE_ERR_HIP = -7
MOE_ERR_DEVICE = -8

MOE_DEV_BAD_EXPERT_ID = 1
MOE_DEV_BAD_SLOT = 2
MOE_DEV_CHAIN_TIMEOUT = 4

MOE_FMT_MXFP4 = 1
MOE_FMT_Q2G32 = 2
MOE_FMT_Q4G32 = 3
FORMATS = {"mxfp4": MOE_FMT_MXFP4, "q2": MOE_FMT_Q2G32, "q4": MOE_FMT_Q4G32}

MOE_LAYOUT_ROWS = 0
MOE_LAYOUT_TILES = 1

MOE_SLOT_SKIP = -2

# Every symbol include/moe.h declares.
EXPORTS = (
    "moe_workspace_bytes", "moe_workspace_init", "moe_route_topk", "moe_dispatch",
    "moe_expert_ffn", "moe_combine", "moe_layer_workspace_bytes", "moe_layer",
    "moe_status_str", "moe_read_device_status", "moe_read_device_status_bits", "moe_qmat_bytes", "moe_pack_qmat",
    "moe_bank_reset", "moe_bank_plan", "moe_bank_fetch", "moe_layer_banked",
    "moe_layer_shared_workspace_bytes", "moe_layer_shared",
    "moe_workspace_bytes_mx8", "moe_expert_ffn_mx8", "moe_layer_mx8_workspace_bytes", "moe_layer_mx8",
    "moe_workspace_bytes_mx4", "moe_expert_ffn_mx4", "moe_layer_mx4_workspace_bytes", "moe_layer_mx4",
    "moe_slab_layout", "moe_bank_slots", "moe_layer_noalloc",
    # include/moe_peak.h
    "moe_peak_stream", "moe_peak_mfma", "moe_peak_hold",
)


class MoeError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_str(code)} ({code})")


class moe_shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("f", ctypes.c_int32)]


class moe_qmat(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("layout", ctypes.c_int32), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("mins", ctypes.c_void_p)]


class moe_experts(ctypes.Structure):
    _fields_ = [("gate", moe_qmat), ("up", moe_qmat), ("down", moe_qmat),
                ("slot_of_expert", ctypes.c_void_p), ("num_slots", ctypes.c_int32),
                ("slot_bytes", ctypes.c_uint64)]


class moe_bank(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("num_slots", ctypes.c_int32), ("slot_of_expert", ctypes.c_void_p),
                ("expert_of_slot", ctypes.c_void_p), ("last_use", ctypes.c_void_p), ("clock", ctypes.c_uint64),
                ("copy_stream", ctypes.c_void_p), ("ev_copied", ctypes.c_void_p), ("ev_computed", ctypes.c_void_p)]


class moe_bank_stats(ctypes.Structure):
    _fields_ = [("active", ctypes.c_int32), ("hits", ctypes.c_int32), ("misses", ctypes.c_int32),
                ("passes", ctypes.c_int32), ("bytes_paged", ctypes.c_int64)]


_LIB = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        # torch first: its HIP runtime is the one the library must share
        # (stream handles and device pointers come from it).
        _torch()
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`"
                " (there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "moe_workspace_bytes": (_SZ, [_P]),
            "moe_layer_workspace_bytes": (_SZ, [_P]),
            "moe_workspace_init": (_I, [_P, _SZ, _P]),
            "moe_route_topk": (_I, [_P, _P, _P, _P, _P, _P, _P, _P]),
            "moe_dispatch": (_I, [_P, _P, _P, _P, _P, _P, _SZ, _P]),
            "moe_expert_ffn": (_I, [_P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
            "moe_combine": (_I, [_P, _P, _P, _P, _P, _P]),
            "moe_layer": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
            "moe_status_str": (ctypes.c_char_p, [_I]),
            "moe_read_device_status": (_I, [_P, _P]),
            "moe_read_device_status_bits": (_I, [_P, _P, _P]),
            "moe_qmat_bytes": (_SZ, [_I, _I, _I, _I, _I, _P, _P, _P]),
            "moe_pack_qmat": (_I, [_P, _P, _I, _I, _I, _P]),
            "moe_layer_shared_workspace_bytes": (_SZ, [_P]),
            "moe_layer_shared": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
            "moe_workspace_bytes_mx8": (_SZ, [_P]),
            "moe_expert_ffn_mx8": (_I, [_P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
            "moe_layer_mx8_workspace_bytes": (_SZ, [_P]),
            "moe_layer_mx8": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
            "moe_workspace_bytes_mx4": (_SZ, [_P]),
            "moe_expert_ffn_mx4": (_I, [_P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
            "moe_layer_mx4_workspace_bytes": (_SZ, [_P]),
            "moe_layer_mx4": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
            "moe_bank_reset": (_I, [_P]),
            "moe_bank_plan": (_I, [_P, _P, _I, _P, _P, _P]),
            "moe_bank_fetch": (_I, [_P, _P, _I, _I, _P, _P, _I, _P]),
            "moe_layer_banked": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _P]),
            "moe_slab_layout": (_SZ, [_I, _I, _I, _P]),
            "moe_bank_slots": (_I, [_I, _P, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, _P]),
            "moe_layer_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
            "moe_peak_stream": (_I, [_P, _SZ, ctypes.c_int32, _P, _P]),
            "moe_peak_mfma": (_I, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P]),
            "moe_peak_hold": (_I, [ctypes.c_uint32, _P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def status_str(code: int) -> str:
    return lib().moe_status_str(int(code)).decode()


# ------------------------------------------------------------------ helpers

def _torch():
    import torch
    return torch


def _stream(stream) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _ptr(t, dtype=None, name="tensor", allow_none=False) -> Optional[int]:
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _check(rc: int, where: str) -> None:
    if rc != MOE_OK:
        raise MoeError(rc, where)


@dataclass(frozen=True)
class Shape:
    T: int
    d: int
    E: int
    k: int
    f: int

    def c(self) -> moe_shape:
        return moe_shape(self.T, self.d, self.E, self.k, self.f)


@dataclass
class QMat:
    """One quantised matrix on the device: n rows of K elements per slot, in
    MOE_LAYOUT_ROWS (codes/scales/mins as in include/moe.h) or
    MOE_LAYOUT_TILES (codes/scales; mins None)."""
    codes: object
    scales: object
    mins: object = None
    layout: int = MOE_LAYOUT_TILES

    def c(self, fmt: int, name: str = "qmat") -> moe_qmat:
        torch = _torch()
        codes = _ptr(self.codes, torch.uint8, f"{name}.codes")
        scales = _ptr(self.scales, name=f"{name}.scales")
        mins = _ptr(self.mins, name=f"{name}.mins", allow_none=True)
        return moe_qmat(fmt, self.layout, codes, scales, mins)


def slab_layout(fmt: str, d: int, f: int):
    """moe_slab_layout: (slab bytes, [offsets of gate codes, gate scales, up
    codes, up scales, down codes, down scales]) of one expert."""
    off = (ctypes.c_size_t * 6)()
    n = int(lib().moe_slab_layout(FORMATS[fmt], int(d), int(f), off))
    if n == 0:
        raise MoeError(MOE_ERR_SHAPE, "slab_layout")
    return n, [int(v) for v in off]


def _slab_experts(fmt: str, base: int, num_slots: int, d: int, f: int, soe=None) -> moe_experts:
    """moe_experts of a slab pack whose slot 0 starts at address `base`."""
    fmtc = FORMATS[fmt]
    slab, off = slab_layout(fmt, d, f)
    q = [moe_qmat(fmtc, MOE_LAYOUT_TILES, base + off[2 * m], base + off[2 * m + 1], None) for m in range(3)]
    return moe_experts(q[0], q[1], q[2], soe, num_slots, slab)


@dataclass
class Experts:
    """The gate/up/down packs of one layer (device tensors, tile layout);
    d = hidden size, f = expert FFN size.  A slab pack (``slab`` set: uint8
    [num_slots * slot_bytes], every expert's six arrays in one slab, see
    ``to_slabs``) has no separate QMats."""
    fmt: str
    gate: Optional[QMat]
    up: Optional[QMat]
    down: Optional[QMat]
    slot_of_expert: object = None
    num_slots: int = 0
    d: int = 0
    f: int = 0
    slab: object = None

    def c(self) -> moe_experts:
        torch = _torch()
        fmt = FORMATS[self.fmt]
        soe = _ptr(self.slot_of_expert, torch.int32, "slot_of_expert", allow_none=True)
        if self.slab is not None:
            return _slab_experts(self.fmt, _ptr(self.slab, torch.uint8, "slab"), self.num_slots, self.d, self.f, soe)
        return moe_experts(self.gate.c(fmt, "gate"), self.up.c(fmt, "up"), self.down.c(fmt, "down"), soe,
                           self.num_slots, 0)

    def slot_arrays(self):
        """[(matrix, slot bytes of codes, slot bytes of scales, codes tensor,
        scales tensor)] of a separate-array pack."""
        out = []
        for name, n, K in (("gate", self.f, self.d), ("up", self.f, self.d), ("down", self.d, self.f)):
            cb, sb, _ = moe_qmat_bytes(self.fmt, MOE_LAYOUT_TILES, 1, n, K)
            m = getattr(self, name)
            out.append((name, cb, sb, m.codes, m.scales))
        return out

    def to_slabs(self, pin_host: bool = False, device=None) -> "Experts":
        """A copy as a slab pack (moe_slab_layout): on `device` (default: the
        pack's), or with pin_host in pinned host memory (a slot-bank pool;
        such a pack is passed to the C ABI through _slab_experts)."""
        torch = _torch()
        if self.slab is not None:
            raise ValueError("already a slab pack")
        slab, off = slab_layout(self.fmt, self.d, self.f)
        n = self.num_slots * slab
        if pin_host:
            t = torch.zeros(n, dtype=torch.uint8, pin_memory=True)
        else:
            t = torch.zeros(n, dtype=torch.uint8, device=device or self.gate.codes.device)
        for i, (_, cb, sb, codes, scales) in enumerate(self.slot_arrays()):
            cs = codes.view(torch.uint8).reshape(self.num_slots, cb)
            ss = scales.view(torch.uint8).reshape(self.num_slots, sb)
            view = t.view(self.num_slots, slab)
            view[:, off[2 * i]:off[2 * i] + cb].copy_(cs)
            view[:, off[2 * i + 1]:off[2 * i + 1] + sb].copy_(ss)
        return Experts(self.fmt, None, None, None, self.slot_of_expert, self.num_slots, self.d, self.f, slab=t)

    @staticmethod
    def from_arrays(fmt: str, gate: dict, up: dict, down: dict, device="cuda",
                    slot_of_expert=None) -> "Experts":
        """Row-layout host arrays (numpy; codes uint8 [slots][n][..], scales
        uint8 or uint16 fp16 bits, mins uint16) -> tile-layout device packs
        (copied to the device, then re-laid by moe_pack_qmat)."""
        torch = _torch()
        slots, f = int(gate["codes"].shape[0]), int(gate["codes"].shape[1])
        d = 32 * int(gate["scales"].shape[2])
        soe = None
        if slot_of_expert is not None:
            soe = torch.from_numpy(np.ascontiguousarray(slot_of_expert, dtype=np.int32)).to(device)
        return Experts(fmt, pack_arrays(fmt, gate, f, d, device), pack_arrays(fmt, up, f, d, device),
                       pack_arrays(fmt, down, d, f, device), soe, slots, d, f)


def _dev(a, device):
    torch = _torch()
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a)) if not isinstance(a, torch.Tensor) else a
    if t.dtype == torch.uint16:
        t = t.view(torch.int16)
    return t.contiguous().to(device)


def pack_arrays(fmt: str, m: dict, n: int, K: int, device="cuda", stream=None) -> QMat:
    """One row-layout matrix (host arrays) -> a tile-layout QMat on the device."""
    src = QMat(_dev(m["codes"], device), _dev(m["scales"], device), _dev(m.get("mins"), device),
               MOE_LAYOUT_ROWS)
    slots = int(m["codes"].shape[0])
    return pack_qmat(fmt, src, slots, n, K, stream)


def pack_qmat(fmt: str, src: QMat, slots: int, n: int, K: int, stream=None) -> QMat:
    """Allocate a tile-layout matrix and fill it from the row-layout `src`
    (device tensors) with moe_pack_qmat."""
    torch = _torch()
    cb, sb, _ = moe_qmat_bytes(fmt, MOE_LAYOUT_TILES, slots, n, K)
    if cb == 0:
        raise MoeError(MOE_ERR_SHAPE, "pack_qmat")
    dev = src.codes.device
    dst = QMat(torch.empty(cb, dtype=torch.uint8, device=dev), torch.empty(sb, dtype=torch.uint8, device=dev),
               None, MOE_LAYOUT_TILES)
    moe_pack_qmat(fmt, src, dst, slots, n, K, stream)
    return dst


# ------------------------------------------------------------ C entry points

def moe_qmat_bytes(fmt, layout: int, slots: int, n: int, K: int):
    """(codes, scales, mins) byte sizes of a matrix; zeros if invalid."""
    f = FORMATS.get(fmt, fmt) if isinstance(fmt, str) else fmt
    c, s_, m = ctypes.c_size_t(0), ctypes.c_size_t(0), ctypes.c_size_t(0)
    lib().moe_qmat_bytes(int(f), int(layout), int(slots), int(n), int(K), ctypes.byref(c), ctypes.byref(s_),
                         ctypes.byref(m))
    return int(c.value), int(s_.value), int(m.value)


def moe_pack_qmat(fmt, src: QMat, dst: QMat, slots: int, n: int, K: int, stream=None) -> None:
    f = FORMATS[fmt] if isinstance(fmt, str) else fmt
    s_ = src.c(f, "src")
    d_ = dst.c(f, "dst")
    _check(lib().moe_pack_qmat(ctypes.byref(s_), ctypes.byref(d_), int(slots), int(n), int(K), _stream(stream)),
           "moe_pack_qmat")


def moe_workspace_bytes(shape: Shape) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(shape.c())))


def moe_layer_workspace_bytes(shape: Shape) -> int:
    return int(lib().moe_layer_workspace_bytes(ctypes.byref(shape.c())))


def moe_workspace_init(ws, stream=None) -> None:
    _check(lib().moe_workspace_init(_ptr(ws, name="ws"), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_workspace_init")


def moe_route_topk(shape: Shape, x, w_router, bias, logits, topk_ids, topk_w, stream=None) -> None:
    torch = _torch()
    rc = lib().moe_route_topk(
        ctypes.byref(shape.c()), _ptr(x, (torch.int16, torch.bfloat16, torch.uint16), "x", allow_none=True),
        _ptr(w_router, torch.float32, "w_router", allow_none=True),
        _ptr(bias, torch.float32, "bias", allow_none=True), _ptr(logits, torch.float32, "logits"),
        _ptr(topk_ids, torch.int32, "topk_ids"), _ptr(topk_w, torch.float32, "topk_w"), _stream(stream))
    _check(rc, "moe_route_topk")


def moe_dispatch(shape: Shape, topk_ids, offsets, perm, inv, ws, stream=None) -> None:
    torch = _torch()
    rc = lib().moe_dispatch(
        ctypes.byref(shape.c()), _ptr(topk_ids, torch.int32, "topk_ids"),
        _ptr(offsets, torch.int32, "offsets"), _ptr(perm, torch.int32, "perm"),
        _ptr(inv, torch.int32, "inv"), _ptr(ws, name="ws"), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "moe_dispatch")


def moe_expert_ffn(shape: Shape, x, experts: Experts, offsets, perm, y, ws, stream=None) -> None:
    torch = _torch()
    ex = experts.c()
    rc = lib().moe_expert_ffn(
        ctypes.byref(shape.c()), _ptr(x, (torch.int16, torch.bfloat16, torch.uint16), "x"),
        ctypes.byref(ex), _ptr(offsets, torch.int32, "offsets"), _ptr(perm, torch.int32, "perm"),
        _ptr(y, torch.float32, "y"), _ptr(ws, name="ws"), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "moe_expert_ffn")


def moe_combine(shape: Shape, y, inv, topk_w, out, stream=None) -> None:
    torch = _torch()
    rc = lib().moe_combine(
        ctypes.byref(shape.c()), _ptr(y, torch.float32, "y"), _ptr(inv, torch.int32, "inv"),
        _ptr(topk_w, torch.float32, "topk_w"), _ptr(out, torch.float32, "out"), _stream(stream))
    _check(rc, "moe_combine")


def moe_layer(shape: Shape, x, w_router, bias, logits, experts: Experts, topk_ids, topk_w, out, ws,
              stream=None) -> None:
    torch = _torch()
    ex = experts.c()
    rc = lib().moe_layer(
        ctypes.byref(shape.c()), _ptr(x, (torch.int16, torch.bfloat16, torch.uint16), "x"),
        _ptr(w_router, torch.float32, "w_router", allow_none=True),
        _ptr(bias, torch.float32, "bias", allow_none=True), _ptr(logits, torch.float32, "logits"),
        ctypes.byref(ex), _ptr(topk_ids, torch.int32, "topk_ids"), _ptr(topk_w, torch.float32, "topk_w"),
        _ptr(out, torch.float32, "out"), _ptr(ws, name="ws"), ws.numel() * ws.element_size(),
        _stream(stream))
    _check(rc, "moe_layer")


MOE_NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024


def moe_layer_noalloc(shape: Shape, x, w_router, bias, logits, experts: Experts, topk_ids, topk_w, out,
                      status=None, stream=None) -> None:
    """moe_layer with the library's own per-GPU scratch array as workspace
    (nothing allocated; calls that overlap on one GPU race).  status: a
    device int32/uint32 tensor of one element that device faults are OR-ed
    into, or None."""
    torch = _torch()
    ex = experts.c()
    rc = lib().moe_layer_noalloc(
        ctypes.byref(shape.c()), _ptr(x, (torch.int16, torch.bfloat16, torch.uint16), "x"),
        _ptr(w_router, torch.float32, "w_router", allow_none=True),
        _ptr(bias, torch.float32, "bias", allow_none=True), _ptr(logits, torch.float32, "logits"),
        ctypes.byref(ex), _ptr(topk_ids, torch.int32, "topk_ids"), _ptr(topk_w, torch.float32, "topk_w"),
        _ptr(out, torch.float32, "out"), _ptr(status, (torch.int32, torch.uint32), "status", allow_none=True),
        _stream(stream))
    _check(rc, "moe_layer_noalloc")


def moe_read_device_status(ws, stream=None) -> int:
    """Synchronises the stream; returns the device status bits (0 = clean)."""
    bits = ctypes.c_uint32(0)
    rc = lib().moe_read_device_status_bits(_ptr(ws, name="ws"), ctypes.byref(bits), _stream(stream))
    if rc not in (MOE_OK, MOE_ERR_DEVICE):
        raise MoeError(rc, "moe_read_device_status")
    return int(bits.value)


def check_device_status(ws, where: str, stream=None) -> None:
    """Synchronises the stream and raises MoeError(MOE_ERR_DEVICE) if a
    kernel flagged bad device data or a prefill hand-off timed out (whose y
    rows are then NaN) in the calls on `ws` since its last moe_workspace_init."""
    bits = moe_read_device_status(ws, stream)
    if bits:
        err = MoeError(MOE_ERR_DEVICE, f"{where}: device status {bits:#x}")
        err.bits = bits
        raise err


# --------------------------------------------------------------- conveniences

def alloc_workspace(shape: Shape, layer: bool = False, device="cuda", stream=None):
    """A zero-initialised workspace tensor for `shape` (header cleared)."""
    torch = _torch()
    n = moe_layer_workspace_bytes(shape) if layer else moe_workspace_bytes(shape)
    if n == 0:
        raise MoeError(MOE_ERR_SHAPE, "alloc_workspace")
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    moe_workspace_init(ws, stream)
    return ws


def layer(x, experts: Experts, k: int, *, w_router=None, bias=None, logits=None, ws=None, stream=None,
          check: bool = False):
    """Run the whole layer; returns (out, topk_ids, topk_w, logits).  With
    check=True the stream is synchronised and a nonzero device status word
    (e.g. MOE_DEV_CHAIN_TIMEOUT) raises MoeError."""
    torch = _torch()
    T, d = x.shape
    E = int(w_router.shape[0]) if w_router is not None else int(logits.shape[1])
    f = experts.f
    shape = Shape(T, d, E, k, f)
    dev = x.device
    if logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    out = torch.empty((T, d), dtype=torch.float32, device=dev)
    if ws is None:
        ws = alloc_workspace(shape, layer=True, device=dev, stream=stream)
    moe_layer(shape, x, w_router, bias, logits, experts, ids, w, out, ws, stream)
    if check:
        check_device_status(ws, "layer", stream)
    return out, ids, w, logits


# ------------------------------------------------ MXFP8 / MXFP4 activations

def _ffn_mxq(bits, shape: Shape, x, experts: Experts, offsets, perm, y, ws, stream=None) -> None:
    torch = _torch()
    ex = experts.c()
    name = f"moe_expert_ffn_mx{bits}"
    rc = getattr(lib(), name)(
        ctypes.byref(shape.c()), _ptr(x, (torch.int16, torch.bfloat16, torch.uint16), "x"),
        ctypes.byref(ex), _ptr(offsets, torch.int32, "offsets"), _ptr(perm, torch.int32, "perm"),
        _ptr(y, torch.float32, "y"), _ptr(ws, name="ws"), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, name)


def moe_expert_ffn_mx8(shape: Shape, x, experts: Experts, offsets, perm, y, ws, stream=None) -> None:
    _ffn_mxq(8, shape, x, experts, offsets, perm, y, ws, stream)


def moe_expert_ffn_mx4(shape: Shape, x, experts: Experts, offsets, perm, y, ws, stream=None) -> None:
    _ffn_mxq(4, shape, x, experts, offsets, perm, y, ws, stream)


def _alloc_workspace_mxq(bits, shape: Shape, layer: bool, device, stream):
    torch = _torch()
    fn = getattr(lib(), f"moe_layer_mx{bits}_workspace_bytes" if layer else f"moe_workspace_bytes_mx{bits}")
    n = int(fn(ctypes.byref(shape.c())))
    if n == 0:
        raise MoeError(MOE_ERR_SHAPE, f"alloc_workspace_mx{bits}")
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    moe_workspace_init(ws, stream)
    return ws


def alloc_workspace_mx8(shape: Shape, layer: bool = False, device="cuda", stream=None):
    return _alloc_workspace_mxq(8, shape, layer, device, stream)


def alloc_workspace_mx4(shape: Shape, layer: bool = False, device="cuda", stream=None):
    return _alloc_workspace_mxq(4, shape, layer, device, stream)


def _layer_mxq(bits, x, experts: Experts, k: int, w_router, bias, logits, ws, stream, check):
    torch = _torch()
    T, d = x.shape
    E = int(w_router.shape[0]) if w_router is not None else int(logits.shape[1])
    shape = Shape(T, d, E, k, experts.f)
    dev = x.device
    if logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    out = torch.empty((T, d), dtype=torch.float32, device=dev)
    if ws is None:
        ws = _alloc_workspace_mxq(bits, shape, True, dev, stream)
    ex = experts.c()
    name = f"moe_layer_mx{bits}"
    rc = getattr(lib(), name)(
        ctypes.byref(shape.c()), _ptr(x, (torch.int16, torch.bfloat16, torch.uint16), "x"),
        _ptr(w_router, torch.float32, "w_router", allow_none=True),
        _ptr(bias, torch.float32, "bias", allow_none=True), _ptr(logits, torch.float32, "logits"),
        ctypes.byref(ex), _ptr(ids, torch.int32, "topk_ids"), _ptr(w, torch.float32, "topk_w"),
        _ptr(out, torch.float32, "out"), _ptr(ws, name="ws"), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, name)
    if check:
        check_device_status(ws, f"layer_mx{bits}", stream)
    return out, ids, w, logits


def layer_mx8(x, experts: Experts, k: int, *, w_router=None, bias=None, logits=None, ws=None, stream=None,
              check: bool = False):
    """moe_layer_mx8: the layer with MXFP8 activations in the expert FFN;
    returns (out, topk_ids, topk_w, logits)."""
    return _layer_mxq(8, x, experts, k, w_router, bias, logits, ws, stream, check)


def layer_mx4(x, experts: Experts, k: int, *, w_router=None, bias=None, logits=None, ws=None, stream=None,
              check: bool = False):
    """moe_layer_mx4: the layer with MXFP4 activations in the expert FFN;
    returns (out, topk_ids, topk_w, logits)."""
    return _layer_mxq(4, x, experts, k, w_router, bias, logits, ws, stream, check)


# -------------------------------------------------------------- shared expert

def layer_shared(x, experts: Experts, shared: Experts, k: int, *, w_router=None, bias=None, logits=None,
                 ws=None, stream=None, check: bool = False):
    """moe_layer_shared: the layer plus an always-on shared expert (weight 1,
    slot 0 of `shared`); returns (out, topk_ids, topk_w, logits)."""
    torch = _torch()
    T, d = x.shape
    E = int(w_router.shape[0]) if w_router is not None else int(logits.shape[1])
    shape = Shape(T, d, E, k, experts.f)
    dev = x.device
    if logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    out = torch.empty((T, d), dtype=torch.float32, device=dev)
    if ws is None:
        n = int(lib().moe_layer_shared_workspace_bytes(ctypes.byref(shape.c())))
        if n == 0:
            raise MoeError(MOE_ERR_SHAPE, "layer_shared")
        ws = torch.empty(n, dtype=torch.uint8, device=dev)
        moe_workspace_init(ws, stream)
    ex, sh = experts.c(), shared.c()
    rc = lib().moe_layer_shared(
        ctypes.byref(shape.c()), _ptr(x, (torch.int16, torch.bfloat16, torch.uint16), "x"),
        _ptr(w_router, torch.float32, "w_router", allow_none=True),
        _ptr(bias, torch.float32, "bias", allow_none=True), _ptr(logits, torch.float32, "logits"),
        ctypes.byref(ex), ctypes.byref(sh), _ptr(ids, torch.int32, "topk_ids"), _ptr(w, torch.float32, "topk_w"),
        _ptr(out, torch.float32, "out"), _ptr(ws, name="ws"), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "moe_layer_shared")
    if check:
        check_device_status(ws, "layer_shared", stream)
    return out, ids, w, logits


# ------------------------------------------------------------------ slot bank

class BankState:
    """Host bookkeeping of an N-slot bank over E experts (moe_bank; the
    arrays are numpy, owned here)."""

    def __init__(self, E: int, num_slots: int):
        self.slot_of_expert = np.full(E, -1, dtype=np.int32)
        self.expert_of_slot = np.full(num_slots, -1, dtype=np.int32)
        self.last_use = np.zeros(num_slots, dtype=np.uint64)
        self.c = moe_bank(E, num_slots, self.slot_of_expert.ctypes.data, self.expert_of_slot.ctypes.data,
                          self.last_use.ctypes.data, 0)
        _check(lib().moe_bank_reset(ctypes.byref(self.c)), "moe_bank_reset")

    def plan(self, want) -> list:
        """moe_bank_plan over the distinct expert ids `want`; returns the
        loads [(expert, slot), ...]."""
        w = np.ascontiguousarray(want, dtype=np.int32)
        n = len(w)
        le = np.zeros(max(n, 1), dtype=np.int32)
        ls = np.zeros(max(n, 1), dtype=np.int32)
        nl = ctypes.c_int32(0)
        _check(lib().moe_bank_plan(ctypes.byref(self.c), w.ctypes.data if n else None, n, le.ctypes.data,
                                   ls.ctypes.data, ctypes.byref(nl)), "moe_bank_plan")
        return [(int(le[i]), int(ls[i])) for i in range(nl.value)]


def _hip_runtime():
    """The HIP runtime torch loaded (stream and event handles must come from it)."""
    torch = _torch()
    hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
    for fn in ("hipEventCreateWithFlags", "hipEventDestroy"):
        getattr(hip, fn).restype = ctypes.c_int
    return hip


def bank_slots(fmt: str, prefill_shape: Shape, budget_bytes: int = 0, reserve_bytes: int = 0,
               free_bytes: Optional[int] = None) -> int:
    """moe_bank_slots: the slots of a bank of `budget_bytes` (0 = auto, from
    the device's free memory), clamped so that a call of `prefill_shape`
    still finds its layer workspace and `reserve_bytes` of other buffers."""
    if free_bytes is None:
        free_bytes = int(_torch().cuda.mem_get_info()[0])
    n = ctypes.c_int32(0)
    _check(lib().moe_bank_slots(FORMATS[fmt], ctypes.byref(prefill_shape.c()), int(budget_bytes),
                                int(free_bytes), int(reserve_bytes), ctypes.byref(n)), "moe_bank_slots")
    return int(n.value)


class SlotBank:
    """Experts paged through `num_slots` device slots from a pool of all E
    experts in pinned host memory (moe_layer_banked).  `experts` is a device
    pack of the E experts (tile layout); its bytes are copied once into the
    pinned pool, after which the device pack may be dropped.  Pool and bank
    are slab packs, so a miss is one copy.  With `overlap` the copies run on
    a stream of their own (default priority) and the resident experts' FFN
    runs while the misses land."""

    def __init__(self, experts: Experts, num_slots: int, device="cuda", overlap: bool = True):
        torch = _torch()
        E = experts.num_slots
        self.fmt, self.E, self.num_slots, self.d, self.f = experts.fmt, E, num_slots, experts.d, experts.f
        self.pool = experts.to_slabs(pin_host=True)
        self.pool_c = _slab_experts(self.fmt, self.pool.slab.data_ptr(), E, self.d, self.f)
        slab, _ = slab_layout(self.fmt, self.d, self.f)
        self.slots = Experts(self.fmt, None, None, None, None, num_slots, self.d, self.f,
                             slab=torch.zeros(num_slots * slab, dtype=torch.uint8, device=device))
        self.slot_map = torch.full((E,), MOE_SLOT_SKIP, dtype=torch.int32, device=device)
        self.copy_stream = None
        self._events = []
        if overlap:
            self.copy_stream = torch.cuda.Stream(device=device)
            hip = _hip_runtime()
            for _ in range(2):
                ev = ctypes.c_void_p()
                if hip.hipEventCreateWithFlags(ctypes.byref(ev), 2):     # hipEventDisableTiming
                    raise MoeError(MOE_ERR_HIP, "SlotBank: hipEventCreateWithFlags")
                self._events.append(ev)
        self.state = BankState(E, num_slots)
        self.last_stats = None

    @property
    def state(self) -> BankState:
        return self._state

    @state.setter
    def state(self, st: BankState) -> None:
        # the bank's books, plus this bank's copy stream and events
        self._state = st
        if self.copy_stream is not None:
            st.c.copy_stream = int(self.copy_stream.cuda_stream)
            st.c.ev_copied = self._events[0].value
            st.c.ev_computed = self._events[1].value

    def close(self) -> None:
        """Destroys the bank's events (call when done with the bank)."""
        if self._events:
            torch = _torch()
            torch.cuda.synchronize()
            hip = _hip_runtime()
            for ev in self._events:
                hip.hipEventDestroy(ev)
            self._events = []
            self.copy_stream = None
            self._state.c.copy_stream = None
            self._state.c.ev_copied = None
            self._state.c.ev_computed = None

    def layer(self, x, k: int, *, w_router=None, bias=None, logits=None, ws=None, stream=None,
              check: bool = False):
        """One layer call through the bank (synchronises the stream once);
        returns (out, topk_ids, topk_w, logits) and sets last_stats."""
        torch = _torch()
        T, d = x.shape
        shape = Shape(T, d, self.E, k, self.f)
        dev = x.device
        if logits is None:
            logits = torch.empty((T, self.E), dtype=torch.float32, device=dev)
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        out = torch.empty((T, d), dtype=torch.float32, device=dev)
        if ws is None:
            ws = alloc_workspace(shape, layer=True, device=dev, stream=stream)
        st = moe_bank_stats()
        sl = self.slots.c()
        rc = lib().moe_layer_banked(
            ctypes.byref(shape.c()), _ptr(x, (torch.int16, torch.bfloat16, torch.uint16), "x"),
            _ptr(w_router, torch.float32, "w_router", allow_none=True),
            _ptr(bias, torch.float32, "bias", allow_none=True), _ptr(logits, torch.float32, "logits"),
            ctypes.byref(self.pool_c), ctypes.byref(self.state.c), ctypes.byref(sl),
            _ptr(self.slot_map, torch.int32, "slot_map"), _ptr(ids, torch.int32, "topk_ids"),
            _ptr(w, torch.float32, "topk_w"), _ptr(out, torch.float32, "out"), _ptr(ws, name="ws"),
            ws.numel() * ws.element_size(), _stream(stream), ctypes.byref(st))
        _check(rc, "moe_layer_banked")
        self.last_stats = dict(active=st.active, hits=st.hits, misses=st.misses, passes=st.passes,
                               bytes_paged=int(st.bytes_paged))
        if check:
            check_device_status(ws, "SlotBank.layer", stream)
        return out, ids, w, logits
