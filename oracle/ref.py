"""NumPy float64 oracle of the routed MoE layer (test infrastructure only).

The layer, step by step, as the pages describe it in prose ("antirez ds4:
DeepSeek Metal inference", section 技术深度解析: a router picks the top-2 of
64 fine-grained experts per token, a block-sparse kernel loads only the
activated experts' quantised weights and dequantises them on the fly):

1. router logits        l[t, e] = sum_i x[t, i] * W_r[e, i] (+ b[e])
2. top-k + weights      per token, the k largest logits (ties: lower id),
                        w = softmax over the selected logits
3. dispatch             stable counting sort of the (token, slot) pairs by
                        expert id -> offsets / perm / inv
4. gate/up + SwiGLU     act = bf16(silu(W_g x) * (W_u x))
5. down                 y = W_d act
6. combine              out[t] = sum_j w[t, j] * y[inv[t*k + j]]

Rounding points: the inputs (x is bf16) and the SwiGLU intermediate (act is
rounded to bf16, round-to-nearest-even, directly from float64).  Everything
else is float64.  The dequantised weights are exact in float64.

Library primitives used as single steps: ``numpy.matmul``,
``numpy.lexsort``, ``numpy.argsort(kind="stable")``, ``numpy.exp``.
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------

# OCP Microscaling Formats (MX) v1.0, FP4 (E2M1) element encoding: magnitudes
# for the 3 low bits; bit 3 is the sign (so code 8 is -0).
E2M1_MAGNITUDE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)

# bf16 has 8 significant bits; its smallest subnormal is 2**-133 and values
# at or above 2**128 after rounding overflow to infinity.
_BF16_SIG_BITS = 8
_BF16_MIN_QUANTUM_EXP = -133
_BF16_OVERFLOW = 2.0 ** 128


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def fp16_bits_to_f64(bits) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) -> exact float64 values."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def round_bf16(v) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even.

    Rounds directly from float64 (no intermediate float32), handles bf16
    subnormals and overflow to +-inf.  Returns float64 holding bf16 values.
    """
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        _, e = np.frexp(v)                      # v = m * 2**e, 0.5 <= |m| < 1
        q = np.maximum(e - _BF16_SIG_BITS, _BF16_MIN_QUANTUM_EXP)
        r = np.rint(np.ldexp(v, -q))            # exact power-of-two scaling; rint is half-even
        res = np.ldexp(r, q)
        res = np.where(np.abs(res) >= _BF16_OVERFLOW, np.copysign(np.inf, v), res)
        res = np.where(np.isfinite(v), res, v)
    return res


def e8m0_to_f64(scale_bytes) -> np.ndarray:
    """OCP MX e8m0 shared scale: byte b encodes 2**(b - 127); 255 is NaN.

    NaN scales are rejected (the packs never carry them).
    """
    b = np.asarray(scale_bytes, dtype=np.uint8)
    if np.any(b == 255):
        raise ValueError("e8m0 scale byte 255 (NaN) in an MXFP4 pack")
    return np.ldexp(1.0, b.astype(np.int64) - 127)


def e2m1_to_f64(codes) -> np.ndarray:
    """4-bit e2m1 codes (0..15) -> float64 element values (before scaling)."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_MAGNITUDE[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


def dequant_mxfp4(codes, scales) -> np.ndarray:
    """Decode an MXFP4 matrix pack to float64.

    codes  uint8 [..., n, K/2]: element 2i of a row is the LOW nibble of byte
           i, element 2i+1 the HIGH nibble (reading taken: the pages give no
           packing; low-nibble-first is the common MX/GGUF order).
    scales uint8 [..., n, K/32]: one e8m0 scale per 32 consecutive elements
           along K (the MX block size).
    Returns float64 [..., n, K] with value = e2m1(code) * 2**(scale - 127).
    """
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    lo = e2m1_to_f64(codes & 0x0F)
    hi = e2m1_to_f64(codes >> 4)
    elems = np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)
    s = np.repeat(e8m0_to_f64(scales), 32, axis=-1)
    if s.shape != elems.shape:
        raise ValueError(f"scales {scales.shape} do not match codes {codes.shape}")
    return elems * s


def dequant_q2(codes, scale_bits, min_bits) -> np.ndarray:
    """Decode a 2-bit group-asymmetric matrix pack to float64.

    The pages name "q2 asymmetric" quantisation only ("DwarfStar 4 ... 完整指南",
    section on why ds4 suits a 128 GB Mac Studio).  Reading taken:
      w = scale * q + min, q in {0, 1, 2, 3}, one IEEE fp16 scale and one fp16
      min per group of 32 consecutive elements along K.
    codes uint8 [..., n, K/4]: element 4i+j of a row is bits (2j, 2j+1) of
      byte i (lowest bits first).
    scale_bits, min_bits uint16 [..., n, K/32] (fp16 bit patterns).
    """
    codes = np.asarray(codes, dtype=np.uint8)
    q = np.stack([(codes >> (2 * j)) & 3 for j in range(4)], axis=-1)
    q = q.reshape(*codes.shape[:-1], codes.shape[-1] * 4).astype(np.float64)
    s = np.repeat(fp16_bits_to_f64(scale_bits), 32, axis=-1)
    m = np.repeat(fp16_bits_to_f64(min_bits), 32, axis=-1)
    if s.shape != q.shape or m.shape != q.shape:
        raise ValueError("scale/min shape does not match codes")
    return s * q + m


def dequant_q4(codes, scale_bits, min_bits) -> np.ndarray:
    """Decode a 4-bit group-asymmetric matrix pack to float64.

    The pages name a GPTQ-like 4-bit quantisation with dequantisation at
    inference time ("antirez ds4: DeepSeek Metal inference", section
    技术深度解析) and a q4 model build ("DwarfStar 4 ... 完整指南", section
    性能实测参考), nothing more.  Reading taken (the group-wise affine form of
    the 2-bit pack, with a zero point folded into the min):
      w = scale * q + min, q in {0, ..., 15}, one IEEE fp16 scale and one fp16
      min per group of 32 consecutive elements along K.
    codes uint8 [..., n, K/2]: element 2i of a row is the low nibble of byte
      i, element 2i+1 the high nibble (the order of the MXFP4 pack).
    scale_bits, min_bits uint16 [..., n, K/32] (fp16 bit patterns).
    """
    codes = np.asarray(codes, dtype=np.uint8)
    q = np.stack([codes & 0x0F, codes >> 4], axis=-1)
    q = q.reshape(*codes.shape[:-1], codes.shape[-1] * 2).astype(np.float64)
    s = np.repeat(fp16_bits_to_f64(scale_bits), 32, axis=-1)
    m = np.repeat(fp16_bits_to_f64(min_bits), 32, axis=-1)
    if s.shape != q.shape or m.shape != q.shape:
        raise ValueError("scale/min shape does not match codes")
    return s * q + m


def dequant(mat: dict, slot: int) -> np.ndarray:
    """Dequantise one expert slot of a matrix pack (dict with 'fmt' and arrays)."""
    fmt = mat["fmt"]
    if fmt == "mxfp4":
        return dequant_mxfp4(mat["codes"][slot], mat["scales"][slot])
    if fmt == "q2":
        return dequant_q2(mat["codes"][slot], mat["scales"][slot], mat["mins"][slot])
    if fmt == "q4":
        return dequant_q4(mat["codes"][slot], mat["scales"][slot], mat["mins"][slot])
    raise ValueError(f"unknown format {fmt!r}")


# ---------------------------------------------------------------------------
# Steps of the layer
# ---------------------------------------------------------------------------

def router_logits(x_bits, w_router, bias=None) -> np.ndarray:
    """Step 1: l[t, e] = sum_i x[t, i] * W_r[e, i] + b[e], float64.

    The router stays in full precision: the ds4 guide ("避坑指南") reports
    that community quantisations fail precisely at the MoE router.  x is bf16
    (decoded exactly), W_r and b are float32 (exact in float64).
    """
    x = bf16_bits_to_f64(x_bits)
    w = np.asarray(w_router, dtype=np.float32).astype(np.float64)
    l = x @ w.T
    if bias is not None:
        l = l + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    return l


def route_topk(logits, k: int):
    """Step 2: per token, the k experts with the largest logits, and weights.

    Order: by logit descending, ties to the lower expert id (reading taken:
    the pages say only "top-2"); -0.0 and +0.0 compare equal.  Weights:
    softmax over the selected logits, i.e. softmax over all experts
    renormalised over the top-k (reading taken: no sigmoid gate, no routed
    scaling factor).  Logits must be finite.

    Returns ids int32 [T, k] (in selection order) and w float64 [T, k].
    """
    l = np.asarray(logits, dtype=np.float64)
    if not np.all(np.isfinite(l)):
        raise ValueError("router logits must be finite")
    T, E = l.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    expert = np.arange(E)
    for t in range(T):
        order = np.lexsort((expert, -l[t]))   # primary: -logit ascending; secondary: id
        sel = order[:k]
        ids[t] = sel
        ls = l[t, sel]
        ex = np.exp(ls - ls.max())
        w[t] = ex / ex.sum()
    return ids, w


def dispatch(ids, E: int):
    """Step 3: stable sort of the T*k (token, slot) pairs by expert id.

    Pair p = t*k + j.  offsets[E+1] is the exclusive prefix sum of the per
    expert counts; perm[r] is the pair at sorted row r (pairs of one expert
    keep ascending p); inv[p] is the sorted row of pair p.
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    perm = np.argsort(flat, kind="stable").astype(np.int32)
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(flat.size, dtype=np.int32)
    return offsets, perm, inv


def silu(z):
    """silu(z) = z / (1 + exp(-z)) (the Swish-1 gate of SwiGLU)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(x_bits, k: int, offsets, perm, gate: dict, up: dict, down: dict,
               slot_of_expert=None):
    """Steps 4 and 5 for every sorted row.

    For sorted row r of expert e (token t = perm[r] // k):
      g = W_g[e] x_t,  u = W_u[e] x_t           (float64 over exact weights)
      act_r = bf16_RNE(silu(g) * u)             (the SwiGLU rounding point)
      y_r = W_d[e] act_r                        (float64)
    Only experts with at least one row are dequantised: the block-sparse
    kernel reads no inactive expert's weights.  slot_of_expert maps expert -> pack slot
    (identity when None).

    Returns act float64 [T*k, f] (bf16 values) and y float64 [T*k, d].
    """
    x = bf16_bits_to_f64(x_bits)
    offsets = np.asarray(offsets, dtype=np.int64)
    perm = np.asarray(perm, dtype=np.int64)
    E = offsets.size - 1
    n_rows = int(offsets[-1])
    f = gate["codes"].shape[-2]
    d = down["codes"].shape[-2]
    act = np.zeros((n_rows, f), dtype=np.float64)
    y = np.zeros((n_rows, d), dtype=np.float64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        slot = e if slot_of_expert is None else int(slot_of_expert[e])
        wg = dequant(gate, slot)          # [f, d]
        wu = dequant(up, slot)            # [f, d]
        wd = dequant(down, slot)          # [d, f]
        xt = x[perm[r0:r1] // k]          # [rows, d]
        g = xt @ wg.T
        u = xt @ wu.T
        a = round_bf16(silu(g) * u)
        act[r0:r1] = a
        y[r0:r1] = a @ wd.T
    return act, y


def expert_ffn_rows(x_bits, k: int, offsets, perm, rows, gate: dict, up: dict, down: dict,
                    slot_of_expert=None):
    """Steps 4 and 5 for a chosen subset of sorted rows only (same arithmetic
    as ``expert_ffn``), for checking large calls on sampled outputs.

    Returns act float64 [len(rows), f] and y float64 [len(rows), d].
    """
    x = bf16_bits_to_f64(x_bits)
    offsets = np.asarray(offsets, dtype=np.int64)
    perm = np.asarray(perm, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    expert_of_row = np.searchsorted(offsets, rows, side="right") - 1
    f = gate["codes"].shape[-2]
    d = down["codes"].shape[-2]
    act = np.zeros((rows.size, f), dtype=np.float64)
    y = np.zeros((rows.size, d), dtype=np.float64)
    for e in np.unique(expert_of_row):
        sel = np.nonzero(expert_of_row == e)[0]
        slot = int(e) if slot_of_expert is None else int(slot_of_expert[e])
        wg, wu, wd = dequant(gate, slot), dequant(up, slot), dequant(down, slot)
        xt = x[perm[rows[sel]] // k]
        a = round_bf16(silu(xt @ wg.T) * (xt @ wu.T))
        act[sel] = a
        y[sel] = a @ wd.T
    return act, y


def expert_down(act, offsets, down: dict, rows=None, slot_of_expert=None):
    """Step 5 alone, on a GIVEN bf16 intermediate: y_r = W_d[e] act_r in
    float64 for the sorted rows `rows` (all rows when None).  Used to check
    the down projection of a device given the act it produced itself, so
    that a one-ulp difference at the bf16 rounding point of step 4 is not
    mistaken for an error of step 5."""
    offsets = np.asarray(offsets, dtype=np.int64)
    act = np.asarray(act, dtype=np.float64)
    rows = np.arange(int(offsets[-1])) if rows is None else np.asarray(rows, dtype=np.int64)
    expert_of_row = np.searchsorted(offsets, rows, side="right") - 1
    d = down["codes"].shape[-2]
    y = np.zeros((rows.size, d), dtype=np.float64)
    for e in np.unique(expert_of_row):
        sel = np.nonzero(expert_of_row == e)[0]
        slot = int(e) if slot_of_expert is None else int(slot_of_expert[e])
        y[sel] = act[sel] @ dequant(down, slot).T
    return y


def combine(y, inv, w, k: int):
    """Step 6: out[t] = sum_j w[t, j] * y[inv[t*k + j]], summed in j order."""
    y = np.asarray(y, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    inv = np.asarray(inv, dtype=np.int64)
    T = w.shape[0]
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    for j in range(k):
        out += w[:, j:j + 1] * y[inv[j::k]]
    return out


def layer(x_bits, k: int, gate: dict, up: dict, down: dict, *, logits=None,
          w_router=None, bias=None, slot_of_expert=None):
    """The whole layer.  Pass ``logits`` to route on given logits (e.g. the
    GPU's float32 logits, or a given logit tensor); otherwise they are
    computed in float64 from x, W_r and b.

    Returns a dict with logits, ids, w, offsets, perm, inv, act, y, out.
    """
    if logits is None:
        logits = router_logits(x_bits, w_router, bias)
    logits = np.asarray(logits, dtype=np.float64)
    E = logits.shape[1]
    ids, w = route_topk(logits, k)
    offsets, perm, inv = dispatch(ids, E)
    act, y = expert_ffn(x_bits, k, offsets, perm, gate, up, down, slot_of_expert)
    out = combine(y, inv, w, k)
    return dict(logits=logits, ids=ids, w=w, offsets=offsets, perm=perm, inv=inv,
                act=act, y=y, out=out)


# ---------------------------------------------------------------------------
# Shared expert
# ---------------------------------------------------------------------------

def shared_expert(x_bits, gate: dict, up: dict, down: dict):
    """The always-on shared expert of a DeepSeek block (the pages name it only
    through a knob that prefetches its down projection at decode: Anemll/
    ds4-ssd README, section "Experimental Pro Support").  Every token goes
    through slot 0 of the given packs with the routed experts' SwiGLU and
    rounding point:  ys_t = W_d bf16_RNE(silu(W_g x_t) * (W_u x_t)).
    Returns ys float64 [T, d]."""
    x = bf16_bits_to_f64(x_bits)
    wg, wu, wd = dequant(gate, 0), dequant(up, 0), dequant(down, 0)
    act = round_bf16(silu(x @ wg.T) * (x @ wu.T))
    return act @ wd.T


def layer_shared(x_bits, k: int, gate: dict, up: dict, down: dict, shared: dict, **kw):
    """The layer with a shared expert, weight 1, added after the routed
    terms: out[t] = sum_j w[t, j] y[inv[t*k + j]] + ys[t].  `shared` holds
    the shared expert's gate/up/down packs; other arguments as ``layer``."""
    r = layer(x_bits, k, gate, up, down, **kw)
    r["ys"] = shared_expert(x_bits, shared["gate"], shared["up"], shared["down"])
    r["out"] = r["out"] + r["ys"]
    return r


# ---------------------------------------------------------------------------
# MXFP8 activations (the matrix cores' scaled fp4 x fp8 path)
# ---------------------------------------------------------------------------

# OCP Microscaling Formats (MX) v1.0, FP8 E4M3: sign, 4 exponent bits (bias 7),
# 3 mantissa bits; exponent field 0 is subnormal (m/8 * 2**-6); S.1111.111 is
# NaN and there is no infinity, so the largest finite magnitude is
# 1.75 * 2**8 = 448.  A block of 32 elements shares one E8M0 scale.
E4M3_MAX = 448.0
E4M3_EMAX = 8            # exponent of the largest normal


def e4m3_to_f64(codes) -> np.ndarray:
    """Decode E4M3 codes (uint8) to float64; NaN codes decode to NaN."""
    c = np.asarray(codes).astype(np.int64)
    s, e, m = c >> 7, (c >> 3) & 15, c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def _e4m3_table() -> np.ndarray:
    return e4m3_to_f64(np.arange(256))


def round_e4m3(q) -> np.ndarray:
    """Round float64 values to the nearest E4M3 value (ties to even
    mantissa), saturating magnitudes above 448 to 448."""
    q = np.asarray(q, dtype=np.float64)
    a = np.abs(q)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)                      # below 2**-6 the step is the subnormal 2**-9
    step = 2.0 ** (e - 3.0)
    r = np.round(a / step) * step                # numpy rounds half to even
    r = np.minimum(r, E4M3_MAX)
    return np.where(q < 0, -r, r)


def encode_e4m3(v) -> np.ndarray:
    """E4M3 code of values that are exactly representable (and not NaN);
    +0 for zero, the sign bit kept for negative values."""
    v = np.asarray(v, dtype=np.float64)
    table = _e4m3_table()
    pos = table[:127]                            # codes 0..126: the non-negative finite values, increasing
    idx = np.searchsorted(pos, np.abs(v))
    if not np.array_equal(pos[np.minimum(idx, 126)], np.abs(v)):
        raise ValueError("value not representable in E4M3")
    return (idx + np.where(v < 0, 128, 0)).astype(np.uint8)


def quantize_mxfp8(v):
    """Quantise float64 values [..., K] (K a multiple of 32) to MXFP8 along
    the last axis (OCP MX v1.0 conversion): per block of 32, the shared
    scale is 2**(floor(log2(amax)) - 8) (8 = E4M3's largest exponent; E8M0
    byte = that exponent + 127, clamped to 0..254; an all-zero block gets
    byte 0), and each element is v / scale rounded to E4M3 as round_e4m3.
    Returns (codes uint8 [..., K], scale bytes uint8 [..., K/32])."""
    v = np.asarray(v, dtype=np.float64)
    blocks = v.reshape(v.shape[:-1] + (v.shape[-1] // 32, 32))
    amax = np.abs(blocks).max(axis=-1)
    with np.errstate(divide="ignore"):
        ex = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - E4M3_EMAX, -127.0)
    sbyte = np.clip(ex + 127.0, 0, 254)
    scale = 2.0 ** (sbyte - 127.0)
    q = round_e4m3(blocks / scale[..., None])
    return encode_e4m3(q).reshape(v.shape), sbyte.astype(np.uint8)


def mxfp8_to_f64(codes, scale_bytes) -> np.ndarray:
    """Values of MXFP8 data [..., K] with scale bytes [..., K/32]."""
    c = np.asarray(codes)
    vals = e4m3_to_f64(c).reshape(c.shape[:-1] + (c.shape[-1] // 32, 32))
    return (vals * 2.0 ** (np.asarray(scale_bytes, dtype=np.float64) - 127.0)[..., None]).reshape(c.shape)


# ---------------------------------------------------------------------------
# MXFP4 activations (OCP MX v1.0: E2M1 elements, one E8M0 scale per 32)
# ---------------------------------------------------------------------------

E2M1_MAX = 6.0
E2M1_EMAX = 2            # exponent of the largest normal (6 = 1.5 * 2**2)


def round_e2m1(q) -> np.ndarray:
    """Round float64 values to the nearest E2M1 value (ties to the even
    mantissa), saturating magnitudes above 6 to 6.  Below 1 the step is the
    subnormal step 0.5; in [2**e, 2**(e+1)) it is 2**(e-1)."""
    q = np.asarray(q, dtype=np.float64)
    a = np.abs(q)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, 0.0)
    step = 2.0 ** (e - 1.0)
    r = np.round(a / step) * step                # numpy rounds half to even
    r = np.minimum(r, E2M1_MAX)
    return np.where(q < 0, -r, r)


def encode_e2m1(v) -> np.ndarray:
    """E2M1 code (0..15) of values that are exactly representable; +0 for
    zero, the sign bit (8) for negative nonzero values."""
    v = np.asarray(v, dtype=np.float64)
    idx = np.searchsorted(E2M1_MAGNITUDE, np.abs(v))
    if not np.array_equal(E2M1_MAGNITUDE[np.minimum(idx, 7)], np.abs(v)):
        raise ValueError("value not representable in E2M1")
    return (idx + np.where(v < 0, 8, 0)).astype(np.uint8)


def quantize_mxfp4(v):
    """Quantise float64 values [..., K] (K a multiple of 32) to MXFP4 along
    the last axis (OCP MX v1.0 conversion): per block of 32, the shared
    scale is 2**(floor(log2(amax)) - 2) (2 = E2M1's largest exponent; E8M0
    byte = that exponent + 127, clamped to 0..254; an all-zero block gets
    byte 0), and each element is v / scale rounded to E2M1 as round_e2m1.
    Returns (codes uint8 [..., K], one 4-bit code per element, and scale
    bytes uint8 [..., K/32])."""
    v = np.asarray(v, dtype=np.float64)
    blocks = v.reshape(v.shape[:-1] + (v.shape[-1] // 32, 32))
    amax = np.abs(blocks).max(axis=-1)
    with np.errstate(divide="ignore"):
        ex = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - E2M1_EMAX, -127.0)
    sbyte = np.clip(ex + 127.0, 0, 254)
    scale = 2.0 ** (sbyte - 127.0)
    q = round_e2m1(blocks / scale[..., None])
    return encode_e2m1(q).reshape(v.shape), sbyte.astype(np.uint8)


def mxfp4_act_to_f64(codes, scale_bytes) -> np.ndarray:
    """Values of MXFP4 data [..., K] (one code per element) with scale
    bytes [..., K/32]."""
    c = np.asarray(codes)
    vals = e2m1_to_f64(c).reshape(c.shape[:-1] + (c.shape[-1] // 32, 32))
    return (vals * 2.0 ** (np.asarray(scale_bytes, dtype=np.float64) - 127.0)[..., None]).reshape(c.shape)


def _expert_ffn_mx(x_bits, k, offsets, perm, gate, up, down, quantize, decode, slot_of_expert):
    """Steps 4 and 5 with the token rows and the SwiGLU output each
    quantised along their contraction axis by `quantize` (values back by
    `decode`) in place of the bf16 rounding point; products and sums are
    float64.  Returns act float64 [T*k, f] (the quantised values), its codes
    and scale bytes, and y float64 [T*k, d]."""
    xq, xs = quantize(bf16_bits_to_f64(x_bits))
    xv = decode(xq, xs)
    offsets = np.asarray(offsets, dtype=np.int64)
    perm = np.asarray(perm, dtype=np.int64)
    E = offsets.size - 1
    R = perm.size
    f, d = gate["codes"].shape[1], down["codes"].shape[1]
    h = np.zeros((R, f))
    y = np.zeros((R, d))
    wd = {}
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 <= r0:
            continue
        slot = e if slot_of_expert is None else int(slot_of_expert[e])
        xt = xv[perm[r0:r1] // k]
        h[r0:r1] = silu(xt @ dequant(gate, slot).T) * (xt @ dequant(up, slot).T)
        wd[e] = dequant(down, slot)
    aq, asc = quantize(h)
    act = decode(aq, asc)
    for e, w in wd.items():
        r0, r1 = offsets[e], offsets[e + 1]
        y[r0:r1] = act[r0:r1] @ w.T
    return act, aq, asc, y


def expert_ffn_mx8(x_bits, k: int, offsets, perm, gate: dict, up: dict, down: dict, slot_of_expert=None):
    """Steps 4 and 5 with MXFP8 activations (the matrix cores' native scaled
    fp4 x fp8 products): the token rows x_t and the SwiGLU output are each
    quantised to MXFP8 (quantize_mxfp8).  Returns act, its codes, its scale
    bytes and y, as _expert_ffn_mx."""
    return _expert_ffn_mx(x_bits, k, offsets, perm, gate, up, down, quantize_mxfp8, mxfp8_to_f64, slot_of_expert)


def expert_ffn_mx4(x_bits, k: int, offsets, perm, gate: dict, up: dict, down: dict, slot_of_expert=None):
    """Steps 4 and 5 with MXFP4 activations (the matrix cores' native scaled
    fp4 x fp4 products): the token rows x_t and the SwiGLU output are each
    quantised to MXFP4 (quantize_mxfp4).  Returns act, its codes (one per
    element), its scale bytes and y, as _expert_ffn_mx."""
    return _expert_ffn_mx(x_bits, k, offsets, perm, gate, up, down, quantize_mxfp4, mxfp4_act_to_f64,
                          slot_of_expert)


def _layer_mx(ffn, x_bits, k, gate, up, down, logits, w_router, bias):
    if logits is None:
        logits = router_logits(x_bits, w_router, bias)
    logits = np.asarray(logits, dtype=np.float64)
    ids, w = route_topk(logits, k)
    offsets, perm, inv = dispatch(ids, logits.shape[1])
    act, aq, asc, y = ffn(x_bits, k, offsets, perm, gate, up, down)
    out = combine(y, inv, w, k)
    return dict(logits=logits, ids=ids, w=w, offsets=offsets, perm=perm, inv=inv, act=act, act_codes=aq,
                act_scales=asc, y=y, out=out)


def layer_mx8(x_bits, k: int, gate: dict, up: dict, down: dict, *, logits=None, w_router=None, bias=None):
    """The layer with MXFP8 activations in the expert FFN (routing and
    combine as ``layer``)."""
    return _layer_mx(expert_ffn_mx8, x_bits, k, gate, up, down, logits, w_router, bias)


def layer_mx4(x_bits, k: int, gate: dict, up: dict, down: dict, *, logits=None, w_router=None, bias=None):
    """The layer with MXFP4 activations in the expert FFN (routing and
    combine as ``layer``)."""
    return _layer_mx(expert_ffn_mx4, x_bits, k, gate, up, down, logits, w_router, bias)
