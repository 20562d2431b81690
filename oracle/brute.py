"""Scalar pure-Python oracle of the routed MoE layer (test infrastructure only).

A second, deliberately naive implementation used to pin ``oracle.ref`` on tiny
inputs.  It shares no helper with ``oracle.ref``:

* e2m1 is decoded from its bit fields (1 sign, 2 exponent bits with bias 1,
  1 mantissa bit; exponent field 0 is subnormal), per the OCP Microscaling
  Formats (MX) v1.0 specification -- not from a value table;
* bf16 rounding searches the ordered bf16 bit patterns with exact rational
  comparisons (``fractions.Fraction``) and breaks ties to the even pattern;
* top-k tries every k-subset and keeps the one whose members all beat every
  non-member (logit descending, ties to the lower id);
* the dispatch walks the experts in order and collects their pairs;
* every dot product is an explicit loop summed with ``math.fsum`` (exactly
  rounded), so its only rounding is the final one.

Use it on inputs of a few hundred thousand multiply-adds at most.
"""

from __future__ import annotations

import itertools
import math
import struct
from fractions import Fraction


def bf16_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]


def fp16_value(bits: int) -> float:
    return struct.unpack("<e", struct.pack("<H", bits & 0xFFFF))[0]


def e2m1_value(code: int) -> float:
    sign = -1.0 if (code >> 3) & 1 else 1.0
    exp_field = (code >> 1) & 3
    mant = code & 1
    if exp_field == 0:                       # subnormal: 2**(1 - bias) * (m / 2)
        mag = 0.5 * mant
    else:                                    # normal: 2**(e - bias) * (1 + m / 2)
        mag = 2.0 ** (exp_field - 1) * (1.0 + 0.5 * mant)
    return sign * mag


def e8m0_value(byte: int) -> float:
    if byte == 255:
        raise ValueError("e8m0 NaN")
    return 2.0 ** (byte - 127)


def round_bf16(v: float) -> float:
    """Nearest bf16 value to v (exact comparison), ties to the even pattern."""
    if v != v or v in (math.inf, -math.inf):
        return v
    target = Fraction(abs(v))
    # positive finite bf16 patterns 0x0000..0x7F7F increase with their value
    lo, hi = 0, 0x7F7F
    if target >= Fraction(bf16_value(hi)):
        below = hi
    else:
        while hi - lo > 1:                   # invariant: value(lo) <= target < value(hi)
            mid = (lo + hi) // 2
            if Fraction(bf16_value(mid)) <= target:
                lo = mid
            else:
                hi = mid
        below = lo
    a = Fraction(bf16_value(below))
    if below == 0x7F7F:
        # past the largest finite bf16: rounds to inf once at or beyond the
        # midpoint to 2**128 (the next exponent step)
        mid_to_inf = a + (Fraction(2) ** 128 - a) / 2
        if target > mid_to_inf or (target == mid_to_inf):
            return math.copysign(math.inf, v)
        return math.copysign(float(a), v)
    b = Fraction(bf16_value(below + 1))
    da, db = target - a, b - target
    if da < db:
        pick = below
    elif db < da:
        pick = below + 1
    else:
        pick = below if below % 2 == 0 else below + 1
    return math.copysign(bf16_value(pick), v)


def silu(z: float) -> float:
    if z < -700.0:            # exp(-z) overflows: z / inf is -0
        return -0.0
    return z / (1.0 + math.exp(-z))


def dequant_row(mat: dict, slot: int, row: int, K: int) -> list:
    """One dequantised row (length K) of a matrix pack."""
    out = []
    if mat["fmt"] == "mxfp4":
        codes = mat["codes"][slot][row]
        scales = mat["scales"][slot][row]
        for i in range(K):
            byte = int(codes[i // 2])
            code = (byte & 0xF) if i % 2 == 0 else (byte >> 4)
            out.append(e2m1_value(code) * e8m0_value(int(scales[i // 32])))
    elif mat["fmt"] == "q2":
        codes = mat["codes"][slot][row]
        sc = mat["scales"][slot][row]
        mn = mat["mins"][slot][row]
        for i in range(K):
            q = (int(codes[i // 4]) >> (2 * (i % 4))) & 3
            out.append(fp16_value(int(sc[i // 32])) * q + fp16_value(int(mn[i // 32])))
    elif mat["fmt"] == "q4":
        codes = mat["codes"][slot][row]
        sc = mat["scales"][slot][row]
        mn = mat["mins"][slot][row]
        for i in range(K):
            byte = int(codes[i // 2])
            q = (byte & 0xF) if i % 2 == 0 else (byte >> 4)
            out.append(fp16_value(int(sc[i // 32])) * q + fp16_value(int(mn[i // 32])))
    else:
        raise ValueError(mat["fmt"])
    return out


def beats(l, a: int, b: int) -> bool:
    return l[a] > l[b] or (l[a] == l[b] and a < b)


def route_topk(logits, k: int):
    T = len(logits)
    ids, ws = [], []
    for t in range(T):
        l = [float(v) for v in logits[t]]
        E = len(l)
        chosen = None
        for subset in itertools.combinations(range(E), k):
            rest = [e for e in range(E) if e not in subset]
            if all(beats(l, a, b) for a in subset for b in rest):
                chosen = subset
                break
        # order the chosen set: count how many members each one beats
        order = sorted(chosen, key=lambda a: -sum(beats(l, a, b) for b in chosen))
        m = max(l[e] for e in order)
        ex = [math.exp(l[e] - m) for e in order]
        s = math.fsum(ex)
        ids.append(list(order))
        ws.append([v / s for v in ex])
    return ids, ws


def dispatch(ids, E: int):
    flat = [e for row in ids for e in row]
    perm = []
    offsets = [0]
    for e in range(E):
        for p, ep in enumerate(flat):
            if ep == e:
                perm.append(p)
        offsets.append(len(perm))
    inv = [0] * len(flat)
    for r, p in enumerate(perm):
        inv[p] = r
    return offsets, perm, inv


def layer(x_bits, k: int, gate: dict, up: dict, down: dict, *, logits=None,
          w_router=None, bias=None):
    """Whole layer, scalar.  Returns a dict of Python lists."""
    T = len(x_bits)
    d = len(x_bits[0])
    x = [[bf16_value(int(b)) for b in row] for row in x_bits]
    if logits is None:
        E = len(w_router)
        logits = []
        for t in range(T):
            row = []
            for e in range(E):
                s = math.fsum(x[t][i] * float(w_router[e][i]) for i in range(d))
                if bias is not None:
                    s = math.fsum([s, float(bias[e])])
                row.append(s)
            logits.append(row)
    E = len(logits[0])
    ids, ws = route_topk(logits, k)
    offsets, perm, inv = dispatch(ids, E)
    f = len(gate["codes"][0])
    act, y = [], []
    cache = {}
    for e in range(E):
        for r in range(offsets[e], offsets[e + 1]):
            if e not in cache:
                cache[e] = (
                    [dequant_row(gate, e, n, d) for n in range(f)],
                    [dequant_row(up, e, n, d) for n in range(f)],
                    [dequant_row(down, e, n, f) for n in range(d)],
                )
            wg, wu, wd = cache[e]
            xt = x[perm[r] // k]
            a_row = []
            for n in range(f):
                g = math.fsum(wg[n][i] * xt[i] for i in range(d))
                u = math.fsum(wu[n][i] * xt[i] for i in range(d))
                a_row.append(round_bf16(silu(g) * u))
            act.append(a_row)
            y.append([math.fsum(wd[n][i] * a_row[i] for i in range(f)) for n in range(d)])
    out = []
    for t in range(T):
        out.append([math.fsum(ws[t][j] * y[inv[t * k + j]][n] for j in range(k))
                    for n in range(d)])
    return dict(logits=logits, ids=ids, w=ws, offsets=offsets, perm=perm, inv=inv,
                act=act, y=y, out=out)
