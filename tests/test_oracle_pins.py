"""Pins of the CPU oracle against facts that do not come from the oracle itself:
the published e2m1/e8m0 encodings (golden fixtures), hand-decoded packs,
closed forms, library routines (torch, numpy), brute force on tiny inputs and
exact invariants.  CPU only."""

import itertools
import math
import os

import numpy as np
import pytest
import torch

import synthetic
from oracle import brute, ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_fixture(name):
    rows = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            rows.setdefault(key, []).extend(vals)
    return rows


# ----------------------------------------------------------------- formats

def test_e2m1_table_matches_published_encoding():
    codes, values = [], []
    with open(os.path.join(GOLDEN, "e2m1.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                c, bits, v = line.split()
                assert int(bits, 2) == int(c)
                codes.append(int(c))
                values.append(float(v))
    assert codes == list(range(16))
    got = ref.e2m1_to_f64(np.arange(16, dtype=np.uint8))
    for c in range(16):
        assert got[c] == values[c] and math.copysign(1, got[c]) == math.copysign(1, values[c])
        b = brute.e2m1_value(c)      # bit-field decode, independent of the table
        assert b == values[c] and math.copysign(1, b) == math.copysign(1, values[c])


def test_e8m0_closed_form():
    b = np.array([0, 1, 119, 123, 126, 127, 128, 254], dtype=np.uint8)
    assert list(ref.e8m0_to_f64(b)) == [2.0 ** (int(v) - 127) for v in b]
    assert ref.e8m0_to_f64(np.array([127], np.uint8))[0] == 1.0
    with pytest.raises(ValueError):
        ref.e8m0_to_f64(np.array([255], np.uint8))


def test_mxfp4_hand_decoded_row():
    fx = _read_fixture("mxfp4_row.txt")
    codes = np.array([int(v, 16) for v in fx["bytes"]], np.uint8)[None, :]
    scales = np.array([int(v) for v in fx["scales"]], np.uint8)[None, :]
    want = np.array([float(v) for v in fx["values"]])
    got = ref.dequant_mxfp4(codes, scales)[0]
    assert got.shape == want.shape == (64,)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))          # code 8 is -0
    mat = dict(fmt="mxfp4", codes=codes[None], scales=scales[None])
    assert brute.dequant_row(mat, 0, 0, 64) == list(want)


def test_q2_hand_decoded_row():
    fx = _read_fixture("q2_row.txt")
    codes = np.array([int(v, 16) for v in fx["bytes"]], np.uint8)[None, :]
    sc = np.array([int(v, 16) for v in fx["scales"]], np.uint16)[None, :]
    mn = np.array([int(v, 16) for v in fx["mins"]], np.uint16)[None, :]
    want = np.array([float(v) for v in fx["values"]])
    got = ref.dequant_q2(codes, sc, mn)[0]
    assert np.array_equal(got, want)
    mat = dict(fmt="q2", codes=codes[None], scales=sc[None], mins=mn[None])
    assert brute.dequant_row(mat, 0, 0, 64) == list(want)


def test_q4_hand_decoded_row():
    fx = _read_fixture("q4_row.txt")
    codes = np.array([int(v, 16) for v in fx["bytes"]], np.uint8)[None, :]
    sc = np.array([int(v, 16) for v in fx["scales"]], np.uint16)[None, :]
    mn = np.array([int(v, 16) for v in fx["mins"]], np.uint16)[None, :]
    want = np.array([float(v) for v in fx["values"]])
    got = ref.dequant_q4(codes, sc, mn)[0]
    assert got.shape == want.shape == (64,)
    assert np.array_equal(got, want)
    mat = dict(fmt="q4", codes=codes[None], scales=sc[None], mins=mn[None])
    assert brute.dequant_row(mat, 0, 0, 64) == list(want)


def test_mxfp4_values_exact_in_bf16():
    """Every e2m1 code times a scale 2**-8..2**-4 is a bf16 value, so MXFP4
    weights can be widened to bf16 for matrix cores with no rounding."""
    for s in range(119, 124):
        for c in range(16):
            v = brute.e2m1_value(c) * 2.0 ** (s - 127)
            assert brute.round_bf16(v) == v


def test_q2_values_exact_in_fp32():
    """scale*q + min of fp16 scale/min is exact in float32 for the workload's
    ranges, so a float32 dequantisation with one FMA loses nothing."""
    rng = np.random.default_rng(7)
    sc = rng.uniform(0.005, 0.02, 20000).astype(np.float16).astype(np.float64)
    mn = rng.uniform(-0.04, 0.0, 20000).astype(np.float16).astype(np.float64)
    for q in range(4):
        w = sc * q + mn
        assert np.array_equal(w.astype(np.float32).astype(np.float64), w)


def test_q4_values_exact_in_fp32():
    """scale*q + min of fp16 scale/min is exact in float32 for q = 0..15 and
    the generator's ranges (an fp16 significand times a 4-bit integer needs
    15 bits), so the device's float32 group sums lose nothing to the format."""
    rng = np.random.default_rng(8)
    sc = rng.uniform(0.001, 0.004, 20000).astype(np.float16).astype(np.float64)
    mn = rng.uniform(-0.04, 0.0, 20000).astype(np.float16).astype(np.float64)
    for q in range(16):
        w = sc * q + mn
        assert np.array_equal(w.astype(np.float32).astype(np.float64), w)


def test_q4_one_plus_q_over_16_exact_in_bf16():
    """1 + q/16 (q = 0..15) is a bf16 value with the bit pattern 0x3F80 | q << 3:
    the device multiplies bf16(1 + q/16) operands and applies scale and min
    per group, so this pins that the operand carries q exactly."""
    for q in range(16):
        v = 1.0 + q / 16.0
        assert brute.round_bf16(v) == v
        assert brute.bf16_value(0x3F80 | (q << 3)) == v


# ------------------------------------------------------------ bf16 rounding

def test_round_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(3)
    v = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
        # exact ties between two bf16 neighbours (low 16 bits = 0x8000)
        ((rng.integers(0, 2 ** 31, 4000, dtype=np.uint64) & ~np.uint64(0xFFFF)) | np.uint64(0x8000))
        .astype(np.uint32).view(np.float32).astype(np.float64),
        np.array([0.0, -0.0, 1e-40, -1e-40, 1e-45, 3.3e38, -3.39e38]),
    ]).astype(np.float32)
    v = v[np.isfinite(v)]
    want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = ref.round_bf16(v.astype(np.float64))
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_round_bf16_direct_from_float64():
    # no double rounding: 1 + 2**-8 + 2**-30 is just above the tie -> rounds up
    assert ref.round_bf16(np.array([1.0 + 2.0 ** -8 + 2.0 ** -30]))[0] == 1.0 + 2.0 ** -7
    assert ref.round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0              # tie -> even
    assert ref.round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6  # tie -> even (up)
    assert ref.round_bf16(np.array([3.4e38]))[0] == math.inf
    # against the independent rational search on random float64 values
    rng = np.random.default_rng(5)
    v = rng.standard_normal(3000) * 10.0 ** rng.integers(-40, 38, 3000)
    got = ref.round_bf16(v)
    for a, b in zip(v, got):
        assert brute.round_bf16(float(a)) == b


# ------------------------------------------------------------------ routing

def test_router_logits_closed_form():
    T, d, E = 3, 64, 5
    x = synthetic.to_bf16_bits(np.random.default_rng(1).standard_normal((T, d)).astype(np.float32))
    xv = np.array([[brute.bf16_value(int(b)) for b in row] for row in x])
    wr = np.zeros((E, d), np.float32)
    for e in range(E):
        wr[e, 3 * e] = 1.0                # one-hot rows pick x[:, 3e]
        wr[e, 3 * e + 1] = -2.0
    bias = np.arange(E, dtype=np.float32) * 0.25
    got = ref.router_logits(x, wr, bias)
    want = xv[:, 0:3 * E:3] - 2.0 * xv[:, 1:3 * E + 1:3] + bias[None, :]
    assert np.array_equal(got, want)


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(11)
    for trial in range(60):
        E = 8
        l = rng.integers(-3, 4, size=(3, E)).astype(np.float64) * 0.5   # many exact ties
        if trial % 7 == 0:
            l[:] = 0.0
            l[0, 2] = -0.0
        for k in (1, 2, 3, 8):
            ids, w = ref.route_topk(l, k)
            bids, bw = brute.route_topk(l, k)
            assert ids.tolist() == bids
            assert np.allclose(w, bw, rtol=0, atol=1e-15)


def test_topk_tie_rules():
    l = np.array([[1.0, 2.0, 2.0, 0.5], [0.0, -0.0, 0.0, -1.0]])
    ids, _ = ref.route_topk(l, 2)
    assert ids.tolist() == [[1, 2], [0, 1]]
    with pytest.raises(ValueError):
        ref.route_topk(np.array([[0.0, np.nan]]), 1)


def test_topk_weights_sum_to_one_and_full_softmax():
    rng = np.random.default_rng(12)
    l = rng.standard_normal((50, 16)) * 3
    for k in (1, 2, 5):
        _, w = ref.route_topk(l, k)
        assert np.all(np.abs(w.sum(1) - 1.0) < 1e-15)
    ids, w = ref.route_topk(l, 16)                 # k = E: plain softmax
    sm = torch.softmax(torch.from_numpy(l), dim=1).numpy()
    assert np.allclose(np.take_along_axis(sm, ids.astype(np.int64), 1), w, rtol=1e-14, atol=0)


# ----------------------------------------------------------------- dispatch

def test_dispatch_against_brute_and_invariants():
    rng = np.random.default_rng(13)
    for T, E, k in [(1, 64, 2), (7, 8, 2), (33, 16, 3), (100, 5, 1), (0, 4, 2)]:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]) if T else np.zeros((0, k), np.int32)
        off, perm, inv = ref.dispatch(ids, E)
        boff, bperm, binv = brute.dispatch(ids.tolist(), E)
        assert off.tolist() == boff and perm.tolist() == bperm and inv.tolist() == binv
        assert off[0] == 0 and off[-1] == T * k and np.all(np.diff(off) >= 0)
        assert sorted(perm.tolist()) == list(range(T * k))
        assert np.array_equal(inv[perm], np.arange(T * k))
        flat = ids.reshape(-1)
        for e in range(E):
            seg = perm[off[e]:off[e + 1]]
            assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)   # stable


# ---------------------------------------------------------------------- FFN

def _small_case(fmt, T=3, d=64, E=4, k=2, f=32, seed=0, **kw):
    return synthetic.make_case(T, d, E, k, f, fmt, seed=seed, router="device", **kw)


def _dense_weights_brute(mat, slot, n, K):
    return np.array([brute.dequant_row(mat, slot, r, K) for r in range(n)])


@pytest.mark.parametrize("fmt", ["mxfp4", "q2", "q4"])
def test_single_expert_is_dense_swiglu(fmt):
    """E = 1, k = 1: the layer is a dense SwiGLU MLP (torch float64)."""
    c = _small_case(fmt, T=5, d=64, E=1, k=1, f=32, seed=4)
    r = ref.layer(c["x"], 1, c["gate"], c["up"], c["down"], w_router=c["w_router"])
    x = torch.tensor([[brute.bf16_value(int(b)) for b in row] for row in c["x"]], dtype=torch.float64)
    wg = torch.from_numpy(_dense_weights_brute(c["gate"], 0, 32, 64))
    wu = torch.from_numpy(_dense_weights_brute(c["up"], 0, 32, 64))
    wd = torch.from_numpy(_dense_weights_brute(c["down"], 0, 64, 32))
    h = torch.nn.functional.silu(x @ wg.T) * (x @ wu.T)
    act = torch.tensor([[brute.round_bf16(float(v)) for v in row] for row in h], dtype=torch.float64)
    out = act @ wd.T
    assert np.allclose(r["out"], out.numpy(), rtol=1e-12, atol=1e-12)
    assert np.array_equal(r["w"], np.ones((5, 1)))


def test_identity_experts_closed_form():
    """Hand-built weights: gate = I, up = 2I, down = cyclic shift.  Then
    out[t, n] = bf16(silu(x[t, n+1]) * 2 x[t, n+1]) (indices mod 32)."""
    d = f = 32
    E, k, T = 2, 1, 3
    def eye_pack(code):
        codes = np.zeros((E, d, d // 2), np.uint8)
        for n in range(d):
            codes[:, n, n // 2] |= code << (4 * (n % 2))
        return dict(fmt="mxfp4", codes=codes, scales=np.full((E, d, 1), 127, np.uint8))
    gate, up = eye_pack(2), eye_pack(4)           # e2m1 code 2 = 1.0, code 4 = 2.0
    down = dict(fmt="mxfp4", codes=np.zeros((E, d, f // 2), np.uint8),
                scales=np.full((E, d, 1), 127, np.uint8))
    for n in range(d):
        kk = (n + 1) % f
        down["codes"][:, n, kk // 2] |= 2 << (4 * (kk % 2))
    xv = np.array([[(i - 16) / 8.0 + 0.125 * t for i in range(d)] for t in range(T)], np.float32)
    x = synthetic.to_bf16_bits(xv)
    logits = np.array([[1.0, 0.0], [0.0, 1.0], [2.0, 2.0]], np.float32)
    r = ref.layer(x, k, gate, up, down, logits=logits)
    for t in range(T):
        for n in range(d):
            xi = float(xv[t, (n + 1) % d])
            want = brute.round_bf16(xi / (1 + math.exp(-xi)) * 2 * xi)
            assert r["out"][t, n] == want


@pytest.mark.parametrize("fmt", ["mxfp4", "q2", "q4"])
def test_ref_matches_brute_small(fmt):
    for seed, (T, d, E, k, f) in enumerate([(3, 64, 4, 2, 32), (6, 32, 8, 3, 64), (2, 96, 3, 3, 32)]):
        c = _small_case(fmt, T=T, d=d, E=E, k=k, f=f, seed=seed, zipf=1.1 if seed == 1 else None)
        r = ref.layer(c["x"], k, c["gate"], c["up"], c["down"], w_router=c["w_router"], bias=c["bias"])
        b = brute.layer(c["x"], k, c["gate"], c["up"], c["down"], w_router=c["w_router"], bias=c["bias"])
        assert np.allclose(r["logits"], b["logits"], rtol=0, atol=1e-14)
        assert r["ids"].tolist() == b["ids"]
        assert r["perm"].tolist() == b["perm"] and r["offsets"].tolist() == b["offsets"]
        assert np.array_equal(r["act"], np.array(b["act"]))
        scale = np.abs(np.array(b["out"])).max()
        assert np.allclose(r["out"], b["out"], rtol=0, atol=1e-12 * scale)


def test_ref_matches_brute_tiny_workload():
    c = synthetic.workload(0)
    r = ref.layer(c["x"], c["k"], c["gate"], c["up"], c["down"], logits=c["logits"])
    b = brute.layer(c["x"], c["k"], c["gate"], c["up"], c["down"], logits=c["logits"])
    assert r["ids"].tolist() == b["ids"] and r["perm"].tolist() == b["perm"]
    assert np.array_equal(r["act"], np.array(b["act"]))
    assert np.allclose(r["out"], b["out"], rtol=0, atol=1e-12 * np.abs(r["out"]).max())


def test_k_equals_E_is_softmax_mixture():
    c = _small_case("mxfp4", T=4, d=64, E=3, k=3, f=32, seed=9)
    r = ref.layer(c["x"], 3, c["gate"], c["up"], c["down"], w_router=c["w_router"])
    x = torch.tensor([[brute.bf16_value(int(b)) for b in row] for row in c["x"]], dtype=torch.float64)
    p = torch.softmax(x @ torch.from_numpy(c["w_router"].astype(np.float64)).T, dim=1)
    mix = torch.zeros((4, 64), dtype=torch.float64)
    for e in range(3):
        wg = torch.from_numpy(_dense_weights_brute(c["gate"], e, 32, 64))
        wu = torch.from_numpy(_dense_weights_brute(c["up"], e, 32, 64))
        wd = torch.from_numpy(_dense_weights_brute(c["down"], e, 64, 32))
        h = torch.nn.functional.silu(x @ wg.T) * (x @ wu.T)
        act = torch.tensor([[brute.round_bf16(float(v)) for v in row] for row in h], dtype=torch.float64)
        mix += p[:, e:e + 1] * (act @ wd.T)
    assert np.allclose(r["out"], mix.numpy(), rtol=1e-12, atol=1e-12 * float(mix.abs().max()))


def test_token_permutation_invariance():
    c = _small_case("mxfp4", T=9, d=64, E=6, k=2, f=32, seed=21)
    r = ref.layer(c["x"], 2, c["gate"], c["up"], c["down"], w_router=c["w_router"])
    pi = np.random.default_rng(0).permutation(9)
    r2 = ref.layer(c["x"][pi], 2, c["gate"], c["up"], c["down"], w_router=c["w_router"])
    assert np.array_equal(r2["ids"], r["ids"][pi])
    assert np.allclose(r2["out"], r["out"][pi], rtol=0, atol=1e-13 * np.abs(r["out"]).max())


def test_power_of_two_scale_invariance():
    c = _small_case("mxfp4", T=4, d=64, E=4, k=2, f=32, seed=22)
    base = ref.layer(c["x"], 2, c["gate"], c["up"], c["down"], w_router=c["w_router"])["out"]
    for which in ("up", "down"):
        m = dict(c[which])
        m["scales"] = m["scales"] + np.uint8(1)
        mats = {"gate": c["gate"], "up": c["up"], "down": c["down"], which: m}
        out = ref.layer(c["x"], 2, mats["gate"], mats["up"], mats["down"], w_router=c["w_router"])["out"]
        assert np.array_equal(out, 2.0 * base)
    q = _small_case("q2", T=4, d=64, E=4, k=2, f=32, seed=23)
    base = ref.layer(q["x"], 2, q["gate"], q["up"], q["down"], w_router=q["w_router"])["out"]
    m = dict(q["down"])
    # x2 in binary16 is exact (normal and subnormal values alike)
    m["scales"] = (m["scales"].view(np.float16) * np.float16(2)).view(np.uint16)
    m["mins"] = (m["mins"].view(np.float16) * np.float16(2)).view(np.uint16)
    out = ref.layer(q["x"], 2, q["gate"], q["up"], m, w_router=q["w_router"])["out"]
    assert np.array_equal(out, 2.0 * base)


def test_combine_order_and_weights():
    y = np.arange(12, dtype=np.float64).reshape(6, 2)
    inv = np.array([5, 0, 1, 4, 2, 3])
    w = np.array([[0.25, 0.75], [0.5, 0.5], [1.0, 0.0]])
    out = ref.combine(y, inv, w, 2)
    want = np.array([0.25 * y[5] + 0.75 * y[0], 0.5 * y[1] + 0.5 * y[4], y[2]])
    assert np.array_equal(out, want)


# ---------------------------------------------------------------- shared expert

@pytest.mark.parametrize("fmt", ["mxfp4", "q2", "q4"])
def test_shared_expert_is_dense_swiglu(fmt):
    """The shared expert is a dense SwiGLU MLP over every token (torch
    float64 on the scalar twin's dequantised rows and bf16 rounding)."""
    c = _small_case(fmt, T=6, d=64, E=4, k=2, f=32, seed=12)
    sh = synthetic.make_shared(c, seed=3)
    ys = ref.shared_expert(c["x"], sh["gate"], sh["up"], sh["down"])
    x = torch.tensor([[brute.bf16_value(int(b)) for b in row] for row in c["x"]], dtype=torch.float64)
    wg = torch.from_numpy(_dense_weights_brute(sh["gate"], 0, 32, 64))
    wu = torch.from_numpy(_dense_weights_brute(sh["up"], 0, 32, 64))
    wd = torch.from_numpy(_dense_weights_brute(sh["down"], 0, 64, 32))
    h = torch.nn.functional.silu(x @ wg.T) * (x @ wu.T)
    act = torch.tensor([[brute.round_bf16(float(v)) for v in row] for row in h], dtype=torch.float64)
    assert np.allclose(ys, (act @ wd.T).numpy(), rtol=1e-12, atol=1e-12)


def test_shared_expert_with_zero_down_adds_nothing():
    """All-zero MXFP4 down codes make the shared expert's output exactly 0,
    so the layer with it equals the layer without it."""
    c = _small_case("mxfp4", T=5, d=64, E=4, k=2, f=32, seed=13)
    sh = synthetic.make_shared(c, seed=4)
    sh["down"] = dict(sh["down"], codes=np.zeros_like(sh["down"]["codes"]))
    a = ref.layer(c["x"], 2, c["gate"], c["up"], c["down"], w_router=c["w_router"])
    b = ref.layer_shared(c["x"], 2, c["gate"], c["up"], c["down"], sh, w_router=c["w_router"])
    assert np.array_equal(a["out"], b["out"]) and not np.any(b["ys"])


def test_shared_expert_is_one_more_routed_slot():
    """With weight 1 the shared expert is the same as routing every token to
    one extra expert: the oracle layer over E + 1 experts with k + 1 slots
    whose last slot is that expert with weight 1 (built by hand here)."""
    c = _small_case("q4", T=4, d=64, E=3, k=1, f=32, seed=14)
    sh = synthetic.make_shared(c, seed=5)
    r = ref.layer_shared(c["x"], 1, c["gate"], c["up"], c["down"], sh, w_router=c["w_router"])
    ids = np.concatenate([r["ids"], np.full((4, 1), 3)], axis=1)
    w = np.concatenate([r["w"], np.ones((4, 1))], axis=1)
    packs = {m: {n: np.concatenate([c[m][n], sh[m][n]]) if n != "fmt" else "q4" for n in c[m]}
             for m in ("gate", "up", "down")}
    offsets, perm, inv = ref.dispatch(ids, 4)
    _, y = ref.expert_ffn(c["x"], 2, offsets, perm, packs["gate"], packs["up"], packs["down"])
    out = ref.combine(y, inv, w, 2)
    assert np.allclose(r["out"], out, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------- MXFP8 activations

def test_e4m3_decode_against_spec_and_torch():
    """E4M3 (OCP MX v1.0 FP8): largest normal 448 (0x7E), smallest normal
    2**-6 (0x08), smallest subnormal 2**-9 (0x01), 1.0 = 0x38, NaN at
    S.1111.111; every finite code equals torch's float8_e4m3fn decoding."""
    t = ref.e4m3_to_f64(np.arange(256))
    assert t[0x7E] == 448.0 and t[0x08] == 2.0 ** -6 and t[0x01] == 2.0 ** -9 and t[0x38] == 1.0
    assert t[0xFE] == -448.0 and np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    tt = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    fin = ~np.isnan(t)
    assert np.array_equal(np.isnan(tt), ~fin)
    assert np.array_equal(t[fin], tt[fin])


def test_e4m3_rounding_against_torch():
    """round_e4m3 is round-to-nearest-even with saturation: equal to torch's
    float8_e4m3fn cast of the value clamped to [-448, 448], on random values
    over the whole range and on every midpoint between neighbours."""
    rng = np.random.default_rng(21)
    v = (rng.standard_normal(20000) * 2.0 ** rng.integers(-12, 10, 20000)).astype(np.float32).astype(np.float64)
    pos = np.unique(np.abs(ref.e4m3_to_f64(np.arange(127))))
    mids = (pos[1:] + pos[:-1]) / 2
    v = np.concatenate([v, mids, -mids, [500.0, -1e6, 0.0]])
    want = torch.from_numpy(np.clip(v, -448.0, 448.0)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(ref.round_e4m3(v), want)


def test_mxfp8_quantizer_rules():
    rng = np.random.default_rng(22)
    v = rng.standard_normal((5, 128)) * 2.0 ** rng.integers(-20, 20, (5, 1))
    v[2, 32:64] = 0.0
    codes, sb = ref.quantize_mxfp8(v)
    vals = ref.mxfp8_to_f64(codes, sb)
    blocks = np.abs(v).reshape(5, 4, 32).max(axis=-1)
    scale = 2.0 ** (sb.astype(np.float64) - 127)
    nz = blocks > 0
    # the block maximum lands in [2**8, 2**9) before rounding
    assert np.all((blocks[nz] / scale[nz] >= 256) & (blocks[nz] / scale[nz] < 512))
    assert sb[2, 1] == 0 and not np.any(vals[2, 32:64])
    # within half an E4M3 step (relative 2**-4) of the input where no
    # saturation applies (scaled magnitude <= 448); above it, exactly 448
    err = np.abs(vals - v) / np.maximum(np.abs(v), 1e-300)
    scaled = np.abs(v) / scale.repeat(32, axis=1)
    normal = (scaled >= 2.0 ** -6) & (scaled <= 448)
    assert np.all(err[normal] <= 2.0 ** -4 + 1e-15)
    assert np.all(np.abs(vals[scaled > 464]) == 448 * scale.repeat(32, axis=1)[scaled > 464])
    c2, s2 = ref.quantize_mxfp8(vals)
    assert np.array_equal(c2, codes) and np.array_equal(s2, sb)


def test_mx8_single_expert_is_dense_swiglu_with_fp8_casts():
    """E = 1, k = 1 with MXFP8 activations: a dense SwiGLU MLP in torch
    float64 where both activations go through torch's float8_e4m3fn cast
    with the block scale of the largest magnitude (an independent route to
    the same quantisation)."""
    c = _small_case("mxfp4", T=5, d=64, E=1, k=1, f=32, seed=23)
    r = ref.layer_mx8(c["x"], 1, c["gate"], c["up"], c["down"], w_router=c["w_router"])

    def mx8(t):
        b = t.reshape(t.shape[0], -1, 32)
        amax = b.abs().amax(dim=-1, keepdim=True)
        sc = torch.exp2(torch.floor(torch.log2(amax)) - 8)
        q = torch.clamp(b / sc, -448, 448).to(torch.float8_e4m3fn).to(torch.float64)
        return (q * sc).reshape(t.shape)

    x = torch.tensor([[brute.bf16_value(int(b)) for b in row] for row in c["x"]], dtype=torch.float64)
    wg = torch.from_numpy(_dense_weights_brute(c["gate"], 0, 32, 64))
    wu = torch.from_numpy(_dense_weights_brute(c["up"], 0, 32, 64))
    wd = torch.from_numpy(_dense_weights_brute(c["down"], 0, 64, 32))
    xq = mx8(x)
    act = mx8(torch.nn.functional.silu(xq @ wg.T) * (xq @ wu.T))
    assert np.allclose(r["out"], (act @ wd.T).numpy(), rtol=1e-12, atol=1e-12)


def test_mx8_layer_close_to_bf16_layer():
    """MXFP8 activations move out by about their rounding (relative 2**-5
    per element on average), no more: a dropped scale or transposed
    operand would not stay within a few per cent of the bf16 layer."""
    c = _small_case("mxfp4", T=12, d=256, E=8, k=2, f=128, seed=24)
    a = ref.layer(c["x"], 2, c["gate"], c["up"], c["down"], w_router=c["w_router"])
    b = ref.layer_mx8(c["x"], 2, c["gate"], c["up"], c["down"], w_router=c["w_router"])
    assert np.array_equal(a["ids"], b["ids"])
    rel = np.linalg.norm(b["out"] - a["out"]) / np.linalg.norm(a["out"])
    assert 1e-3 < rel < 0.05, rel


# ---------------------------------------------- helpers that judge GPU results

@pytest.mark.parametrize("fmt", ["mxfp4", "q2", "q4"])
def test_expert_down_equals_expert_ffn_given_its_act(fmt):
    """ref.expert_down judges the device's down projection from the device's
    own act.  Given the oracle's act it must return the oracle's y, on every
    row and on any subset of rows, with the slot map applied (a permuted map
    over more slots than experts)."""
    T, d, E, k, f = 11, 96, 6, 3, 64
    c = synthetic.make_case(T, d, E, k, f, fmt, seed=31, slots=9, zipf=1.1)
    soe = np.array([8, 2, 5, 0, 7, 3], np.int32)
    r = ref.layer(c["x"], k, c["gate"], c["up"], c["down"], w_router=c["w_router"], bias=c["bias"],
                  slot_of_expert=soe)
    y_all = ref.expert_down(r["act"], r["offsets"], c["down"], slot_of_expert=soe)
    assert np.allclose(y_all, r["y"], rtol=0, atol=1e-13 * np.abs(r["y"]).max())
    rows = np.array([0, 4, 5, 17, T * k - 1])
    y_sub = ref.expert_down(r["act"][rows], r["offsets"], c["down"], rows=rows, slot_of_expert=soe)
    assert np.allclose(y_sub, r["y"][rows], rtol=0, atol=1e-13 * np.abs(r["y"]).max())
    # against the scalar twin: explicit fsum dot products over its own dequantised rows
    e_of = np.searchsorted(r["offsets"], rows, side="right") - 1
    for i, (row, e) in enumerate(zip(rows, e_of)):
        for m in (0, 37, d - 1):
            wrow = brute.dequant_row(c["down"], int(soe[e]), m, f)
            want = math.fsum(float(a) * w for a, w in zip(r["act"][row], wrow))
            assert abs(y_sub[i, m] - want) <= 1e-13 * max(1.0, abs(want))


def test_expert_down_uses_the_given_act_not_its_own():
    """One flipped act element moves y by exactly that difference times the
    weight column (a dropped or transposed operand fails this)."""
    c = synthetic.make_case(4, 64, 3, 2, 32, "mxfp4", seed=32)
    r = ref.layer(c["x"], 2, c["gate"], c["up"], c["down"], w_router=c["w_router"])
    act = r["act"].copy()
    act[3, 7] += 0.25
    y = ref.expert_down(act, r["offsets"], c["down"])
    e = int(np.searchsorted(r["offsets"], 3, side="right") - 1)
    col = np.array([brute.dequant_row(c["down"], e, m, 32)[7] for m in range(64)])
    assert np.allclose(y[3] - r["y"][3], 0.25 * col, rtol=0, atol=1e-13)
    assert np.array_equal(np.delete(y, 3, axis=0), np.delete(r["y"], 3, axis=0))


@pytest.mark.parametrize("fmt", ["mxfp4", "q2", "q4"])
def test_expert_ffn_rows_equals_expert_ffn(fmt):
    """ref.expert_ffn_rows judges sampled rows of large calls: on any subset
    of sorted rows (spanning several experts, in any order) it must equal
    ref.expert_ffn on those rows, with a non-identity slot map."""
    T, d, E, k, f = 13, 128, 7, 2, 64
    c = synthetic.make_case(T, d, E, k, f, fmt, seed=33, slots=10, zipf=1.1)
    soe = np.array([9, 0, 4, 1, 8, 2, 6], np.int32)
    r = ref.layer(c["x"], k, c["gate"], c["up"], c["down"], w_router=c["w_router"], bias=c["bias"],
                  slot_of_expert=soe)
    for rows in (np.arange(T * k), np.array([1, 2, 3, 10, 20, 25]), np.array([25, 0, 14, 3]), np.array([T * k - 1])):
        act, y = ref.expert_ffn_rows(c["x"], k, r["offsets"], r["perm"], rows, c["gate"], c["up"], c["down"],
                                     slot_of_expert=soe)
        assert np.array_equal(act, r["act"][rows])
        assert np.allclose(y, r["y"][rows], rtol=0, atol=1e-13 * np.abs(r["y"]).max())
    # the slot map matters: identity slots give different rows
    act_id, _ = ref.expert_ffn_rows(c["x"], k, r["offsets"], r["perm"], np.arange(T * k), c["gate"], c["up"],
                                    c["down"])
    assert not np.array_equal(act_id, r["act"])


# ------------------------------------------------- MXFP4 activations

def _e2m1_nearest_brute(v):
    """Nearest E2M1 value by search over the 8 magnitudes, written out:
    the closest magnitude, a tie going to the even code (even mantissa),
    magnitudes above 6 clamped to 6; the sign kept, zero made +0."""
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    a = min(abs(v), 6.0)
    best = 0
    for c in range(8):
        dc, db = abs(mags[c] - a), abs(mags[best] - a)
        if dc < db or (dc == db and c % 2 == 0 and best % 2 == 1):
            best = c
    m = mags[best]
    return -m if (v < 0 and m > 0) else m


def test_e2m1_rounding_against_search():
    """round_e2m1 (step arithmetic) against a search over the E2M1 values
    with the tie rule spelled out, on random values, every midpoint and
    values around the clamp."""
    rng = np.random.default_rng(41)
    v = rng.standard_normal(20000) * 2.0 ** rng.integers(-3, 4, 20000)
    mags = ref.E2M1_MAGNITUDE
    mids = (mags[1:] + mags[:-1]) / 2
    v = np.concatenate([v, mids, -mids, mids + 1e-9, mids - 1e-9, [5.99, 6.0, 6.5, 7.0, 7.01, 1e9, -1e9, 0.0]])
    got = ref.round_e2m1(v)
    want = np.array([_e2m1_nearest_brute(float(t)) for t in v])
    assert np.array_equal(got, want)


def test_mxfp4_act_hand_worked_block():
    fx = _read_fixture("mxfp4_act_block.txt")
    va = np.array([float(t) for t in fx["values_a"]])
    ca = np.array([int(t) for t in fx["codes_a"]], np.uint8)
    assert va.size == 32 and ca.size == 32
    v = np.stack([va, va * 2.0 ** -20])
    codes, sb = ref.quantize_mxfp4(v)
    assert sb[0, 0] == int(fx["scale_a"][0]) and sb[1, 0] == int(fx["scale_b"][0])
    assert np.array_equal(codes[0], ca) and np.array_equal(codes[1], ca)
    vals = ref.mxfp4_act_to_f64(codes, sb)
    assert np.array_equal(vals[1], vals[0] * 2.0 ** -20)


def test_mxfp4_act_quantizer_rules():
    rng = np.random.default_rng(42)
    v = rng.standard_normal((5, 128)) * 2.0 ** rng.integers(-20, 20, (5, 1))
    v[2, 32:64] = 0.0
    codes, sb = ref.quantize_mxfp4(v)
    vals = ref.mxfp4_act_to_f64(codes, sb)
    blocks = np.abs(v).reshape(5, 4, 32).max(axis=-1)
    scale = 2.0 ** (sb.astype(np.float64) - 127)
    nz = blocks > 0
    # the block maximum lands in [4, 8) before rounding
    assert np.all((blocks[nz] / scale[nz] >= 4) & (blocks[nz] / scale[nz] < 8))
    assert sb[2, 1] == 0 and not np.any(vals[2, 32:64])
    # within half an E2M1 step of the input where no clamp applies: the step
    # is 0.5 below 2, 1 in [2, 4), 2 in [4, 6]; above 6, exactly 6 * scale
    sc = scale.repeat(32, axis=1)
    scaled = np.abs(v) / sc
    half = np.where(scaled < 2, 0.25, np.where(scaled < 4, 0.5, 1.0))
    ok = scaled <= 6
    assert np.all(np.abs(vals - v)[ok] <= half[ok] * sc[ok] * (1 + 1e-12))
    assert np.all(np.abs(vals[~ok]) == 6 * sc[~ok])
    # quantising the quantised values again changes nothing
    c2, s2 = ref.quantize_mxfp4(vals)
    assert np.array_equal(c2, codes) and np.array_equal(s2, sb)


def test_mx4_single_expert_is_dense_swiglu_with_fp4_casts():
    """E = 1, k = 1 with MXFP4 activations: a dense SwiGLU MLP in torch
    float64 where both activations go through a nearest-value search over
    the E2M1 grid with the block scale of the largest magnitude (an
    independent route to the same quantisation)."""
    c = _small_case("mxfp4", T=5, d=64, E=1, k=1, f=32, seed=43)
    r = ref.layer_mx4(c["x"], 1, c["gate"], c["up"], c["down"], w_router=c["w_router"])

    def mx4(t):
        b = t.reshape(t.shape[0], -1, 32)
        amax = b.abs().amax(dim=-1, keepdim=True)
        sc = torch.exp2(torch.floor(torch.log2(amax)) - 2)
        q = torch.tensor([_e2m1_nearest_brute(float(u)) for u in (b / sc).flatten()],
                         dtype=torch.float64).reshape(b.shape)
        return (q * sc).reshape(t.shape)

    x = torch.tensor([[brute.bf16_value(int(b)) for b in row] for row in c["x"]], dtype=torch.float64)
    wg = torch.from_numpy(_dense_weights_brute(c["gate"], 0, 32, 64))
    wu = torch.from_numpy(_dense_weights_brute(c["up"], 0, 32, 64))
    wd = torch.from_numpy(_dense_weights_brute(c["down"], 0, 64, 32))
    xq = mx4(x)
    act = mx4(torch.nn.functional.silu(xq @ wg.T) * (xq @ wu.T))
    assert np.allclose(r["out"], (act @ wd.T).numpy(), rtol=1e-12, atol=1e-12)


def test_mx4_layer_close_to_bf16_layer():
    """MXFP4 activations move out by about their rounding (E2M1 keeps one
    mantissa bit: relative errors of several per cent per element), no
    more: a dropped scale or transposed operand would not stay within a
    few tens of per cent of the bf16 layer."""
    c = _small_case("mxfp4", T=12, d=256, E=8, k=2, f=128, seed=44)
    a = ref.layer(c["x"], 2, c["gate"], c["up"], c["down"], w_router=c["w_router"])
    b = ref.layer_mx4(c["x"], 2, c["gate"], c["up"], c["down"], w_router=c["w_router"])
    m = ref.layer_mx8(c["x"], 2, c["gate"], c["up"], c["down"], w_router=c["w_router"])
    assert np.array_equal(a["ids"], b["ids"])
    rel = np.linalg.norm(b["out"] - a["out"]) / np.linalg.norm(a["out"])
    rel8 = np.linalg.norm(m["out"] - a["out"]) / np.linalg.norm(a["out"])
    assert 2 * rel8 < rel < 0.3, (rel, rel8)
