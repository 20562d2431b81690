"""Parity of the HIP path (through the C ABI) with the CPU oracle: the five
workloads at their full sizes (every row), ragged shapes spanning several
tiles, and the degenerate cases of routing and dispatch."""

import zlib

import numpy as np
import pytest
import torch

import quantized_routed_moe_amd as qm
import synthetic
from gpu_util import (assert_act_close, assert_close, check_against_oracle, device_case, run_layer,
                      run_steps)
from oracle import ref

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("c", [0, 1, 2, 4])
def test_workload_full(c):
    case = synthetic.workload(c)
    _say(f"workload {c}: T={case['T']} d={case['d']} E={case['E']} k={case['k']} f={case['f']} {case['fmt']}")
    dc = device_case(case)
    g = run_steps(dc)
    assert g["status"] == 0
    info = check_against_oracle(case, g, strict=True)
    _say(f"  parity ok {info}")
    lay = run_layer(dc)
    _assert_layer_equals_steps(lay, g)


@pytest.mark.parametrize("T,fmt", [(16, "mxfp4"), (1, "mxfp4"), (16, "q4")])
def test_fanout_k4_full_shape(T, fmt):
    """Top-4 fanout at the full expert shape (d=4096, f=2048, E=64): twice the
    rows per token of the quoted workloads, and the combine over four slots
    (not fused into the down projection)."""
    case = synthetic.make_case(T, 4096, 64, 4, 2048, fmt, seed=7100 + T, zipf=1.1)
    _say(f"k=4 fanout: T={T} d=4096 E=64 k=4 f=2048 {fmt}")
    dc = device_case(case)
    g = run_steps(dc)
    assert g["status"] == 0
    info = check_against_oracle(case, g, strict=True)
    _say(f"  parity ok {info}")
    _assert_layer_equals_steps(run_layer(dc), g)


def _assert_layer_equals_steps(lay, g):
    bad = [n for n in ("ids", "w", "logits", "out") if not np.array_equal(lay[n], g[n])]
    if bad:
        d = np.abs(lay["out"].astype(np.float64) - g["out"])
        raise AssertionError(f"moe_layer differs from the four calls in {bad}; out: {int((d > 0).sum())} of "
                             f"{d.size} differ, max |diff| {d.max():.3e}, max |out| {np.abs(g['out']).max():.3e}")


def test_workload_prefill_full():
    """The prefill chunk (T=2048, Zipf-skewed routing, the single-launch
    grouped FFN) on every one of its 4096 rows: act within the flip bound, y
    and out within the layer's bounds against the pure float64 oracle (and
    against the oracle fed the device's act), and moe_layer equal to the
    four calls bit for bit."""
    case = synthetic.workload(3)
    _say("workload 3 (prefill chunk T=2048), all rows")
    dc = device_case(case)
    g = run_steps(dc)
    assert g["status"] == 0
    info = check_against_oracle(case, g, strict=True)
    _say(f"  parity ok {info}")
    lay = run_layer(dc)
    _assert_layer_equals_steps(lay, g)


@pytest.mark.parametrize("fmt", ["q2", "q4"])
def test_prefill_chunk_other_formats(fmt):
    """The prefill chunk's shape (T=2048, d=4096, E=64, k=2, f=2048, Zipf)
    with the 2-bit and 4-bit packs, on every row."""
    case = synthetic.make_case(2048, 4096, 64, 2, 2048, fmt, seed=3000 + len(fmt), zipf=1.1)
    _say(f"prefill chunk T=2048 {fmt}, all rows")
    dc = device_case(case)
    g = run_steps(dc)
    assert g["status"] == 0
    info = check_against_oracle(case, g, strict=True)
    _say(f"  parity ok {info}")
    _assert_layer_equals_steps(run_layer(dc), g)


@pytest.mark.parametrize("fmt", ["mxfp4", "q2"])
def test_prefill_four_chunks_sampled(fmt):
    """T=8192 (four prefill chunks at once: 192 m-tile positions, ~130 of
    them full) on the grouped launch, checked on the rows of 300 random tokens
    plus the first and last row of every active expert (every m-tile edge
    the dispatch produces), with the combine checked on the sampled tokens;
    moe_layer equal to the four calls bit for bit on every row."""
    T = 8192
    case = synthetic.make_case(T, 4096, 64, 2, 2048, fmt, seed=8192 + len(fmt), zipf=1.1)
    _say(f"four prefill chunks T={T} {fmt}, sampled rows")
    dc = device_case(case)
    g = run_steps(dc)
    assert g["status"] == 0
    rng = np.random.default_rng(11)
    toks = rng.choice(T, size=300, replace=False)
    inv = g["inv"]
    rows = set(int(inv[t * 2 + j]) for t in toks for j in range(2))
    off = g["offsets"]
    for e in range(64):
        if off[e + 1] > off[e]:
            rows.update((int(off[e]), int(off[e + 1]) - 1))
            # the first and last row of every 128-row m-tile of the expert
            for m0 in range(int(off[e]), int(off[e + 1]), 128):
                rows.update((m0, min(m0 + 127, int(off[e + 1]) - 1)))
    rows = np.array(sorted(rows))
    info = check_against_oracle(case, g, rows=rows, strict=True)
    _say(f"  parity ok on {rows.size} rows {info}")
    _assert_layer_equals_steps(run_layer(dc), g)


SHAPES = [
    # T, d, E, k, f        (d, f multiples of 32 but not of 128: ragged K steps)
    (37, 384, 16, 3, 224),
    (3, 96, 4, 2, 64),
    (100, 512, 64, 8, 256),
    (17, 256, 8, 8, 128),
    (1, 32, 1, 1, 32),
    (64, 1024, 32, 2, 512),
    # T*k >= 256 with d % 512 == 0 and f % 256 == 0: the LDS-tiled grouped path
    # (ffn_grouped.hip for MXFP4, ffn_grouped_q.hip for Q2 and Q4)
    (300, 512, 8, 2, 256),
    (700, 1024, 16, 2, 512),
    (257, 512, 64, 4, 768),
]


@pytest.mark.parametrize("fmt", ["mxfp4", "q2", "q4"])
@pytest.mark.parametrize("shape", SHAPES)
def test_ragged_shapes(fmt, shape):
    T, d, E, k, f = shape
    case = synthetic.make_case(T, d, E, k, f, fmt, seed=zlib.crc32(repr((fmt,) + shape).encode()) % 1000, zipf=1.1)
    _say(f"shape {shape} {fmt}")
    g = run_steps(device_case(case))
    assert g["status"] == 0
    check_against_oracle(case, g)


def _given(case, logits):
    case = dict(case)
    case["logits"] = np.asarray(logits, dtype=np.float32)
    case["w_router"] = None
    case["bias"] = None
    return case


def test_one_expert_takes_every_token():
    base = synthetic.make_case(40, 256, 8, 2, 128, "mxfp4", seed=3)
    lg = np.random.default_rng(1).standard_normal((40, 8)).astype(np.float32)
    lg[:, 5] = 50.0
    case = _given(base, lg)
    g = run_steps(device_case(case))
    check_against_oracle(case, g)
    assert np.all(g["ids"][:, 0] == 5)


@pytest.mark.parametrize("fmt", ["mxfp4", "q2", "q4"])
def test_one_expert_takes_every_token_grouped(fmt):
    base = synthetic.make_case(300, 512, 8, 2, 256, fmt, seed=13)
    lg = np.random.default_rng(4).standard_normal((300, 8)).astype(np.float32)
    lg[:, 2] = 40.0
    case = _given(base, lg)
    g = run_steps(device_case(case))
    check_against_oracle(case, g)
    assert np.all(g["ids"][:, 0] == 2) and g["offsets"][3] - g["offsets"][2] == 300


def test_exact_ties_and_signed_zero():
    base = synthetic.make_case(6, 128, 8, 3, 64, "mxfp4", seed=4)
    lg = np.zeros((6, 8), np.float32)
    lg[1] = [1, 1, 1, 1, 2, 2, 0, 0]
    lg[2] = [-0.0, 0.0, -0.0, 0.0, -1, -1, -1, -1]
    lg[3] = [0.5, -0.0, 0.5, 0.0, 0.5, -2, 3, 0.5]
    lg[4] = np.float32(1e-30) * np.arange(8)
    lg[5] = -np.arange(8, dtype=np.float32)
    case = _given(base, lg)
    g = run_steps(device_case(case))
    check_against_oracle(case, g)
    assert g["ids"][0].tolist() == [0, 1, 2]
    assert g["ids"][2].tolist() == [0, 1, 2]
    assert g["ids"][3].tolist() == [6, 0, 2]


@pytest.mark.parametrize("fmt", ["mxfp4", "q2", "q4"])
def test_single_expert_and_full_fanout(fmt):
    c1 = synthetic.make_case(9, 128, 1, 1, 64, fmt, seed=5)
    check_against_oracle(c1, run_steps(device_case(c1)))
    c2 = synthetic.make_case(9, 128, 8, 8, 64, fmt, seed=6)
    g = run_steps(device_case(c2))
    check_against_oracle(c2, g)
    assert np.all(np.sort(g["ids"], axis=1) == np.arange(8))


def test_zero_tokens_is_a_noop():
    s = qm.Shape(0, 256, 8, 2, 128)
    t = torch.empty(0, device="cuda")
    qm.moe_combine(s, t.float(), t.int(), t.float(), t.float())


def test_slot_indirection():
    case = synthetic.make_case(12, 256, 8, 2, 128, "mxfp4", seed=7, slots=11)
    soe = np.array([10, 3, 0, 7, 1, 9, 2, 5], np.int32)
    case["slot_of_expert"] = soe
    g = run_steps(device_case(case))
    assert g["status"] == 0
    check_against_oracle(case, g)


def test_bad_slot_raises_status_and_zeroes_rows():
    case = synthetic.make_case(12, 256, 8, 2, 128, "mxfp4", seed=8, slots=8)
    lg = np.random.default_rng(2).standard_normal((12, 8)).astype(np.float32)
    lg[:, 6] = 9.0                          # every token routes to expert 6
    case = _given(case, lg)
    case["slot_of_expert"] = np.array([0, 1, 2, 3, 4, 5, 99, 7], np.int32)
    g = run_steps(device_case(case))
    assert g["status"] == qm.MOE_DEV_BAD_SLOT
    rows6 = np.arange(g["offsets"][6], g["offsets"][7])
    assert rows6.size == 12 and np.all(g["y"][rows6] == 0.0)


def test_dispatch_experts_missing_from_waves():
    """Regression: with few experts and skewed routing many (wave, expert)
    pairs of the dispatch scan hold no pair; their counts must read as zero.
    Two 1024-pair tiles, E = 8."""
    T, k, E = 750, 2, 8
    rng = np.random.default_rng(5)
    p = np.array([0.5, 0.3, 0.12, 0.05, 0.02, 0.006, 0.003, 0.001])
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    s = qm.Shape(T, 64, E, k, 32)
    dev_ids = torch.from_numpy(ids).cuda()
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
    ws = qm.alloc_workspace(s)
    qm.moe_dispatch(s, dev_ids, offsets, perm, inv, ws)
    assert qm.moe_read_device_status(ws) == 0
    off, pm, iv = ref.dispatch(ids, E)
    assert np.array_equal(offsets.cpu().numpy(), off)
    assert np.array_equal(perm.cpu().numpy(), pm)
    assert np.array_equal(inv.cpu().numpy(), iv)


def test_dispatch_bad_ids():
    s = qm.Shape(5, 64, 4, 2, 32)
    ids = torch.tensor([[0, 1], [7, 2], [3, -1], [1, 0], [2, 3]], dtype=torch.int32, device="cuda")
    offsets = torch.empty(5, dtype=torch.int32, device="cuda")
    perm = torch.empty(10, dtype=torch.int32, device="cuda")
    inv = torch.empty(10, dtype=torch.int32, device="cuda")
    ws = qm.alloc_workspace(s)
    qm.moe_dispatch(s, ids, offsets, perm, inv, ws)
    assert qm.moe_read_device_status(ws) == qm.MOE_DEV_BAD_EXPERT_ID
    off, pm, iv = offsets.cpu().numpy(), perm.cpu().numpy(), inv.cpu().numpy()
    assert off.tolist() == [0, 2, 4, 6, 8]
    assert pm.tolist() == [0, 7, 1, 6, 3, 8, 4, 9, 2, 5]
    assert np.array_equal(iv[pm], np.arange(10))


@pytest.mark.parametrize("T,k,E", [(1, 1, 64), (1, 2, 64), (21, 3, 8), (32, 2, 64), (65, 1, 16), (130, 1, 64)])
@pytest.mark.parametrize("with_bad", [False, True])
def test_dispatch_either_side_of_the_one_wave_size(T, k, E, with_bad):
    """Batches of at most 64 pairs take the one-wave dispatch kernel, larger
    ones the 1024-thread kernel: both give the stable order by expert id,
    ids outside [0, E) last in pair order, offsets[E] = number of valid pairs."""
    rng = np.random.default_rng(T * 7 + k + E)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    if with_bad:
        ids.flat[rng.choice(T * k, size=max(1, T * k // 5), replace=False)] = rng.choice([-3, E, E + 9])
    s = qm.Shape(T, 64, E, k, 32)
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
    ws = qm.alloc_workspace(s)
    qm.moe_dispatch(s, torch.from_numpy(ids).cuda(), offsets, perm, inv, ws)
    assert qm.moe_read_device_status(ws) == (qm.MOE_DEV_BAD_EXPERT_ID if with_bad else 0)
    flat = ids.reshape(-1)
    bucket = np.where((flat >= 0) & (flat < E), flat, E)
    want_perm = np.argsort(bucket, kind="stable")
    want_off = np.searchsorted(np.sort(bucket), np.arange(E + 1), side="left")
    assert np.array_equal(offsets.cpu().numpy(), want_off)
    assert np.array_equal(perm.cpu().numpy(), want_perm)
    assert np.array_equal(inv.cpu().numpy()[want_perm], np.arange(T * k))
    if not with_bad:
        off, pm, iv = ref.dispatch(ids, E)
        assert np.array_equal(want_off, off) and np.array_equal(want_perm, pm)


def test_determinism_and_token_permutation():
    case = synthetic.make_case(29, 512, 16, 2, 256, "mxfp4", seed=9, zipf=1.1)
    dc = device_case(case)
    a, b = run_steps(dc), run_steps(dc)
    for n in ("logits", "ids", "w", "perm", "y", "out", "act"):
        assert np.array_equal(a[n], b[n]), n
    pi = np.random.default_rng(3).permutation(29)
    case2 = dict(case)
    case2["x"] = case["x"][pi]
    c = run_steps(device_case(case2))
    assert np.array_equal(c["ids"], a["ids"][pi])
    assert np.array_equal(c["out"], a["out"][pi])


@pytest.mark.parametrize("c", [1, 4])
def test_power_of_two_scaling(c):
    """+1 on every down-projection scale exponent doubles the output exactly."""
    case = synthetic.workload(c)
    a = run_steps(device_case(case))
    case2 = dict(case)
    d2 = dict(case["down"])
    if case["fmt"] == "mxfp4":
        d2["scales"] = d2["scales"] + np.uint8(1)
    else:
        # x2 in binary16 is exact (normal and subnormal values alike)
        d2["scales"] = (d2["scales"].view(np.float16) * np.float16(2)).view(np.uint16)
        d2["mins"] = (d2["mins"].view(np.float16) * np.float16(2)).view(np.uint16)
    case2["down"] = d2
    b = run_steps(device_case(case2))
    assert np.array_equal(b["out"], 2.0 * a["out"])


@pytest.mark.parametrize("shape", [(1, 256, 8, 1, 128), (3, 512, 16, 2, 256), (8, 256, 64, 3, 128),
                                   (5, 384, 8, 8, 160), (7, 1024, 32, 2, 512), (1, 256, 64, 64, 128),
                                   (16, 256, 64, 2, 128), (32, 256, 16, 2, 128), (12, 384, 8, 1, 160),
                                   (20, 256, 32, 3, 128), (8, 256, 64, 16, 128), (33, 256, 16, 2, 128)])
@pytest.mark.parametrize("fmt", ["mxfp4", "q2", "q4"])
def test_layer_small_T_fused_path_equals_steps(shape, fmt):
    """moe_layer's small-batch path (T <= 8, T*k <= 64: logits-only router
    launch, routing inside every gate/up workgroup, scatter-add combine for
    k <= 2) gives exactly what the four entry points give; the shapes with
    T > 8 or T*k > 64 take the general path."""
    T, d, E, k, f = shape
    case = synthetic.make_case(T, d, E, k, f, fmt, seed=zlib.crc32(repr(shape).encode()) % 997, zipf=1.1)
    dc = device_case(case)
    g = run_steps(dc)
    check_against_oracle(case, g)
    lay = run_layer(dc)
    _assert_layer_equals_steps(lay, g)


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 6, 7, 8, 9, 17, 32])
def test_router_every_small_batch_size(T):
    """The small-batch router runs one kernel instantiation per token count
    (1 to 8 rows per workgroup; larger batches in groups of 8).  Each token's
    logits match the float64 oracle within 1e-4 and equal, bit for bit, the
    logits the same token gets in a batch of its own: a token's sum is formed
    the same way whatever the batch."""
    case = synthetic.make_case(T, 4096, 64, 2, 128, "mxfp4", seed=600 + T, zipf=1.1)
    dc = device_case(case)
    s = dc["shape"]
    _say(f"router T={T}")
    logits = torch.empty((T, s.E), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, s.k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, s.k), dtype=torch.float32, device="cuda")
    qm.moe_route_topk(s, dc["x"], dc["w_router"], dc["bias"], logits, ids, w)
    got = logits.cpu().numpy()
    l64 = ref.router_logits(case["x"], case["w_router"], case["bias"])
    assert np.abs(got - l64).max() <= 1e-4
    s1 = qm.Shape(1, s.d, s.E, s.k, s.f)
    one = torch.empty((1, s.E), dtype=torch.float32, device="cuda")
    i1 = torch.empty((1, s.k), dtype=torch.int32, device="cuda")
    w1 = torch.empty((1, s.k), dtype=torch.float32, device="cuda")
    for t in range(T):
        qm.moe_route_topk(s1, dc["x"][t:t + 1].contiguous(), dc["w_router"], dc["bias"], one, i1, w1)
        assert np.array_equal(one.cpu().numpy()[0], got[t]), f"token {t}"


def test_layer_repeated_on_one_workspace():
    """Back-to-back moe_layer calls sharing one workspace give identical
    results, leave the device status clean and the rest of the header zero."""
    case = synthetic.workload(1)
    dc = device_case(case)
    s = dc["shape"]
    ws = qm.alloc_workspace(s, layer=True)
    outs = []
    for _ in range(4):
        out, ids, w, lg = qm.layer(dc["x"], dc["experts"], s.k, w_router=dc["w_router"], bias=dc["bias"], ws=ws)
        outs.append(out.cpu().numpy())
    assert qm.moe_read_device_status(ws) == 0
    words = ws[:256].view(torch.int32).cpu().numpy()
    assert not words[16:32].any(), words[16:32]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    g = run_steps(dc)
    assert np.array_equal(outs[0], g["out"])


# ---------------------------------------------------------------- tile layout

def _tiles_mxfp4(codes, scales):
    """The tile layout of include/moe.h restated with numpy reshapes:
    block (slot, tile, step), piece L = 16 g + r holds group 4 step + g of row
    16 tile + r; padding groups have zero codes and scale byte 127."""
    slots, n, half = codes.shape
    G, S, NT = half // 16, -(-half // 64), n // 16
    cg = np.zeros((slots, n, 4 * S, 16), np.uint8)
    cg[:, :, :G] = codes.reshape(slots, n, G, 16)
    sg = np.full((slots, n, 4 * S), 127, np.uint8)
    sg[:, :, :G] = scales
    c = cg.reshape(slots, NT, 16, S, 4, 16).transpose(0, 1, 3, 4, 2, 5)
    s = sg.reshape(slots, NT, 16, S, 4).transpose(0, 1, 3, 4, 2)
    return c.reshape(-1), s.reshape(-1)


def _tiles_q2(codes, scales, mins):
    """Q2: piece L = 16 g + r holds elements 8g..8g+7 of each group 4 step + j
    of row 16 tile + r as two words; word t: even elements of groups 2t and
    2t+1 in bytes 0 and 1, odd elements in bytes 2 and 3 (2 bits each,
    ascending).  The step's scale words are row-major: (row r, group j) at
    4 r + j, each (scale | min << 16) (zero for padding)."""
    slots, n, quarter = codes.shape
    G, S, NT = quarter // 8, -(-quarter // 32), n // 16
    cg = np.zeros((slots, n, 4 * S, 8), np.uint8)
    cg[:, :, :G] = codes.reshape(slots, n, G, 8)
    # [slot, tile, step, g, r, j, byte] -> 16-bit chunk of elements 8g..8g+7
    b = cg.reshape(slots, NT, 16, S, 4, 4, 2).transpose(0, 1, 3, 5, 2, 4, 6).astype(np.uint32)
    h = b[..., 0] | (b[..., 1] << 8)
    q = [(h >> (2 * e)) & 3 for e in range(8)]                    # element 8g+e
    ev = q[0] | (q[2] << 2) | (q[4] << 4) | (q[6] << 6)
    od = q[1] | (q[3] << 2) | (q[5] << 4) | (q[7] << 6)
    w = [ev[..., 2 * t] | (ev[..., 2 * t + 1] << 8) | (od[..., 2 * t] << 16) | (od[..., 2 * t + 1] << 24)
         for t in range(2)]
    c = np.stack(w, axis=-1).astype("<u4")
    sm = np.zeros((slots, n, 4 * S), np.uint32)
    sm[:, :, :G] = scales.astype(np.uint32) | (mins.astype(np.uint32) << 16)
    s = sm.reshape(slots, NT, 16, S, 4).transpose(0, 1, 3, 2, 4)
    return np.ascontiguousarray(c).reshape(-1).view(np.uint8), np.ascontiguousarray(s.reshape(-1)).view(np.uint8)


def _tiles_q4(codes, scales, mins):
    """Q4: piece L = 16 g + r holds elements 8g..8g+7 of each group 4 step + j
    of row 16 tile + r as four words; word j: the nibble of element 8g+2h at
    bits 4h..4h+3 and that of element 8g+2h+1 at bits 16+4h..19+4h.  Scale
    words as Q2."""
    slots, n, half = codes.shape
    G, S, NT = half // 16, -(-half // 64), n // 16
    cg = np.zeros((slots, n, 4 * S, 16), np.uint8)
    cg[:, :, :G] = codes.reshape(slots, n, G, 16)
    # [slot, tile, step, g, r, j, h]: byte 4g + h of group 4 step + j of row 16 tile + r
    b = cg.reshape(slots, NT, 16, S, 4, 4, 4).transpose(0, 1, 3, 5, 2, 4, 6).astype(np.uint32)
    w = np.zeros(b.shape[:-1], np.uint32)
    for h in range(4):
        w |= (b[..., h] & 0xF) << (4 * h)
        w |= (b[..., h] >> 4) << (16 + 4 * h)
    c = w.astype("<u4")
    sm = np.zeros((slots, n, 4 * S), np.uint32)
    sm[:, :, :G] = scales.astype(np.uint32) | (mins.astype(np.uint32) << 16)
    s = sm.reshape(slots, NT, 16, S, 4).transpose(0, 1, 3, 2, 4)
    return np.ascontiguousarray(c).reshape(-1).view(np.uint8), np.ascontiguousarray(s.reshape(-1)).view(np.uint8)


@pytest.mark.parametrize("fmt", ["mxfp4", "q2", "q4"])
@pytest.mark.parametrize("n,K", [(48, 224), (16, 32), (32, 512)])
def test_pack_layout(fmt, n, K):
    rng = np.random.default_rng(n * 7 + K)
    m = synthetic.make_matrix(fmt, 3, n, K, rng)
    q = qm.pack_arrays(fmt, m, n, K)
    got_c, got_s = q.codes.cpu().numpy(), q.scales.cpu().numpy()
    if fmt == "mxfp4":
        want_c, want_s = _tiles_mxfp4(m["codes"], m["scales"])
    elif fmt == "q2":
        want_c, want_s = _tiles_q2(m["codes"], m["scales"], m["mins"])
    else:
        want_c, want_s = _tiles_q4(m["codes"], m["scales"], m["mins"])
    assert np.array_equal(got_c, want_c)
    assert np.array_equal(got_s, want_s)


@pytest.mark.parametrize("fmt", ["mxfp4", "q2", "q4"])
def test_repeated_ids_within_a_token(fmt):
    """moe_dispatch takes ids from any source: tokens that name expert 3 twice
    give it 20 rows of 12 tokens (two 16-row column tiles, the second ragged)."""
    T, d, E, k, f = 12, 256, 8, 2, 160
    case = synthetic.make_case(T, d, E, k, f, fmt, seed=21)
    dc = device_case(case)
    ids = np.full((T, k), 3, np.int32)
    ids[::3, 1] = 5
    s = dc["shape"]
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
    y = torch.full((T * k, d), float("nan"), dtype=torch.float32, device="cuda")
    ws = qm.alloc_workspace(s)
    qm.moe_dispatch(s, torch.from_numpy(ids).cuda(), offsets, perm, inv, ws)
    qm.moe_expert_ffn(s, dc["x"], dc["experts"], offsets, perm, y, ws)
    assert qm.moe_read_device_status(ws) == 0
    off, pm, _ = ref.dispatch(ids, E)
    assert np.array_equal(offsets.cpu().numpy(), off) and off[4] - off[3] == 20
    assert np.array_equal(perm.cpu().numpy(), pm)
    act_dev = ws[256:256 + T * k * f * 2].view(torch.int16).view(torch.bfloat16).float().reshape(T * k, f)
    act_dev = act_dev.cpu().numpy()
    act, _ = ref.expert_ffn(case["x"], k, off, pm, case["gate"], case["up"], case["down"])
    assert_act_close(act_dev, act)
    assert_close(y.cpu().numpy(), ref.expert_down(act_dev, off, case["down"]), "y (given device act)")
