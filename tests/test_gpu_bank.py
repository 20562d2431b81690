"""The expert slot bank on the GPU (through the C ABI): a layer call through
an N-slot bank paged from pinned host memory equals moe_layer over the full
device pack bit for bit (an expert's rows do not depend on its slot or on the
pass that computes it), its hit / miss / pass counts equal the oracle's
replay of the same routing, and experts left out of a call with
MOE_SLOT_SKIP leave their rows untouched."""

import numpy as np
import pytest
import torch

import quantized_routed_moe_amd as qm
import synthetic
from gpu_util import assert_close, device_case
from oracle import bank as ob
from oracle import ref

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _bank_sequence(case, N, steps, seeds, overlap=True):
    """Runs `steps` layer calls (one seeded x each) through a fresh N-slot
    bank (copies on a stream of their own when `overlap`) and through
    moe_layer; returns the per-call routing and stats."""
    dc = device_case(case)
    s = dc["shape"]
    bank = qm.SlotBank(dc["experts"], N, overlap=overlap)
    ws = qm.alloc_workspace(s, layer=True)
    calls, stats = [], []
    for i in range(steps):
        xc = synthetic.make_case(case["T"], case["d"], case["E"], case["k"], case["f"], case["fmt"],
                                 seed=seeds + i, zipf=1.1)["x"]
        x = torch.from_numpy(xc.view(np.int16)).cuda()
        out_b, ids_b, w_b, lg_b = bank.layer(x, s.k, w_router=dc["w_router"], bias=dc["bias"], ws=ws)
        assert qm.moe_read_device_status(ws) == 0
        out_r, ids_r, w_r, lg_r = qm.layer(x, dc["experts"], s.k, w_router=dc["w_router"], bias=dc["bias"])
        for n, a, b in (("ids", ids_b, ids_r), ("w", w_b, w_r), ("logits", lg_b, lg_r), ("out", out_b, out_r)):
            assert torch.equal(a, b), f"call {i}: {n} differs from moe_layer"
        calls.append(sorted(set(ids_b.cpu().numpy().ravel().tolist())))
        stats.append(bank.last_stats)
    return dc, bank, calls, stats


def _check_stats(case, N, calls, stats):
    expect = ob.run_layer_calls(case["E"], N, calls)
    per_expert = sum(sum(qm.moe_qmat_bytes(case["fmt"], qm.MOE_LAYOUT_TILES, 1, n, K)[:2])
                     for n, K in ((case["f"], case["d"]), (case["f"], case["d"]), (case["d"], case["f"])))
    for i, (st, ex) in enumerate(zip(stats, expect)):
        misses = sum(len(p) for p in ex["loads"])
        got = (st["active"], st["hits"], st["misses"], st["passes"], st["bytes_paged"])
        assert got == (ex["active"], ex["hits"], misses, ex["passes"], misses * per_expert), (i, got, ex)


@pytest.mark.parametrize("overlap", [True, False])
def test_bank_decode_shape(overlap):
    """Decode (T=1, d=4096, E=64, top-2, f=2048, MXFP4) through an 8-slot bank."""
    case = synthetic.workload(1)
    N = 8
    _say(f"slot bank: decode shape, N=8, 24 calls, overlap={overlap}")
    dc, bank, calls, stats = _bank_sequence(case, N, 24, 500, overlap=overlap)
    _check_stats(case, N, calls, stats)
    assert sum(st["misses"] for st in stats) > 0 and sum(st["hits"] for st in stats) > 0
    # one call against the oracle, routed on the device's logits
    x = dc["x"]
    out, ids, w, lg = bank.layer(x, 2, w_router=dc["w_router"], bias=dc["bias"])
    o = ref.layer(case["x"], 2, case["gate"], case["up"], case["down"], logits=lg.cpu().numpy())
    assert np.array_equal(ids.cpu().numpy(), o["ids"])
    assert_close(out.cpu().numpy(), o["out"], "banked out vs oracle")
    bank.close()


@pytest.mark.parametrize("overlap", [True, False])
@pytest.mark.parametrize("fmt", ["mxfp4", "q2", "q4"])
def test_bank_multi_pass_grouped(fmt, overlap):
    """128 tokens x top-2 over 16 experts with 3 slots: every call needs
    several passes; MXFP4 takes the grouped (LDS-tiled) FFN path.  With the
    copy stream, a pass's copies wait for the previous pass's FFN, which
    reads the slots they overwrite."""
    case = synthetic.make_case(128, 512, 16, 2, 256, fmt, seed=61, zipf=1.1)
    N = 3
    _say(f"slot bank: T=128 d=512 E=16 f=256 {fmt}, N=3, 6 calls, overlap={overlap}")
    _, bank, calls, stats = _bank_sequence(case, N, 6, 900, overlap=overlap)
    bank.close()
    _check_stats(case, N, calls, stats)
    assert max(st["passes"] for st in stats) >= 3


def test_bank_one_slot_short_batches():
    """One slot: a pass per active expert, every call pages."""
    case = synthetic.make_case(5, 256, 8, 2, 128, "q4", seed=77)
    _say("slot bank: T=5 d=256 E=8 f=128 q4, N=1, 5 calls")
    _, _, calls, stats = _bank_sequence(case, 1, 5, 300)
    _check_stats(case, 1, calls, stats)


def test_skip_slot_leaves_rows_untouched():
    case = synthetic.make_case(40, 256, 8, 2, 128, "mxfp4", seed=88)
    dc = device_case(case)
    s = dc["shape"]
    T, E, k = s.T, s.E, s.k
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
    ws = qm.alloc_workspace(s)
    qm.moe_route_topk(s, dc["x"], dc["w_router"], None, logits, ids, w)
    qm.moe_dispatch(s, ids, offsets, perm, inv, ws)
    full = torch.full((T * k, s.d), float("nan"), device="cuda")
    qm.moe_expert_ffn(s, dc["x"], dc["experts"], offsets, perm, full, ws)
    skip = [1, 4, 6]
    soe = torch.tensor([qm.MOE_SLOT_SKIP if e in skip else e for e in range(E)], dtype=torch.int32, device="cuda")
    ex = qm.Experts(dc["experts"].fmt, dc["experts"].gate, dc["experts"].up, dc["experts"].down, soe, E, s.d, s.f)
    part = torch.full((T * k, s.d), float("nan"), device="cuda")
    qm.moe_expert_ffn(s, dc["x"], ex, offsets, perm, part, ws)
    assert qm.moe_read_device_status(ws) == 0
    off = offsets.cpu().numpy()
    full, part = full.cpu().numpy(), part.cpu().numpy()
    for e in range(E):
        rows = slice(off[e], off[e + 1])
        if e in skip:
            assert np.isnan(part[rows]).all()
        else:
            assert np.array_equal(part[rows], full[rows])
    assert sum(off[e + 1] - off[e] for e in skip) > 0
