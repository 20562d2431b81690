"""Behaviour of the one-call layer beyond plain parity, on the GPU through
the C ABI: an expert mapped to MOE_SLOT_SKIP contributes zero on every FFN
path (fused scatter-add, combine kernel, grouped single launch); a pack
whose experts live in slabs (moe_experts.slot_bytes) gives the same bits as
separate arrays; and a prefill hand-off that gives up (forced from the host
through the workspace's poll-limit word) leaves NaN in the affected y rows
and a status bit that the checked layer turns into an error."""

import numpy as np
import pytest
import torch

import quantized_routed_moe_amd as qm
import synthetic
from gpu_util import assert_close, device_case
from oracle import ref

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


SKIP_CASES = [
    # T, d, E, k, f, fmt: fused small-batch path (k <= 2), combine kernel (k = 3),
    # the general skinny path, and the grouped single launch
    (1, 512, 8, 2, 256, "mxfp4"),
    (6, 512, 8, 3, 256, "q2"),
    (24, 512, 16, 3, 256, "q4"),
    (300, 512, 8, 2, 256, "mxfp4"),
    (300, 512, 8, 2, 256, "q2"),
]


@pytest.mark.parametrize("T,d,E,k,f,fmt", SKIP_CASES)
def test_layer_skipped_expert_contributes_zero(T, d, E, k, f, fmt):
    case = synthetic.make_case(T, d, E, k, f, fmt, seed=4400 + T, router="given")
    _say(f"skipped expert in moe_layer: T={T} d={d} E={E} k={k} f={f} {fmt}")
    dc = device_case(case)
    r = ref.layer(case["x"], k, case["gate"], case["up"], case["down"], logits=case["logits"])
    active = [e for e in range(E) if r["offsets"][e + 1] > r["offsets"][e]]
    skip = active[len(active) // 2]
    soe = np.arange(E, dtype=np.int32)
    soe[skip] = qm.MOE_SLOT_SKIP
    ex = dc["experts"]
    ex2 = qm.Experts(ex.fmt, ex.gate, ex.up, ex.down, torch.from_numpy(soe).cuda(), E, d, f)
    ws = qm.alloc_workspace(dc["shape"], layer=True)
    ws_bytes = ws.numel()
    # poison the workspace's y region: a skipped expert must not read as stale data
    ws[256:].view(torch.uint8).fill_(0xFF)
    qm.moe_workspace_init(ws)
    out, ids, w, _ = qm.layer(dc["x"], ex2, k, logits=dc["logits_in"].clone(), ws=ws, check=True)
    assert ws.numel() == ws_bytes
    y = r["y"].copy()
    y[r["offsets"][skip]:r["offsets"][skip + 1]] = 0.0
    want = ref.combine(y, r["inv"], r["w"], k)
    assert np.array_equal(ids.cpu().numpy(), r["ids"])
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    assert_close(got, want, "out with one expert skipped")
    # tokens that never routed to the skipped expert are unchanged
    full, _, _, _ = qm.layer(dc["x"], ex, k, logits=dc["logits_in"].clone())
    untouched = ~np.any(r["ids"] == skip, axis=1)
    assert np.array_equal(got[untouched], full.cpu().numpy()[untouched])


@pytest.mark.parametrize("T,fmt", [(1, "mxfp4"), (16, "q2"), (5, "q4"), (300, "mxfp4"), (300, "q4")])
def test_slab_pack_equals_separate_arrays(T, fmt):
    d, f, E = (4096, 2048, 64) if T < 300 else (512, 256, 8)
    case = synthetic.make_case(T, d, E, 2, f, fmt, seed=4500 + T, zipf=1.1)
    _say(f"slab pack: T={T} d={d} E={E} f={f} {fmt}")
    dc = device_case(case)
    slabs = dc["experts"].to_slabs()
    a = qm.layer(dc["x"], dc["experts"], 2, w_router=dc["w_router"], bias=dc["bias"], check=True)
    b = qm.layer(dc["x"], slabs, 2, w_router=dc["w_router"], bias=dc["bias"], check=True)
    for n, u, v in zip(("out", "ids", "w", "logits"), a, b):
        assert torch.equal(u, v), n


@pytest.mark.parametrize("fmt", ["mxfp4", "q2"])
def test_prefill_handoff_timeout_gives_nan_and_status(fmt):
    """Workspace header word 32 = 1 makes every down tile of the single-launch
    grouped FFN give up at once: its y rows must be NaN (never a product of
    unfinished act rows), MOE_DEV_CHAIN_TIMEOUT raised, the checked layer
    raises, and a normal call on a fresh workspace is unaffected."""
    case = synthetic.make_case(300, 512, 8, 2, 256, fmt, seed=4600)
    _say(f"forced prefill hand-off timeout: T=300 d=512 E=8 f=256 {fmt}")
    dc = device_case(case)
    s = dc["shape"]
    T, E, k = s.T, s.E, s.k
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
    y = torch.zeros((T * k, s.d), dtype=torch.float32, device="cuda")
    ws = qm.alloc_workspace(s)
    ws.view(torch.int32)[32] = 1            # poll limit word: give up at once
    qm.moe_route_topk(s, dc["x"], dc["w_router"], None, logits, ids, w)
    qm.moe_dispatch(s, ids, offsets, perm, inv, ws)
    qm.moe_expert_ffn(s, dc["x"], dc["experts"], offsets, perm, y, ws)
    bits = qm.moe_read_device_status(ws)
    assert bits & qm.MOE_DEV_CHAIN_TIMEOUT
    assert torch.isnan(y).all(), "every down tile gave up: every y row must be NaN"
    # the checked one-call layer turns it into an error
    wsl = qm.alloc_workspace(s, layer=True)
    wsl.view(torch.int32)[32] = 1
    with pytest.raises(qm.MoeError) as e:
        qm.layer(dc["x"], dc["experts"], k, w_router=dc["w_router"], ws=wsl, check=True)
    assert e.value.code == qm.MOE_ERR_DEVICE and e.value.bits & qm.MOE_DEV_CHAIN_TIMEOUT
    # default limit: clean
    out, ids2, _, lg = qm.layer(dc["x"], dc["experts"], k, w_router=dc["w_router"], check=True)
    r = ref.layer(case["x"], k, case["gate"], case["up"], case["down"], logits=lg.cpu().numpy())
    assert np.array_equal(ids2.cpu().numpy(), r["ids"])
    assert_close(out.cpu().numpy(), r["out"], "out after the forced timeout")


def test_q_grouped_group_sum_out_of_range_gives_nan():
    """The 2-bit / 4-bit grouped FFN keeps each group's input sum as two
    fp16 halves: a token whose group sum exceeds fp16's range (here 32
    elements of 4096 in one group) gets NaN in its output row, never a
    finite wrong value; every other token still matches the oracle."""
    case = synthetic.make_case(300, 512, 8, 2, 256, "q2", seed=4700)
    x = case["x"].copy()
    big = np.float32(4096.0).view(np.uint32) >> 16            # bf16 bits of 4096 (exact)
    x[5, 64:96] = big
    case["x"] = x
    _say("2-bit grouped FFN, one group sum past fp16's range: T=300 d=512 E=8 f=256")
    dc = device_case(case)
    out, ids, w, lg = qm.layer(dc["x"], dc["experts"], 2, w_router=dc["w_router"], bias=dc["bias"])
    out = out.cpu().numpy()
    assert np.isnan(out[5]).all()
    r = ref.layer(case["x"], 2, case["gate"], case["up"], case["down"], logits=lg.cpu().numpy())
    keep = np.arange(300) != 5
    assert np.array_equal(ids.cpu().numpy(), r["ids"])
    assert_close(out[keep], r["out"][keep], "out of the other tokens")
