"""moe_layer captured into a HIP graph and replayed: every replay equals the
eager call bit for bit, with other eager layer calls (different inputs and
experts) and synchronisations between the replays.  The layer enqueues
kernels only (no memset nodes, no allocation, no host synchronisation), so
a caller may capture it; the benchmark replays its decode steps this way."""

from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

import quantized_routed_moe_amd as qm
import synthetic
from gpu_util import HipGraph, device_case

pytestmark = pytest.mark.gpu

CASES = [
    # (T, d, E, k, f), format: the small-batch routed path (T <= 8, k <= 2,
    # MXFP4, Q2 and Q4), the skinny four-kernel path and the grouped path
    ((1, 256, 8, 2, 128), "mxfp4"),
    ((1, 256, 8, 2, 128), "q2"),
    ((1, 256, 8, 2, 128), "q4"),
    ((16, 256, 16, 2, 128), "q4"),
    ((5, 512, 16, 2, 256), "mxfp4"),
    ((16, 256, 16, 2, 128), "q2"),
    ((12, 256, 8, 3, 128), "mxfp4"),
    ((300, 512, 8, 2, 256), "mxfp4"),
    ((300, 512, 8, 2, 256), "q2"),
]


def _buffers(dc):
    s = dc["shape"]
    dev = dc["x"].device
    return dict(
        logits=dc["logits_in"].clone() if dc["logits_in"] is not None
        else torch.empty((s.T, s.E), dtype=torch.float32, device=dev),
        ids=torch.empty((s.T, s.k), dtype=torch.int32, device=dev),
        w=torch.empty((s.T, s.k), dtype=torch.float32, device=dev),
        out=torch.empty((s.T, s.d), dtype=torch.float32, device=dev),
        ws=qm.alloc_workspace(s, layer=True, device=dev))


def _layer(dc, b, stream):
    qm.moe_layer(dc["shape"], dc["x"], dc["w_router"], dc["bias"], b["logits"], dc["experts"], b["ids"], b["w"],
                 b["out"], b["ws"], stream)


def _poison(b):
    b["ids"].fill_(-7)
    b["w"].fill_(float("nan"))
    b["out"].fill_(float("nan"))


@pytest.mark.parametrize("shape,fmt", CASES)
def test_layer_graph_replays_equal_eager(shape, fmt):
    T, d, E, k, f = shape
    seed = zlib.crc32(repr((shape, fmt, "graph")).encode()) % 1000
    print(f"graph replay: shape {shape} {fmt} seed {seed}", flush=True)
    da = device_case(synthetic.make_case(T, d, E, k, f, fmt, seed=seed, zipf=1.1))
    db = device_case(synthetic.make_case(T, d, E, k, f, fmt, seed=seed + 1, zipf=1.1))
    stream = torch.cuda.Stream()
    ba, bb = _buffers(da), _buffers(db)
    with torch.cuda.stream(stream):
        _layer(da, ba, stream)
        stream.synchronize()
        want = {n: ba[n].cpu().numpy().copy() for n in ("out", "ids", "w", "logits")}
        _layer(db, bb, stream)
        stream.synchronize()
        want_b = bb["out"].cpu().numpy().copy()
        g = HipGraph()
        try:
            g.capture(lambda: _layer(da, ba, stream), stream)
            for rep in range(3):
                _poison(ba)
                g.launch(stream)
                stream.synchronize()
                for n, v in want.items():
                    assert np.array_equal(ba[n].cpu().numpy(), v, equal_nan=False), f"replay {rep}: {n} differs"
                # eager work between replays: another layer on other inputs and experts
                _poison(bb)
                _layer(db, bb, stream)
                stream.synchronize()
                assert np.array_equal(bb["out"].cpu().numpy(), want_b), f"eager call after replay {rep} differs"
        finally:
            g.close()
        assert qm.moe_read_device_status(ba["ws"], stream) == 0
        assert qm.moe_read_device_status(bb["ws"], stream) == 0


def test_single_launch_ffn_replays_with_new_inputs():
    """The prefill FFN runs as one launch whose down tiles wait on ready
    flags raised by the gate/up tiles.  Each replay of a captured call must
    wait for its own gate/up tiles, not trust flags left by the previous
    replay: between replays the token rows change and act is poisoned with
    NaN (the flags are left alone), so a down tile that read act early would
    show up in y."""
    shape, fmt = (300, 512, 8, 2, 256), "mxfp4"
    T, d, E, k, f = shape
    seed = zlib.crc32(repr((shape, fmt, "chain")).encode()) % 1000
    print(f"single-launch FFN replays: shape {shape} {fmt} seed {seed}", flush=True)
    dc = device_case(synthetic.make_case(T, d, E, k, f, fmt, seed=seed, zipf=1.1))
    s = dc["shape"]
    dev = dc["x"].device
    stream = torch.cuda.Stream()
    gen = torch.Generator(device="cpu").manual_seed(seed)
    xs = [dc["x"]] + [(torch.randn((T, d), generator=gen) * (1 + r)).to(torch.bfloat16).view(torch.int16).to(dev)
                      for r in range(3)]
    with torch.cuda.stream(stream):
        logits = torch.empty((T, E), dtype=torch.float32, device=dev)
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
        perm = torch.empty((T * k,), dtype=torch.int32, device=dev)
        inv = torch.empty((T * k,), dtype=torch.int32, device=dev)
        ws_ref = qm.alloc_workspace(s, device=dev, stream=stream)
        qm.moe_route_topk(s, dc["x"], dc["w_router"], dc["bias"], logits, ids, w, stream)
        qm.moe_dispatch(s, ids, offsets, perm, inv, ws_ref, stream)
        want = []
        for x in xs:                          # eager results, own workspace
            y = torch.empty((T * k, d), dtype=torch.float32, device=dev)
            qm.moe_expert_ffn(s, x, dc["experts"], offsets, perm, y, ws_ref, stream)
            stream.synchronize()
            want.append(y.cpu().numpy().copy())
        assert not np.array_equal(want[0], want[1])
        x_buf = xs[0].clone()
        y = torch.empty((T * k, d), dtype=torch.float32, device=dev)
        ws = qm.alloc_workspace(s, device=dev, stream=stream)
        act = ws[256:256 + T * k * f * 2]
        g = HipGraph()
        try:
            g.capture(lambda: qm.moe_expert_ffn(s, x_buf, dc["experts"], offsets, perm, y, ws, stream), stream)
            for rep in range(2 * len(xs)):
                r = rep % len(xs)
                x_buf.copy_(xs[r])
                act.view(torch.int16).fill_(0x7fc0)          # bf16 NaN
                y.fill_(float("nan"))
                stream.synchronize()
                g.launch(stream)
                stream.synchronize()
                assert np.array_equal(y.cpu().numpy(), want[r]), f"replay {rep} (inputs {r}) differs"
        finally:
            g.close()
        assert qm.moe_read_device_status(ws, stream) == 0
        assert qm.moe_read_device_status(ws_ref, stream) == 0
