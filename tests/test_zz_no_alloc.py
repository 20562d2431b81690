"""moe_layer_noalloc (the entry point for callers that cannot allocate:
its workspace is the library's per-GPU scratch array) against moe_layer
through the C ABI: identical outputs bit for bit on two calls in a row, the
second with a smaller input, for each FFN path it can take; shapes past the
array's size are rejected before any work is enqueued."""

import numpy as np
import pytest
import torch

import quantized_routed_moe_amd as qm
import synthetic
from gpu_util import device_case

pytestmark = pytest.mark.gpu


def _outputs(dc, call):
    s = dc["shape"]
    logits = dc["logits_in"].clone() if dc["logits_in"] is not None else torch.full(
        (s.T, s.E), float("nan"), dtype=torch.float32, device="cuda")
    ids = torch.full((s.T, s.k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((s.T, s.k), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((s.T, s.d), float("nan"), dtype=torch.float32, device="cuda")
    call(s, logits, ids, w, out)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (out, ids, w, logits)]


def _reference(dc):
    ws = qm.alloc_workspace(dc["shape"], layer=True)

    def call(s, logits, ids, w, out):
        qm.moe_layer(s, dc["x"], dc["w_router"], dc["bias"], logits, dc["experts"], ids, w, out, ws)
    res = _outputs(dc, call)
    assert qm.moe_read_device_status(ws) == 0
    return res


def _noalloc(dc, status):
    def call(s, logits, ids, w, out):
        qm.moe_layer_noalloc(s, dc["x"], dc["w_router"], dc["bias"], logits, dc["experts"], ids, w, out, status)
    return _outputs(dc, call)


PAIRS = [
    # (first call, second smaller call): T, d, E, k, f, fmt
    ((16, 4096, 64, 2, 2048, "q2"), (1, 4096, 64, 2, 2048, "q2")),            # skinny paths, decode shape
    ((5, 4096, 64, 2, 2048, "mxfp4"), (1, 4096, 64, 2, 2048, "mxfp4")),       # routed small batch
    ((300, 1024, 16, 2, 512, "mxfp4"), (40, 1024, 16, 3, 512, "mxfp4")),      # grouped, then combine kernel
    ((24, 512, 8, 4, 256, "q4"), (3, 512, 8, 4, 256, "q4")),
    ((300, 1024, 16, 2, 512, "q2"), (140, 512, 8, 2, 256, "q4")),      # the 2-bit / 4-bit grouped launch
]


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_equals_moe_layer_twice(first, second):
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for i, (T, d, E, k, f, fmt) in enumerate((first, second)):
        print(f"moe_layer_noalloc call {i}: T={T} d={d} E={E} k={k} f={f} {fmt}", flush=True)
        case = synthetic.make_case(T, d, E, k, f, fmt, seed=5100 + 10 * i + T, zipf=1.1)
        dc = device_case(case)
        want = _reference(dc)
        got = _noalloc(dc, status)
        for name, a, b in zip(("out", "ids", "w", "logits"), got, want):
            assert np.array_equal(a, b), f"call {i}: {name} differs from moe_layer"
        assert int(status.item()) == 0


def test_noalloc_rejects_shapes_past_the_scratch_array():
    case = synthetic.make_case(4, 256, 8, 2, 128, "mxfp4", seed=5200)
    dc = device_case(case)
    big = qm.Shape(2048, 4096, 64, 2, 2048)
    assert qm.moe_layer_workspace_bytes(big) > qm.MOE_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((2048, 4096), dtype=torch.int16, device="cuda")
    t = torch.zeros(16, device="cuda")
    ids = torch.zeros((2048, 2), dtype=torch.int32, device="cuda")
    with pytest.raises(qm.MoeError) as e:
        qm.moe_layer_noalloc(big, x, None, None, torch.zeros((2048, 64), device="cuda"), dc["experts"], ids,
                             torch.zeros((2048, 2), device="cuda"), torch.zeros((2048, 4096), device="cuda"))
    assert e.value.code == qm.MOE_ERR_WORKSPACE
    del t
