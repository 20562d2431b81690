"""The layer with a shared expert (moe_layer_shared) on the GPU against the
oracle: routing bit-exact on the device logits, out within the layer's
tolerance, on the skinny path (decode, verify, two-bit and four-bit
batches, the small-batch routing) and the single-launch grouped path
(shared m-tiles, a ragged last one included)."""

import numpy as np
import pytest
import torch

import quantized_routed_moe_amd as qm
import synthetic
from gpu_util import assert_close, device_case
from oracle import ref

pytestmark = pytest.mark.gpu

CASES = [
    # T, d, E, k, f, fmt, zipf
    (1, 4096, 64, 2, 2048, "mxfp4", None),
    (5, 4096, 64, 2, 2048, "mxfp4", None),
    (16, 4096, 64, 2, 2048, "q2", 1.1),
    (16, 4096, 64, 2, 2048, "q4", 1.1),
    (40, 4096, 64, 4, 2048, "mxfp4", 1.1),
    (256, 4096, 16, 2, 2048, "mxfp4", 1.1),
    (300, 4096, 16, 2, 2048, "mxfp4", 1.1),
    (2048, 4096, 64, 2, 2048, "mxfp4", 1.1),    # the prefill chunk's shape and routing
    (300, 4096, 16, 2, 2048, "q2", 1.1),        # the 2-bit / 4-bit grouped path
    (2048, 4096, 64, 2, 2048, "q4", 1.1),
]


@pytest.mark.parametrize("T,d,E,k,f,fmt,zipf", CASES)
def test_layer_shared_matches_oracle(T, d, E, k, f, fmt, zipf):
    print(f"shared expert: T={T} d={d} E={E} k={k} f={f} {fmt}", flush=True)
    case = synthetic.make_case(T, d, E, k, f, fmt, seed=8100 + T, zipf=zipf)
    sh = synthetic.make_shared(case, seed=8200 + T)
    dc = device_case(case)
    sh_dev = qm.Experts.from_arrays(fmt, sh["gate"], sh["up"], sh["down"], "cuda")
    out, ids, w, lg = qm.layer_shared(dc["x"], dc["experts"], sh_dev, k, w_router=dc["w_router"], bias=dc["bias"])
    r = ref.layer_shared(case["x"], k, case["gate"], case["up"], case["down"], sh, logits=lg.cpu().numpy())
    assert np.array_equal(ids.cpu().numpy(), r["ids"])
    assert np.allclose(w.cpu().numpy(), r["w"], rtol=0, atol=1e-6)
    assert_close(out.cpu().numpy(), r["out"], "out with the shared expert")
    # the routed part is the one moe_layer computes
    base, ids2, _, _ = qm.layer(dc["x"], dc["experts"], k, w_router=dc["w_router"], bias=dc["bias"])
    assert torch.equal(ids, ids2)
    assert_close((out - base).cpu().numpy(), r["ys"], "shared expert alone")


def test_layer_shared_repeats_bit_exact():
    case = synthetic.make_case(256, 512, 16, 2, 256, "mxfp4", seed=8300, zipf=1.1)
    sh = synthetic.make_shared(case, seed=8301)
    dc = device_case(case)
    sh_dev = qm.Experts.from_arrays("mxfp4", sh["gate"], sh["up"], sh["down"], "cuda")
    a = qm.layer_shared(dc["x"], dc["experts"], sh_dev, 2, w_router=dc["w_router"], bias=dc["bias"])[0]
    b = qm.layer_shared(dc["x"], dc["experts"], sh_dev, 2, w_router=dc["w_router"], bias=dc["bias"])[0]
    assert torch.equal(a, b)
