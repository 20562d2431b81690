"""MXFP8 activations on the block-scaled fp4 x fp8 matrix cores
(moe_expert_ffn_mx8 / moe_layer_mx8) against the oracle's MXFP8 layer:
the quantised token rows bit-exact (both sides quantise the same bf16
values), the quantised SwiGLU output equal up to rare one-step rounding
flips (fp32 against float64 before the rounding), y and out from the
device's act within the layer's tolerance, out against the pure oracle
within its relative L2 bound, and
moe_layer_mx8 equal to the separate calls bit for bit."""

import numpy as np
import pytest
import torch

import quantized_routed_moe_amd as qm
import synthetic
from gpu_util import assert_close, device_case
from oracle import ref

pytestmark = pytest.mark.gpu


def _al(v):
    return (v + 255) // 256 * 256


def _carve(T, d, E, k, f):
    """Byte offsets of the MXFP8 workspace (the library's layout: header,
    act codes, act scales, ready flags, token codes, token scales)."""
    R = T * k
    rpad = R + 128
    aq = 256
    as_ = aq + _al(R * f)
    mt = -(-R // 128) + min(E, R)
    flags = as_ + _al((f // 32) * rpad)
    xq = flags + _al(mt * (f // 256) * 8)
    xs = xq + _al(R * d)
    return dict(aq=aq, as_=as_, xq=xq, xs=xs, rpad=rpad, R=R)


def _run(case):
    dc = device_case(case)
    s = dc["shape"]
    T, E, k, d, f = s.T, s.E, s.k, s.d, s.f
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
    y = torch.full((T * k, d), float("nan"), device="cuda")
    out = torch.full((T, d), float("nan"), device="cuda")
    ws = qm.alloc_workspace_mx8(s)
    qm.moe_route_topk(s, dc["x"], dc["w_router"], dc["bias"], logits, ids, w)
    qm.moe_dispatch(s, ids, offsets, perm, inv, ws)
    qm.moe_expert_ffn_mx8(s, dc["x"], dc["experts"], offsets, perm, y, ws)
    qm.moe_combine(s, y, inv, w, out)
    assert qm.moe_read_device_status(ws) == 0
    c = _carve(T, d, E, k, f)
    R, rp = c["R"], c["rpad"]
    wsh = ws.cpu().numpy()
    g = dict(logits=logits, ids=ids, w=w, offsets=offsets, perm=perm, inv=inv, y=y, out=out)
    g = {n: v.cpu().numpy() for n, v in g.items()}
    g["xq"] = wsh[c["xq"]:c["xq"] + R * d].reshape(R, d)
    g["xs"] = wsh[c["xs"]:c["xs"] + (d // 32) * rp].reshape(d // 32, rp)[:, :R].T
    g["aq"] = wsh[c["aq"]:c["aq"] + R * f].reshape(R, f)
    g["as"] = wsh[c["as_"]:c["as_"] + (f // 32) * rp].reshape(f // 32, rp)[:, :R].T
    return dc, g


CASES = [
    # T, d, E, k, f, zipf
    (64, 512, 8, 2, 256, None),
    (100, 1024, 16, 4, 512, 1.1),
    (3, 512, 8, 2, 256, None),
    (256, 4096, 16, 2, 2048, 1.1),
    (2048, 4096, 64, 2, 2048, 1.1),     # the prefill chunk's shape and routing
]


@pytest.mark.parametrize("T,d,E,k,f,zipf", CASES)
def test_mx8_ffn_matches_oracle(T, d, E, k, f, zipf):
    print(f"mx8: T={T} d={d} E={E} k={k} f={f}", flush=True)
    case = synthetic.make_case(T, d, E, k, f, "mxfp4", seed=9100 + T, zipf=zipf)
    dc, g = _run(case)
    o = ref.layer_mx8(case["x"], k, case["gate"], case["up"], case["down"], logits=g["logits"])
    for n in ("ids", "offsets", "perm", "inv"):
        assert np.array_equal(g[n], o[n]), n
    # token rows: the same bf16 values quantised on both sides -> identical bytes
    xq, xs = ref.quantize_mxfp8(ref.bf16_bits_to_f64(case["x"]))
    tok = g["perm"] // k
    assert np.array_equal(g["xq"], xq[tok]) and np.array_equal(g["xs"], xs[tok])
    # SwiGLU output: rare one-step flips and scale changes only
    codes_diff = g["aq"] != o["act_codes"]
    assert codes_diff.mean() <= 2e-3, codes_diff.mean()
    assert (g["as"] != o["act_scales"]).mean() <= 2e-3
    # y against the oracle's down projection of the device act
    act_dev = ref.mxfp8_to_f64(g["aq"], g["as"])
    offs = g["offsets"]
    y_ref = np.zeros_like(o["y"])
    for e in range(E):
        if offs[e + 1] > offs[e]:
            y_ref[offs[e]:offs[e + 1]] = act_dev[offs[e]:offs[e + 1]] @ ref.dequant(case["down"], e).T
    assert_close(g["y"], y_ref, "y (device act)")
    assert_close(g["out"], ref.combine(y_ref, g["inv"], g["w"], k), "out (device act)")
    # Against the pure oracle only the relative L2 bound: an act element
    # that fp32 and float64 round to neighbouring E4M3 values moves by one
    # E4M3 step (2**-3 relative, 32 times a bf16 step), which alone can move
    # an out element past 5e-3 * rms.
    rel = np.linalg.norm(g["out"] - o["out"]) / np.linalg.norm(o["out"])
    assert rel <= 1e-3, rel


def test_mx8_layer_equals_steps():
    case = synthetic.make_case(100, 1024, 16, 4, 512, "mxfp4", seed=9300, zipf=1.1)
    dc, g = _run(case)
    out, ids, w, lg = qm.layer_mx8(dc["x"], dc["experts"], 4, w_router=dc["w_router"], bias=dc["bias"])
    assert np.array_equal(ids.cpu().numpy(), g["ids"])
    assert np.array_equal(out.cpu().numpy(), g["out"])


def test_mx8_rejects_what_it_cannot_run():
    case = synthetic.make_case(8, 256, 8, 2, 128, "q2", seed=9400)
    dc = device_case(case)
    with pytest.raises(qm.MoeError) as e:
        qm.layer_mx8(dc["x"], dc["experts"], 2, w_router=dc["w_router"])
    assert e.value.code == qm.MOE_ERR_UNSUPPORTED
