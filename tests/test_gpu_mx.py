"""MXFP8 and MXFP4 activations on the block-scaled matrix cores
(moe_expert_ffn_mx8 / moe_layer_mx8: fp4 x fp8 products; moe_expert_ffn_mx4
/ moe_layer_mx4: fp4 x fp4 products) against the oracle's quantised-
activation layers:
- the quantised token rows bit-exact (both sides quantise the same bf16
  values);
- the quantised SwiGLU output equal up to rare rounding flips (fp32 against
  float64 before the rounding), each flip to a neighbouring value;
- y and out from the device's act within the layer's tolerance;
- out against the pure oracle within a relative L2 bound that allows for
  those flips;
- the one-call layers equal to the separate calls bit for bit."""

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


def _carve(T, d, E, k, f, bits):
    """Byte offsets of the quantised-activation workspace (the library's
    layout: header, act codes, act scales, ready flags, token codes, token
    scales)."""
    R = T * k
    rpad = R + 128
    aq = 256
    as_ = aq + _al(R * f * bits // 8)
    mt = -(-R // 128) + min(E, R)
    flags = as_ + _al((f // 32) * rpad)
    xq = flags + _al(mt * (f // 256) * 8)
    xs = xq + _al(R * d * bits // 8)
    return dict(aq=aq, as_=as_, xq=xq, xs=xs, rpad=rpad, R=R)


def _codes(raw, bits):
    """One code per element: E4M3 bytes as they are, E2M1 nibbles unpacked
    (the even element in the low nibble)."""
    if bits == 8:
        return raw
    out = np.empty(raw.shape[:-1] + (raw.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = raw & 15
    out[..., 1::2] = raw >> 4
    return out


MX = {
    8: dict(quant=ref.quantize_mxfp8, dec=ref.mxfp8_to_f64, layer=ref.layer_mx8,
            values=lambda: np.unique(ref.e4m3_to_f64(np.arange(256))[~np.isnan(ref.e4m3_to_f64(np.arange(256)))]),
            elem=ref.e4m3_to_f64, block_max=2.0 ** 8, rel_pure=1e-3),
    # E2M1's midpoints are far apart next to the fp32 rounding of act, so
    # flips are rarer than E4M3's (none at all on these cases); one would move
    # its element by up to half its value
    4: dict(quant=ref.quantize_mxfp4, dec=ref.mxfp4_act_to_f64, layer=ref.layer_mx4,
            values=lambda: np.unique(ref.e2m1_to_f64(np.arange(16))), elem=ref.e2m1_to_f64, block_max=4.0,
            rel_pure=1e-3),
}


def _run(case, bits):
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
    ws = qm.alloc_workspace_mx8(s) if bits == 8 else qm.alloc_workspace_mx4(s)
    ffn = qm.moe_expert_ffn_mx8 if bits == 8 else qm.moe_expert_ffn_mx4
    qm.moe_route_topk(s, dc["x"], dc["w_router"], dc["bias"], logits, ids, w)
    qm.moe_dispatch(s, ids, offsets, perm, inv, ws)
    ffn(s, dc["x"], dc["experts"], offsets, perm, y, ws)
    qm.moe_combine(s, y, inv, w, out)
    assert qm.moe_read_device_status(ws) == 0
    c = _carve(T, d, E, k, f, bits)
    R, rp = c["R"], c["rpad"]
    wsh = ws.cpu().numpy()
    g = dict(logits=logits, ids=ids, w=w, offsets=offsets, perm=perm, inv=inv, y=y, out=out)
    g = {n: v.cpu().numpy() for n, v in g.items()}
    g["xq"] = _codes(wsh[c["xq"]:c["xq"] + R * d * bits // 8].reshape(R, d * bits // 8), bits)
    g["xs"] = wsh[c["xs"]:c["xs"] + (d // 32) * rp].reshape(d // 32, rp)[:, :R].T
    g["aq"] = _codes(wsh[c["aq"]:c["aq"] + R * f * bits // 8].reshape(R, f * bits // 8), bits)
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


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("T,d,E,k,f,zipf", CASES)
def test_mx_ffn_matches_oracle(T, d, E, k, f, zipf, bits):
    print(f"mx{bits}: T={T} d={d} E={E} k={k} f={f}", flush=True)
    m = MX[bits]
    case = synthetic.make_case(T, d, E, k, f, "mxfp4", seed=9100 + T, zipf=zipf)
    dc, g = _run(case, bits)
    o = m["layer"](case["x"], k, case["gate"], case["up"], case["down"], logits=g["logits"])
    for n in ("ids", "offsets", "perm", "inv"):
        assert np.array_equal(g[n], o[n]), n
    # token rows: the same bf16 values quantised on both sides -> identical codes
    xq, xs = m["quant"](ref.bf16_bits_to_f64(case["x"]))
    tok = g["perm"] // k
    assert np.array_equal(g["xq"], xq[tok]) and np.array_equal(g["xs"], xs[tok])
    # SwiGLU output: rare flips and scale changes only; where the block scale
    # agrees, a flipped element lands on a neighbouring value
    codes_diff = g["aq"] != o["act_codes"]
    scale_diff = g["as"] != o["act_scales"]
    print(f"  act code flips {codes_diff.mean():.2e}, scale flips {scale_diff.mean():.2e}", flush=True)
    assert codes_diff.mean() <= 2e-3, codes_diff.mean()
    assert scale_diff.mean() <= 2e-3
    # or, for an element so far below its block's largest magnitude that the
    # fp32 accumulation error of the gate/up dot products spans several of
    # its steps, moves by less than 2**-12 of that magnitude (in element
    # units the block maximum is at least 2**8 for E4M3, 4 for E2M1, so for
    # E2M1 this still means a neighbour)
    same_scale = np.repeat(~scale_diff, 32, axis=1)
    vals = m["values"]()
    ev_dev = m["elem"](g["aq"][codes_diff & same_scale])
    ev_ref = m["elem"](o["act_codes"][codes_diff & same_scale])
    step = np.abs(np.searchsorted(vals, ev_dev) - np.searchsorted(vals, ev_ref))
    far = step != 1
    if far.any():
        print(f"  flips past a neighbour: {list(zip(ev_dev[far], ev_ref[far]))[:8]}", flush=True)
    assert np.all((step == 1) | (np.abs(ev_dev - ev_ref) <= 2.0 ** -12 * m["block_max"])), step.max()
    # y against the oracle's down projection of the device act
    act_dev = m["dec"](g["aq"], g["as"])
    offs = g["offsets"]
    y_ref = np.zeros_like(o["y"])
    for e in range(E):
        if offs[e + 1] > offs[e]:
            y_ref[offs[e]:offs[e + 1]] = act_dev[offs[e]:offs[e + 1]] @ ref.dequant(case["down"], e).T
    assert_close(g["y"], y_ref, "y (device act)")
    assert_close(g["out"], ref.combine(y_ref, g["inv"], g["w"], k), "out (device act)")
    # Against the pure oracle only the relative L2 bound: an act element that
    # fp32 and float64 round to neighbouring values moves by one step of the
    # element format (E4M3: 2**-3 relative, 32 bf16 steps; E2M1: up to half
    # the value), which alone can move an out element past 5e-3 * rms.
    rel = np.linalg.norm(g["out"] - o["out"]) / np.linalg.norm(o["out"])
    print(f"  out rel L2 against the pure oracle {rel:.2e}", flush=True)
    assert rel <= m["rel_pure"], rel


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("T,k", [(100, 4), (300, 2)])
def test_mx_layer_equals_steps(bits, T, k):
    case = synthetic.make_case(T, 1024, 16, k, 512, "mxfp4", seed=9300 + T, zipf=1.1)
    dc, g = _run(case, bits)
    layer = qm.layer_mx8 if bits == 8 else qm.layer_mx4
    out, ids, w, lg = layer(dc["x"], dc["experts"], k, w_router=dc["w_router"], bias=dc["bias"])
    assert np.array_equal(ids.cpu().numpy(), g["ids"])
    assert np.array_equal(out.cpu().numpy(), g["out"])


@pytest.mark.parametrize("bits", [8, 4])
def test_mx_rejects_what_it_cannot_run(bits):
    case = synthetic.make_case(8, 256, 8, 2, 128, "q2", seed=9400)
    dc = device_case(case)
    layer = qm.layer_mx8 if bits == 8 else qm.layer_mx4
    with pytest.raises(qm.MoeError) as e:
        layer(dc["x"], dc["experts"], 2, w_router=dc["w_router"])
    assert e.value.code == qm.MOE_ERR_UNSUPPORTED
