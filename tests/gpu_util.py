"""Helpers of the GPU parity tests: move a synthetic case to the device, run
the layer through the C ABI (step by step or in one call) and compare with
the oracle at the stated tolerances."""

from __future__ import annotations

import numpy as np
import torch

import quantized_routed_moe_amd as qm
from oracle import ref

# Tolerances for floating-point outputs (out and y):
#   relative L2 error <= 1e-3 and every element within 5e-3 * rms(reference).
REL_L2 = 1e-3
ELEM_RMS = 5e-3
LOGIT_ABS = 1e-4       # device fp32 logits vs float64 oracle logits
WEIGHT_ABS = 1e-6      # device routing weights vs float64 softmax of the same logits
ACT_FLIP_FRAC = 1e-3   # fraction of act elements allowed to differ ...
ACT_ABS_RMS = 1e-5     # ... each by at most max(one bf16 ulp, 1e-5 * rms(act)).
# The absolute floor: g and u are fp32 sums of d products, so their rounding
# error is ~1e-7..1e-6 of their rms; for act values near zero that error alone
# exceeds one bf16 ulp, whatever the kernel.


def device_case(case: dict, dev="cuda") -> dict:
    x = torch.from_numpy(case["x"].view(np.int16)).to(dev)
    out = dict(x=x, shape=qm.Shape(case["T"], case["d"], case["E"], case["k"], case["f"]))
    out["w_router"] = None if case["w_router"] is None else torch.from_numpy(case["w_router"]).to(dev)
    out["bias"] = None if case["bias"] is None else torch.from_numpy(case["bias"]).to(dev)
    out["logits_in"] = None if case["logits"] is None else torch.from_numpy(case["logits"]).to(dev)
    out["experts"] = qm.Experts.from_arrays(case["fmt"], case["gate"], case["up"], case["down"], dev,
                                            slot_of_expert=case.get("slot_of_expert"))
    return out


def run_steps(dc: dict) -> dict:
    """The four entry points in sequence; returns host numpy results."""
    s = dc["shape"]
    dev = dc["x"].device
    T, E, k = s.T, s.E, s.k
    logits = dc["logits_in"].clone() if dc["logits_in"] is not None else torch.empty((T, E), dtype=torch.float32, device=dev)
    ids = torch.full((T, k), -7, dtype=torch.int32, device=dev)
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device=dev)
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=dev)
    perm = torch.full((T * k,), -7, dtype=torch.int32, device=dev)
    inv = torch.full((T * k,), -7, dtype=torch.int32, device=dev)
    y = torch.full((T * k, s.d), float("nan"), dtype=torch.float32, device=dev)
    out = torch.full((T, s.d), float("nan"), dtype=torch.float32, device=dev)
    ws = qm.alloc_workspace(s, device=dev)
    qm.moe_route_topk(s, dc["x"], dc["w_router"], dc["bias"], logits, ids, w)
    qm.moe_dispatch(s, ids, offsets, perm, inv, ws)
    qm.moe_expert_ffn(s, dc["x"], dc["experts"], offsets, perm, y, ws)
    qm.moe_combine(s, y, inv, w, out)
    status = qm.moe_read_device_status(ws)
    act = ws[256:256 + T * k * s.f * 2].view(torch.int16).view(torch.bfloat16).float()
    res = dict(logits=logits, ids=ids, w=w, offsets=offsets, perm=perm, inv=inv, y=y, out=out,
               act=act.reshape(T * k, s.f))
    res = {n: v.cpu().numpy() for n, v in res.items()}
    res["status"] = status
    return res


def run_layer(dc: dict, ws=None) -> dict:
    """moe_layer in one call; the workspace's device status must stay clean."""
    s = dc["shape"]
    logits = dc["logits_in"].clone() if dc["logits_in"] is not None else None
    if ws is None:
        ws = qm.alloc_workspace(s, layer=True, device=dc["x"].device)
    out, ids, w, lg = qm.layer(dc["x"], dc["experts"], s.k, w_router=dc["w_router"], bias=dc["bias"],
                               logits=logits, ws=ws)
    status = qm.moe_read_device_status(ws)
    assert status == 0, f"device status {status:#x}"
    return dict(out=out.cpu().numpy(), ids=ids.cpu().numpy(), w=w.cpu().numpy(), logits=lg.cpu().numpy())


def assert_close(got, want, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    if want.size == 0:
        return
    err = got - want
    rms = float(np.sqrt(np.mean(want ** 2)))
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(want), 1e-300))
    worst = float(np.max(np.abs(err)))
    assert rel <= REL_L2, f"{what}: relative L2 error {rel:.3e} > {REL_L2}"
    assert worst <= ELEM_RMS * rms, f"{what}: max |err| {worst:.3e} > {ELEM_RMS} * rms {rms:.3e}"


def bf16_ulp(v):
    v = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(np.where(v > 0, v, 1.0))
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def assert_act_close(got, want, what="act"):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    diff = got != want
    n = int(diff.sum())
    assert n <= max(1, ACT_FLIP_FRAC * want.size), f"{what}: {n} of {want.size} bf16 values differ"
    if n:
        rms = float(np.sqrt(np.mean(want ** 2)))
        ulp = np.maximum(bf16_ulp(got[diff]), bf16_ulp(want[diff]))
        over = np.abs(got[diff] - want[diff]) > np.maximum(ulp, ACT_ABS_RMS * rms)
        if np.any(over):
            gv, wv = got[diff][over], want[diff][over]
            detail = ", ".join(f"({a:.6g} vs {b:.6g})" for a, b in list(zip(gv, wv))[:8])
            raise AssertionError(f"{what}: {int(over.sum())} of {n} differing values exceed one bf16 ulp; "
                                 f"rms(act)={rms:.4g}; got vs want: {detail}")


def check_against_oracle(case: dict, g: dict, *, rows=None, check_logits=True, strict=False) -> dict:
    """Compare device results `g` (from run_steps) with the oracle.

    Routing is judged on the device's float32 logits (bit-exact ids, perm,
    inv, offsets); the float64 oracle logits must agree within LOGIT_ABS.
    act is compared with the oracle's act (ACT_FLIP_FRAC / one ulp).  y is
    compared with the oracle's down projection of the DEVICE act, and out
    with the oracle's combine of that y, at REL_L2 / ELEM_RMS: fp32 and
    float64 sums round to bf16 differently on ~1e-3 of the act elements,
    and one such ulp on a large activation moves a y element by more than
    5e-3*rms on some shapes.  With strict=True (the five workloads) the
    device y and out must ALSO meet REL_L2 / ELEM_RMS against the pure
    oracle.
    With `rows`, the FFN is checked on those sorted rows only."""
    k, E = case["k"], case["E"]
    info = {}
    if case["logits"] is not None:
        assert np.array_equal(g["logits"], case["logits"])
    elif check_logits:
        l64 = ref.router_logits(case["x"], case["w_router"], case["bias"])
        err = np.abs(g["logits"] - l64).max()
        assert err <= LOGIT_ABS, f"logits error {err:.3e}"
        ids64, _ = ref.route_topk(l64, k)
        info["fp64_route_mismatch_tokens"] = int(np.sum(np.any(ids64 != g["ids"], axis=1)))
    ids, w = ref.route_topk(g["logits"], k)
    assert np.array_equal(g["ids"], ids), "top-k ids differ from the oracle on the device logits"
    assert np.abs(g["w"] - w).max() <= WEIGHT_ABS
    offsets, perm, inv = ref.dispatch(ids, E)
    assert np.array_equal(g["offsets"], offsets)
    assert np.array_equal(g["perm"], perm)
    assert np.array_equal(g["inv"], inv)
    soe = case.get("slot_of_expert")
    if rows is None:
        act, y = ref.expert_ffn(case["x"], k, offsets, perm, case["gate"], case["up"], case["down"], soe)
        assert_act_close(g["act"], act)
        y_dev_act = ref.expert_down(g["act"], offsets, case["down"], slot_of_expert=soe)
        assert_close(g["y"], y_dev_act, "y (given device act)")
        assert_close(g["out"], ref.combine(y_dev_act, inv, w, k), "out (given device act)")
        if strict:
            assert_close(g["y"], y, "y")
            assert_close(g["out"], ref.combine(y, inv, w, k), "out")
    else:
        act, y = ref.expert_ffn_rows(case["x"], k, offsets, perm, rows, case["gate"], case["up"],
                                     case["down"], soe)
        assert_act_close(g["act"][rows], act)
        y_dev_act = ref.expert_down(g["act"][rows], offsets, case["down"], rows=rows, slot_of_expert=soe)
        assert_close(g["y"][rows], y_dev_act, "y (sampled rows, given device act)")
        if strict:
            assert_close(g["y"][rows], y, "y (sampled rows)")
        # combine checked on tokens whose every pair was sampled
        rowset = set(int(r) for r in rows)
        toks = [t for t in range(case["T"]) if all(int(inv[t * k + j]) in rowset for j in range(k))]
        if toks:
            ymap = {int(r): y_dev_act[i] for i, r in enumerate(rows)}
            out = np.stack([sum(w[t, j] * ymap[int(inv[t * k + j])] for j in range(k)) for t in toks])
            assert_close(g["out"][toks], out, "out (sampled tokens)")
        info["sampled_tokens"] = len(toks)
    info["active_experts"] = int(np.sum(np.diff(offsets) > 0))
    info["act_flips"] = int(np.sum(g["act"][rows if rows is not None else slice(None)] != act))
    return info


class HipGraph:
    """Stream capture into a HIP graph through the HIP runtime (no torch
    graph machinery): capture(fn, stream) records what fn enqueues on
    `stream`, launch(stream) replays it."""

    def __init__(self):
        import ctypes
        import os
        self._c = ctypes
        self.hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
        for name in ("hipStreamBeginCapture", "hipStreamEndCapture", "hipGraphInstantiate", "hipGraphLaunch",
                     "hipGraphExecDestroy", "hipGraphDestroy"):
            getattr(self.hip, name).restype = ctypes.c_int
        self.graph = ctypes.c_void_p()
        self.exe = ctypes.c_void_p()

    def _ok(self, rc, what):
        assert rc == 0, f"{what} returned hipError {rc}"

    def capture(self, fn, stream) -> None:
        c = self._c
        s = c.c_void_p(stream.cuda_stream)
        self._ok(self.hip.hipStreamBeginCapture(s, 1), "hipStreamBeginCapture")   # thread-local mode
        try:
            fn()
        finally:
            self._ok(self.hip.hipStreamEndCapture(s, c.byref(self.graph)), "hipStreamEndCapture")
        self._ok(self.hip.hipGraphInstantiate(c.byref(self.exe), self.graph, None, None, c.c_size_t(0)),
                 "hipGraphInstantiate")

    def launch(self, stream) -> None:
        self._ok(self.hip.hipGraphLaunch(self.exe, self._c.c_void_p(stream.cuda_stream)), "hipGraphLaunch")

    def close(self) -> None:
        if self.exe:
            self.hip.hipGraphExecDestroy(self.exe)
        if self.graph:
            self.hip.hipGraphDestroy(self.graph)
        self.exe = self._c.c_void_p()
        self.graph = self._c.c_void_p()
