"""Seeded synthetic inputs for the routed MoE layer.

This module only draws random inputs; it holds none of the layer's
arithmetic (no dequantisation, routing, sorting or matrix products).  Both the
GPU path's tests/bench and the CPU oracle consume the exact bytes it returns.

Every tensor i of workload c is drawn from its own stream
``numpy.random.default_rng(1000 * c + i)`` (plus ``seed_offset``), so the order
in which tensors are generated does not matter.

Workloads (d = hidden size, f = expert FFN size, E experts, top-k):

  0 tiny           T=4,    d=256,  E=8,  k=2, f=128,  MXFP4, logits given N(0,1)
  1 decode         T=1,    d=4096, E=64, k=2, f=2048, MXFP4, router on device
  2 spec-verify    T=5,    d=4096, E=64, k=2, f=2048, MXFP4, correlated tokens
  3 prefill chunk  T=2048, d=4096, E=64, k=2, f=2048, MXFP4, Zipf(1.1) router bias
  4 two-bit        T=16,   d=4096, E=64, k=2, f=2048, Q2,    Zipf(1.1) router bias
  (5-8: the 4-bit pack at 16 and 1 tokens, the 2-bit and 4-bit packs at the
  prefill chunk's size; not among the quoted configurations)

Value recipe:
  x        bf16(N(0,1))   (workload 2: bf16(base + 0.3 * noise_t), base/noise N(0,1))
  W_r      float32 N(0, 1/d)
  bias     b_e = -1.1 * ln(e + 1)  (log of a Zipf(s=1.1) prior over expert rank)
  MXFP4    codes uniform over all 16 e2m1 codes (each nibble), e8m0 scale bytes
           uniform over {119..123} (scales 2**-8 .. 2**-4)
  Q2       codes uniform over {0..3}, fp16 scale U[0.005, 0.02], fp16 min U[-0.04, 0]
  Q4       codes uniform over {0..15}, fp16 scale U[0.001, 0.004], fp16 min U[-0.04, 0]
           (the same weight range as Q2: 15 steps of a quarter of Q2's scale)
"""

from __future__ import annotations

import math

import numpy as np

WORKLOADS = {
    0: dict(name="tiny", T=4, d=256, E=8, k=2, f=128, fmt="mxfp4", router="given"),
    1: dict(name="decode", T=1, d=4096, E=64, k=2, f=2048, fmt="mxfp4", router="device"),
    2: dict(name="spec-verify", T=5, d=4096, E=64, k=2, f=2048, fmt="mxfp4", router="device",
            correlated=True),
    3: dict(name="prefill", T=2048, d=4096, E=64, k=2, f=2048, fmt="mxfp4", router="device",
            zipf=1.1),
    4: dict(name="two-bit", T=16, d=4096, E=64, k=2, f=2048, fmt="q2", router="device",
            zipf=1.1),
    # the 4-bit group-asymmetric pack (not among the quoted configurations)
    5: dict(name="four-bit", T=16, d=4096, E=64, k=2, f=2048, fmt="q4", router="device",
            zipf=1.1),
    6: dict(name="four-bit decode", T=1, d=4096, E=64, k=2, f=2048, fmt="q4", router="device"),
    # the prefill chunk with the 2-bit and 4-bit packs (not quoted configurations)
    7: dict(name="two-bit prefill", T=2048, d=4096, E=64, k=2, f=2048, fmt="q2", router="device", zipf=1.1),
    8: dict(name="four-bit prefill", T=2048, d=4096, E=64, k=2, f=2048, fmt="q4", router="device", zipf=1.1),
}

# stream ids within a workload
_S_X, _S_X2, _S_WR, _S_LOGITS = 0, 1, 2, 3
_S_MAT = {"gate": 10, "up": 20, "down": 30}
_S_SHARED = {"gate": 40, "up": 50, "down": 60}


def _rng(stream: int, seed: int) -> np.random.Generator:
    return np.random.default_rng(stream + seed)


def to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Nearest-even bf16 bit patterns of float32 samples (input preparation)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _fp16_bits(v: np.ndarray) -> np.ndarray:
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def make_matrix(fmt: str, slots: int, n: int, K: int, rng: np.random.Generator) -> dict:
    """Random quantised pack for `slots` experts of an n x K matrix (K contiguous)."""
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    if fmt == "mxfp4":
        codes = rng.integers(0, 256, size=(slots, n, K // 2), dtype=np.uint8)
        scales = rng.integers(119, 124, size=(slots, n, K // 32), dtype=np.uint8)
        return dict(fmt="mxfp4", codes=codes, scales=scales)
    if fmt == "q2":
        codes = rng.integers(0, 256, size=(slots, n, K // 4), dtype=np.uint8)
        scales = _fp16_bits(rng.uniform(0.005, 0.02, size=(slots, n, K // 32)))
        mins = _fp16_bits(rng.uniform(-0.04, 0.0, size=(slots, n, K // 32)))
        return dict(fmt="q2", codes=codes, scales=scales, mins=mins)
    if fmt == "q4":
        codes = rng.integers(0, 256, size=(slots, n, K // 2), dtype=np.uint8)
        scales = _fp16_bits(rng.uniform(0.001, 0.004, size=(slots, n, K // 32)))
        mins = _fp16_bits(rng.uniform(-0.04, 0.0, size=(slots, n, K // 32)))
        return dict(fmt="q4", codes=codes, scales=scales, mins=mins)
    raise ValueError(fmt)


def zipf_bias(E: int, s: float) -> np.ndarray:
    return np.array([-s * math.log(e + 1) for e in range(E)], dtype=np.float32)


def make_case(T: int, d: int, E: int, k: int, f: int, fmt: str = "mxfp4", *,
              router: str = "device", seed: int = 0, slots: int | None = None,
              zipf: float | None = None, correlated: bool = False) -> dict:
    """One seeded layer input.  router='given' draws float32 N(0,1) logits;
    router='device' draws W_r ~ N(0, 1/d) (and a Zipf bias if zipf is set)."""
    slots = E if slots is None else slots
    if correlated:
        base = _rng(_S_X, seed).standard_normal(d, dtype=np.float32)
        noise = _rng(_S_X2, seed).standard_normal((T, d), dtype=np.float32)
        xf = base[None, :] + np.float32(0.3) * noise
    else:
        xf = _rng(_S_X, seed).standard_normal((T, d), dtype=np.float32)
    case = dict(T=T, d=d, E=E, k=k, f=f, fmt=fmt, slots=slots, x=to_bf16_bits(xf),
                logits=None, w_router=None, bias=None)
    if router == "given":
        case["logits"] = _rng(_S_LOGITS, seed).standard_normal((T, E), dtype=np.float32)
    else:
        wr = _rng(_S_WR, seed).standard_normal((E, d), dtype=np.float32)
        case["w_router"] = (wr / np.float32(math.sqrt(d))).astype(np.float32)
        if zipf is not None:
            case["bias"] = zipf_bias(E, zipf)
    case["gate"] = make_matrix(fmt, slots, f, d, _rng(_S_MAT["gate"], seed))
    case["up"] = make_matrix(fmt, slots, f, d, _rng(_S_MAT["up"], seed))
    case["down"] = make_matrix(fmt, slots, d, f, _rng(_S_MAT["down"], seed))
    return case


def workload(c: int, seed_offset: int = 0) -> dict:
    """The seeded inputs of workload c (0..4)."""
    w = WORKLOADS[c]
    return make_case(w["T"], w["d"], w["E"], w["k"], w["f"], w["fmt"], router=w["router"],
                     seed=1000 * c + seed_offset, zipf=w.get("zipf"),
                     correlated=w.get("correlated", False))


def make_shared(case: dict, seed: int = 0) -> dict:
    """A shared expert for `case`: one slot of gate/up/down packs in the
    case's format, drawn like the routed experts from streams of their own."""
    fmt, d, f = case["fmt"], case["d"], case["f"]
    return {"gate": make_matrix(fmt, 1, f, d, _rng(_S_SHARED["gate"], seed)),
            "up": make_matrix(fmt, 1, f, d, _rng(_S_SHARED["up"], seed)),
            "down": make_matrix(fmt, 1, d, f, _rng(_S_SHARED["down"], seed))}
