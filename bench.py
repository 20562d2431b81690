"""Benchmark of the routed MoE layer on one MI355X.

A step is one pass of the whole layer -- router logits, top-k, dispatch,
fused-dequant SwiGLU expert FFN, combine -- over one batch of tokens, with
every input already resident in HBM.  Consecutive steps use different weight
pools ("layers") and different token batches, cycling through enough pools
that a layer's experts are evicted from the 256 MB Infinity Cache before the
layer comes round again (as in a real decode pass over a deep MoE model).

Timed regions over the same K steps: (1) the one-call layer, moe_layer,
enqueued call by call from Python (eager_ms_per_step); (1g) the same K
calls captured once into a HIP graph and replayed -- its throughput is
`value` (tokens/s) and ms_per_step; (2) the four entry points with HIP
events around moe_expert_ffn on the launch stream -- the average FFN
duration gives the roofline figure.

Prints ONE JSON line.  Headline workload: decode, T=1, d=4096, E=64, k=2,
f=2048, MXFP4 experts; by default the same line also carries a `workloads`
map with every quoted configuration (0-4: tiny, decode, verify, prefill,
two-bit), each with its own value, roofline and oracle baseline, and
`measured_peaks`: this box's cold HBM read stream, a decode-sized cold
stream replayed from a HIP graph, and the dense bf16, fp4 x fp8 and
fp4 x fp4 matrix loops (include/moe_peak.h), against which every roofline
also reports `frac_measured`.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 0..8]

Workloads 0-4 are the configurations the targets are quoted on; 5 and 6
run the 4-bit group-asymmetric pack at 16 tokens and at 1 token, 7 and 8 the
2-bit and 4-bit packs at the prefill chunk's size (2048 tokens).  --bank N
runs the workload through an N-slot expert bank paged from pinned host
memory instead (its own JSON line: paging included, PCIe roofline);
--shared adds an always-on shared expert (moe_layer_shared; its own JSON line);
--mx8 / --mx4 run the prefill with MXFP8 / MXFP4 activations.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0         # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
MFMA_FP8_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 matrix, published (the fp4 x fp8 products run at it)
MFMA_FP4_PEAK_TFLOPS = 10100.0  # MI355X dense fp4 / fp6 matrix, published (the fp4 x fp4 products)
METRIC = "MoE layer tokens/s; decode weight-stream GB/s; prefill expert TFLOP/s"

# HBM bytes per moe_expert_ffn call from rocprofv3 counter runs of the current
# FFN kernels (--pmc FETCH_SIZE, then --pmc WRITE_SIZE, one dispatch each;
# FETCH_SIZE x 2.0 and WRITE_SIZE x 1.0 KiB, the factors a plain 256 MiB copy
# reads), summed over the kernels of the call.  Workloads 3, 4, 7 and 8 route a
# different number of experts each step: theirs is the average of the counted
# steps.  Must be re-measured (or removed) whenever an FFN kernel changes.
MEASURED_FFN_TRAFFIC = {
    0: (2 * (213.0 + 113.0) + (2.0 + 8.0)) * 1024,
    1: (2 * (13158.0 + 4435.2) + (8.0 + 32.0)) * 1024,
    2: (2 * (18469.3 + 9103.3) + (40.0 + 160.0)) * 1024,
    3: (2 * 422740.3 + 98328.8) * 1024,
    4: (2 * (27882.0 + 14209.4) + (310.9 + 512.0)) * 1024,
    5: (2 * (43124.4 + 19622.7) + (310.9 + 512.0)) * 1024,
    6: (2 * (15467.8 + 5203.2) + (8.0 + 32.0)) * 1024,
    7: (2 * (8211.1 + 292317.6) + (1024.0 + 90128.4)) * 1024,
    8: (2 * (8211.2 + 483074.4) + (1024.0 + 90129.0)) * 1024,
}

MX_BYTES_PER_EXPERT = lambda d, f: 3 * d * f // 2 + 3 * d * f // 32      # codes + e8m0 scales
Q2_BYTES_PER_EXPERT = lambda d, f: 3 * d * f // 4 + 3 * d * f // 32 * 4  # codes + fp16 scale + min
Q4_BYTES_PER_EXPERT = lambda d, f: 3 * d * f // 2 + 3 * d * f // 32 * 4  # codes + fp16 scale + min
BYTES_PER_EXPERT = {"mxfp4": MX_BYTES_PER_EXPERT, "q2": Q2_BYTES_PER_EXPERT, "q4": Q4_BYTES_PER_EXPERT}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    import synthetic
    p.add_argument("--workload", type=int, default=None, choices=sorted(synthetic.WORKLOADS),
                   help="one workload only (default: workload 1 as the headline, plus every quoted "
                        "configuration 0-4 in a `workloads` map of the same line)")
    p.add_argument("--no-peaks", action="store_true",
                   help="skip the measured stream and matrix-core peaks (include/moe_peak.h)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--mx8", action="store_true",
                   help="MXFP8 activations on the block-scaled fp4 x fp8 matrix cores (moe_layer_mx8)")
    p.add_argument("--mx4", action="store_true",
                   help="MXFP4 activations on the block-scaled fp4 x fp4 matrix cores (moe_layer_mx4)")
    p.add_argument("--shared", action="store_true",
                   help="run the workload with a shared expert (moe_layer_shared)")
    p.add_argument("--bank", type=int, default=0, metavar="N",
                   help="run the workload through an N-slot expert bank paged from pinned host memory")
    p.add_argument("--cpu-sample-steps", type=int, default=0,
                   help="oracle steps timed on the host (0 = automatic)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="instead of the layer: copy MIB MiB device-to-device 5 times (a plain copy "
                        "of known size, to scale the FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


def copy_calibration(mib: int) -> None:
    import torch

    n = mib * 2 ** 20
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 5}), flush=True)


def make_pool(torch, w, gen, dev):
    """One layer's experts on the device: uniform codes, scales as in the
    synthetic recipe (e8m0 bytes 119..123; Q2 fp16 scale U[.005,.02], min
    U[-.04,0]; Q4 fp16 scale U[.001,.004], min U[-.04,0])."""
    import quantized_routed_moe_amd as qm

    E, d, f = w["E"], w["d"], w["f"]

    def mat(n, K):
        # drawn in the row layout, then re-laid into the tile layout the
        # kernels read (moe_pack_qmat); the row copy is dropped
        if w["fmt"] == "mxfp4":
            codes = torch.randint(0, 256, (E, n, K // 2), dtype=torch.uint8, device=dev, generator=gen)
            scales = torch.randint(119, 124, (E, n, K // 32), dtype=torch.uint8, device=dev, generator=gen)
            rows = qm.QMat(codes, scales, None, qm.MOE_LAYOUT_ROWS)
        else:
            q2 = w["fmt"] == "q2"
            codes = torch.randint(0, 256, (E, n, K // 4 if q2 else K // 2), dtype=torch.uint8, device=dev, generator=gen)
            lo, span = (0.005, 0.015) if q2 else (0.001, 0.003)
            sc = (torch.rand((E, n, K // 32), device=dev, generator=gen) * span + lo).half().view(torch.int16)
            mn = (torch.rand((E, n, K // 32), device=dev, generator=gen) * -0.04).half().view(torch.int16)
            rows = qm.QMat(codes, sc.contiguous(), mn.contiguous(), qm.MOE_LAYOUT_ROWS)
        return qm.pack_qmat(w["fmt"], rows, E, n, K)

    return qm.Experts(w["fmt"], mat(f, d), mat(f, d), mat(d, f), None, E, d, f)


def cpu_baseline(c, steps):
    """The oracle as it stands, timed on this host on `steps` seeded steps of
    the same workload (input generation excluded)."""
    import numpy as np

    import synthetic
    from oracle import ref

    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        blas = 1
    total, tokens = 0.0, 0
    for i in range(steps):
        case = synthetic.workload(c, seed_offset=17 + i)
        t0 = time.perf_counter()
        ref.layer(case["x"], case["k"], case["gate"], case["up"], case["down"], logits=case["logits"],
                  w_router=case["w_router"], bias=case["bias"])
        total += time.perf_counter() - t0
        tokens += case["T"]
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    return dict(value=tokens / total, unit="tokens/s", cores=int(blas), kind="oracle",
                sample=f"{steps} seeded step(s) of the workload ({tokens} tokens), NumPy float64 oracle, "
                       f"{total:.1f} s of host time; input generation not timed; BLAS threads {blas} of "
                       f"{affinity} cores in the process affinity mask")


def bank_main(args):
    """--bank N: K layer calls of the workload through an N-slot expert bank
    whose misses are copied from a pinned host pool of all E experts (one
    layer).  Each call synchronises once (the host learns which experts have
    rows), so the calls run eagerly.  `value` includes the paging; the
    roofline figure is the host -> device copy rate of moe_bank_fetch against
    PCIe 5.0 x16 (63 GB/s per direction)."""
    import ctypes

    import numpy as np
    import torch

    import quantized_routed_moe_amd as qm
    import synthetic

    c, N = args.workload, args.bank
    w = synthetic.WORKLOADS[c]
    T, d, E, k, f = w["T"], w["d"], w["E"], w["k"], w["f"]
    if not 1 <= N <= E:
        raise SystemExit(f"--bank must be in 1..{E}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1000 * c + 321)
    pool = make_pool(torch, w, gen, dev)
    bank = qm.SlotBank(pool, N, dev)
    del pool
    torch.cuda.empty_cache()
    wr = (torch.randn((E, d), device=dev, generator=gen) / math.sqrt(d)).contiguous()
    b = torch.from_numpy(synthetic.zipf_bias(E, w["zipf"])).to(dev) if w.get("zipf") else None
    n_x = 4 if T >= 1024 else 61
    xs = torch.randn((n_x, T, d), device=dev, generator=gen).to(torch.bfloat16).view(torch.int16).contiguous()
    shape = qm.Shape(T, d, E, k, f)
    ws = qm.alloc_workspace(shape, layer=True, device=dev)
    for i in range(args.warmup):
        bank.layer(xs[i % n_x], k, w_router=wr, bias=b, ws=ws)
    torch.cuda.synchronize()
    K = args.steps
    tot = dict(active=0, hits=0, misses=0, passes=0, bytes_paged=0)
    t0 = time.perf_counter()
    for i in range(K):
        bank.layer(xs[(args.warmup + i) % n_x], k, w_router=wr, bias=b, ws=ws)
        for n in tot:
            tot[n] += bank.last_stats[n]
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert qm.moe_read_device_status(ws) == 0

    # the copy engine alone: moe_bank_fetch of min(N, 8) experts, HIP events
    L = qm.lib()
    hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
    stream = torch.cuda.current_stream().cuda_stream
    n_f = min(N, 8)
    le = (ctypes.c_int32 * n_f)(*range(n_f))
    ls = (ctypes.c_int32 * n_f)(*range(n_f))
    sl = bank.slots.c()
    per_expert = BYTES_PER_EXPERT[w["fmt"]](d, f)
    ev = [ctypes.c_void_p(), ctypes.c_void_p()]
    for e_ in ev:
        hip.hipEventCreate(ctypes.byref(e_))
    rates = []
    for _ in range(5):
        hip.hipEventRecord(ev[0], ctypes.c_void_p(stream))
        if L.moe_bank_fetch(ctypes.byref(bank.pool_c), ctypes.byref(sl), d, f, le, ls, n_f, ctypes.c_void_p(stream)):
            raise RuntimeError("moe_bank_fetch failed")
        hip.hipEventRecord(ev[1], ctypes.c_void_p(stream))
        hip.hipEventSynchronize(ev[1])
        ms = ctypes.c_float()
        hip.hipEventElapsedTime(ctypes.byref(ms), ev[0], ev[1])
        rates.append(n_f * per_expert / (ms.value / 1e3) / 1e9)
    for e_ in ev:
        hip.hipEventDestroy(e_)
    # the fetched slots now hold experts 0..n_f-1: the bank's books are stale
    bank.state = qm.BankState(E, N)
    pcie = float(np.median(rates))
    peak = 63.0
    res = {
        "metric": "MoE layer tokens/s through an expert slot bank (paging included)",
        "value": round(T * K / elapsed, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / K * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w['name']} through a {N}-slot bank: T={T} d={d} E={E} k={k} f={f} {w['fmt']}",
                   "T": T, "d": d, "E": E, "k": k, "f": f, "format": w["fmt"], "bank_slots": N,
                   "parallelism": "none (1 GPU)"},
        "launch": "eager; one host synchronisation per call",
        "bank": {"hit_rate": round(tot["hits"] / max(tot["active"], 1), 4),
                 "misses_per_call": round(tot["misses"] / K, 3), "passes_per_call": round(tot["passes"] / K, 3),
                 "bytes_paged_per_call": round(tot["bytes_paged"] / K),
                 "device_bytes": N * per_expert, "pool_host_bytes": E * per_expert},
        "roofline": {"bound": "pcie", "achieved": round(pcie, 2), "peak": peak, "unit": "GB/s",
                     "frac": round(pcie / peak, 4), "traffic": None,
                     "kernel": f"moe_bank_fetch of {n_f} experts (host -> device DMA)"},
    }
    print(json.dumps(res), flush=True)


def shared_main(args):
    """--shared: K layer steps of moe_layer_shared (the routed experts plus an
    always-on shared expert of the same format and size), captured into a HIP
    graph and replayed, as `value` in main().  The roofline divides the
    algorithmic bytes (or flops) of all experts the step runs, shared expert
    included, by the whole layer step: a lower bound for the FFN's own rate."""
    import ctypes

    import numpy as np
    import torch

    import quantized_routed_moe_amd as qm
    import synthetic

    c = args.workload
    w = synthetic.WORKLOADS[c]
    T, d, E, k, f = w["T"], w["d"], w["E"], w["k"], w["f"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1000 * c + 555)
    per_expert = BYTES_PER_EXPERT[w["fmt"]](d, f)
    n_pools = max(2, min(24, 1 + math.ceil(512 * 2 ** 20 / ((min(E, max(2, T * k)) + 1) * per_expert))))
    pools = [make_pool(torch, w, gen, dev) for _ in range(n_pools)]
    shareds = [make_pool(torch, dict(w, E=1), gen, dev) for _ in range(n_pools)]
    routers = []
    for _ in range(n_pools):
        wr = torch.randn((E, d), device=dev, generator=gen) / math.sqrt(d)
        b = torch.from_numpy(synthetic.zipf_bias(E, w["zipf"])).to(dev) if w.get("zipf") else None
        routers.append((wr.contiguous(), b))
    n_x = 4 if T >= 1024 else 61
    xs = torch.randn((n_x, T, d), device=dev, generator=gen).to(torch.bfloat16).view(torch.int16).contiguous()
    shape = qm.Shape(T, d, E, k, f)
    L = qm.lib()
    sc = shape.c()
    ws = torch.empty(int(L.moe_layer_shared_workspace_bytes(ctypes.byref(sc))), dtype=torch.uint8, device=dev)
    qm.moe_workspace_init(ws)
    logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, k), dtype=torch.float32, device=dev)
    out = torch.empty((T, d), dtype=torch.float32, device=dev)
    hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
    torch.cuda.synchronize()
    torch.cuda.set_stream(torch.cuda.Stream())
    stream = torch.cuda.current_stream().cuda_stream
    ex_c = [p_.c() for p_ in pools]
    sh_c = [p_.c() for p_ in shareds]

    def layer_step(j):
        p = j % n_pools
        wr, b = routers[p]
        if L.moe_layer_shared(ctypes.byref(sc), xs.data_ptr() + (j % n_x) * T * d * 2, wr.data_ptr(),
                              None if b is None else b.data_ptr(), logits.data_ptr(), ctypes.byref(ex_c[p]),
                              ctypes.byref(sh_c[p]), ids.data_ptr(), tw.data_ptr(), out.data_ptr(), ws.data_ptr(),
                              ws.numel(), stream):
            raise RuntimeError("moe_layer_shared failed")

    for i in range(args.warmup):
        layer_step(i)
    torch.cuda.synchronize()
    K = args.steps
    t0 = time.perf_counter()
    for i in range(K):
        layer_step(args.warmup + i)
    torch.cuda.synchronize()
    eager = time.perf_counter() - t0
    for fn in ("hipStreamBeginCapture", "hipStreamEndCapture", "hipGraphInstantiate", "hipGraphLaunch"):
        getattr(hip, fn).restype = ctypes.c_int
    graph, gexec = ctypes.c_void_p(), ctypes.c_void_p()
    sp = ctypes.c_void_p(stream)
    if hip.hipStreamBeginCapture(sp, 1):
        raise RuntimeError("hipStreamBeginCapture failed")
    try:
        for i in range(K):
            layer_step(args.warmup + i)
    finally:
        if hip.hipStreamEndCapture(sp, ctypes.byref(graph)):
            raise RuntimeError("hipStreamEndCapture failed")
    if hip.hipGraphInstantiate(ctypes.byref(gexec), graph, None, None, ctypes.c_size_t(0)):
        raise RuntimeError("hipGraphInstantiate failed")
    hip.hipGraphLaunch(gexec, sp)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    hip.hipGraphLaunch(gexec, sp)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    hip.hipGraphExecDestroy(gexec)
    hip.hipGraphDestroy(graph)
    assert qm.moe_read_device_status(ws) == 0
    # activated routed experts per step (routing replayed untimed)
    U = []
    wsr = qm.alloc_workspace(shape, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    inv = torch.empty(T * k, dtype=torch.int32, device=dev)
    for i in range(K):
        j = args.warmup + i
        wr, b = routers[j % n_pools]
        qm.moe_route_topk(shape, xs[j % n_x], wr, b, logits, ids, tw)
        qm.moe_dispatch(shape, ids, offsets, perm, inv, wsr)
        U.append(int((offsets[1:] - offsets[:-1] > 0).sum().item()))
    U_mean = float(np.mean(U))
    step_s = elapsed / K
    rows = T * k + T
    layer_bytes = (U_mean + 1) * per_expert + T * d * 2 + rows * f * 4 + rows * d * 8 + T * d * 4
    flops = 2.0 * rows * 3 * d * f
    if T * k >= 1024:
        ach, peak, unit, bound = flops / step_s / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s", "mfma"
    else:
        ach, peak, unit, bound = layer_bytes / step_s / 1e9, HBM_PEAK_GBPS, "GB/s", "hbm"
    res = {
        "metric": "MoE layer tokens/s with a shared expert",
        "value": round(T * K / elapsed, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w['name']} + shared expert: T={T} d={d} E={E} k={k} f={f} {w['fmt']}",
                   "T": T, "d": d, "E": E, "k": k, "f": f, "format": w["fmt"], "shared_experts": 1,
                   "weight_pools": n_pools, "parallelism": "none (1 GPU)"},
        "launch": "HIP graph of the K steps, replayed once",
        "eager_ms_per_step": round(eager / K * 1e3, 5),
        "active_experts_mean": U_mean,
        "roofline": {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
                     "frac": round(ach / peak, 4), "traffic": None,
                     "kernel": "moe_layer_shared, whole layer step (routed + shared experts' work / step time)"},
    }
    print(json.dumps(res), flush=True)


def _hip(torch):
    import ctypes
    hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
    for fn in ("hipStreamBeginCapture", "hipStreamEndCapture", "hipGraphInstantiate", "hipGraphLaunch",
               "hipGraphExecDestroy", "hipGraphDestroy", "hipEventCreate", "hipEventRecord",
               "hipEventSynchronize", "hipEventElapsedTime", "hipEventDestroy", "hipMemcpyAsync"):
        getattr(hip, fn).restype = ctypes.c_int
    return hip


class Events:
    """HIP event pairs recorded on a raw stream (torch.cuda.Event sees only
    torch's current stream)."""

    def __init__(self, hip, n):
        import ctypes
        self.c, self.hip = ctypes, hip
        self.ev = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            hip.hipEventCreate(ctypes.byref(a))
            hip.hipEventCreate(ctypes.byref(b))
            self.ev.append((a, b))

    def ms(self):
        out = []
        for a, b in self.ev:
            m = self.c.c_float()
            self.hip.hipEventElapsedTime(self.c.byref(m), a, b)
            out.append(m.value)
        return out

    def close(self):
        for a, b in self.ev:
            self.hip.hipEventDestroy(a)
            self.hip.hipEventDestroy(b)
        self.ev = []


def capture_replay(hip, stream, fn, K):
    """fn(i) for i < K captured once into a HIP graph on `stream` (a created
    stream), replayed once to warm, then timed over one replay (seconds)."""
    import ctypes

    import torch

    graph, gexec = ctypes.c_void_p(), ctypes.c_void_p()
    sp = ctypes.c_void_p(stream)

    def ok(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} returned hipError {rc}")

    ok(hip.hipStreamBeginCapture(sp, 1), "hipStreamBeginCapture")       # thread-local capture
    try:
        for i in range(K):
            fn(i)
    finally:
        ok(hip.hipStreamEndCapture(sp, ctypes.byref(graph)), "hipStreamEndCapture")
    ok(hip.hipGraphInstantiate(ctypes.byref(gexec), graph, None, None, ctypes.c_size_t(0)), "hipGraphInstantiate")
    ok(hip.hipGraphLaunch(gexec, sp), "hipGraphLaunch")                  # warm replay
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ok(hip.hipGraphLaunch(gexec, sp), "hipGraphLaunch")
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    hip.hipGraphExecDestroy(gexec)
    hip.hipGraphDestroy(graph)
    return elapsed


def measure_peaks(stream_bytes_decode):
    """Measured roofline of this box, in this process (include/moe_peak.h):
      * hbm_GBps: one cold 1 GiB read stream (the Infinity Cache evicted by
        reading another 1 GiB first), median of 5, event-timed;
      * hbm_GBps_decode_stream: K back-to-back reads of `stream_bytes_decode`
        bytes (the decode FFN call's algorithmic bytes), each from a
        different buffer (24 buffers, > 256 MB, so every read is cold),
        replayed from a HIP graph -- the rate a kernel of that size can
        reach, launch included;
      * bf16_TFLOPs / fp8_TFLOPs / fp4_TFLOPs: the dense matrix-core loops
        (bf16 32x32x16, scaled fp4 x fp8 and fp4 x fp4 32x32x64), median of 5."""
    import ctypes

    import numpy as np
    import torch

    import quantized_routed_moe_amd as qm

    L = qm.lib()
    hip = _hip(torch)
    torch.cuda.synchronize()
    torch.cuda.set_stream(torch.cuda.Stream())
    stream = torch.cuda.current_stream().cuda_stream
    sp = ctypes.c_void_p(stream)
    big = 1 << 30
    bufs = [torch.empty(big, dtype=torch.uint8, device="cuda") for _ in range(2)]
    for b in bufs:
        b.fill_(7)
    sink = torch.empty(1 << 16, dtype=torch.int32, device="cuda")
    ev = Events(hip, 5)
    for i, (a, b) in enumerate(ev.ev):
        if L.moe_peak_stream(bufs[(i + 1) % 2].data_ptr(), big, 0, sink.data_ptr(), sp):   # evict
            raise RuntimeError("moe_peak_stream failed")
        hip.hipEventRecord(a, sp)
        if L.moe_peak_stream(bufs[i % 2].data_ptr(), big, 0, sink.data_ptr(), sp):
            raise RuntimeError("moe_peak_stream failed")
        hip.hipEventRecord(b, sp)
    torch.cuda.synchronize()
    hbm = big / (float(np.median(ev.ms())) / 1e3) / 1e9
    ev.close()
    del bufs
    # decode-sized cold streams replayed from a graph
    nb = stream_bytes_decode // 16 * 16
    small = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(24)]
    for b in small:
        b.fill_(3)
    K = 48
    secs = capture_replay(hip, stream, lambda i: L.moe_peak_stream(small[i % 24].data_ptr(), nb, 0,
                                                                    sink.data_ptr(), sp), K)
    dec = nb * K / secs / 1e9
    del small
    torch.cuda.empty_cache()
    res = {"hbm_GBps": round(hbm, 1), "hbm_GBps_decode_stream": round(dec, 1),
           "decode_stream_bytes": nb, "decode_stream_us": round(secs / K * 1e6, 3)}
    fsink = torch.empty(4096, dtype=torch.float32, device="cuda")
    for kind, name, per in ((0, "bf16_TFLOPs", 32768), (1, "fp8_TFLOPs", 131072), (2, "fp4_TFLOPs", 131072)):
        iters = {0: 4000, 1: 2000, 2: 4000}[kind]
        ev = Events(hip, 5)
        L.moe_peak_mfma(kind, iters, 0, fsink.data_ptr(), sp)           # warm
        for a, b in ev.ev:
            hip.hipEventRecord(a, sp)
            if L.moe_peak_mfma(kind, iters, 0, fsink.data_ptr(), sp):
                raise RuntimeError("moe_peak_mfma failed")
            hip.hipEventRecord(b, sp)
        torch.cuda.synchronize()
        flop = 1024 * 4 * iters * 8 * per
        res[name] = round(flop / (float(np.median(ev.ms())) / 1e3) / 1e12, 1)
        ev.close()
    return res


def run_workload(c, args, mx=0, peaks=None, cpu=True):
    """Times workload c (see the module docstring): returns its result dict
    (value, ms_per_step, roofline, cpu_baseline, ...)."""
    import ctypes

    import numpy as np
    import torch

    import quantized_routed_moe_amd as qm
    import synthetic

    w = synthetic.WORKLOADS[c]
    T, d, E, k, f = w["T"], w["d"], w["E"], w["k"], w["f"]
    shape = qm.Shape(T, d, E, k, f)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1000 * c + 123)

    per_expert = BYTES_PER_EXPERT[w["fmt"]](d, f)
    touched_guess = min(E, max(2, T * k)) * per_expert
    n_pools = 1 + math.ceil(512 * 2 ** 20 / touched_guess)
    n_pools = max(2, min(n_pools, 24))
    pools = [make_pool(torch, w, gen, dev) for _ in range(n_pools)]
    routers = []
    for _ in range(n_pools):
        if w["router"] == "given":
            routers.append(None)
        else:
            wr = torch.randn((E, d), device=dev, generator=gen) / math.sqrt(d)
            b = torch.from_numpy(synthetic.zipf_bias(E, w["zipf"])).to(dev) if w.get("zipf") else None
            routers.append((wr.contiguous(), b))
    n_x = 4 if T >= 1024 else 61
    if w.get("correlated"):
        base = torch.randn((n_x, 1, d), device=dev, generator=gen)
        xs = (base + 0.3 * torch.randn((n_x, T, d), device=dev, generator=gen)).to(torch.bfloat16)
    else:
        xs = torch.randn((n_x, T, d), device=dev, generator=gen).to(torch.bfloat16)
    xs = xs.view(torch.int16).contiguous()
    given = torch.randn((n_x, T, E), device=dev, generator=gen) if w["router"] == "given" else None

    logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, k), dtype=torch.float32, device=dev)
    offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    perm = torch.empty((T * k,), dtype=torch.int32, device=dev)
    inv = torch.empty((T * k,), dtype=torch.int32, device=dev)
    y = torch.empty((T * k, d), dtype=torch.float32, device=dev)
    out = torch.empty((T, d), dtype=torch.float32, device=dev)
    if mx and (w["fmt"] != "mxfp4" or d % 512 or f % 256):
        raise SystemExit(f"--mx{mx} needs MXFP4 experts with d % 512 == 0 and f % 256 == 0")
    ws = (qm.alloc_workspace_mx8(shape, layer=True, device=dev) if mx == 8 else
          qm.alloc_workspace_mx4(shape, layer=True, device=dev) if mx == 4 else
          qm.alloc_workspace(shape, layer=True, device=dev))

    # Raw C-ABI calls with precomputed arguments keep the host far ahead of
    # the GPU, so HIP event pairs measure kernels, not launch latency.
    L = qm.lib()
    hip = _hip(torch)
    # a created stream (default priority): the legacy null stream cannot be
    # captured; what was enqueued so far is finished first
    torch.cuda.synchronize()
    torch.cuda.set_stream(torch.cuda.Stream())
    stream = torch.cuda.current_stream().cuda_stream
    sc = shape.c()
    sh = ctypes.byref(sc)
    ex_c = [p_.c() for p_ in pools]
    ex_ref = [ctypes.byref(e) for e in ex_c]
    xb, xstride = xs.data_ptr(), T * d * 2
    lg_p, ids_p, tw_p = logits.data_ptr(), ids.data_ptr(), tw.data_ptr()
    off_p, perm_p, inv_p = offsets.data_ptr(), perm.data_ptr(), inv.data_ptr()
    y_p, out_p, ws_p, ws_n = y.data_ptr(), out.data_ptr(), ws.data_ptr(), ws.numel()
    ffn_ws_n = (int(getattr(L, f"moe_workspace_bytes_mx{mx}")(ctypes.byref(shape.c()))) if mx else
                qm.moe_workspace_bytes(shape))
    ffn_call = getattr(L, f"moe_expert_ffn_mx{mx}") if mx else L.moe_expert_ffn
    layer_call = getattr(L, f"moe_layer_mx{mx}") if mx else L.moe_layer
    wr_p = [None if r is None else r[0].data_ptr() for r in routers]
    b_p = [None if (r is None or r[1] is None) else r[1].data_ptr() for r in routers]
    given_p = None if given is None else given.data_ptr()

    def set_logits(j):
        if given is not None:    # given router logits are an input: copy them in
            hip.hipMemcpyAsync(ctypes.c_void_p(lg_p), ctypes.c_void_p(given_p + (j % n_x) * T * E * 4),
                               ctypes.c_size_t(T * E * 4), 3, ctypes.c_void_p(stream))

    def step(j, ev=None):
        p = j % n_pools
        xp = xb + (j % n_x) * xstride
        set_logits(j)
        rc = L.moe_route_topk(sh, xp, wr_p[p], b_p[p], lg_p, ids_p, tw_p, stream)
        rc |= L.moe_dispatch(sh, ids_p, off_p, perm_p, inv_p, ws_p, ws_n, stream)
        if ev is not None:
            hip.hipEventRecord(ev[0], ctypes.c_void_p(stream))
        rc |= ffn_call(sh, xp, ex_ref[p], off_p, perm_p, y_p, ws_p, ffn_ws_n, stream)
        if ev is not None:
            hip.hipEventRecord(ev[1], ctypes.c_void_p(stream))
        rc |= L.moe_combine(sh, y_p, inv_p, tw_p, out_p, stream)
        if rc:
            raise RuntimeError("a C-ABI call failed")

    def layer_step(j):
        p = j % n_pools
        set_logits(j)
        if layer_call(sh, xb + (j % n_x) * xstride, wr_p[p], b_p[p], lg_p, ex_ref[p], ids_p, tw_p, out_p,
                      ws_p, ws_n, stream):
            raise RuntimeError("moe_layer failed")

    for i in range(args.warmup):
        layer_step(i)
        step(i)
    torch.cuda.synchronize()
    K = args.steps

    # Timed region 1 (eager): K steps of the one-call layer, moe_layer, each
    # call enqueued from Python.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        layer_step(args.warmup + i)
    torch.cuda.synchronize()
    eager_elapsed = time.perf_counter() - t0

    # Timed region 1g (value): the same K steps captured once into a HIP
    # graph and replayed.  Every kernel of every step runs; the graph only
    # removes the per-launch work of the command processor between the
    # dependent launches (decode steps are a few launches of a few us each).
    elapsed = capture_replay(hip, stream, lambda i: layer_step(args.warmup + i), K)

    # Timed region 2 (roofline): the same K steps through the four entry
    # points, with HIP events around moe_expert_ffn on the same stream.  A
    # hold kernel first keeps the stream busy while the host enqueues the
    # steps (it is slower per step than the GPU at small T), so the steps
    # then run back to back from the queue and each event pair times the
    # FFN call's kernels, not gaps waiting for the host.  Untimed steps
    # worth ~20 ms of GPU time (from the graph's step time) run first: after
    # the idle hold the clocks take some milliseconds to settle (at the
    # prefill chunk the first ~30 calls measured 10-30 % slower).  The
    # four-call step time comes from one more event pair around the loop.
    n_settle = min(4 * K, max(args.warmup, int(0.02 / (elapsed / K)) + 1))
    evs = Events(hip, K + 1)
    torch.cuda.synchronize()
    if L.moe_peak_hold(min(1000000, 100 * (K + n_settle) + 2000), stream):
        raise RuntimeError("moe_peak_hold failed")
    for i in range(n_settle):
        step(args.warmup + i)
    hip.hipEventRecord(evs.ev[K][0], ctypes.c_void_p(stream))
    for i in range(K):
        step(args.warmup + i, evs.ev[i])
    hip.hipEventRecord(evs.ev[K][1], ctypes.c_void_p(stream))
    torch.cuda.synchronize()
    all_ms = evs.ms()
    ffn_ms, steps_elapsed = all_ms[:K], all_ms[K] / 1e3
    evs.close()
    assert qm.moe_read_device_status(ws) == 0

    # activated experts per timed step (routing replayed untimed; it is deterministic)
    U = []
    for i in range(K):
        j = args.warmup + i
        p = j % n_pools
        set_logits(j)
        L.moe_route_topk(sh, xb + (j % n_x) * xstride, wr_p[p], b_p[p], lg_p, ids_p, tw_p, stream)
        L.moe_dispatch(sh, ids_p, off_p, perm_p, inv_p, ws_p, ws_n, stream)
        U.append(int((offsets[1:] - offsets[:-1] > 0).sum().item()))
    U_mean = float(np.mean(U))

    weight_bytes = U_mean * per_expert
    if mx:   # x read, token codes write+read, act codes write+read, y write (scale bytes left out)
        act_bytes = T * d * 2 + (T * k * d + T * k * f) * mx // 8 * 2 + T * k * d * 4
    else:    # x read, act write+read, y write
        act_bytes = T * d * 2 + T * k * f * 2 * 2 + T * k * d * 4
    ffn_bytes = weight_bytes + act_bytes
    ffn_avg_s = float(np.mean(ffn_ms)) / 1e3
    flops = 2.0 * T * k * 3 * d * f
    gbps = ffn_bytes / ffn_avg_s / 1e9
    tflops = flops / ffn_avg_s / 1e12

    traffic = MEASURED_FFN_TRAFFIC.get(c)
    traffic = None if traffic is None else round(traffic)
    if mx:
        traffic = None
    if T * k >= 1024:
        peak = {8: MFMA_FP8_PEAK_TFLOPS, 4: MFMA_FP4_PEAK_TFLOPS}.get(mx, MFMA_BF16_PEAK_TFLOPS)
        roof = dict(bound="mfma", achieved=round(tflops, 2), peak=peak, unit="TFLOP/s",
                    frac=round(tflops / peak, 4), traffic=traffic)
        mpeak = None if peaks is None else peaks.get({8: "fp8_TFLOPs", 4: "fp4_TFLOPs"}.get(mx, "bf16_TFLOPs"))
        if mpeak:
            roof["measured_peak"] = mpeak
            roof["frac_measured"] = round(tflops / mpeak, 4)
        roof["hbm_GBps_of_call"] = round(gbps, 1)
    else:
        roof = dict(bound="hbm", achieved=round(gbps, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=round(gbps / HBM_PEAK_GBPS, 4), traffic=traffic)
        if peaks is not None:
            roof["measured_peak"] = peaks["hbm_GBps"]
            roof["frac_measured"] = round(gbps / peaks["hbm_GBps"], 4)
    roof["traffic_unit"] = "HBM bytes per call (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
    roof["kernel"] = (f"moe_expert_ffn_mx{mx} (token quantisation, then one launch of block-scaled fp4 x fp{mx} tiles)" if mx
                      else "moe_expert_ffn (one launch: gate/up + SwiGLU tiles, then down tiles)" if T * k >= 256 and w["fmt"] == "mxfp4"
                      else "moe_expert_ffn (token group sums, then one launch: gate/up + SwiGLU tiles, then down tiles)"
                      if T * k >= 256
                      else "moe_expert_ffn (gate/up + SwiGLU kernel, down kernel)")
    roof["algorithmic_bytes_per_launch"] = round(ffn_bytes)
    roof["algorithmic_flop_per_launch"] = round(flops)
    roof["avg_launch_ms"] = round(ffn_avg_s * 1e3, 5)
    p10, p50, p90 = np.percentile(np.asarray(ffn_ms) * 1e3, [10, 50, 90])
    roof["launch_us_p10_p50_p90"] = [round(float(p10), 2), round(float(p50), 2), round(float(p90), 2)]

    res = {
        "value": round(T * K / elapsed, 2),
        "unit": "tokens/s",
        "ms_per_step": round(elapsed / K * 1e3, 5),
        "dtype": f"mxfp{mx} activations x mxfp4 weights" if mx else "bf16",
        "config": {"workload": f"{w['name']}{f' (MXFP{mx} activations)' if mx else ''}: T={T} d={d} E={E} k={k} f={f} {w['fmt']}",
                   "T": T, "d": d, "E": E, "k": k, "f": f, "format": w["fmt"],
                   "weight_pools": n_pools, "parallelism": "none (1 GPU)"},
        "weight_stream_GBps": round(gbps, 1),
        "expert_TFLOPs": round(tflops, 3),
        "active_experts_mean": U_mean,
        "launch": "HIP graph of the K steps, replayed once",
        "eager_ms_per_step": round(eager_elapsed / K * 1e3, 5),
        "four_call_ms_per_step": round(steps_elapsed / K * 1e3, 5),
        "roofline": roof,
    }
    del pools, routers, xs, ws, y
    torch.cuda.empty_cache()
    if cpu and not args.no_cpu_baseline and not mx:
        n = args.cpu_sample_steps or {0: 200, 1: 6, 2: 4, 3: 1, 4: 3, 5: 3, 6: 6, 7: 1, 8: 1}[c]
        res["cpu_baseline"] = cpu_baseline(c, n)
    return res


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the layer runs on one GPU; --gpus must be 1 "
                                   "(expert-parallel sharding is designed, not built)"}))
        sys.exit(2)
    if args.bank or args.shared:
        if args.workload is None:
            args.workload = 1
        (bank_main if args.bank else shared_main)(args)
        return

    import synthetic

    head = 1 if args.workload is None else args.workload
    w = synthetic.WORKLOADS[head]
    peaks = None
    if not args.no_peaks:
        peaks = measure_peaks(MX_BYTES_PER_EXPERT(w["d"], w["f"]) * 2 + 57344)
    if args.mx8 and args.mx4:
        raise SystemExit("--mx8 and --mx4 exclude each other")
    r = run_workload(head, args, mx=8 if args.mx8 else 4 if args.mx4 else 0, peaks=peaks)
    res = {
        "metric": METRIC,
        "value": r["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": r["dtype"],
        "data": "synthetic",
    }
    res.update({n: v for n, v in r.items() if n not in res})
    if peaks is not None:
        res["measured_peaks"] = peaks
    if args.workload is None and not (args.mx8 or args.mx4):
        # the other configurations in the same run, each with its own
        # roofline and oracle baseline (the headline is workload 1)
        res["workloads"] = {}
        for c in (0, 1, 2, 3, 4):
            rc = r if c == head else run_workload(c, args, peaks=peaks)
            keep = ("value", "unit", "ms_per_step", "roofline", "cpu_baseline", "active_experts_mean",
                    "weight_stream_GBps", "expert_TFLOPs", "eager_ms_per_step")
            res["workloads"][synthetic.WORKLOADS[c]["name"]] = dict(
                {"config": rc["config"]["workload"]}, **{n: rc[n] for n in keep if n in rc})
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
