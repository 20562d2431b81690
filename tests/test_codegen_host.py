"""Compiled-code guards (host only: hipcc cross-compiles for gfx950 here).

The single-launch prefill FFN keeps several stages of global -> LDS copies
in flight and waits for each stage with an explicit count of its own
loads.  If the compiler cannot tell a stage's LDS reads apart from the
copies still in flight, it inserts a wait for ALL of them (vmcnt(0)) in
front of the multiplies, which serialises loads and matrix work: a second
__shared__ object in the kernel once did exactly that and cost ~25 % of the
prefill FFN call.  This test fails if any block of the kernel's K loop (a
block holding matrix instructions) waits for every outstanding vector
memory operation."""

import os
import re
import shutil
import subprocess

import pytest

from quantized_routed_moe_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "quantized_routed_moe_amd", "csrc", "ffn_grouped.hip")


def _mfma_blocks(asm: str, kernel: str):
    i = asm.index(kernel + ":")
    j = asm.index(".Lfunc_end", i)
    blocks, cur = [], []
    for line in asm[i:j].split("\n"):
        t = line.strip()
        if not t or t.startswith(";"):
            continue
        if t.endswith(":") or t.startswith(".LBB"):
            if cur:
                blocks.append(cur)
            cur = []
            continue
        if not t.startswith("."):
            cur.append(t)
    if cur:
        blocks.append(cur)
    return [b for b in blocks if any(x.startswith("v_mfma") for x in b)]


def test_grouped_k_loop_never_waits_for_every_copy(tmp_path):
    hipcc = _build.hipcc()
    if not os.path.exists(hipcc) and shutil.which(hipcc) is None:
        pytest.skip("hipcc not available")
    out = tmp_path / "ffn_grouped.s"
    flags = [f for f in _build.COMMON if f not in ("-fPIC",)]
    r = subprocess.run([hipcc, *flags, "--offload-device-only", "-S", SRC, "-o", str(out)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    kernels = re.findall(r"^(_ZN5qrmoe26ffn_grouped_chained_kernel\w+):", asm, re.M)
    assert len(kernels) == 3, kernels                        # bf16, MXFP8 and MXFP4 operands
    for k in kernels:
        blocks = _mfma_blocks(asm, k)
        assert blocks, k
        full = [x for b in blocks for x in b if x == "s_waitcnt vmcnt(0)"]
        assert not full, f"{k}: {len(full)} waits for every copy in flight inside the K loop"
