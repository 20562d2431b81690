"""The roofline measurement kernels of include/moe_peak.h on the GPU, through
the C ABI: the read stream reads every byte it is given (the xor of its
per-workgroup words equals the xor of the buffer's 32-bit words), the
matrix-core loops finish with finite sums, and the hold kernel keeps its
stream busy for at least the time asked for."""

import numpy as np
import pytest
import torch

import quantized_routed_moe_amd as qm

pytestmark = pytest.mark.gpu


def _stream():
    return torch.cuda.current_stream().cuda_stream


@pytest.mark.parametrize("nbytes,wgs", [(16, 0), (1 << 20, 0), ((1 << 20) + 48, 7), (3 << 22, 2048)])
def test_peak_stream_reads_every_word(nbytes, wgs):
    print(f"moe_peak_stream: {nbytes} bytes, workgroups {wgs}", flush=True)
    rng = np.random.default_rng(nbytes + wgs)
    words = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    g = wgs or 2048
    sink = torch.zeros(g, dtype=torch.int32, device="cuda")
    assert qm.lib().moe_peak_stream(buf.data_ptr(), nbytes, wgs, sink.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_peak_mfma_sums_are_finite(kind):
    print(f"moe_peak_mfma: kind {kind}", flush=True)
    sink = torch.full((64 * 4,), float("nan"), dtype=torch.float32, device="cuda")
    assert qm.lib().moe_peak_mfma(kind, 3, 64, sink.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    s = sink.cpu().numpy()
    assert np.isfinite(s).all() and (s != 0).any()


@pytest.mark.parametrize("us", [200, 2000])
def test_peak_hold_holds_the_stream(us):
    print(f"moe_peak_hold: {us} us", flush=True)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    assert qm.lib().moe_peak_hold(us, _stream()) == 0
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    assert us / 1e3 <= ms < us / 1e3 + 20.0, ms
