"""GPU checks of the measurement helpers: q4_read_probe (the plain
streaming read the benchmark times as the decode GEMV's read ceiling) and
q4_mfma_probe (back-to-back matrix instructions on random operands: the
GEMMs' measured ceiling)."""
import pytest
import torch

import w4_gemm_amd as q4

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_read_probe_reads_and_leaves_sink():
    """The measurement helper streams a whole buffer (sizes with and without
    a partial last group of pieces) and leaves its sink alone for ordinary
    data."""
    sink = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    for nbytes in (1024, 8 * 1024 * 3 + 5 * 1024, 124780544):
        buf = torch.full((nbytes,), 3, dtype=torch.uint8, device=DEV)
        q4.q4_read_probe(buf, sink)
        torch.cuda.synchronize()
        assert int(sink.item()) == 7


@pytest.mark.parametrize("kind,peak", [("fp4", 10100.0), ("bf16", 2500.0), ("fp16", 2500.0), ("fp8", 5000.0),
                                       ("fp4_copy", 10100.0), ("fp4_mix", 10100.0), ("bf16_mix", 2500.0)])
def test_mfma_probe_rate(kind, peak):
    """The probe reports its operation count, leaves the sink alone, and
    runs at a positive rate no higher than the published dense peak (plus
    timing slack).  The three instruction-mix kinds read a 64 KB window at
    the sink."""
    n = q4.PROBE_MIX_SINK if kind.endswith(("_copy", "_mix")) else 1
    sink = torch.full((n,), 7, dtype=torch.int32, device=DEV)
    iters = 512
    flops = q4.q4_mfma_probe(kind, iters, sink)
    per = 2 * 16 * 16 * (128 if kind.startswith("fp4") or kind == "fp8" else 32)
    waves = flops / (iters * 8 * per)
    assert waves == int(waves) and int(waves) % 8 == 0 and waves > 0
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        q4.q4_mfma_probe(kind, iters, sink)
    e1.record()
    torch.cuda.synchronize()
    tflops = 5 * flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    print(f"{kind}: {tflops:.0f} TFLOP/s", flush=True)
    assert 0 < tflops < 1.05 * peak
    assert torch.all(sink == 7)
    assert q4.q4_mfma_probe(kind, 0, sink) == 0.0
