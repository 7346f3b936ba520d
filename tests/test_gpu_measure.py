"""GPU check of the measurement helper q4_read_probe (the plain streaming
read the benchmark times as the decode GEMV's read ceiling)."""
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
