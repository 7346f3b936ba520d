"""GPU parity of q4_relayout: a weight quantized row-major and moved to the
tiled layout is, byte for byte, the weight quantized tiled (codes, scales,
the padding rows of the last tile and the NVFP4 global scale), and the
reverse move gives the row-major quantization back.  Both quantizations are
themselves checked bit-exact against the oracle in test_gpu_quantize.py;
here the row-major side is also compared with the oracle directly, and the
tiled result is read back through the layout's definition (untile)."""
import pytest
import torch

import oracle
import w4_gemm_amd as q4
from q4_helpers import assert_quant_equal, log, to_f32

pytestmark = pytest.mark.gpu
FMTS = ("int4", "mxfp4", "nvfp4", "int4_zp")
DEV = "cuda:0"


def _bytes(t: torch.Tensor) -> bytes:
    return t.detach().contiguous().cpu().view(torch.uint8).numpy().tobytes()


def _same(a: q4.Q4Tensor, b: q4.Q4Tensor):
    assert _bytes(a.codes) == _bytes(b.codes)
    assert _bytes(a.scales) == _bytes(b.scales)
    if a.global_scale is not None:
        assert _bytes(a.global_scale) == _bytes(b.global_scale)


def _weight(rows, cols, seed):
    g = torch.Generator().manual_seed(seed)
    w = torch.randn(rows, cols, generator=g) * 0.02
    w[torch.rand(rows, cols, generator=g) < 0.001] *= 30.0          # outliers
    w[: min(rows, 2), :64] = 0.0                                      # all-zero blocks
    return w.to(torch.bfloat16)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(16, 512), (37, 1024), (130, 2048), (1, 512)])
def test_relayout_matches_tiled_quantization(fmt, shape):
    rows, cols = shape
    log("relayout", fmt, shape)
    w = _weight(rows, cols, rows * 7 + cols)
    wd = w.to(DEV)
    qr = q4.quantize(wd, fmt, layout="rows")
    qt = q4.quantize(wd, fmt, layout="tiled")
    moved = q4.relayout(qr, "tiled")
    back = q4.relayout(qt, "rows")
    torch.cuda.synchronize()
    _same(moved, qt)
    _same(back, qr)
    # both results against the oracle's quantization (the tiled one read back
    # through the layout's definition)
    ref = oracle.quantize(fmt, to_f32(w))
    assert_quant_equal(moved, ref, fmt)
    assert_quant_equal(back, ref, fmt)


@pytest.mark.parametrize("fmt", ("mxfp4", "nvfp4"))
def test_relayout_same_layout_copies(fmt):
    w = _weight(40, 1024, 5).to(DEV)
    for lay in ("rows", "tiled"):
        a = q4.quantize(w, fmt, layout=lay)
        b = q4.relayout(a, lay)
        torch.cuda.synchronize()
        _same(a, b)


def test_relayout_empty_copies_global_scale():
    a = q4.empty_q4("nvfp4", 0, 512, device=DEV)
    a.global_scale.fill_(0.125)
    b = q4.relayout(a, "tiled")
    torch.cuda.synchronize()
    assert float(b.global_scale.item()) == 0.125


def test_gemm_on_relayout_weights_is_the_tiled_gemm():
    """W4A16 (NVFP4) and W4A4 (MXFP4): the tiled kernels on weights moved from
    row-major give bit-identical outputs to those on weights quantized tiled."""
    g = torch.Generator(device=DEV).manual_seed(11)
    M, N, K = 96, 272, 1024
    A = torch.randn(M, K, device=DEV, generator=g).bfloat16()
    W = (torch.randn(N, K, device=DEV, generator=g) * 0.02).bfloat16()
    C1 = torch.empty(M, N, device=DEV, dtype=torch.bfloat16)
    C2 = torch.empty_like(C1)
    qt = q4.quantize(W, "nvfp4", layout="tiled")
    qm = q4.relayout(q4.quantize(W, "nvfp4", layout="rows"), "tiled")
    q4.q4_gemm(A, qt, C1)
    q4.q4_gemm(A, qm, C2)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)
    qa = q4.quantize(A, "mxfp4", layout="tiled")
    wt = q4.quantize(W, "mxfp4", layout="tiled")
    wm = q4.relayout(q4.quantize(W, "mxfp4", layout="rows"), "tiled")
    q4.q4_gemm(qa, wt, C1)
    q4.q4_gemm(qa, wm, C2)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)


def _offset_scales(q: q4.Q4Tensor, copy: bool) -> q4.Q4Tensor:
    """The same tensor with its scales 4 bytes off 16-byte alignment."""
    nb = q.scales.numel() * q.scales.element_size()
    buf = torch.empty(nb + 64, dtype=torch.uint8, device=DEV)
    base = (-buf.data_ptr()) % 16
    off = buf[base + 4: base + 4 + nb]
    if copy:
        off.copy_(q.scales.reshape(-1).view(torch.uint8))
    out = q4.Q4Tensor(q.fmt, q.rows, q.cols, q.codes, off.view(q.scales.dtype).reshape(q.scales.shape),
                      q.global_scale, q.layout)
    assert out.scales.data_ptr() % 16 == 4
    return out


@pytest.mark.parametrize("fmt", FMTS)
def test_relayout_scales_at_any_alignment(fmt):
    """Scales aligned to 16 bytes move in whole row groups, others byte by byte;
    both give the other layout's quantization exactly, in both directions."""
    rows, cols = 37, 1024
    log("relayout unaligned scales", fmt)
    wd = _weight(rows, cols, 99).to(DEV)
    qr = q4.quantize(wd, fmt, layout="rows")
    qt = q4.quantize(wd, fmt, layout="tiled")
    moved = q4.relayout(_offset_scales(qr, True), "tiled")       # unaligned source
    dst = _offset_scales(q4.empty_q4(fmt, rows, cols, device=DEV, layout="rows"), False)
    q4.q4_relayout(qt, dst)                                       # unaligned destination
    torch.cuda.synchronize()
    _same(moved, qt)
    _same(dst, qr)


@pytest.mark.parametrize("fmt", ("mxfp4", "nvfp4"))
def test_relayout_full_decode_weight(fmt):
    """The 28672 x 8192 decode weight (the launch the benchmark times): both
    directions byte-equal to the other layout's quantization, which is itself
    checked against the oracle on sampled rows in test_gpu_quantize.py."""
    log("relayout full", fmt)
    g = torch.Generator(device=DEV).manual_seed(17)
    w = (torch.randn(28672, 8192, device=DEV, generator=g) * 0.02).bfloat16()
    qr = q4.quantize(w, fmt, layout="rows")
    qt = q4.quantize(w, fmt, layout="tiled")
    del w
    moved = q4.relayout(qr, "tiled")
    torch.cuda.synchronize()
    assert torch.equal(moved.codes, qt.codes) and torch.equal(moved.scales, qt.scales)
    del moved
    back = q4.relayout(qt, "rows")
    torch.cuda.synchronize()
    assert torch.equal(back.codes, qr.codes) and torch.equal(back.scales, qr.scales)
    if fmt == "nvfp4":
        assert torch.equal(back.global_scale, qr.global_scale)
