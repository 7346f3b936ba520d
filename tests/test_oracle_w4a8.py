"""Pins of the oracle's W4A8 pieces: per-token FP8 (E4M3) activation
quantization and the W4A8 product.

Each test ties the oracle to something other than itself: the values the
"Quantization chains" page prints for one outlier setting an E4M3 scale
(tests/golden/e4m3_chains.json), torch's float8_e4m3fn cast running the
pages' own fp8_per_row formula ("Quantization in deployment", formats.py),
invariants of the per-row scale, and a brute-force decode of codes and scales
written out here from the bit fields.
"""
import json
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_fp8_rows_one_outlier_sets_the_scale():
    g = golden("e4m3_chains.json")["printed"]
    a = np.array([[g["tensor_absmax"], g["small_value"], g["second_value"]],
                  [g["block_absmax"], g["small_value"], g["second_value"]]], dtype=np.float32)
    q = oracle.quantize_fp8_rows(a)
    deq = oracle.dequant_fp8_rows(q)
    assert abs(q.scales[0] - g["tensor_scale"]) < 5e-4                  # 100/448 = 0.223
    assert deq[0, 0] == g["tensor_absmax"]
    assert deq[0, 1] == g["small_value_stored"]                          # 0.0002 -> 0
    assert abs(deq[0, 2] - g["second_value_stored"]) < 5e-7               # 0.000436
    assert round(abs(deq[0, 2] - g["second_value"]) / g["second_value"] * 100) == g["second_value_error_pct"]
    assert q.scales[1] == np.float32(1.0) / np.float32(448.0)             # the block's own scale
    for k, x in ((1, g["small_value"]), (2, g["second_value"])):
        assert round(abs(deq[1, k] - x) / x * 100, 1) == g["block_error_pct"]   # 4.1 %


def _fp8_per_row_torch(a):
    """The pages' fp8_per_row, executed by torch on the CPU."""
    x = torch.from_numpy(a)
    scale = x.abs().amax(dim=-1, keepdim=True).clamp(min=1e-12) / 448.0
    y = (x / scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return y.view(torch.uint8).numpy(), scale[:, 0].numpy()


def test_fp8_rows_match_torch_float8_cast():
    rng = np.random.default_rng(7)
    rows = [rng.standard_normal(512).astype(np.float32) * s for s in (1.0, 1e-3, 30.0)]
    r = rng.standard_normal(512).astype(np.float32)
    r[rng.choice(512, 3, replace=False)] *= 50.0                         # outliers
    rows.append(r)
    rows.append((rng.random(512) * 1e-6).astype(np.float32) - 5e-7)      # tiny, both signs
    # a row whose scale is exactly 1 (amax 448) holding every midpoint between
    # neighbouring E4M3 values: the ties go to the even code
    ev = np.array([oracle.e4m3_value(c) for c in range(127)])
    mids = ((ev[:-1] + ev[1:]) / 2).astype(np.float32)
    m = np.zeros(512, dtype=np.float32)
    m[0] = 448.0
    m[1:1 + len(mids)] = mids
    m[1 + len(mids):1 + 2 * len(mids)] = -mids
    rows.append(m)
    # bf16-exact inputs, as the GPU path sees them
    a = torch.from_numpy(np.stack(rows)).bfloat16().float().numpy()
    a[0, 5] = -0.0
    q = oracle.quantize_fp8_rows(a)
    ref_codes, ref_scales = _fp8_per_row_torch(a)
    assert np.array_equal(q.scales, ref_scales)
    # torch maps -0.0 to 0x80 as well; compare every byte
    assert np.array_equal(q.codes, ref_codes)
    assert q.codes[0, 5] == 0x80


def test_fp8_rows_invariants():
    rng = np.random.default_rng(11)
    a = torch.from_numpy(rng.standard_normal((6, 256)).astype(np.float32)).bfloat16().float().numpy()
    q = oracle.quantize_fp8_rows(a)
    # the largest magnitude of every row lands on +-448
    big = np.abs(a).argmax(axis=1)
    assert all((q.codes[i, big[i]] & 0x7F) == 0x7E for i in range(6))
    # sign symmetry
    qn = oracle.quantize_fp8_rows(-a)
    assert np.array_equal(qn.codes, q.codes ^ 0x80) and np.array_equal(qn.scales, q.scales)
    # a power of two moves only the scale
    for j in (-3, -1, 2, 5):
        qj = oracle.quantize_fp8_rows(a * np.float32(2.0 ** j))
        assert np.array_equal(qj.codes, q.codes)
        assert np.array_equal(qj.scales, q.scales * np.float32(2.0 ** j))
    # an all-zero row: scale 1e-12/448, codes 0
    qz = oracle.quantize_fp8_rows(np.zeros((1, 64), dtype=np.float32))
    assert qz.scales[0] == np.float32(1e-12) / np.float32(448.0)
    assert not qz.codes.any()


def _e4m3(c):
    e, m = (c >> 3) & 15, c & 7
    v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
    return -v if c & 0x80 else v


def test_w4a8_brute_force_decode():
    rng = np.random.default_rng(3)
    M, N, K = 3, 5, 256
    a = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).bfloat16().float().numpy()
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    qw = oracle.quantize("int4", w)
    qa = oracle.quantize_fp8_rows(a)
    got = oracle.gemm_w4a8(a, qw)
    sw = qw.scales.view(np.float16).astype(np.float64)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                b = int(qw.codes[n, k // 2])
                nib = b & 0xF if k % 2 == 0 else b >> 4
                wq = nib - 16 if nib >= 8 else nib
                av = np.float32(_e4m3(int(qa.codes[m, k]))) * qa.scales[m]
                acc += float(av) * float(np.float32(wq * sw[n, k // 128]))
            assert abs(acc - got[m, n]) <= 1e-12 * max(1.0, abs(acc))


def test_w4a8_one_hot_rows_pick_weight_columns():
    rng = np.random.default_rng(5)
    N, K = 40, 512
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    qw = oracle.quantize("int4", w)
    cols = [0, 7, 128, 300, 511]
    a = np.zeros((len(cols), K), dtype=np.float32)
    for i, c in enumerate(cols):
        a[i, c] = 448.0                      # row scale exactly 1, code 0x7E
    qa = oracle.quantize_fp8_rows(a)
    assert np.all(qa.scales == 1.0)
    got = oracle.gemm_w4a8(a, qw)
    wd = oracle.dequant(qw).astype(np.float64)
    for i, c in enumerate(cols):
        assert np.array_equal(got[i], 448.0 * wd[:, c])
