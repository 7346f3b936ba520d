"""The seeded input generators: determinism, the stated recipe, routing."""
import numpy as np
import torch

from w4_gemm_amd import workloads


def test_normal_stream_is_deterministic_and_thread_independent():
    a = workloads.normal_f32("t/x", 3 * workloads.CHUNK + 17, seed=5)
    b = workloads.normal_f32("t/x", 3 * workloads.CHUNK + 17, seed=5)
    assert np.array_equal(a, b)
    c = workloads.normal_f32("t/x", 3 * workloads.CHUNK + 17, seed=6)
    assert not np.array_equal(a, c)
    # a shorter draw is a prefix (chunks are independent of the total)
    assert np.array_equal(workloads.normal_f32("t/x", 100, seed=5), a[:100])
    assert abs(a.mean()) < 0.01 and abs(a.std() - 1) < 0.01


def test_matrix_outliers_and_channels():
    m = workloads.matrix("t/w", 64, 512, 0.02, seed=1, outlier_frac=0.001, outlier_mult=20.0)
    assert m.dtype == torch.bfloat16 and m.shape == (64, 512)
    z = workloads.normal_f32("t/w", 64 * 512, seed=1) * np.float32(0.02)
    idx = workloads.choose("t/w", 64 * 512, round(0.001 * 64 * 512), seed=1)
    z[idx] *= np.float32(20.0)
    assert torch.equal(m, torch.from_numpy(z.reshape(64, 512)).to(torch.bfloat16))
    a = workloads.matrix("t/a", 8, 1000, 1.0, seed=2, channel_frac=0.01, channel_mult=10.0)
    ch = workloads.choose("t/a", 1000, 10, seed=2)
    base = workloads.matrix("t/a", 8, 1000, 1.0, seed=2)
    ratio = (a.float() / base.float())[:, ch]
    assert torch.allclose(ratio, torch.full_like(ratio, 10.0), rtol=1e-2)


def test_route_top_k_and_counting_sort():
    logits = workloads.normal_f32("t/logits", 256 * 64, seed=0).reshape(256, 64)
    r = workloads.route(logits, 8)
    assert r.offsets[0] == 0 and r.offsets[-1] == 256 * 8
    assert np.all(np.diff(r.offsets) >= 0)
    for t in range(256):
        # brute force: the 8 largest logits, ties to the lower expert id
        order = sorted(range(64), key=lambda e: (-logits[t, e], e))[:8]
        assert sorted(order) == sorted(r.topk_ids[t].tolist())
    for e in range(64):
        toks = r.gather[r.offsets[e]:r.offsets[e + 1]]
        assert np.all(np.diff(toks) > 0)              # tokens ascending within an expert
        assert all(e in r.topk_ids[t] for t in toks)
