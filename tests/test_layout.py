"""The tiled layout's definition (include/q4.h) written out element by element,
checked against the array rearrangement the GPU tests use to read tiled
tensors back (q4_helpers.untile)."""
import numpy as np
import pytest

from q4_helpers import untile


def tile_by_definition(codes, scales, fmt, rows, cols):
    """Row-major -> tiled, one element at a time from the header's formulas."""
    RT, S = (rows + 15) // 16, cols // 128
    Q = S // 4
    tc = np.zeros(RT * S * 1024, np.uint8)
    for r in range(rows):
        t, n = divmod(r, 16)
        for k in range(0, cols, 2):             # one byte = elements k, k+1
            s, rem = divmod(k, 128)
            g, j = divmod(rem, 32)
            l = 16 * g + n
            tc[(t * S + s) * 1024 + 16 * l + j // 2] = codes[r, k // 2]
    if fmt == "mxfp4":
        ts = np.zeros(RT * Q * 256, np.uint8)
        for r in range(rows):
            t, n = divmod(r, 16)
            for b in range(cols // 32):
                s, g = divmod(b, 4)
                q, i = divmod(s, 4)
                ts[((t * Q + q) * 64 + 16 * g + n) * 4 + i] = scales[r, b]
    elif fmt == "nvfp4":
        ts = np.zeros(RT * Q * 512, np.uint8)
        for r in range(rows):
            t, n = divmod(r, 16)
            for b in range(cols // 16):
                s, rem = divmod(b, 8)
                g, h = divmod(rem, 2)
                q, i = divmod(s, 4)
                ts[((t * Q + q) * 64 + 16 * g + n) * 8 + 2 * i + h] = scales[r, b]
    else:
        ts = np.zeros(RT * Q * 64, np.uint16)
        for r in range(rows):
            t, n = divmod(r, 16)
            for s in range(cols // 128):
                q, i = divmod(s, 4)
                ts[((t * Q + q) * 16 + n) * 4 + i] = scales[r, s]
    return tc, ts


@pytest.mark.parametrize("fmt,g,dt", [("mxfp4", 32, np.uint8), ("nvfp4", 16, np.uint8),
                                      ("int4", 128, np.uint16)])
@pytest.mark.parametrize("rows,cols", [(16, 512), (21, 1024), (3, 512)])
def test_untile_inverts_the_definition(fmt, g, dt, rows, cols):
    rng = np.random.default_rng(rows * cols + g)
    codes = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(0, 256 if dt == np.uint8 else 65536, (rows, cols // g)).astype(dt)
    tc, ts = tile_by_definition(codes, scales, fmt, rows, cols)
    c2, s2 = untile(tc, ts, fmt, rows, cols)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
