"""The number-theoretic fact the INT4 quantizers use in place of a division,
checked in numpy fp32 on the CPU (no GPU, no oracle: it is a property of
fp32 arithmetic on bf16 values and fp16 scales).

INT4 codes are clamp(rne(w / s), -8, 7), or clamp(rne(w / s) + z, -8, 7)
with a zero point, for a bf16 value w and an fp16 scale s ("LLM
quantization", the absmax and zero-point recipes).  A bf16 quotient over an
fp16 scale is either exactly a half-integer or at least 2^-12 away from
one, so with r within 1 ulp of 1/s and y = fl(w r), clamping y and rounding
it to a multiple of 2^-14 (fl(c + 768)) recovers every tie exactly and
keeps every other quotient on its side; fl(. + 1.5 2^23 - 768) then rounds
to the integer with ties to even.  The kernels' construction, restated
here, is compared with the correctly rounded division for every finite bf16
value against a spread of fp16 scales (all exponents, subnormals included),
for the correctly rounded reciprocal and both its neighbours."""
import numpy as np

f32 = np.float32
MAGIC_BITS = 0x4B400000  # bits of 1.5 * 2^23


def _bf16_values():
    bits = np.arange(1 << 16, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    return x[np.isfinite(x)]


def _snap_code(y, lo, hi, snap=True):
    c = np.minimum(np.maximum(y, f32(lo)), f32(hi))
    t = (c + f32(768)).astype(f32) if snap else c
    n = (t + f32(12582912 - (768 if snap else 0))).astype(f32)
    return (n.view(np.uint32).astype(np.int64) - MAGIC_BITS).astype(np.int32)


def _mismatches(scales, snap=True):
    x = _bf16_values()
    bad = 0
    with np.errstate(all="ignore"):
        for i in range(0, scales.size, 64):
            s = scales[i:i + 64][:, None]
            q = np.rint(x[None, :] / s)                     # fl(w / s), then rne
            q_int4 = np.clip(q, -8, 7).astype(np.int32)
            q_wide = np.clip(q, -64, 64).astype(np.int32)
            rn = (f32(1) / s).astype(f32)
            for r in (np.nextafter(rn, f32(0)), rn, np.nextafter(rn, f32(np.inf))):
                y = (x[None, :] * r).astype(f32)
                bad += int(np.count_nonzero(_snap_code(y, -8, 7, snap) != q_int4))
                k = _snap_code(y, -16, 16, snap)
                for z in (-8, -3, 0, 7):
                    bad += int(np.count_nonzero(np.clip(k + z, -8, 7) != np.clip(q_wide + z, -8, 7)))
    return bad


def _fp16_scales(stride):
    return np.arange(1, 0x7C00, stride, dtype=np.uint16).view(np.float16).astype(np.float32)


def test_int4_code_without_division_matches_rne_of_quotient():
    scales = _fp16_scales(29)
    assert scales.min() < 2.0 ** -14 and scales.max() > 32768  # subnormal and top binade
    assert _mismatches(scales) == 0


def test_int4_code_without_the_snap_is_wrong_somewhere():
    # the same construction without the 2^-14 rounding: the product's error
    # flips exact ties (the check above is sensitive to that mistake)
    assert _mismatches(_fp16_scales(29 * 16), snap=False) > 0
