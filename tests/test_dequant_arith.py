"""Host check of the exactness argument behind the matrix-core kernels' INT4
dequantization.

Those kernels compute (q - z) s as one fused multiply-add on an fp16 operand
built by OR-ing a code nibble into 0x6400:
    fma(1024 + q, s, -(1024 + z) s)            (low nibble of a byte)
    fma(1024 + 16 q, s / 16, -(64 + z) s)      (high nibble)
with the biases derived from -z s by fma(-1024, s, -z s), fma(-64, s, -z s)
and the scale s / 16.  Their outputs equal the binary32 product (q - z) s
that q4_dequantize rounds only if every one of those terms is exactly a
binary32 value (an fma whose exact result is representable returns it) and
the fp16 operands are exact.  This checks that for every finite fp16 scale
(the INT4 formats store fp16 scales), every code q and zero-point z.
"""

import numpy as np


def _all_scales():
    bits = np.arange(0, 0x7C00, dtype=np.uint16)  # +0 .. largest finite fp16
    return bits.view(np.float16).astype(np.float64)


def _exact_f32(v):
    """True where the float64 value v is exactly a binary32 value."""
    return v.astype(np.float32).astype(np.float64) == v


def test_fp16_operands_are_exact():
    q = np.arange(16, dtype=np.uint16)
    lo = (0x6400 | q).view(np.float16).astype(np.float64)
    hi = (0x6400 | (q << 4)).view(np.float16).astype(np.float64)
    assert np.array_equal(lo, 1024.0 + q)
    assert np.array_equal(hi, 1024.0 + 16.0 * q)


def test_every_term_is_a_binary32_value():
    s = _all_scales()
    assert _exact_f32(s / 16.0).all()
    for z in range(16):
        bias = -float(z) * s
        b1 = -(1024.0 + z) * s
        b16 = -(64.0 + z) * s
        # float64 holds these products exactly (at most 11 + 11 bits)
        assert _exact_f32(bias).all(), z
        assert _exact_f32(b1).all(), z
        assert _exact_f32(b16).all(), z
        for q in range(16):
            prod = float(q - z) * s
            assert _exact_f32(prod).all(), (q, z)
            # the two fma forms give the product itself
            assert np.array_equal((1024.0 + q) * s + b1, prod)
            assert np.array_equal((1024.0 + 16.0 * q) * (s / 16.0) + b16, prod)


def test_a_plausible_slip_is_caught():
    """The same check rejects a bias that is not exact: (1024 + z) s rounded
    through fp16 (the scale's own format) loses bits for most scales."""
    s = _all_scales()
    s = s[s < 32.0]  # where (1024 + z) s fits fp16
    b1_f16 = (-(1024.0 + 7) * s).astype(np.float16).astype(np.float64)
    assert not np.array_equal((1024.0 + 3) * s + b1_f16, float(3 - 7) * s)
