"""Pins of the oracle's FP4 format (a reading: "Loading a model in 4-bit",
"Developer", names the fp4 quant type beside nf4 but prints no codebook, so
this format's parity is unpinned against the pages).

The reading: the E2M1 element values (sign, two exponent bits, one mantissa
bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6) divided by 6 and scaled by the block absmax
as NF4's table is; coding to the nearest entry with ties to the lower index.
The tests pin the oracle to that definition: the table against the E2M1
decode of every code, the coding against an exact-rational brute force,
values on the E2M1 grid round-tripping exactly, and the product against
numpy on the dequantized weights.
"""

from fractions import Fraction as Fr

import numpy as np
import pytest
import torch

from oracle import exact

FP4 = 4
F16, BF16 = 0, 1


def f16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def bits16(vals):
    return np.asarray(vals, dtype=np.float32).astype(np.float16).view(np.uint16)


def unpack(packed):
    p = np.asarray(packed, dtype=np.uint8)
    return np.stack([p & 0xF, (p >> 4) & 0xF], axis=-1).reshape(p.shape[:-1] + (-1,))


def test_table_is_e2m1_over_six(orc):
    t = orc.fp4_table()
    # the E2M1 magnitudes from the bit fields, written out independently
    mags = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    for c in range(16):
        want = exact.rn32(Fr(mags[c & 7]) * (-1 if c & 8 else 1) / 6)
        assert Fr(float(t[c])) == want, c
        assert exact.FP4_TABLE[c] == want, c
    assert np.signbit(t[8]) and not np.signbit(t[0])   # code 8 is -0
    assert t[7] == 1.0 and t[15] == -1.0


def test_nearest_at_decision_points(orc):
    mags = sorted(set(abs(v) for v in exact.FP4_TABLE))
    xs = [0.0, -0.0, 1.0, -1.0, 1e-30, -1e-30]
    ties = 0
    for a, b in zip(mags[:-1], mags[1:]):
        m = (a + b) / 2
        for sgn in (1, -1):
            x0 = np.float32(float(exact.rn32(sgn * m)))
            if Fr(float(x0)) == sgn * m:
                ties += 1
            v = x0
            for _ in range(3):
                xs.append(float(v))
                v = np.nextafter(v, np.float32(2))
            v = x0
            for _ in range(3):
                xs.append(float(v))
                v = np.nextafter(v, np.float32(-2))
    assert ties >= 2            # +-rn32(1/12)/2: exact binary32 midpoints
    rng = np.random.default_rng(12)
    xs += rng.uniform(-1, 1, 5000).astype(np.float32).tolist()
    for x in xs:
        assert orc.fp4_nearest(x) == exact.fp4_nearest(Fr(x)), x
    # the tie between +0 and -0 keeps code 0; a tie between two levels keeps
    # the lower index (the smaller magnitude, for either sign)
    assert orc.fp4_nearest(-0.0) == 0
    assert orc.fp4_nearest(np.float32(1 / 24)) in (0, 1)
    assert orc.fp4_nearest(0.125) == 1 and orc.fp4_nearest(-0.125) == 9


@pytest.mark.parametrize("g", [32, 64, 128])
def test_quantize_matches_exact_brute_force(orc, g):
    rng = np.random.default_rng(300 + g)
    rows = []
    for sigma, mu in [(1e-6, 0.0), (0.02, 0.0), (0.02, 0.01), (1.0, 0.0), (300.0, 0.0)]:
        rows.append(bits16(rng.standard_normal((4, g)).astype(np.float32) * np.float32(sigma)
                           + np.float32(mu)))
    special = np.zeros((3, g), np.float32)
    special[1, 3] = -0.5
    special[2, :] = -0.25
    rows.append(bits16(special))
    w = np.concatenate(rows, 0)
    codes, scales, zeros = orc.quantize(FP4, g, w)
    assert zeros is None and scales.dtype == np.float32
    nib = unpack(codes)
    for r in range(w.shape[0]):
        want, c, _ = exact.quantize_group(FP4, w[r].tolist())
        assert nib[r].tolist() == want, r
        assert Fr(float(scales[r, 0])) == c, r
    assert np.all(nib[w.shape[0] - 3] == 0)             # a zero block: all +0


def test_e2m1_grid_round_trips(orc):
    """Blocks of E2M1 values times 2^k whose absmax is 6 * 2^k code to the
    exact level and dequantize to the same value in either dtype."""
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -1.5, -2, -3, -4, -6, 6], np.float32)
    rows = []
    for k in (-6, 0, 3):
        rng = np.random.default_rng(k + 50)
        v = rng.permutation(np.tile(grid, 4)) * np.float32(2.0 ** k)
        v[0] = 6 * 2.0 ** k
        rows.append(v)
    w = bits16(np.stack(rows))
    codes, scales, zeros = orc.quantize(FP4, 64, w)
    for out_t in (F16, BF16):
        out = orc.dequantize(FP4, 64, codes, scales, zeros, 3, 64, out_t)
        ov = f16(out) if out_t == F16 else (out.astype(np.uint32) << 16).view(np.float32)
        assert np.array_equal(ov, f16(w)), out_t


def test_dequant_is_one_product_then_one_rounding(orc):
    rng = np.random.default_rng(5)
    w = bits16(rng.standard_normal((8, 128)).astype(np.float32) * np.float32(0.05))
    codes, scales, zeros = orc.quantize(FP4, 32, w)
    nib = unpack(codes)
    out = orc.dequantize(FP4, 32, codes, scales, zeros, 8, 128, BF16)
    for r in range(8):
        for k in range(0, 128, 7):
            c = Fr(float(scales[r, k // 32]))
            v = exact.round_binary(exact.rn32(exact.FP4_TABLE[nib[r, k]] * c), 8, -126)
            got = float((np.uint32(out[r, k]) << np.uint32(16)).view(np.float32))
            assert Fr(got) == v, (r, k)


def test_matmul_reference(orc):
    N, K, M, g = 24, 256, 3, 64
    rng = np.random.default_rng(8)
    w = bits16(rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02))
    codes, scales, zeros = orc.quantize(FP4, g, w)
    xf = rng.standard_normal((M, K)).astype(np.float32)
    x = torch.from_numpy(xf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    xv = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    deq = orc.dequantize(FP4, g, codes, scales, zeros, N, K, BF16)
    wv = (deq.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    y, ad = orc.matmul(FP4, g, BF16, x, codes, scales, zeros, N, K)
    assert np.allclose(y, xv @ wv.T, rtol=1e-12, atol=1e-15)
    assert np.allclose(ad, np.abs(xv) @ np.abs(wv).T, rtol=1e-12, atol=1e-15)
