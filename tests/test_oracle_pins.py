"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these tests re-types the oracle's formulas: they compare it with the
printed table, with library conversions (numpy fp16, torch bf16), with an
exact-rational brute force over all 16 levels, with closed-form special cases,
with invariants and error bounds that follow from the definitions, and with
numpy's matmul.  A plausible mistake in the oracle (wrong table entry, wrong
nibble order, wrong tie rule, round-half-away instead of half-even, scale /8
instead of /7, grouping along the wrong axis, a sign error in the zero-point,
a dropped term in the product) fails at least one of them.
"""

import os
from fractions import Fraction as Fr

import numpy as np
import pytest
import torch

from oracle import exact

HERE = os.path.dirname(os.path.abspath(__file__))
NF4, SYM, ASYM = 0, 1, 2
F16, BF16 = 0, 1


def page_table_decimals():
    with open(os.path.join(HERE, "golden", "nf4_table.txt")) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


def f16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def bits16(vals):
    return np.asarray(vals, dtype=np.float32).astype(np.float16).view(np.uint16)


def unpack_page(packed):
    """The page's unpack expression: low nibble, then high nibble, per byte."""
    p = np.asarray(packed, dtype=np.uint8)
    return np.stack([p & 0xF, (p >> 4) & 0xF], axis=-1).reshape(p.shape[:-1] + (-1,))


def zero_points(zeros, ngroups):
    return unpack_page(zeros[None, :])[0][:ngroups]


# ---------------------------------------------------------------- P1 table
def test_nf4_table_is_the_printed_one(orc):
    dec = page_table_decimals()
    assert len(dec) == 16
    want = np.array([np.float32(d) for d in dec], dtype=np.float32)
    got = orc.nf4_table()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert np.all(np.diff(got) > 0)
    assert got[0] == -1.0 and got[7] == 0.0 and got[15] == 1.0
    # the exact mini-oracle reads the same decimals
    assert [float(q) for q in exact.NF4_TABLE] == [float(v) for v in want]


# ---------------------------------------------------------- P2 conversions
def test_f16_decode_all_patterns(orc):
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.f16_bits_to_f32(allb)
    want = allb.view(np.float16).astype(np.float32)
    fin = np.isfinite(want)
    assert np.array_equal(got[fin].view(np.uint32), want[fin].view(np.uint32))
    assert np.all(np.isnan(got[np.isnan(want)]))


def _f32_probe_values():
    rng = np.random.default_rng(7)
    r = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    r = r[np.isfinite(r)]
    # every fp16 value, the exact midpoints between neighbours, and one ulp
    # (binary32) either side of each midpoint: where rounding decides
    h = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mid = ((h[:-1] + h[1:]) / 2).astype(np.float32)   # exact in binary32
    near = np.concatenate([mid, np.nextafter(mid, np.float32(np.inf)),
                           np.nextafter(mid, np.float32(-np.inf)), h.astype(np.float32),
                           np.float32([65504, 65519.996, 65520, 65536, 1e30])])
    v = np.concatenate([r, near, -near]).astype(np.float32)
    return v


def test_f32_to_f16_matches_numpy(orc):
    v = _f32_probe_values()
    got = orc.f32_to_f16_bits(v)
    with np.errstate(over="ignore"):
        want = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def test_f32_to_bf16_matches_torch(orc):
    rng = np.random.default_rng(8)
    r = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    # add exact bf16 midpoints (low half 0x8000) with both parities, and +-1
    mids = (r & 0xFFFF0000) | 0x8000
    v = np.concatenate([r, mids, mids + 1, mids - 1]).view(np.float32)
    v = v[np.isfinite(v)]
    got = orc.f32_to_bf16_bits(v)
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- P3 packing
def test_packing_low_nibble_first(orc):
    # A block with max|w| = 1 has c = 1, so w = fp16(Q[i]) codes to i (the
    # fp16 rounding of Q[i] is far below half of any table gap).
    dec = page_table_decimals()
    q16 = np.array([np.float32(d) for d in dec], dtype=np.float32).astype(np.float16)
    rng = np.random.default_rng(3)
    want = rng.integers(0, 16, size=(4, 128))
    want[:, 0] = 15                      # forces c = 1 in the first block
    want[:, 64] = 0                      # and in the second
    want[0, 2], want[0, 3] = 1, 2        # codes 1, 2 at elements 2, 3
    w = q16[want].view(np.uint16)
    codes, scales, _ = orc.quantize(NF4, 64, w)
    assert np.all(scales == 1.0)
    assert np.array_equal(unpack_page(codes), want)
    # element 2t is the low nibble of byte t, element 2t+1 the high nibble
    assert codes[0, 1] == 0x21


def test_dequant_of_unit_block_is_the_table(orc):
    dec = page_table_decimals()
    q32 = np.array([np.float32(d) for d in dec], dtype=np.float32)
    w = np.tile(q32.astype(np.float16), 4)[None, :].view(np.uint16)   # 1 x 64, c = 1
    codes, scales, _ = orc.quantize(NF4, 64, w)
    assert np.array_equal(unpack_page(codes)[0], np.tile(np.arange(16), 4))
    out16 = orc.dequantize(NF4, 64, codes, scales, None, 1, 64, F16)
    assert np.array_equal(out16[0, :16], q32.astype(np.float16).view(np.uint16))
    outbf = orc.dequantize(NF4, 64, codes, scales, None, 1, 64, BF16)
    want_bf = torch.from_numpy(q32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(outbf[0, :16], want_bf)


# ------------------------------------------------------- P4 NF4 coding exact
def test_nf4_exhaustive_fp16_unit_block(orc):
    """Every finite fp16 w in [-1, 1] in a block whose absmax is 1 (so x = w)
    codes to the brute-force nearest entry, ties to the lower index."""
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = allb.view(np.float16).astype(np.float32)
    sel = allb[np.isfinite(vals) & (np.abs(vals) <= 1.0)]
    assert sel.size == 30722
    n63 = (sel.size + 62) // 63
    padded = np.concatenate([sel, np.zeros(n63 * 63 - sel.size, np.uint16)])
    rows = np.concatenate([np.full((n63, 1), 0x3C00, np.uint16), padded.reshape(n63, 63)], 1)
    codes, scales, _ = orc.quantize(NF4, 64, rows)
    assert np.all(scales == 1.0)
    got = unpack_page(codes)[:, 1:].reshape(-1)[: sel.size]
    table = [exact.NF4_TABLE[i] for i in range(16)]
    for b, c in zip(sel.tolist(), got.tolist()):
        x = exact.f16_value(b)
        d = [abs(x - q) for q in table]
        assert c == d.index(min(d)), hex(b)


def test_nf4_nearest_at_decision_points(orc):
    table = exact.NF4_TABLE
    xs = []
    ties = 0
    for i in range(15):
        m = (table[i] + table[i + 1]) / 2
        x0 = np.float32(float(exact.rn32(m)))
        if Fr(float(x0)) == m:
            ties += 1
            assert orc.lib().orc_nf4_nearest(x0) == i      # exact tie -> lower index
        v = x0
        for _ in range(4):
            xs.append(v)
            v = np.nextafter(v, np.float32(2))
        v = x0
        for _ in range(4):
            xs.append(v)
            v = np.nextafter(v, np.float32(-2))
    assert ties >= 1
    rng = np.random.default_rng(11)
    xs = np.concatenate([np.array(xs, np.float32),
                         rng.uniform(-1, 1, 20000).astype(np.float32),
                         np.float32([0.0, -0.0, 1e-30, -1e-30, 1.0, -1.0])])
    got = orc.nf4_nearest(xs)
    for x, c in zip(xs.tolist(), got.tolist()):
        assert c == exact.nf4_nearest(Fr(x)), x


def _groups_for_exact(fmt, seed, n_groups=12, g=32):
    rng = np.random.default_rng(seed)
    rows = []
    for sigma, mu in [(1e-6, 0.0), (3e-5, 1e-5), (0.02, 0.0), (0.02, 0.01), (1.0, 0.0),
                      (300.0, 0.0), (0.02, -0.05)]:
        v = rng.standard_normal((n_groups, g)).astype(np.float32) * np.float32(sigma) + np.float32(mu)
        rows.append(bits16(v))
    # degenerate groups: all zero, one non-zero, all equal, all negative
    special = np.zeros((4, g), np.float32)
    special[1, 5] = 0.5
    special[2, :] = 0.25
    special[3, :] = -np.abs(rng.standard_normal(g)).astype(np.float32)
    rows.append(bits16(special))
    return np.concatenate(rows, 0)


@pytest.mark.parametrize("fmt", [NF4, SYM, ASYM])
def test_quantize_matches_exact_brute_force(orc, fmt):
    w = _groups_for_exact(fmt, 100 + fmt)
    codes, scales, zeros = orc.quantize(fmt, 32, w)
    nib = unpack_page(codes)
    zp = zero_points(zeros, w.shape[0]) if fmt == ASYM else None
    for r in range(w.shape[0]):
        want, s, z = exact.quantize_group(fmt, w[r].tolist())
        assert nib[r].tolist() == want, (fmt, r)
        got_s = Fr(float(scales[r, 0])) if fmt == NF4 else exact.f16_value(int(scales[r, 0]))
        assert got_s == s, (fmt, r)
        if fmt == ASYM:
            assert int(zp[r]) == z, r


def test_int4_sym_half_integers_round_to_even(orc):
    # max|w| = 7 gives s = 1 exactly; w = k + 1/2 lands on exact ties.
    w = np.zeros((1, 32), np.float32)
    w[0, :10] = [7.0, 0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, -3.5, 6.5]
    codes, scales, _ = orc.quantize(SYM, 32, bits16(w))
    assert f16(scales)[0, 0] == 1.0
    q = unpack_page(codes)[0, :10].astype(int) - 8
    assert q.tolist() == [7, 0, 2, 2, 4, 0, -2, -2, -4, 6]


def test_int4_asym_closed_form_case(orc):
    # range [0, 15] gives s = 1, z = 0; range [-7.5, 7.5] gives s = 1, and
    # z = round_half_even(7.5) = 8.
    w = np.zeros((2, 32), np.float32)
    w[0, :4] = [15.0, 0.0, 2.5, 14.5]
    w[1, :5] = [-7.5, 7.5, 0.0, 0.5, -3.25]
    codes, scales, zeros = orc.quantize(ASYM, 32, bits16(w))
    assert np.all(f16(scales) == 1.0)
    z = zero_points(zeros, 2)
    assert z.tolist() == [0, 8]
    nib = unpack_page(codes)
    assert nib[0, :4].tolist() == [15, 0, 2, 14]
    # -7.5 -> round(-7.5) = -8 -> q = 0; 7.5 -> 8 -> 16 -> clamp 15; 0 -> 8;
    # 0.5 -> 0 -> 8; -3.25 -> -3 -> 5
    assert nib[1, :5].tolist() == [0, 15, 8, 8, 5]


# ------------------------------------------------- P5 INT4 exhaustive absmax
def _all_positive_f16():
    b = np.arange(1, 0x7C00, dtype=np.uint16)
    return b


def test_int4_sym_exhaustive_absmax(orc):
    a = _all_positive_f16()
    n = a.size
    w = np.zeros((2 * n, 32), np.uint16)
    w[:n, 0] = a
    w[n:, 0] = a | 0x8000                      # the same magnitude, negative
    codes, scales, _ = orc.quantize(SYM, 32, w)
    s = f16(scales[:, 0])
    av = f16(a)
    nib = unpack_page(codes)
    normal = s[:n] >= np.float32(2.0 ** -14)
    # a normal scale appears exactly from some absmax on (monotone)
    first = np.argmax(normal)
    assert np.all(normal[first:]) and not np.any(normal[:first])
    assert 4.27e-4 < av[first] < 4.28e-4
    # scale is a/7 to within fp32 then fp16 rounding
    rel = np.abs(s[:n][normal].astype(np.float64) * 7 - av[normal]) / av[normal]
    assert rel.max() <= 2.0 ** -11 + 2.0 ** -23
    # with a normal scale the absmax codes to the top level, -absmax to -7:
    # level -8 (nibble 0) never occurs
    assert np.all(nib[:n][normal, 0] == 15)
    assert np.all(nib[n:][normal, 0] == 1)
    assert (av[normal].astype(np.float64) / s[:n][normal]).max() < 7.5
    # zeros elsewhere code to the zero level
    assert np.all(nib[:, 1:] == 8)
    # scale 0 only for absmax below half of the smallest subnormal times 7
    zero = s[:n] == 0
    assert np.all(av[zero] <= 7 * 2.0 ** -25) and np.all(av[~zero] > 7 * 2.0 ** -25 * 0.99)


def test_int4_asym_exhaustive_range(orc):
    a = _all_positive_f16()
    n = a.size
    w = np.zeros((n, 32), np.uint16)
    w[:, 0] = a | 0x8000                       # lo = -a
    w[:, 1] = np.flip(a)                       # hi = some other magnitude
    codes, scales, zeros = orc.quantize(ASYM, 32, w)
    s = f16(scales[:, 0]).astype(np.float64)
    z = zero_points(zeros, n).astype(int)
    nib = unpack_page(codes).astype(int)
    normal = s >= 2.0 ** -14
    lo = -f16(a).astype(np.float64)
    # zero is exactly a level: w = 0 codes to z and dequantizes to 0
    assert np.all(nib[normal, 2] == z[normal])
    # the zero-point needs no clamping with a normal scale
    assert np.all(-lo[normal] / s[normal] <= 15.5)
    # the low end codes to level 0
    assert np.all(nib[normal, 0] == 0)


# ----------------------------------------------- P6/P7 invariants and bounds
def _rand_w(N, K, seed, sigma=0.02, mu=0.0):
    rng = np.random.default_rng(seed)
    return bits16(rng.standard_normal((N, K)).astype(np.float32) * np.float32(sigma) + np.float32(mu))


def _ulp(v, out_t):
    v = np.abs(v).astype(np.float64)
    if out_t == F16:
        e = np.floor(np.log2(np.maximum(v, 2.0 ** -14)))
        return 2.0 ** (e - 10)
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -126)))
    return 2.0 ** (e - 7)


@pytest.mark.parametrize("fmt", [NF4, SYM, ASYM])
@pytest.mark.parametrize("g", [32, 64, 128])
def test_invariants_and_error_bound(orc, fmt, g):
    N, K = 96, 512
    w = _rand_w(N, K, 1000 + 10 * fmt + g, mu=0.001 if fmt == ASYM else 0.0)
    codes, scales, zeros = orc.quantize(fmt, g, w)
    G = K // g
    nib = unpack_page(codes)
    assert codes.shape == (N, K // 2) and scales.shape == (N, G)
    assert nib.min() >= 0 and nib.max() <= 15
    wv = f16(w).astype(np.float64)
    wg = wv.reshape(N, G, g)
    ng = nib.reshape(N, G, g).astype(np.int64)
    table = orc.nf4_table().astype(np.float64)
    if fmt == NF4:
        c = scales.astype(np.float64)
        # the stored absmax is the group's max |w| (grouping along K)
        assert np.array_equal(c, np.abs(wg).max(-1))
        # every group has a code at an end of the table
        assert np.all(((ng == 0) | (ng == 15)).any(-1))
        x = (wg.astype(np.float32) / c[..., None].astype(np.float32)).astype(np.float64)
        d = np.abs(x[..., None] - table)                    # brute force, 16 levels
        assert np.all(np.take_along_axis(d, ng[..., None], -1)[..., 0] <= d.min(-1))
        step = c[..., None]
        half_gap = 0.5 * np.diff(table).max()
        recon_bound = step * half_gap * (1 + 2.0 ** -20)
    else:
        s = f16(scales).astype(np.float64)
        assert np.all(s >= 2.0 ** -14)
        if fmt == SYM:
            level = ng - 8
            assert np.all(((ng == 1) | (ng == 15)).any(-1))
            assert not np.any(ng == 0)
            bound = 0.5 + 2.0 ** -20
        else:
            z = zero_points(zeros, N * G).reshape(N, G).astype(np.int64)
            level = ng - z[..., None]
            assert np.all(((ng == 0) | (ng == 15)).any(-1))
            bound = 0.5 + 15 * 2.0 ** -11 + 2.0 ** -20
        recon = level * s[..., None]
        assert np.all(np.abs(recon - wg) <= bound * s[..., None])
        recon_bound = bound * s[..., None]
    for out_t in (F16, BF16):
        out = orc.dequantize(fmt, g, codes, scales, zeros, N, K, out_t)
        ov = (f16(out) if out_t == F16 else
              (out.astype(np.uint32) << 16).view(np.float32)).astype(np.float64)
        err = np.abs(ov.reshape(N, G, g) - wg)
        assert np.all(err <= recon_bound + 0.5 * _ulp(ov, out_t).reshape(N, G, g) + 1e-30)


@pytest.mark.parametrize("fmt", [NF4, SYM, ASYM])
def test_dequant_is_deterministic_function_of_codes(orc, fmt):
    # dequant(quant(w)) is a fixed point: re-quantizing the dequantized fp16
    # weights gives back the same codes for NF4/sym (levels are exact points).
    w = _rand_w(16, 256, 77 + fmt)
    codes, scales, zeros = orc.quantize(fmt, 64, w)
    out = orc.dequantize(fmt, 64, codes, scales, zeros, 16, 256, F16)
    if fmt == NF4:
        codes2, scales2, _ = orc.quantize(fmt, 64, out)
        # absmax survives exactly only when fp16(c * Q[extreme]) == c, i.e. always
        assert np.array_equal(scales2, scales)
        assert np.array_equal(codes2, codes)


# -------------------------------------------------------------- P8 product
@pytest.mark.parametrize("fmt,act_t", [(NF4, F16), (SYM, BF16), (ASYM, BF16), (NF4, BF16), (3, BF16)])
def test_matmul_reference(orc, fmt, act_t):
    N, K, M, g = 40, 256, 3, 32
    w = _rand_w(N, K, 5 + fmt)
    codes, scales, zeros = orc.quantize(fmt, g, w)
    rng = np.random.default_rng(9)
    xf = rng.standard_normal((M, K)).astype(np.float32)
    if act_t == F16:
        x = bits16(xf)
        xv = f16(x).astype(np.float64)
    else:
        x = torch.from_numpy(xf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        xv = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    deq = orc.dequantize(fmt, g, codes, scales, zeros, N, K, act_t)
    wv = (f16(deq) if act_t == F16 else (deq.astype(np.uint32) << 16).view(np.float32)).astype(np.float64)
    y, ad = orc.matmul(fmt, g, act_t, x, codes, scales, zeros, N, K)
    ref = xv @ wv.T                                    # numpy (BLAS) product
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-15)
    assert np.allclose(ad, np.abs(xv) @ np.abs(wv).T, rtol=1e-12, atol=1e-15)
    # sampled rows give the same numbers as the full product
    rows = np.array([3, 0, 39, 17])
    ys, _ = orc.matmul(fmt, g, act_t, x, codes, scales, zeros, N, K, rows=rows)
    assert np.array_equal(ys, y[:, rows])
    # one-hot x picks one dequantized weight exactly; zero x gives zero
    onehot = np.zeros((2, K), np.uint16)
    onehot[0, 7] = 0x3C00 if act_t == F16 else 0x3F80
    yo, _ = orc.matmul(fmt, g, act_t, onehot, codes, scales, zeros, N, K)
    assert np.array_equal(yo[0], wv[:, 7])
    assert np.all(yo[1] == 0)


# ------------------------------------------------------ P9 byte arithmetic
def test_oracle_bits_per_weight(orc):
    import json
    with open(os.path.join(HERE, "golden", "footprints.json")) as f:
        fp = json.load(f)
    N, K = 8, 1024
    w = _rand_w(N, K, 1)
    bits = {}
    for fmt, g in [(NF4, 64), (SYM, 128), (ASYM, 32)]:
        codes, scales, zeros = orc.quantize(fmt, g, w)
        nbytes = codes.nbytes + scales.nbytes + (zeros.nbytes if zeros is not None else 0)
        bits[fmt] = nbytes * 8 / (N * K)
    nf = fp["nf4_absmax_bits"]
    assert bits[NF4] - 4 == nf["printed_bits"] == nf["absmax_bits"] / nf["block"]
    assert bits[SYM] == 4.125
    assert bits[ASYM] == 4.625


def test_output_rounding_term(orc):
    """The tolerance's output-rounding term is half the spacing of the
    output dtype at the reference: bf16 spacing at [8, 16) is 2^-4, fp16
    spacing at [1, 2) is 2^-10; and it is the largest error of that
    rounding (torch's conversion, checked on a sweep)."""
    assert orc.half_ulp(np.array([8.03]), BF16)[0] == 2.0 ** -5
    assert orc.half_ulp(np.array([1.5]), F16)[0] == 2.0 ** -11
    # (float32 inputs: one rounding, as the kernels' fp32 accumulators get)
    v = (np.random.default_rng(3).standard_normal(20000) * 50).astype(np.float32)
    for act, dt in ((BF16, torch.bfloat16), (F16, torch.float16)):
        r = torch.from_numpy(v).to(dt).double().numpy()
        assert np.all(np.abs(r - v) <= orc.half_ulp(v, act))
    t0 = orc.tolerance(np.array([1.0]))
    t1 = orc.tolerance(np.array([1.0]), np.array([8.03]), BF16)
    assert t0[0] == 2e-3 + 1e-3 and t1[0] == t0[0] + 2.0 ** -5
