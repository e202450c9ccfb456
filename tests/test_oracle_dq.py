"""Pins of the oracle's double quantization of the NF4 block constants.

The pages say only that the per-block absmax constants are quantized again in
blocks of 256 to 8 bits, and that this brings their cost from 0.5 to about
0.127 bits per parameter (about 0.4 bits saved).  The oracle reads the 8-bit
code as symmetric absmax int8 coding (scale = run max / 127, nearest level,
ties to even) with one binary32 constant per run of 256 absmax values in flat
group order.  These tests pin that reading without retyping it: the printed
bit figures, closed-form runs whose second-level scale is a power of two (so
every quotient is exact), the tie rule on exact halves, a brute-force nearest
level over all 128 levels, flat order across row boundaries, the partial last
run, the all-zero run, and the identity with plain NF4 when the absmax values
are representable exactly.
"""

import json
import os

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
NF4, NF4_DQ = 0, 3
F16, BF16 = 0, 1


def _bits16(vals):
    return np.asarray(vals, dtype=np.float32).astype(np.float16).view(np.uint16)


def _weights_with_absmax(c, g, N, seed=0):
    """fp16 weights [N, G*g] whose group absmax values are exactly c (flat,
    N*G values, each exactly representable in fp16): one element of each
    group carries +-c, the others are smaller in magnitude."""
    c = np.asarray(c, dtype=np.float32).reshape(N, -1)
    G = c.shape[1]
    rng = np.random.default_rng(seed)
    w = rng.uniform(-0.9, 0.9, size=(N, G, g)).astype(np.float32) * c[..., None]
    pos = rng.integers(0, g, size=(N, G))
    sign = np.where(rng.integers(0, 2, size=(N, G)) == 1, 1.0, -1.0).astype(np.float32)
    np.put_along_axis(w, pos[..., None], (sign * c)[..., None], axis=-1)
    wb = _bits16(w.reshape(N, G * g))
    # the fp16 rounding of the smaller elements cannot exceed c
    assert np.all(np.abs(wb.view(np.float16).astype(np.float32)).reshape(N, G, g).max(-1) == c)
    return wb


def test_printed_bit_figures(orc):
    """0.5 bits per parameter of fp32 absmax at g = 64, about 0.127 with the
    constants coded in 8 bits per run of 256, about 0.4 bits saved."""
    with open(os.path.join(HERE, "golden", "footprints.json")) as f:
        fp = json.load(f)["nf4_absmax_bits"]
    N, K, g = 64, 1024, fp["block"]             # N*K/g = 1024 constants, 4 runs
    rng = np.random.default_rng(3)
    w = _bits16(rng.standard_normal((N, K)).astype(np.float32) * 0.02)
    _, s_nf4, _ = orc.quantize(NF4, g, w)
    _, s_dq, _ = orc.quantize(NF4_DQ, g, w)
    bits_nf4 = s_nf4.nbytes * 8 / (N * K)
    bits_dq = s_dq.nbytes * 8 / (N * K)
    assert bits_nf4 == fp["printed_bits"]
    assert abs(bits_dq - fp["printed_dq_bits"]) < 5e-4
    assert round(bits_nf4 - bits_dq, 1) == 0.4
    assert orc.DQ_BLOCK == fp["dq_block"]
    qc, _ = orc.dq_split(s_dq, N * K // g)
    assert qc.dtype == np.uint8 and qc.size * 8 == fp["dq_bits"] * (N * K // g)


@pytest.mark.parametrize("g", [32, 64, 128])
def test_codes_are_those_of_nf4(orc, g):
    """Only the constants change: the 4-bit codes are made with the exact
    absmax, and the 8-bit codes are the second-level coding of NF4's absmax
    array."""
    N, K = 21, 1536                              # N*K/g crosses several runs
    rng = np.random.default_rng(g)
    w = _bits16(rng.standard_normal((N, K)).astype(np.float32) * 0.03)
    c1, s1, _ = orc.quantize(NF4, g, w)
    c2, s2buf, _ = orc.quantize(NF4_DQ, g, w)
    assert np.array_equal(c1, c2)
    qc, s2 = orc.dq_split(s2buf, N * K // g)
    qc_ref, s2_ref = orc.double_quant(s1.reshape(-1))
    assert np.array_equal(qc, qc_ref) and np.array_equal(s2, s2_ref)


def test_power_of_two_scale_is_exact(orc):
    """Run max 127 gives s2 = 1 exactly, so every integer absmax 0..127 is its
    own code and the DQ dequantization equals plain NF4's bit for bit."""
    g, N = 64, 4
    c = (np.arange(N * 128) % 128).astype(np.float32)   # 2 runs of 256, max 127
    K = g * c.size // N
    w = _weights_with_absmax(c, g, N, seed=1)
    codes, sb, _ = orc.quantize(NF4_DQ, g, w)
    qc, s2 = orc.dq_split(sb, c.size)
    assert np.array_equal(s2, np.ones(2, np.float32))
    assert np.array_equal(qc, c.astype(np.uint8))
    c0, s0, _ = orc.quantize(NF4, g, w)
    for out_t in (F16, BF16):
        a = orc.dequantize(NF4_DQ, g, codes, sb, None, N, K, out_t)
        b = orc.dequantize(NF4, g, c0, s0, None, N, K, out_t)
        assert np.array_equal(a, b)


def test_exact_halves_round_to_even(orc):
    """Run max 254 gives s2 = 2: odd absmax values sit exactly between two
    levels and go to the even one (1 -> 0, 3 -> 2, 5 -> 2, 7 -> 4, ...)."""
    g, N = 32, 2
    odd = np.arange(1, 255, 2, dtype=np.float32)              # 127 odd values
    c = np.concatenate([odd, [254.0], np.zeros(128, np.float32)])
    w = _weights_with_absmax(c, g, N, seed=2)
    _, sb, _ = orc.quantize(NF4_DQ, g, w)
    qc, s2 = orc.dq_split(sb, c.size)
    assert s2[0] == 2.0
    half = odd / 2.0                                          # k + 0.5
    even = np.where(np.floor(half) % 2 == 0, np.floor(half), np.ceil(half))
    assert np.array_equal(qc[:127], even.astype(np.uint8))
    assert qc[127] == 127 and np.all(qc[128:] == 0)


def test_nearest_level_brute_force(orc):
    """For absmax values from real weights, each 8-bit code is the nearest of
    the 128 levels q * s2 (brute force in fp64), the run max codes to 127, and
    s2 is the binary32 quotient of the run max by 127."""
    N, K, g = 50, 2048, 64                       # 1600 constants: 6 full runs + 64
    rng = np.random.default_rng(11)
    w = _bits16(rng.standard_normal((N, K)).astype(np.float32)
                * rng.uniform(0.005, 0.05, size=(N, 1)).astype(np.float32))
    _, s_nf4, _ = orc.quantize(NF4, g, w)
    c = s_nf4.reshape(-1).astype(np.float64)
    _, sb, _ = orc.quantize(NF4_DQ, g, w)
    qc, s2 = orc.dq_split(sb, c.size)
    assert s2.size == 7
    run = np.arange(c.size) // 256
    step = s2.astype(np.float64)[run]
    levels = np.arange(128, dtype=np.float64)
    dist = np.abs(c[:, None] - levels[None, :] * step[:, None])
    chosen = dist[np.arange(c.size), qc.astype(np.int64)]
    # fp32 division may move a near-tie by a hair: allow 2^-20 of a step
    assert np.all(chosen <= dist.min(1) + step * 2.0 ** -20)
    assert np.all(chosen <= step * (0.5 + 2.0 ** -20))
    for b in range(s2.size):
        cb = c[run == b]
        assert s2[b] == np.float32(np.float32(cb.max()) / np.float32(127.0))
        assert qc[run == b][np.argmax(cb)] == 127


def test_runs_follow_flat_group_order(orc):
    """Runs of 256 constants cross row boundaries (flat order r*G + j): with
    G = 100, run 0 holds rows 0, 1 and the first 56 groups of row 2."""
    g, N, G = 32, 3, 100
    c = np.ones(N * G, np.float32)
    c[2 * G + 55] = 127.0 / 64.0                 # in run 0: s2 = 1/64 exactly
    w = _weights_with_absmax(c, g, N, seed=5)
    _, sb, _ = orc.quantize(NF4_DQ, g, w)
    qc, s2 = orc.dq_split(sb, N * G)
    assert s2[0] == 1.0 / 64.0
    assert s2[1] == np.float32(np.float32(1.0) / np.float32(127.0))
    exp = np.full(N * G, 64, np.uint8)
    exp[2 * G + 55] = 127
    exp[256:] = 127
    assert np.array_equal(qc, exp)
    # the buffer layout: codes, zero padding up to 16 bytes, then s2
    off = orc.dq_s2_offset(N * G)
    assert off == 304 and sb.size == 304 + 8 and np.all(sb[300:304] == 0)


def test_zero_run_and_partial_last_run(orc):
    """An all-zero run has s2 = 0 and codes 0 and dequantizes to zeros; the
    short last run takes its own max."""
    g, N = 128, 3
    c = np.zeros(300, np.float32)
    c[256:] = np.linspace(0.25, 8.0, 44).astype(np.float16).astype(np.float32)
    w = _weights_with_absmax(c, g, N, seed=6)
    codes, sb, _ = orc.quantize(NF4_DQ, g, w)
    qc, s2 = orc.dq_split(sb, 300)
    assert s2[0] == 0.0 and np.all(qc[:256] == 0)
    assert s2[1] == np.float32(np.float32(8.0) / np.float32(127.0))
    assert qc[-1] == 127
    out = orc.dequantize(NF4_DQ, g, codes, sb, None, N, 100 * g, F16)
    deq = out.view(np.float16).astype(np.float32).reshape(-1)
    assert np.all(deq[:256 * g] == 0)
    # the recovered absmax of the last run is within half a step of c
    chat = qc[256:].astype(np.float64) * np.float64(s2[1])
    assert np.all(np.abs(chat - c[256:]) <= 0.5 * s2[1] * (1 + 2.0 ** -20))


def test_dequant_uses_recovered_absmax(orc):
    """DQ dequantization equals plain NF4 dequantization with the absmax
    array replaced by the recovered constants q * s2 (binary32)."""
    N, K, g = 12, 2048, 64
    rng = np.random.default_rng(21)
    w = _bits16(rng.standard_normal((N, K)).astype(np.float32) * 0.02)
    codes, sb, _ = orc.quantize(NF4_DQ, g, w)
    qc, s2 = orc.dq_split(sb, N * K // g)
    chat = (qc.astype(np.float32) * s2[np.arange(qc.size) // 256]).astype(np.float32)
    for out_t in (F16, BF16):
        a = orc.dequantize(NF4_DQ, g, codes, sb, None, N, K, out_t)
        b = orc.dequantize(NF4, g, codes, chat.reshape(N, -1), None, N, K, out_t)
        assert np.array_equal(a, b)
