"""GPU parity: libq4's HIP kernels against the CPU oracle, through the C ABI.

Codes, packed bytes, scales, zero-points and dequantized fp16/bf16 values must
be bit-identical; GEMV/GEMM outputs must satisfy
|y - y_ref(fp64)| <= 2e-3 * sum_k |x_k * what_k| + 1e-3 for every output.
Inputs come from the shared seeded generators (bit_group_wise_amd.synth) and
from exhaustive fp16 sweeps.
"""

import numpy as np
import pytest
import torch

import oracle
from bit_group_wise_amd import q4, synth
from _helpers import DEV, TORCH_ACT, assert_product_ok, assert_quant_equal, dev16, host16

pytestmark = pytest.mark.gpu

FMTS = [q4.NF4, q4.INT4_SYM, q4.INT4_ASYM, q4.NF4_DQ, q4.FP4]
GS = [32, 64, 128]


def bits16(v):
    return np.asarray(v, np.float32).astype(np.float16).view(np.uint16)


def special_rows(K, seed):
    """Rows that exercise degenerate groups: all zero, a single non-zero,
    values so small that the INT4 scale is subnormal or zero, huge values,
    all negative, all positive."""
    rng = np.random.default_rng(seed)
    rows = np.zeros((8, K), np.float32)
    rows[1, 3] = 0.5
    rows[2] = rng.standard_normal(K) * 1e-6
    rows[3] = rng.standard_normal(K) * 2e-7
    rows[4] = rng.standard_normal(K) * 3000.0
    rows[5] = -np.abs(rng.standard_normal(K)) * 0.02
    rows[6] = np.abs(rng.standard_normal(K)) * 0.02 + 0.01
    rows[7] = rng.standard_normal(K) * 0.02
    rows[7, ::7] = 0.0
    return bits16(rows)


# ------------------------------------------------------------------ codec
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("g", GS)
@pytest.mark.parametrize("shape", [(96, 1024), (37, 384), (1, 128), (3, 640)])
def test_quantize_dequantize_bit_exact(fmt, g, shape):
    N, K = shape
    w = synth.weight_f16_bits(N, K, seed=1000 + N + fmt, mu=0.001 if fmt == q4.INT4_ASYM else 0.0)
    w = np.concatenate([w, special_rows(K, 7)], 0)
    N = w.shape[0]
    q, (oc, os_, oz) = assert_quant_equal(fmt, g, w, tag=f"fmt{fmt} g{g} {shape}")
    for act in (q4.F16, q4.BF16):
        out = q4.dequantize(q, TORCH_ACT[act])
        torch.cuda.synchronize()
        ref = oracle.dequantize(fmt, g, oc, os_, oz, N, K, act)
        got = host16(out)
        bad = np.argwhere(got != ref)
        assert bad.size == 0, f"dequant act{act} differs at {bad[:5].tolist()}"


def all_finite_f16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = b.view(np.float16)
    return b[np.isfinite(v)]


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_exhaustive_fp16(fmt):
    """Every finite fp16 value, in groups of 32 drawn in several orders (so
    each value meets many different group scales), plus every value in a
    unit-absmax NF4 block."""
    vals = all_finite_f16()
    rng = np.random.default_rng(42)
    rows = []
    for _ in range(4):
        p = vals[rng.permutation(vals.size)]
        rows.append(p[: (p.size // 128) * 128].reshape(-1, 128))
    # sorted by magnitude: neighbouring magnitudes share groups
    mag = vals[np.argsort(np.abs(vals.view(np.float16).astype(np.float32)), kind="stable")]
    rows.append(mag[: (mag.size // 128) * 128].reshape(-1, 128))
    w = np.concatenate(rows, 0)
    for g in GS:
        assert_quant_equal(fmt, g, w, tag=f"exhaustive fmt{fmt} g{g}")
    if fmt in (q4.NF4, q4.FP4):
        unit = vals[np.abs(vals.view(np.float16).astype(np.float32)) <= 1.0]
        n63 = (unit.size + 62) // 63
        pad = np.concatenate([unit, np.zeros(n63 * 63 - unit.size, np.uint16)])
        blk = np.concatenate([np.full((n63, 1), 0x3C00, np.uint16), pad.reshape(n63, 63)], 1)
        assert_quant_equal(fmt, 64, blk, tag="unit blocks")


@pytest.mark.parametrize("fmt", [q4.INT4_SYM, q4.INT4_ASYM])
def test_quantize_every_absmax(fmt):
    """Groups [a, -a/3, 0...] for every positive fp16 a: every scale value,
    the subnormal-scale and zero-scale regimes."""
    a = np.arange(1, 0x7C00, dtype=np.uint16)
    w = np.zeros((a.size, 32), np.uint16)
    w[:, 0] = a
    w[:, 1] = bits16(-a.view(np.float16).astype(np.float32) / 3)
    assert_quant_equal(fmt, 32, w, tag="every absmax")


def test_quantize_outliers_config_shape():
    w = synth.weight_f16_bits(512, 4096, seed=201, outlier_seed=202)
    assert_quant_equal(q4.INT4_SYM, 128, w, tag="outliers")


def test_determinism():
    w = synth.weight_f16_bits(256, 2048, seed=5)
    x = dev16(synth.act_bits(1, 2048, 6, q4.BF16), q4.BF16)
    outs = []
    for _ in range(2):
        q = q4.quantize(dev16(w), q4.NF4, 64)
        y = q4.gemv(x, q)
        z = q4.gemm(x, q)
        torch.cuda.synchronize()
        outs.append((q.codes.cpu().numpy(), host16(y), host16(z)))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)


# ------------------------------------------------------------------ products
def _setup(fmt, g, N, K, M, act, seed):
    w = synth.weight_f16_bits(N, K, seed=seed, mu=0.001 if fmt == q4.INT4_ASYM else 0.0)
    q, (oc, os_, oz) = assert_quant_equal(fmt, g, w)
    xb = synth.act_bits(M, K, seed + 1, act)
    return q, (oc, os_, oz), xb


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("act", [q4.F16, q4.BF16])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 7, 8, 13, 16])
def test_gemv_tolerance(fmt, act, M):
    for g, K in [(32, 2080), (64, 2112), (128, 2176)]:   # 65, 66, 68 chunks: ragged lanes
        N = 75
        q, (oc, os_, oz), xb = _setup(fmt, g, N, K, M, act, seed=300 + M + g)
        y = q4.gemv(dev16(xb, act), q)
        torch.cuda.synchronize()
        yr, ad = oracle.matmul(fmt, g, act, xb, oc, os_, oz, N, K)
        assert_product_ok(y, yr, ad, tag=f"gemv fmt{fmt} act{act} M{M} g{g}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("act", [q4.F16, q4.BF16])
def test_gemv_special_inputs(fmt, act):
    g, N, K = 64, 40, 512
    q, (oc, os_, oz), _ = _setup(fmt, g, N, K, 1, act, seed=77)
    deq = host16(q4.dequantize(q, TORCH_ACT[act]))
    one = 0x3C00 if act == q4.F16 else 0x3F80
    x = np.zeros((3, K), np.uint16)
    x[0, 5] = one
    x[1, K - 1] = one
    y = host16(q4.gemv(dev16(x, act), q))
    torch.cuda.synchronize()
    assert np.all((y[2] & 0x7FFF) == 0)           # zero x gives exactly zero
    # every weight enters as the value q4_dequantize writes: a one-hot x
    # returns the dequantized weight exactly (zeros compared as values)
    as_f = (lambda b: b.view(np.float16).astype(np.float32)) if act == q4.F16 else \
        (lambda b: (b.astype(np.uint32) << 16).view(np.float32))
    assert np.array_equal(as_f(y[0]), as_f(deq[:, 5]))
    assert np.array_equal(as_f(y[1]), as_f(deq[:, K - 1]))
    yr, ad = oracle.matmul(fmt, g, act, x, oc, os_, oz, N, K)
    assert_product_ok(torch.from_numpy(y.view(np.int16)).view(TORCH_ACT[act]), yr, ad)


def test_gemv_rows_consistent_with_m1():
    """Row m of a batched GEMV is the M = 1 GEMV of x[m] within tolerance."""
    fmt, g, act, N, K = q4.NF4, 64, q4.BF16, 128, 1024
    q, (oc, os_, oz), xb = _setup(fmt, g, N, K, 5, act, seed=9)
    yb = q4.gemv(dev16(xb, act), q).float().cpu().numpy()
    for m in range(5):
        y1 = q4.gemv(dev16(xb[m:m + 1], act), q).float().cpu().numpy()
        yr, ad = oracle.matmul(fmt, g, act, xb[m:m + 1], oc, os_, oz, N, K)
        assert np.all(np.abs(yb[m] - y1[0]) <= 2 * oracle.tolerance(ad[0]))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("act", [q4.F16, q4.BF16])
@pytest.mark.parametrize("M,N,K,g", [(1, 64, 256, 64), (37, 200, 288, 32), (128, 128, 512, 128),
                                     (300, 136, 1024, 64), (17, 1000, 160, 32)])
def test_gemm_tolerance(fmt, act, M, N, K, g):
    q, (oc, os_, oz), xb = _setup(fmt, g, N, K, M, act, seed=M + N)
    y = q4.gemm(dev16(xb, act), q)
    torch.cuda.synchronize()
    yr, ad = oracle.matmul(fmt, g, act, xb, oc, os_, oz, N, K)
    assert_product_ok(y, yr, ad, tag=f"gemm fmt{fmt} act{act} {M}x{N}x{K}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("act", [q4.F16, q4.BF16])
def test_gemm_skinny_row_blocks_and_slices(fmt, act):
    """q4_gemm up to 96 activation rows runs the skinny product with 1, 2 or
    4 blocks of 16 rows per launch, and past 64 rows as consecutive launches
    over row slices: every row count class, ragged N and K, against the
    oracle."""
    for M, N, K, g in [(31, 200, 288, 32), (33, 136, 1088, 64), (64, 72, 384, 128),
                       (65, 200, 288, 32), (80, 136, 576, 64), (96, 1000, 160, 32)]:
        q, (oc, os_, oz), xb = _setup(fmt, g, N, K, M, act, seed=M + N + K)
        y = q4.gemm(dev16(xb, act), q)
        torch.cuda.synchronize()
        yr, ad = oracle.matmul(fmt, g, act, xb, oc, os_, oz, N, K)
        assert_product_ok(y, yr, ad, tag=f"gemm fmt{fmt} act{act} {M}x{N}x{K}")


def test_gemm_matches_library_matmul():
    """Cross-check against torch.matmul on the dequantized weights."""
    fmt, g, act, M, N, K = q4.INT4_ASYM, 32, q4.BF16, 256, 384, 1024
    q, (oc, os_, oz), xb = _setup(fmt, g, N, K, M, act, seed=11)
    x = dev16(xb, act)
    y = q4.gemm(x, q).float()
    wd = q4.dequantize(q, torch.bfloat16).float()
    ref = torch.matmul(x.float(), wd.t().contiguous())
    yr, ad = oracle.matmul(fmt, g, act, xb, oc, os_, oz, N, K)
    tol = torch.from_numpy(oracle.tolerance(ad)).to(DEV).float()
    assert torch.all((y - ref).abs() <= 2 * tol)
