"""Long rows.  The largest K q4_gemm accepts (Q4_GEMM_MAX_K): a 256-row tile
of x then spans exactly 2^31 bytes, the end of the GEMM's 32-bit buffer
view.  The sampled x rows are zero except near both ends of K, so a dword
the view failed to cover (read as zero) would change those outputs
completely.  And q4_gemv on rows of about half a million weights, every
format."""

import numpy as np
import pytest
import torch

import oracle
from bit_group_wise_amd import q4, synth
from _helpers import DEV, assert_product_ok, dev16

pytestmark = pytest.mark.gpu


def test_gemm_at_max_k():
    K = 4194304
    N, M, g, fmt = 16, 256, 128, q4.INT4_SYM
    w = synth.weight_f16_bits(N, K, seed=901)
    oc, os_, oz = oracle.quantize(fmt, g, w)
    q = q4.quantize(dev16(w), fmt, g)
    torch.cuda.synchronize()
    assert np.array_equal(q.codes.cpu().numpy(), oc)
    # x rows 0 and 255 (the tile's first and last): values only in the first
    # and last 64 columns; all other rows zero
    xs = np.zeros((2, K), np.uint16)
    ends = synth.act_bits(2, 128, seed=902, act_t=q4.BF16)
    xs[:, :64] = ends[:, :64]
    xs[:, -64:] = ends[:, 64:]
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    xd = dev16(xs, q4.BF16)
    x[0] = xd[0]
    x[M - 1] = xd[1]
    y = q4.gemm(x, q)
    torch.cuda.synchronize()
    yr, ad = oracle.matmul(fmt, g, q4.BF16, xs, oc, os_, oz, N, K)
    assert_product_ok(y[[0, M - 1]], yr, ad, tag="gemm K = Q4_GEMM_MAX_K")
    # the last dword alone (x only in the last 2 columns) is seen
    xs2 = np.zeros((1, K), np.uint16)
    xs2[0, -2:] = ends[1, -2:]
    x[M - 1] = dev16(xs2, q4.BF16)[0]
    y = q4.gemm(x, q)
    torch.cuda.synchronize()
    yr, ad = oracle.matmul(fmt, g, q4.BF16, xs2, oc, os_, oz, N, K)
    assert np.any(yr != 0)
    assert_product_ok(y[[M - 1]], yr, ad, tag="gemm K = Q4_GEMM_MAX_K, last dword")
    del x
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", [q4.NF4, q4.INT4_SYM, q4.INT4_ASYM, q4.NF4_DQ, q4.FP4])
def test_gemv_long_rows(fmt):
    """q4_gemv on rows of 524,416 weights (129 stages of the M <= 2 GEMV, x
    read from L2 instead of staged in LDS; for double quantization, 16 to 65
    runs of 256 groups per row), the magnitude changing every 4096 columns,
    at M = 1, 2 (vector ALUs) and 4, 16 (skinny product) against the
    oracle."""
    K, N = 524416, 9
    for g in (32, 128):
        v = synth.normal_f32((N, K), 950 + g, 0.02)
        v *= np.exp2((np.arange(K) // 4096) % 9 - 4).astype(np.float32)[None, :]
        w = synth.to_f16_bits(v)
        oc, os_, oz = oracle.quantize(fmt, g, w)
        q = q4.quantize(dev16(w), fmt, g)
        for M in (1, 2, 4, 16):
            print(f"gemv long rows fmt{fmt} g{g} M{M}", flush=True)
            xb = synth.act_bits(M, K, 960 + M, q4.BF16)
            y = q4.gemv(dev16(xb, q4.BF16), q)
            torch.cuda.synchronize()
            yr, ad = oracle.matmul(fmt, g, q4.BF16, xb, oc, os_, oz, N, K)
            assert_product_ok(y, yr, ad, tag=f"gemv long rows fmt{fmt} g{g} M{M}")
