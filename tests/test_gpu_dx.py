"""Backward product dX = dY . What (q4_gemm_dx) against the oracle.

Every format, group size and activation dtype on shapes with ragged M, N and
K against the tile (256 x 128 output, 64 rows of W per step): one tile, a
partial tile in every direction, N not a multiple of 64.  Weights have rows
of very different magnitude, so a row read in place of another is off by a
large factor.  A 7B-style shape (M = 2048, N = 14336, K = 4096) is checked
on sampled columns, and one case against torch's matmul on the dequantized
weight.
"""

import numpy as np
import pytest
import torch

import oracle
from bit_group_wise_amd import q4, synth
from _helpers import DEV, TORCH_ACT, assert_product_ok, assert_quant_equal, dev16

pytestmark = pytest.mark.gpu

SHAPES = [(256, 64, 128), (37, 200, 288), (300, 136, 1024), (513, 1032, 160), (1, 8, 32)]


@pytest.mark.parametrize("act", [q4.BF16, q4.F16])
@pytest.mark.parametrize("fmt", [q4.NF4, q4.INT4_SYM, q4.INT4_ASYM, q4.NF4_DQ, q4.FP4])
def test_dx_against_oracle(fmt, act):
    for g in (32, 64, 128):
        for M, N, K in SHAPES:
            if K % g:
                continue
            tag = f"dx fmt{fmt} act{act} g{g} {M}x{N}x{K}"
            print(tag, flush=True)
            w = synth.weight_rowscaled_f16_bits(N, K, seed=M + N + K + g)
            q, (oc, os_, oz) = assert_quant_equal(fmt, g, w)
            dyb = synth.act_bits(M, N, 7 + M, act)
            dx = q4.gemm_dx(dev16(dyb, act), q)
            torch.cuda.synchronize()
            ref, ad = oracle.matmul_dx(fmt, g, act, dyb, oc, os_, oz, N, K)
            assert_product_ok(dx, ref, ad, tag=tag)


def test_dx_7b_shape_sampled():
    """M = 2048, N = 14336, K = 4096 (INT4-asym g32, bf16): sampled columns at
    tile edges and at random."""
    M, N, K, g, act = 2048, 14336, 4096, 32, q4.BF16
    w = synth.weight_f16_bits(N, K, seed=401, mu=0.001)
    q, (oc, os_, oz) = assert_quant_equal(q4.INT4_ASYM, g, w)
    dyb = synth.act_bits(M, N, 403, act)
    dx = q4.gemm_dx(dev16(dyb, act), q)
    torch.cuda.synchronize()
    cols = np.concatenate([[0, 1, 127, 128, 4095], np.random.default_rng(5).choice(K, 11, replace=False)])
    rows = np.concatenate([[0, 255, 256, 2047], np.random.default_rng(6).choice(M, 4, replace=False)])
    ref, ad = oracle.matmul_dx(q4.INT4_ASYM, g, act, dyb[rows], oc, os_, oz, N, K, cols=cols)
    got = dx[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols).to(DEV)]
    assert_product_ok(got, ref, ad, tag="dx 7b sampled")


def test_dx_matches_library_matmul():
    """dY @ dequantize(W) with torch (fp32) agrees within the same bound."""
    fmt, g, act, M, N, K = q4.NF4, 64, q4.BF16, 384, 512, 768
    w = synth.weight_f16_bits(N, K, seed=12)
    q = q4.quantize(dev16(w), fmt, g)
    dy = dev16(synth.act_bits(M, N, 13, act), act)
    dx = q4.gemm_dx(dy, q).float()
    wd = q4.dequantize(q, torch.bfloat16).float()
    ref = torch.matmul(dy.float(), wd)
    # (plus half a bf16 ulp of the result: dX is rounded once to bf16)
    tol = 2e-3 * torch.matmul(dy.float().abs(), wd.abs()) + 1e-3 + ref.abs() * 2.0 ** -8
    assert bool(((dx - ref).abs() <= tol).all())


def test_dx_rejects():
    q = q4.alloc_quantized(q4.NF4, 64, 12, 128, DEV)
    dy = torch.zeros((2, 12), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(q4.Q4Error):
        q4.gemm_dx(dy, q)          # N % 8 != 0
