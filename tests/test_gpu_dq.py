"""NF4 with double-quantized absmax on the GPU: every kernel against the
oracle on weights whose rows differ in magnitude by up to 2^10, so that a
group given another run's second-level constant (or another group's 8-bit
code) is off by a large factor.

Shapes put run boundaries (every 256 groups, flat order) inside rows, inside
a GEMV stage, inside a GEMM span of 256 k and at ragged row ends: K / g of 65,
33, 3 and 9 groups per row.  Quantize and dequantize are bit-exact; products
meet the tolerance |y - y_ref| <= 2e-3 sum|x what| + 1e-3; the chain equals
consecutive GEMVs bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle
from bit_group_wise_amd import q4, synth
from _helpers import DEV, TORCH_ACT, assert_product_ok, assert_quant_equal, dev16, host16

pytestmark = pytest.mark.gpu

SHAPES = [(75, 2080, 32), (300, 1056, 32), (37, 384, 128), (200, 576, 64), (4099, 4096, 64)]


def _weight(N, K, seed):
    return synth.weight_rowscaled_f16_bits(N, K, seed)


@pytest.mark.parametrize("N,K,g", SHAPES)
def test_dq_quantize_dequantize_bit_exact(N, K, g):
    w = _weight(N, K, 500 + N)
    print(f"dq codec {N}x{K} g{g}", flush=True)
    q, (oc, os_, oz) = assert_quant_equal(q4.NF4_DQ, g, w, tag=f"dq {N}x{K} g{g}")
    qc, s2 = q4.dq_parts(q)
    assert s2.numel() == (N * K // g + 255) // 256
    for act in (q4.F16, q4.BF16):
        got = host16(q4.dequantize(q, TORCH_ACT[act]))
        ref = oracle.dequantize(q4.NF4_DQ, g, oc, os_, oz, N, K, act)
        bad = np.argwhere(got != ref)
        assert bad.size == 0, f"dq dequant act{act} differs at {bad[:5].tolist()}"


@pytest.mark.parametrize("act", [q4.BF16, q4.F16])
@pytest.mark.parametrize("N,K,g", SHAPES[:4])
def test_dq_products(N, K, g, act):
    w = _weight(N, K, 700 + K)
    q, (oc, os_, oz) = assert_quant_equal(q4.NF4_DQ, g, w)
    for M in (1, 2, 4, 16, 17, 300):
        print(f"dq product {N}x{K} g{g} act{act} M{M}", flush=True)
        xb = synth.act_bits(M, K, 900 + M, act)
        x = dev16(xb, act)
        yr, ad = oracle.matmul(q4.NF4_DQ, g, act, xb, oc, os_, oz, N, K)
        if M <= 16:
            y = q4.gemv(x, q)
            torch.cuda.synchronize()
            assert_product_ok(y, yr, ad, tag=f"dq gemv M{M} {N}x{K} g{g}")
        y = q4.gemm(x, q)
        torch.cuda.synchronize()
        assert_product_ok(y, yr, ad, tag=f"dq gemm M{M} {N}x{K} g{g}")


def test_dq_large_rows_sampled():
    """4099 x 4096 (runs of 256 groups = 4 rows at g = 64; a ragged last
    workgroup of rows): GEMV, skinny product and GEMM on sampled rows."""
    N, K, g = 4099, 4096, 64
    w = _weight(N, K, 41)
    q, (oc, os_, oz) = assert_quant_equal(q4.NF4_DQ, g, w)
    rows = np.concatenate([np.arange(0, 8), np.arange(4090, 4099),
                           np.random.default_rng(3).choice(N, 40, replace=False)])
    for M in (1, 8, 64):
        xb = synth.act_bits(M, K, 77 + M, q4.BF16)
        x = dev16(xb, q4.BF16)
        yr, ad = oracle.matmul(q4.NF4_DQ, g, q4.BF16, xb, oc, os_, oz, N, K, rows=rows)
        y = (q4.gemv(x, q) if M <= 16 else q4.gemm(x, q))[:, torch.from_numpy(rows).to(DEV)]
        torch.cuda.synchronize()
        assert_product_ok(y, yr, ad, tag=f"dq large M{M}")


def test_dq_chain_matches_gemv():
    """A chain of double-quantized GEMVs, one reading the previous output,
    equals consecutive q4_gemv calls bit for bit."""
    tasks, ref = [], []
    prev = None
    for i, (N, K) in enumerate([(2080, 1024), (300, 2080), (4096, 300 // 4 * 4)]):
        K = K if K % 32 == 0 else (K // 32) * 32
        q = q4.quantize(dev16(_weight(N, K, 60 + i)), q4.NF4_DQ, 32)
        x = dev16(synth.act_bits(1, K, 80 + i, q4.BF16), q4.BF16)
        y = torch.empty((1, N), dtype=torch.bfloat16, device=DEV)
        tasks.append((x, q, y))
        ref.append(q4.gemv(x, q))
    # a dependent task: x is the first task's output
    qd = q4.quantize(dev16(_weight(640, 2080, 99)), q4.NF4_DQ, 32)
    tasks.append((tasks[0][2], qd, torch.empty((1, 640), dtype=torch.bfloat16, device=DEV)))
    ref.append(q4.gemv(ref[0], qd))
    outs = q4.gemv_chain(tasks)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(outs, ref)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"task {i} differs"


def test_dq_long_rows_gemv():
    """Rows longer than the runs of 256 groups a stage can touch (K / g of
    769, 641 and 528 groups, so runs also start inside rows), with the
    magnitude changing every 2048 columns so that every run has its own
    second-level constant: the M <= 2 GEMV (which picks a stage's runs from
    the stage's first group) and the skinny product against the oracle."""
    for g, K in [(32, 24608), (64, 41024), (128, 67584)]:
        N = 5
        v = synth.normal_f32((N, K), 4100 + g, 0.02, 0.0)
        v *= np.exp2((np.arange(K) // 2048) % 9 - 4).astype(np.float32)[None, :]
        w = synth.to_f16_bits(v)
        q, (oc, os_, oz) = assert_quant_equal(q4.NF4_DQ, g, w, tag=f"dq long rows g{g}")
        for act in (q4.BF16, q4.F16):
            for M in (1, 2, 4):
                print(f"dq long rows g{g} K{K} act{act} M{M}", flush=True)
                xb = synth.act_bits(M, K, 4200 + M, act)
                y = q4.gemv(dev16(xb, act), q)
                torch.cuda.synchronize()
                yr, ad = oracle.matmul(q4.NF4_DQ, g, act, xb, oc, os_, oz, N, K)
                assert_product_ok(y, yr, ad, tag=f"dq long rows g{g} act{act} M{M}")
