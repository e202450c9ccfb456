"""No kernel reads past the buffers it is given.

Every input here is the front slice of a larger device buffer whose tail
holds values that would show in the result if read: bf16/fp16 Inf behind the
activations (0 * Inf is NaN, and Inf times a non-zero weight is Inf), 0xff
bytes behind codes, scales and zero-points (codes 15, NaN scales).  The
shapes are ragged in every direction a kernel tiles: M not a multiple of the
GEMM's 256-row tile, K not a multiple of its 256-column span nor of the
GEMV's 4096-column stage, N not a multiple of the backward product's 64-row
step.  The tails stay mapped, so a stray read returns the planted values
rather than faulting; the outputs must be finite and match the oracle.
"""

import numpy as np
import pytest
import torch

import oracle
from bit_group_wise_amd import q4, synth
from _helpers import DEV, TORCH_ACT, assert_product_ok, dev16

pytestmark = pytest.mark.gpu

TAIL = 1 << 20  # elements (or bytes) of planted tail behind every input


def inf_tailed(bits: np.ndarray, act: int) -> torch.Tensor:
    """A device tensor holding `bits` whose storage continues with Inf."""
    n = bits.size
    inf = 0x7C00 if act == q4.F16 else 0x7F80
    buf = torch.full((n + TAIL,), inf, dtype=torch.int16, device=DEV)
    buf[:n] = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).ravel()).to(DEV)
    return buf[:n].view(TORCH_ACT[act]).view(bits.shape)


def ff_tailed(t: torch.Tensor) -> torch.Tensor:
    """A copy of t (any dtype) whose storage continues with 0xff bytes."""
    nb = t.numel() * t.element_size()
    buf = torch.full((nb + TAIL,), 0xFF, dtype=torch.uint8, device=DEV)
    buf[:nb] = t.contiguous().view(torch.uint8).view(-1)
    return buf[:nb].view(t.dtype).view(t.shape)


def tailed_weight(q: q4.QuantizedWeight) -> q4.QuantizedWeight:
    """The same weight with codes, scales and zero-points in 0xff-tailed
    storage (the padding the size helpers add is part of the tail: its
    contents are never used as values)."""
    z = ff_tailed(q.zeros) if q.zeros is not None else None
    return q4.QuantizedWeight(q.fmt, q.g, q.N, q.K, ff_tailed(q.codes), ff_tailed(q.scales), z)


def _setup(fmt, g, N, K, seed):
    w = synth.weight_f16_bits(N, K, seed=seed, mu=0.001 if fmt == q4.INT4_ASYM else 0.0)
    q = q4.quantize(dev16(w), fmt, g)
    torch.cuda.synchronize()
    return tailed_weight(q), oracle.quantize(fmt, g, w)


FMTS = [q4.NF4, q4.INT4_SYM, q4.INT4_ASYM, q4.NF4_DQ, q4.FP4]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("act", [q4.BF16, q4.F16])
def test_gemm_ragged_inf_tail(fmt, act):
    for M, N, K, g in [(37, 200, 288, 32), (300, 136, 1088, 64), (17, 72, 384, 128)]:
        q, (oc, os_, oz) = _setup(fmt, g, N, K, seed=M + K)
        xb = synth.act_bits(M, K, seed=M + 1, act_t=act)
        y = q4.gemm(inf_tailed(xb, act), q)
        torch.cuda.synchronize()
        yr, ad = oracle.matmul(fmt, g, act, xb, oc, os_, oz, N, K)
        assert_product_ok(y, yr, ad, tag=f"gemm fmt{fmt} act{act} {M}x{N}x{K}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("act", [q4.BF16, q4.F16])
def test_gemv_ragged_inf_tail(fmt, act):
    """M = 1, 2 (one row per wave; x in registers, staged in LDS, or read
    from L2 for long rows) and the skinny product (M = 5)."""
    for M, N, K, g in [(1, 75, 2112, 64), (2, 75, 4224, 32), (1, 9, 40960, 128),
                       (2, 9, 20480, 64), (5, 75, 2176, 128)]:
        q, (oc, os_, oz) = _setup(fmt, g, N, K, seed=N + K)
        xb = synth.act_bits(M, K, seed=M + 3, act_t=act)
        y = q4.gemv(inf_tailed(xb, act), q)
        torch.cuda.synchronize()
        yr, ad = oracle.matmul(fmt, g, act, xb, oc, os_, oz, N, K)
        assert_product_ok(y, yr, ad, tag=f"gemv fmt{fmt} act{act} M{M} {N}x{K}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("act", [q4.BF16, q4.F16])
def test_chain_ragged_inf_tail(fmt, act):
    """Tasks whose last stage is partial (K = 11008, 2176) or single-row,
    every input Inf- or 0xff-tailed; independent and waiting tasks."""
    tasks, refs = [], []
    for i, (N, K, g) in enumerate([(77, 11008, 64), (5, 2176, 128), (1, 4096, 32),
                                   (130, 1024, 64)]):
        if K % g:
            continue
        q, (oc, os_, oz) = _setup(fmt, g, N, K, seed=i + 11)
        g_used = q.g
        xb = synth.act_bits(1, K, seed=i + 21, act_t=act)
        tasks.append((inf_tailed(xb, act), q, None, q4.TASK_NO_WAIT if i % 2 else 0))
        refs.append((xb, oc, os_, oz, N, K, g_used))
    # one chain per group size (a chain shares format and group size)
    by_g = {}
    for t, r in zip(tasks, refs):
        by_g.setdefault(r[6], []).append((t, r))
    for g, items in by_g.items():
        outs = q4.gemv_chain([t for t, _ in items])
        torch.cuda.synchronize()
        for y, (_, (xb, oc, os_, oz, N, K, _g)) in zip(outs, items):
            yr, ad = oracle.matmul(fmt, g, act, xb, oc, os_, oz, N, K)
            assert_product_ok(y, yr, ad, tag=f"chain fmt{fmt} act{act} {N}x{K} g{g}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("act", [q4.BF16, q4.F16])
def test_gemm_dx_ragged_inf_tail(fmt, act):
    for M, N, K, g in [(37, 136, 256, 64), (300, 72, 384, 32), (5, 520, 128, 128)]:
        q, (oc, os_, oz) = _setup(fmt, g, N, K, seed=M + N)
        dyb = synth.act_bits(M, N, seed=M + 5, act_t=act)
        dx = q4.gemm_dx(inf_tailed(dyb, act), q)
        torch.cuda.synchronize()
        ref, ad = oracle.matmul_dx(fmt, g, act, dyb, oc, os_, oz, N, K)
        assert_product_ok(dx, ref, ad, tag=f"gemm_dx fmt{fmt} act{act} {M}x{N}x{K}")
