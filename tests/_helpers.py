"""Shared helpers of the GPU parity tests: moving bit patterns between numpy
and torch device tensors, and comparing GPU results with the oracle."""

import numpy as np
import torch

import oracle
from bit_group_wise_amd import q4

DEV = "cuda:0"
TORCH_ACT = {q4.F16: torch.float16, q4.BF16: torch.bfloat16}


def dev16(bits: np.ndarray, act_t: int = q4.F16) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).to(DEV)
    return t.view(TORCH_ACT[act_t])


def host16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def gpu_quantize(fmt, g, w_bits):
    q = q4.quantize(dev16(w_bits), fmt, g)
    torch.cuda.synchronize()
    codes = q.codes.cpu().numpy()
    if fmt in (q4.NF4, q4.NF4_DQ, q4.FP4):   # float32 [N, G], or the NF4_DQ byte buffer
        scales = q.scales.cpu().numpy()
    else:
        scales = q.scales.view(torch.int16).cpu().numpy().view(np.uint16)
    zeros = q.zeros.cpu().numpy() if q.zeros is not None else None
    return q, codes, scales, zeros


def assert_quant_equal(fmt, g, w_bits, tag=""):
    """GPU quantize == oracle quantize, bit for bit; returns the GPU weight."""
    q, codes, scales, zeros = gpu_quantize(fmt, g, w_bits)
    oc, os_, oz = oracle.quantize(fmt, g, w_bits)
    bad = np.argwhere(codes != oc)
    assert bad.size == 0, f"{tag} codes differ at {bad[:5].tolist()} gpu={codes[tuple(bad[0])]:#x} orc={oc[tuple(bad[0])]:#x}"
    if fmt in (q4.NF4, q4.FP4):
        assert np.array_equal(scales.view(np.uint32), os_.view(np.uint32)), f"{tag} scales differ"
    elif fmt == q4.NF4_DQ:
        # 8-bit absmax codes, the zero gap and the binary32 constants
        assert scales.shape == os_.shape, f"{tag} scale buffer sizes differ"
        bad = np.argwhere(scales != os_)
        assert bad.size == 0, f"{tag} double-quantized scales differ at bytes {bad[:5].ravel().tolist()}"
    else:
        assert np.array_equal(scales, os_), f"{tag} scales differ"
    if fmt == q4.INT4_ASYM:
        assert np.array_equal(zeros, oz), f"{tag} zero-points differ"
    return q, (oc, os_, oz)


def assert_product_ok(y_gpu: torch.Tensor, y_ref: np.ndarray, absdot: np.ndarray, tag=""):
    """|y - y_ref| <= 2e-3 * sum|x * what| + 1e-3 + half an ulp of y_ref in
    the output dtype, for every output."""
    yv = y_gpu.float().cpu().numpy().astype(np.float64)
    assert yv.shape == y_ref.shape
    err = np.abs(yv - y_ref)
    act = q4.F16 if y_gpu.dtype == torch.float16 else q4.BF16
    tol = oracle.tolerance(absdot, y_ref, act)
    worst = np.unravel_index(np.argmax(err - tol), err.shape)
    assert np.all(np.isfinite(yv)), f"{tag} non-finite output"
    assert np.all(err <= tol), (f"{tag} out of tolerance at {worst}: gpu={yv[worst]} ref={y_ref[worst]} "
                                f"err={err[worst]} tol={tol[worst]}")
    return float((err / tol).max())
