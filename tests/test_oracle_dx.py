"""Pins of the oracle's backward product dX = dY . What (the gradient path
through the frozen dequantized weights in QLoRA).

Not retyped from the oracle: the product is checked against numpy's matmul on
the oracle's own dequantized weights (a different route: dequantize, then a
BLAS product), against the forward oracle through the adjoint identity
<dX, x> = <dY, x . What^T> (a transposed index in either function fails it),
one-hot and zero gradients, and column sampling.
"""

import numpy as np
import pytest
import torch

NF4, SYM, ASYM, NF4_DQ = 0, 1, 2, 3
F16, BF16 = 0, 1


def _bits16(v):
    return np.asarray(v, np.float32).astype(np.float16).view(np.uint16)


def _act_bits(a, act_t):
    a = np.asarray(a, np.float32)
    if act_t == F16:
        return _bits16(a)
    return torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _act_vals(b, act_t):
    if act_t == F16:
        return b.view(np.float16).astype(np.float64)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _setup(orc, fmt, g, N, K, seed):
    rng = np.random.default_rng(seed)
    w = _bits16(rng.standard_normal((N, K)).astype(np.float32) * 0.02
                + (0.001 if fmt == ASYM else 0.0))
    return orc.quantize(fmt, g, w)


@pytest.mark.parametrize("fmt,g,act_t", [(NF4, 64, BF16), (SYM, 32, F16), (ASYM, 128, BF16),
                                         (NF4_DQ, 32, BF16)])
def test_dx_equals_numpy_on_dequantized(orc, fmt, g, act_t):
    N, K, M = 48, 256, 5
    codes, scales, zeros = _setup(orc, fmt, g, N, K, 10 + fmt)
    rng = np.random.default_rng(20 + fmt)
    dy = _act_bits(rng.standard_normal((M, N)), act_t)
    wd = _act_vals(orc.dequantize(fmt, g, codes, scales, zeros, N, K, act_t), act_t)
    dx, ad = orc.matmul_dx(fmt, g, act_t, dy, codes, scales, zeros, N, K)
    dyv = _act_vals(dy, act_t)
    assert dx.shape == (M, K)
    assert np.allclose(dx, dyv @ wd, rtol=1e-12, atol=1e-15)
    assert np.allclose(ad, np.abs(dyv) @ np.abs(wd), rtol=1e-12, atol=1e-15)
    cols = np.array([0, 255, 17, 128])
    dxs, _ = orc.matmul_dx(fmt, g, act_t, dy, codes, scales, zeros, N, K, cols=cols)
    assert np.array_equal(dxs, dx[:, cols])


@pytest.mark.parametrize("fmt", [NF4, ASYM])
def test_adjoint_of_forward(orc, fmt):
    """<dY . What, x> == <dY, x . What^T>, the forward oracle on the right."""
    N, K, g, act_t = 40, 192, 32, BF16
    codes, scales, zeros = _setup(orc, fmt, g, N, K, 30 + fmt)
    rng = np.random.default_rng(31)
    dy = _act_bits(rng.standard_normal((1, N)), act_t)
    x = _act_bits(rng.standard_normal((1, K)), act_t)
    dx, adx = orc.matmul_dx(fmt, g, act_t, dy, codes, scales, zeros, N, K)
    y, ady = orc.matmul(fmt, g, act_t, x, codes, scales, zeros, N, K)
    lhs = float(dx[0] @ _act_vals(x, act_t)[0])
    rhs = float(_act_vals(dy, act_t)[0] @ y[0])
    scale = float(np.abs(dx[0]) @ np.abs(_act_vals(x, act_t)[0])) + 1e-300
    assert abs(lhs - rhs) <= 1e-12 * scale
    # and a transposed reading (dx from What^T rows) would break it
    assert abs(lhs) > 1e-6


def test_one_hot_and_zero_gradients(orc):
    """dY = e_n gives row n of the dequantized weight exactly; dY = 0 gives 0."""
    N, K, g, act_t = 24, 128, 64, F16
    codes, scales, zeros = _setup(orc, NF4, g, N, K, 40)
    wd = _act_vals(orc.dequantize(NF4, g, codes, scales, zeros, N, K, act_t), act_t)
    dy = np.zeros((3, N), np.uint16)
    dy[0, 5] = 0x3C00
    dy[1, N - 1] = 0x3C00
    dx, _ = orc.matmul_dx(NF4, g, act_t, dy, codes, scales, zeros, N, K)
    assert np.array_equal(dx[0], wd[5])
    assert np.array_equal(dx[1], wd[N - 1])
    assert np.all(dx[2] == 0)


def test_rejects_bad_arguments(orc):
    codes, scales, zeros = _setup(orc, NF4, 64, 8, 128, 50)
    dy = np.zeros((1, 8), np.uint16)
    with pytest.raises(ValueError):
        orc.matmul_dx(NF4, 64, 2, dy, codes, scales, zeros, 8, 128)
    with pytest.raises(ValueError):
        orc.matmul_dx(NF4, 64, BF16, dy, codes, scales, zeros, 8, 128, cols=[128])
