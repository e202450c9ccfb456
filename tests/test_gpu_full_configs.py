"""Parity at the workloads' full sizes, in the launch configurations the
benchmark times.

Quantize and dequantize are compared bit for bit on every weight.  GEMV and
GEMM outputs are compared with the fp64 oracle on sampled weight rows: the
first and last rows, the rows on both sides of every 256-row tile edge the
sample reaches, and seeded random rows.  Every row is checked for all M
activation rows.  The tolerance is |y - y_ref| <= 2e-3 * sum|x * what| + 1e-3.

The inputs are the synthetic tensors of the five workloads (seeds and
distributions in bit_group_wise_amd.synth).  The decode-token shapes are the
row-concatenated q/k/v and gate/up matrices the benchmark launches.
"""

import numpy as np
import pytest
import torch

import oracle
from bit_group_wise_amd import q4, synth
from _helpers import TORCH_ACT, assert_product_ok, assert_quant_equal, dev16, host16

pytestmark = pytest.mark.gpu


def _sample_rows(N: int, seed: int, n_random: int = 48) -> np.ndarray:
    rows = {0, N - 1}
    for edge in range(256, N, 256):
        if len(rows) > 96:
            break
        rows.update((edge - 1, edge))
    rng = np.random.default_rng(seed)
    rows.update(rng.choice(N, size=min(n_random, N), replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def _dequant_equal(q, fmt, g, oc, os_, oz, act):
    N, K = q.N, q.K
    got = host16(q4.dequantize(q, TORCH_ACT[act]))
    want = oracle.dequantize(fmt, g, oc, os_, oz, N, K, act)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"dequant differs at {bad[:5].tolist()}"


def _check_product(fn, q, fmt, g, act, oc, os_, oz, x_bits, rows, tag):
    x = dev16(x_bits, act)
    y = fn(x, q)
    torch.cuda.synchronize()
    ys = y[:, torch.from_numpy(rows).to(y.device)]
    yr, ad = oracle.matmul(fmt, g, act, x_bits, oc, os_, oz, q.N, q.K, rows=rows)
    return assert_product_ok(ys, yr, ad, tag=tag)


@pytest.mark.parametrize("name", ["c1_nf4_1k", "c2_sym_4k"])
def test_small_configs_every_output(name):
    """c1 (NF4 g64 1024^2, fp16 x) and c2 (INT4-sym g128 4096^2 with 0.1 %
    outliers, fp16 x): all weights bit-exact, every GEMV output in tolerance."""
    c = synth.CONFIGS[name]
    (N, K, seed), = c["mats"]
    w = synth.weight_f16_bits(N, K, seed, sigma=c["sigma"], mu=c["mu"],
                              outlier_seed=c.get("outlier_seed"))
    q, (oc, os_, oz) = assert_quant_equal(c["fmt"], c["g"], w, tag=name)
    _dequant_equal(q, c["fmt"], c["g"], oc, os_, oz, c["act"])
    x_bits = synth.act_bits(1, K, c["x_seeds"][0], c["act"])
    _check_product(q4.gemv, q, c["fmt"], c["g"], c["act"], oc, os_, oz, x_bits,
                   np.arange(N, dtype=np.int64), f"{name} gemv")


def test_c3_mlp_gemv_m1_m4_m16():
    """c3: NF4 g64 gate/up 11008x4096 and down 4096x11008, bf16 x at
    M = 1, 4, 16."""
    c = synth.CONFIGS["c3_nf4_mlp"]
    for (N, K, seed), xs in zip(c["mats"], c["x_seeds"]):
        w = synth.weight_f16_bits(N, K, seed, sigma=c["sigma"])
        q, (oc, os_, oz) = assert_quant_equal(c["fmt"], c["g"], w, tag=f"c3 {N}x{K}")
        _dequant_equal(q, c["fmt"], c["g"], oc, os_, oz, c["act"])
        rows = _sample_rows(N, seed)
        for M in c["M"]:
            x_bits = synth.act_bits(M, K, xs, c["act"])
            _check_product(q4.gemv, q, c["fmt"], c["g"], c["act"], oc, os_, oz, x_bits, rows,
                           f"c3 {N}x{K} M{M}")


def test_c4_prefill_gemm_2048():
    """c4: INT4-asym g32 14336x4096 ~ N(0.001, 0.02^2), bf16 x 2048x4096,
    the prefill GEMM."""
    c = synth.CONFIGS["c4_asym_gemm"]
    (N, K, seed), = c["mats"]
    w = synth.weight_f16_bits(N, K, seed, sigma=c["sigma"], mu=c["mu"])
    q, (oc, os_, oz) = assert_quant_equal(c["fmt"], c["g"], w, tag="c4")
    _dequant_equal(q, c["fmt"], c["g"], oc, os_, oz, c["act"])
    x_bits = synth.act_bits(2048, K, c["x_seeds"][0], c["act"])
    rows = _sample_rows(N, seed, n_random=24)
    _check_product(q4.gemm, q, c["fmt"], c["g"], c["act"], oc, os_, oz, x_bits, rows,
                   "c4 gemm")


def _layer0(parts, K):
    return np.concatenate([synth.weight_f16_bits(n, K, synth.llama7b_seed(0, idx))
                           for n, idx in parts], axis=0)


@pytest.mark.parametrize("name,parts,K", [
    ("qkv", [(4096, 0), (4096, 1), (4096, 2)], 4096),
    ("o", [(4096, 3)], 4096),
    ("gate_up", [(11008, 4), (11008, 5)], 4096),
    ("down", [(4096, 6)], 11008),
])
def test_c5_token_launch_shapes(name, parts, K):
    """c5: the decode token's four launch shapes (layer 0, NF4 g64, bf16 x,
    M = 1).  Quantize is row-local, so sampled rows are compared bit for bit
    against the oracle run on those rows alone."""
    w = _layer0(parts, K)
    N = w.shape[0]
    q = q4.quantize(dev16(w), q4.NF4, 64)
    torch.cuda.synchronize()
    rows = _sample_rows(N, 7 * N + K)
    oc, os_, _ = oracle.quantize(q4.NF4, 64, w[rows])
    gc = q.codes.cpu().numpy()[rows]
    gs = q.scales.cpu().numpy()[rows]
    assert np.array_equal(gc, oc), f"{name}: codes differ on sampled rows"
    assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32)), f"{name}: absmax differs"
    x_bits = synth.act_bits(1, K, 5900 if K == 4096 else 5901, synth.BF16)
    y = q4.gemv(dev16(x_bits, q4.BF16), q)
    torch.cuda.synchronize()
    ys = y[:, torch.from_numpy(rows).to(y.device)]
    yr, ad = oracle.matmul(q4.NF4, 64, q4.BF16, x_bits, oc, os_, None, rows.size, K)
    assert_product_ok(ys, yr, ad, tag=f"c5 {name}")


def test_c5_token_shapes_double_quantized_chain():
    """The decode token's four launch shapes with double-quantized absmax,
    run as one chained launch (as the benchmark's dq leg runs them).  The
    second-level runs cross rows, so the oracle quantizes each whole matrix;
    code bytes and 8-bit absmax codes are compared on sampled rows, the run
    constants in full, and the products on sampled rows."""
    shapes = [("qkv", [(4096, 0), (4096, 1), (4096, 2)], 4096), ("o", [(4096, 3)], 4096),
              ("gate_up", [(11008, 4), (11008, 5)], 4096), ("down", [(4096, 6)], 11008)]
    tasks, refs = [], []
    for name, parts, K in shapes:
        print(f"dq c5 {name}", flush=True)
        w = _layer0(parts, K)
        N = w.shape[0]
        q = q4.quantize(dev16(w), q4.NF4_DQ, 64)
        oc, os_, _ = oracle.quantize(q4.NF4_DQ, 64, w)
        torch.cuda.synchronize()
        rows = _sample_rows(N, 11 * N + K)
        G = K // 64
        gq, gs2 = (t.cpu().numpy() for t in q4.dq_parts(q))
        oq, os2 = oracle.dq_split(os_, N * G)
        assert np.array_equal(q.codes.cpu().numpy()[rows], oc[rows]), f"{name}: codes differ"
        assert np.array_equal(gq[rows], oq.reshape(N, G)[rows]), f"{name}: absmax codes differ"
        assert np.array_equal(gs2.view(np.uint32), os2.view(np.uint32)), f"{name}: run constants"
        x_bits = synth.act_bits(1, K, 5900 if K == 4096 else 5901, synth.BF16)
        tasks.append((dev16(x_bits, q4.BF16), q, None, q4.TASK_NO_WAIT))
        refs.append((name, rows, oracle.matmul(q4.NF4_DQ, 64, q4.BF16, x_bits, oc, os_, None, N,
                                               K, rows=rows)))
    outs = q4.gemv_chain(tasks)
    torch.cuda.synchronize()
    for y, (name, rows, (yr, ad)) in zip(outs, refs):
        ys = y[:, torch.from_numpy(rows).to(y.device)]
        assert_product_ok(ys, yr, ad, tag=f"dq c5 {name}")
