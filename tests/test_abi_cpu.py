"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every symbol include/q4.h declares, reproduces the pages' byte arithmetic
through its size helpers, and rejects bad arguments with the documented
status codes before any HIP call."""

import ctypes
import json
import os
import re

import pytest

from bit_group_wise_amd import q4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))


def header_functions():
    with open(os.path.join(ROOT, "include", "q4.h")) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(q4_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = header_functions()
    assert names == sorted(q4.SIGNATURES), names
    L = q4.lib()
    for n in names:
        assert hasattr(L, n)


def test_status_strings():
    for s in range(5):
        assert q4.status_str(s)
    assert q4.status_str(q4.EALIGN) == "misaligned pointer"


def test_size_helpers_reproduce_page_figures():
    with open(os.path.join(HERE, "golden", "footprints.json")) as f:
        fp = json.load(f)
    # fp16 scale overhead per group size for 8 * 2^30 weights (8B params)
    so = fp["scale_overhead_8b"]
    n = so["params"]
    K = 4096
    N = n // K
    # (the scale buffers carry 16 bytes of trailing padding, not counted)
    for g in (32, 64, 128):
        mib = (q4.scales_bytes(q4.INT4_SYM, N, K, g) - 16) / 2**20
        assert mib == so["printed_mb"][str(g)]
    # 4 bits per weight: codes of 8B params are 4 GB (2^32 bytes)
    assert q4.codes_bytes(N, K) == n // 2
    # NF4 block 64 with 32-bit absmax: 0.5 extra bits per weight
    nb = fp["nf4_absmax_bits"]
    extra_bits = (q4.scales_bytes(q4.NF4, N, K, 64) - 16) * 8 / n
    assert extra_bits == nb["printed_bits"]
    # double quantisation figure (8-bit per block of 64 plus fp32 per 256 blocks)
    dq = nb["dq_bits"] / nb["block"] + 32 / (nb["block"] * nb["dq_block"])
    assert round(dq, 3) == nb["printed_dq_bits"]
    # 7B at 4.2 bits/param: 3.67 GB; FP16 14.00 GB; ratio 3.8x
    b7 = fp["int4_7b"]
    gb = b7["params"] * b7["bits_per_param"] / 8 / 1e9
    assert f"{gb:.2f}" == f"{b7['printed_gb']:.2f}" or abs(gb - b7["printed_gb"]) < 0.01
    assert round(fp["fp16_7b"]["params"] * 2 / 1e9, 2) == fp["fp16_7b"]["printed_gb"]
    assert round(14.00 / gb, 1) == b7["printed_ratio"]
    b70 = fp["int4_70b"]
    assert round(b70["params"] * b70["bits_per_param"] / 8 / 1e9) == b70["printed_gb_approx"]
    # SmolLM2-135M floors at 32/16/8/4 bits
    sm = fp["smollm2"]
    for bits, mb in sm["printed_mb"].items():
        assert round(sm["params"] * int(bits) / 8 / 1e6) == mb
    # the 4-bit floor equals the codes buffer of that many weights
    assert q4.codes_bytes(1, sm["params"] - sm["params"] % 2) == sm["params"] // 2


def test_size_helpers_invalid():
    assert q4.codes_bytes(0, 64) == 0
    assert q4.scales_bytes(q4.NF4, 4, 100, 64) == 0
    assert q4.scales_bytes(7, 4, 128, 64) == 0
    assert q4.zeros_bytes(q4.NF4, 4, 128, 64) == 0
    # padding: at least 16 bytes past the data, to a multiple of 16
    # (9 groups -> 5 bytes of nibbles -> 32; 18 bytes of scales -> 48)
    assert q4.zeros_bytes(q4.INT4_ASYM, 3, 96, 32) == 32
    assert q4.scales_bytes(q4.INT4_SYM, 3, 96, 32) == 48
    assert q4.scales_bytes(q4.NF4, 1, 128, 64) == 32
    # FP4: binary32 absmax like NF4, no zero-points
    assert q4.scales_bytes(q4.FP4, 1, 128, 64) == 32
    assert q4.zeros_bytes(q4.FP4, 4, 128, 64) == 0
    # NF4_DQ: 9 codes padded to 16, one 4-byte constant, then the padding
    assert q4.scales_bytes(q4.NF4_DQ, 3, 96, 32) == 48
    # 1024 groups: 1024 code bytes + 4 constants (0.127 bits per weight) + 16
    assert q4.scales_bytes(q4.NF4_DQ, 64, 1024, 64) == 1024 + 16 + 16
    assert q4.dq_scales_size(1024) * 8 / (64 * 1024) == 0.126953125


# Fake device addresses: validation never dereferences them and returns
# before any HIP call, so no GPU is needed.
A = 0x10000          # 16-byte aligned
MIS = 0x10002        # 2-byte aligned only


def call_quantize(fmt=q4.NF4, g=64, w=A, N=4, K=128, codes=A, scales=A, zeros=None):
    return q4.lib().q4_quantize(fmt, g, w, N, K, codes, scales, zeros, None)


def call_gemv(fmt=q4.NF4, g=64, act=q4.BF16, x=A, M=1, codes=A, scales=A, zeros=None, N=4, K=128,
              y=A, name="q4_gemv"):
    return getattr(q4.lib(), name)(fmt, g, act, x, M, codes, scales, zeros, N, K, y, None)


@pytest.mark.parametrize("kw,status", [
    (dict(fmt=5), q4.EUNSUPPORTED),
    (dict(fmt=q4.NF4_DQ, scales=0x10004), q4.EALIGN),   # NF4_DQ scales need 16 bytes
    (dict(fmt=q4.NF4_DQ, zeros=A), q4.EINVAL),
    (dict(g=16), q4.EUNSUPPORTED),
    (dict(g=256), q4.EUNSUPPORTED),
    (dict(w=None), q4.EINVAL),
    (dict(codes=None), q4.EINVAL),
    (dict(scales=None), q4.EINVAL),
    (dict(N=0), q4.EINVAL),
    (dict(K=-64), q4.EINVAL),
    (dict(K=96), q4.EINVAL),                       # K % 64 != 0
    (dict(zeros=A), q4.EINVAL),                    # zeros for NF4
    (dict(fmt=q4.INT4_ASYM, g=32), q4.EINVAL),     # asym without zeros
    (dict(w=MIS), q4.EALIGN),
    (dict(codes=MIS), q4.EALIGN),
    (dict(scales=MIS), q4.EALIGN),                 # NF4 scales need 4 bytes
    (dict(fmt=q4.FP4, scales=MIS), q4.EALIGN),     # FP4 scales need 4 bytes
    (dict(fmt=q4.FP4, zeros=A), q4.EINVAL),        # zeros for FP4
])
def test_quantize_rejects(kw, status):
    assert call_quantize(**kw) == status


@pytest.mark.parametrize("name", ["q4_gemv", "q4_gemm"])
@pytest.mark.parametrize("kw,status", [
    (dict(act=2), q4.EUNSUPPORTED),
    (dict(M=0), q4.EINVAL),
    (dict(x=None), q4.EINVAL),
    (dict(y=None), q4.EINVAL),
    (dict(x=MIS), q4.EALIGN),
    (dict(y=0x10001), q4.EALIGN),
    (dict(fmt=q4.INT4_SYM, zeros=A), q4.EINVAL),
    (dict(K=2**32), q4.EUNSUPPORTED),
])
def test_products_reject(name, kw, status):
    assert call_gemv(name=name, **kw) == status


def test_gemv_rejects_m_above_16():
    assert call_gemv(M=17) == q4.EUNSUPPORTED


def header_define(name):
    with open(os.path.join(ROOT, "include", "q4.h")) as f:
        m = re.search(r"#define\s+" + name + r"\s+(\d+)", f.read())
    return int(m.group(1))


def test_k_limits():
    """The largest K each product accepts: q4_gemm keeps a 256-row x tile
    view within 2^31 bytes (its 32-bit buffer range), q4_gemv keeps the
    skinny product's 16-row offsets within 31 bits.  One group past the limit
    is rejected before any HIP call."""
    gemm_k, gemv_k = header_define("Q4_GEMM_MAX_K"), header_define("Q4_GEMV_MAX_K")
    assert 256 * gemm_k * 2 <= 2**31
    assert 16 * gemv_k * 2 < 2**31 and 64 * (gemv_k // 2) < 2**31
    for g in (32, 64, 128):
        assert call_gemv(name="q4_gemm", M=32, K=gemm_k + g, g=g) == q4.EUNSUPPORTED
        assert call_gemv(name="q4_gemv", M=1, K=gemv_k + g, g=g) == q4.EUNSUPPORTED
        assert call_gemv(name="q4_gemv", M=16, K=gemv_k + g, g=g) == q4.EUNSUPPORTED


def test_dequantize_rejects():
    L = q4.lib()
    assert L.q4_dequantize(q4.NF4, 64, A, A, None, 4, 128, 5, A, None) == q4.EUNSUPPORTED
    assert L.q4_dequantize(q4.NF4, 64, A, A, None, 4, 128, q4.F16, None, None) == q4.EINVAL
    assert L.q4_dequantize(q4.NF4, 64, A, A, None, 4, 128, q4.F16, MIS, None) == q4.EALIGN
    assert L.q4_dequantize(q4.NF4, 64, A, MIS, None, 4, 128, q4.F16, A, None) == q4.EALIGN


def call_chain(n=2, fmt=q4.NF4, g=64, act=q4.BF16, sync=A, **task_kw):
    arr = (q4.GemvTask * max(n, 1))()
    for i in range(max(n, 1)):
        kw = dict(x=A, codes=A, scales=A, zeros=None, y=A, N=4, K=128, flags=0)
        if i == n - 1:
            kw.update(task_kw)
        arr[i] = q4.GemvTask(**kw)
    return q4.lib().q4_gemv_chain(fmt, g, act, ctypes.addressof(arr), n, sync, None)


def test_gemv_task_layout():
    # q4_gemv_task: five pointers, two int64 sizes, uint32 flags (+4 padding)
    assert ctypes.sizeof(q4.GemvTask) == 64
    assert q4.GemvTask.N.offset == 40 and q4.GemvTask.flags.offset == 56


@pytest.mark.parametrize("kw,status", [
    (dict(fmt=5), q4.EUNSUPPORTED),
    (dict(fmt=q4.NF4_DQ, scales=0x10004), q4.EALIGN),   # NF4_DQ scales need 16 bytes
    (dict(fmt=q4.NF4_DQ, zeros=A), q4.EINVAL),
    (dict(g=16), q4.EUNSUPPORTED),
    (dict(act=2), q4.EUNSUPPORTED),
    (dict(n=0), q4.EINVAL),
    (dict(n=65), q4.EUNSUPPORTED),
    (dict(sync=None), q4.EINVAL),
    (dict(sync=0x10004), q4.EALIGN),
    (dict(x=None), q4.EINVAL),
    (dict(y=None), q4.EINVAL),
    (dict(x=MIS), q4.EALIGN),
    (dict(N=0), q4.EINVAL),
    (dict(K=96), q4.EINVAL),
    (dict(zeros=A), q4.EINVAL),
    (dict(flags=2), q4.EINVAL),
    (dict(K=16384 + 64), q4.EUNSUPPORTED),       # x no longer fits the LDS buffers
    (dict(N=262144, K=16384), q4.EUNSUPPORTED),   # codes 2 GiB: past Q4_GEMV_CHAIN_MAX_CODES
    (dict(sync=0x10040), q4.EALIGN),              # sync words need 128 bytes
])
def test_chain_rejects(kw, status):
    assert call_chain(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(N=12), q4.EUNSUPPORTED),                 # N % 8 != 0
    (dict(N=8 * 524288), q4.EUNSUPPORTED),         # N above Q4_GEMM_DX_MAX_N
    (dict(N=65536, K=65536), q4.EUNSUPPORTED),     # codes above 2 GiB - 129
    (dict(dy=None), q4.EINVAL),
    (dict(dx=None), q4.EINVAL),
    (dict(dx=0x10008), q4.EALIGN),                 # dx needs 16 bytes
    (dict(dy=MIS), q4.EALIGN),
    (dict(fmt=q4.INT4_ASYM), q4.EINVAL),           # asym without zeros
    (dict(act=2), q4.EUNSUPPORTED),
])
def test_gemm_dx_rejects(kw, status):
    a = dict(fmt=q4.NF4, g=64, act=q4.BF16, dy=A, M=4, codes=A, scales=A, zeros=None, N=16,
             K=128, dx=A)
    a.update(kw)
    L = q4.lib()
    assert L.q4_gemm_dx(a["fmt"], a["g"], a["act"], a["dy"], a["M"], a["codes"], a["scales"],
                        a["zeros"], a["N"], a["K"], a["dx"], None) == status
