"""CPU oracle for 4-bit group-wise weight quantization (NF4, INT4-sym, INT4-asym,
NF4 with double-quantized absmax, FP4).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` import this package.  The product library
never imports, links or calls it, and shares no code with it.

The arithmetic lives in plain scalar C (``q4_oracle.c``, built with gcc, no
fast-math) and is reached through ctypes; this module only marshals numpy
arrays.  ``exact.py`` holds a tiny exact-rational re-derivation used to pin the
C code on small inputs.

What the oracle computes, and from which page (titles and sections of the web
pages on 4-bit group-wise quantization):

* "What is 4-bit quantization and why does it matter?", section "How 4-bit
  quantization works": the affine formula, INT4-symmetric levels -8..7 with
  scale max|w|/7, the printed NF4 table, the low-nibble-first unpack.
* "INT4" (AI technologies atlas), "How it works" / "Components": asymmetric
  levels 0..15 with an integer zero-point, FP16 per-group scales.
* "Loading a model in 4-bit", "Block-wise quantisation, stated exactly":
  contiguous blocks, absmax per block, nearest of 16 entries after dividing by
  the absmax, dequantize = absmax times table value; "Where the accuracy goes":
  the product is an ordinary 16-bit matmul on dequantized weights.
* "What is 4-bit quantization and why does it matter?", "QLoRA fine-tunes in
  4-bit": the backward product through the frozen dequantized weights,
  dX = dY . What (matmul_dx).
* Double quantization of the NF4 block constants ("Loading a model in 4-bit",
  the double-quantization flag and "Where the accuracy goes"; the closing
  section on NF4: blocks of 256 constants to 8 bits, 0.5 -> about 0.127 bits
  per parameter).  Read as symmetric absmax int8 coding of each run of 256
  absmax values (flat group order) with a binary32 constant per run.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

NF4, INT4_SYM, INT4_ASYM, NF4_DQ, FP4 = 0, 1, 2, 3, 4
F16, BF16 = 0, 1
FORMAT_NAMES = {NF4: "nf4", INT4_SYM: "int4_sym", INT4_ASYM: "int4_asym", NF4_DQ: "nf4_dq",
                FP4: "fp4"}
DQ_BLOCK = 256

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q4_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int


def build(force: bool = True) -> str:
    """Compile q4_oracle.c into liboracle.so with gcc (IEEE, no contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-Wall", "-Wextra", _SRC, "-lm", "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib() -> ctypes.CDLL:
    """Load the oracle library, building it first if it is not there."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build(force=True)
            L = ctypes.CDLL(_LIB)
            L.orc_quantize.argtypes = [_int, _int, _u16p, _i64, _i64, _u8p, _vp, _u8p]
            L.orc_dequantize.argtypes = [_int, _int, _u8p, _vp, _u8p, _i64, _i64, _int, _u16p]
            L.orc_matmul.argtypes = [_int, _int, _int, _u16p, _i64, _u8p, _vp, _u8p,
                                     _i64, _i64, _i64p, _i64, _f64p, _f64p]
            for f in (L.orc_quantize, L.orc_dequantize, L.orc_matmul):
                f.restype = _int
            L.orc_matmul_dx.argtypes = [_int, _int, _int, _u16p, _i64, _u8p, _vp, _u8p,
                                        _i64, _i64, _i64p, _i64, _f64p, _f64p]
            L.orc_matmul_dx.restype = _int
            L.orc_double_quant.argtypes = [_f32p, _i64, _u8p, _f32p]
            L.orc_double_quant.restype = None
            L.orc_dq_s2_offset.argtypes = [_i64]
            L.orc_dq_s2_offset.restype = _i64
            L.orc_nf4_nearest.argtypes = [ctypes.c_float]
            L.orc_nf4_nearest.restype = _int
            L.orc_fp4_nearest.argtypes = [ctypes.c_float]
            L.orc_fp4_nearest.restype = _int
            L.orc_f32_to_f16_array.argtypes = [_f32p, _u16p, _i64]
            L.orc_f16_to_f32_array.argtypes = [_u16p, _f32p, _i64]
            L.orc_f32_to_bf16_array.argtypes = [_f32p, _u16p, _i64]
            L.orc_nf4_nearest_array.argtypes = [_f32p, _u8p, _i64]
            for f in (L.orc_f32_to_f16_array, L.orc_f16_to_f32_array,
                      L.orc_f32_to_bf16_array, L.orc_nf4_nearest_array):
                f.restype = None
            _lib = L
    return _lib


def _p(a: np.ndarray, t):
    return a.ctypes.data_as(t)


def _check_g(g: int) -> None:
    if g not in (32, 64, 128):
        raise ValueError("group size must be 32, 64 or 128")


def nf4_table() -> np.ndarray:
    """The oracle's codebook, as float32[16]."""
    arr = (ctypes.c_float * 16).in_dll(lib(), "orc_nf4_table")
    return np.array(arr, dtype=np.float32)


def fp4_table() -> np.ndarray:
    """The oracle's FP4 codebook (a reading; parity unpinned against the
    pages), as float32[16]."""
    arr = (ctypes.c_float * 16).in_dll(lib(), "orc_fp4_table")
    return np.array(arr, dtype=np.float32)


def fp4_nearest(x: float) -> int:
    """Nearest FP4 index of a binary32 value (ties to the lower index)."""
    return int(lib().orc_fp4_nearest(float(np.float32(x))))


def f32_to_f16_bits(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().orc_f32_to_f16_array(_p(a, _f32p), _p(out, _u16p), a.size)
    return out


def f16_bits_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib().orc_f16_to_f32_array(_p(h, _u16p), _p(out, _f32p), h.size)
    return out


def f32_to_bf16_bits(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().orc_f32_to_bf16_array(_p(a, _f32p), _p(out, _u16p), a.size)
    return out


def nf4_nearest(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().orc_nf4_nearest_array(_p(x, _f32p), _p(out, _u8p), x.size)
    return out


def dq_s2_offset(n_groups: int) -> int:
    """Byte offset of the second-level constants in an NF4_DQ scales buffer."""
    return int(lib().orc_dq_s2_offset(n_groups))


def dq_scales_size(n_groups: int) -> int:
    """Bytes of an NF4_DQ scales buffer: codes (padded to 16) then s2."""
    return dq_s2_offset(n_groups) + 4 * ((n_groups + DQ_BLOCK - 1) // DQ_BLOCK)


def dq_split(scales, n_groups: int):
    """(qc uint8[n_groups], s2 float32[ceil(n_groups/256)]) of an NF4_DQ
    scales buffer (flat uint8)."""
    b = np.ascontiguousarray(scales, dtype=np.uint8).reshape(-1)
    off = dq_s2_offset(n_groups)
    nb = (n_groups + DQ_BLOCK - 1) // DQ_BLOCK
    return b[:n_groups].copy(), b[off:off + 4 * nb].copy().view(np.float32)


def double_quant(c):
    """Second-level quantization of an absmax array (flat order):
    (qc uint8[n], s2 float32[ceil(n/256)])."""
    c = np.ascontiguousarray(c, dtype=np.float32).reshape(-1)
    n = c.size
    qc = np.zeros(n, dtype=np.uint8)
    s2 = np.zeros((n + DQ_BLOCK - 1) // DQ_BLOCK, dtype=np.float32)
    lib().orc_double_quant(_p(c, _f32p), n, _p(qc, _u8p), _p(s2, _f32p))
    return qc, s2


def quantize(fmt: int, g: int, w_bits: np.ndarray):
    """Quantize fp16 weights given as uint16 bit patterns [N, K].

    Returns (codes uint8[N, K/2], scales, zeros) where scales is float32[N, K/g]
    for NF4 and FP4, uint16 fp16 bits [N, K/g] for INT4 and, for NF4_DQ, the flat
    uint8 buffer of dq_scales_size(N*K/g) bytes (see dq_split); zeros is uint8
    [ceil(N*K/g/2)] for INT4-asym, else None."""
    _check_g(g)
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    N, K = w.shape
    if K % g:
        raise ValueError("K must be a multiple of g")
    G = K // g
    codes = np.zeros((N, K // 2), dtype=np.uint8)
    if fmt == NF4_DQ:
        scales = np.zeros(dq_scales_size(N * G), dtype=np.uint8)
    else:
        scales = np.zeros((N, G), dtype=np.float32 if fmt in (NF4, FP4) else np.uint16)
    zeros = np.zeros(((N * G + 1) // 2,), dtype=np.uint8) if fmt == INT4_ASYM else None
    rc = lib().orc_quantize(fmt, g, _p(w, _u16p), N, K, _p(codes, _u8p),
                            scales.ctypes.data_as(_vp),
                            _p(zeros, _u8p) if zeros is not None else None)
    if rc != 0:
        raise ValueError("orc_quantize rejected its arguments")
    return codes, scales, zeros


def dequantize(fmt: int, g: int, codes, scales, zeros, N: int, K: int, out_t: int) -> np.ndarray:
    """Dequantize to fp16 (F16) or bf16 (BF16) bit patterns, uint16[N, K]."""
    _check_g(g)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales)
    out = np.empty((N, K), dtype=np.uint16)
    z = np.ascontiguousarray(zeros, dtype=np.uint8) if zeros is not None else None
    rc = lib().orc_dequantize(fmt, g, _p(codes, _u8p), scales.ctypes.data_as(_vp),
                              _p(z, _u8p) if z is not None else None, N, K, out_t,
                              _p(out, _u16p))
    if rc != 0:
        raise ValueError("orc_dequantize rejected its arguments")
    return out


def matmul(fmt: int, g: int, act_t: int, x_bits, codes, scales, zeros, N: int, K: int,
           rows=None):
    """fp64 reference y = x . what^T on rows `rows` of W (all rows if None).

    x_bits: uint16 [M, K] activation bit patterns in dtype act_t.
    Returns (y float64 [M, nrows], absdot float64 [M, nrows]) where absdot is
    sum_k |x * what|, the scale of the tolerance."""
    _check_g(g)
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    if x.ndim == 1:
        x = x[None, :]
    M = x.shape[0]
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales)
    z = np.ascontiguousarray(zeros, dtype=np.uint8) if zeros is not None else None
    if rows is None:
        r = None
        nrows = N
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = r.size
    y = np.empty((M, nrows), dtype=np.float64)
    ad = np.empty((M, nrows), dtype=np.float64)
    rc = lib().orc_matmul(fmt, g, act_t, _p(x, _u16p), M, _p(codes, _u8p),
                          scales.ctypes.data_as(_vp), _p(z, _u8p) if z is not None else None,
                          N, K, _p(r, _i64p) if r is not None else None, nrows,
                          _p(y, _f64p), _p(ad, _f64p))
    if rc != 0:
        raise ValueError("orc_matmul rejected its arguments")
    return y, ad


def matmul_dx(fmt: int, g: int, act_t: int, dy_bits, codes, scales, zeros, N: int, K: int,
              cols=None):
    """fp64 reference dx = dy . what on columns `cols` of W (all if None).

    dy_bits: uint16 [M, N] in dtype act_t.  Returns (dx float64 [M, ncols],
    absdot float64 [M, ncols])."""
    _check_g(g)
    dy = np.ascontiguousarray(dy_bits, dtype=np.uint16)
    if dy.ndim == 1:
        dy = dy[None, :]
    M = dy.shape[0]
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales)
    z = np.ascontiguousarray(zeros, dtype=np.uint8) if zeros is not None else None
    if cols is None:
        c = None
        ncols = K
    else:
        c = np.ascontiguousarray(cols, dtype=np.int64)
        ncols = c.size
    dx = np.empty((M, ncols), dtype=np.float64)
    ad = np.empty((M, ncols), dtype=np.float64)
    rc = lib().orc_matmul_dx(fmt, g, act_t, _p(dy, _u16p), M, _p(codes, _u8p),
                             scales.ctypes.data_as(_vp), _p(z, _u8p) if z is not None else None,
                             N, K, _p(c, _i64p) if c is not None else None, ncols,
                             _p(dx, _f64p), _p(ad, _f64p))
    if rc != 0:
        raise ValueError("orc_matmul_dx rejected its arguments")
    return dx, ad


def half_ulp(v: np.ndarray, act_t: int) -> np.ndarray:
    """Half the spacing of the fp16 (F16) or bf16 (BF16) numbers at |v|: the
    largest error of rounding v to that dtype (normal range; the subnormal
    spacing below it)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    mant, emin = (10, -14) if act_t == F16 else (7, -126)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** emin)))
    return 2.0 ** (e - mant - 1)


def tolerance(absdot: np.ndarray, y_ref=None, act_t=None) -> np.ndarray:
    """Per-output bound for a GEMV/GEMM result: 2e-3 * sum|x*what| + 1e-3,
    plus, when the reference and the output dtype are given, half an ulp of
    the reference in that dtype (the output is rounded once to the
    activation dtype, which no implementation can avoid)."""
    t = 2e-3 * absdot + 1e-3
    if y_ref is not None:
        t = t + half_ulp(y_ref, act_t)
    return t
