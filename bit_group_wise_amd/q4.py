"""ctypes binding of libq4 (include/q4.h): argument marshalling only.

Every step of the computation runs in the HIP kernels of ``libq4.so``; this
module allocates outputs with torch (device memory), passes raw pointers and
the current HIP stream, and turns a non-OK status into ``Q4Error``.  If the
library has not been built, loading fails loudly: there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
import threading

NF4, INT4_SYM, INT4_ASYM, NF4_DQ, FP4 = 0, 1, 2, 3, 4
DQ_RUN = 256  # absmax values per second-level constant (NF4_DQ)
F16, BF16 = 0, 1
FORMATS = {"nf4": NF4, "int4_sym": INT4_SYM, "int4_asym": INT4_ASYM, "nf4_dq": NF4_DQ, "fp4": FP4}

OK, EINVAL, EUNSUPPORTED, EALIGN, EHIP = 0, 1, 2, 3, 4

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libq4.so")

# (name, restype, argtypes) of every symbol include/q4.h declares
_vp, _i64, _int, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "q4_codes_bytes": (_sz, [_i64, _i64]),
    "q4_scales_bytes": (_sz, [_int, _i64, _i64, _int]),
    "q4_zeros_bytes": (_sz, [_int, _i64, _i64, _int]),
    "q4_quantize": (_int, [_int, _int, _vp, _i64, _i64, _vp, _vp, _vp, _vp]),
    "q4_dequantize": (_int, [_int, _int, _vp, _vp, _vp, _i64, _i64, _int, _vp, _vp]),
    "q4_gemv": (_int, [_int, _int, _int, _vp, _i64, _vp, _vp, _vp, _i64, _i64, _vp, _vp]),
    "q4_gemm": (_int, [_int, _int, _int, _vp, _i64, _vp, _vp, _vp, _i64, _i64, _vp, _vp]),
    "q4_gemm_dx": (_int, [_int, _int, _int, _vp, _i64, _vp, _vp, _vp, _i64, _i64, _vp, _vp]),
    "q4_gemv_chain": (_int, [_int, _int, _int, ctypes.c_void_p, _int, _vp, _vp]),
    "q4_gemv_chain_static": (_int, [_int, _int, _int, ctypes.c_void_p, _int, _vp]),
    "q4_status_str": (ctypes.c_char_p, [_int]),
}

# q4_gemv_chain limits and the task record (layout of q4_gemv_task)
CHAIN_MAX, CHAIN_MAX_K, CHAIN_SYNC_BYTES, TASK_NO_WAIT = 64, 16384, 1280, 1


class GemvTask(ctypes.Structure):
    _fields_ = [("x", _vp), ("codes", _vp), ("scales", _vp), ("zeros", _vp), ("y", _vp),
                ("N", _i64), ("K", _i64), ("flags", ctypes.c_uint32)]

_lock = threading.Lock()
_lib = None


class Q4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """Load libq4.so (built in-tree by bit_group_wise_amd.build)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is not built; run python -m bit_group_wise_amd.build")
            L = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().q4_status_str(status).decode()


def codes_bytes(N: int, K: int) -> int:
    return lib().q4_codes_bytes(N, K)


def scales_bytes(fmt: int, N: int, K: int, g: int) -> int:
    return lib().q4_scales_bytes(fmt, N, K, g)


def zeros_bytes(fmt: int, N: int, K: int, g: int) -> int:
    return lib().q4_zeros_bytes(fmt, N, K, g)


# ----------------------------------------------------------------- torch glue
def _torch():
    import torch
    return torch


def _stream_ptr(t) -> int | None:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _act_code(dtype) -> int:
    torch = _torch()
    if dtype == torch.float16:
        return F16
    if dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"activation dtype must be float16 or bfloat16, got {dtype}")


def _check(status: int, what: str) -> None:
    if status != OK:
        raise Q4Error(status, what)


def _cuda(t, name):
    if t is not None and (not t.is_cuda or not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous CUDA tensor")


class QuantizedWeight:
    """Packed codes, scales and (INT4-asym) zero-points of an [N, K] weight.

    For NF4_DQ, `scales` is the flat uint8 buffer of 8-bit absmax codes and
    second-level constants (see dq_parts)."""

    def __init__(self, fmt: int, g: int, N: int, K: int, codes, scales, zeros):
        self.fmt, self.g, self.N, self.K = fmt, g, N, K
        self.codes, self.scales, self.zeros = codes, scales, zeros

    def nbytes(self) -> int:
        return (self.codes.numel() + self.scales.numel() * self.scales.element_size()
                + (self.zeros.numel() if self.zeros is not None else 0))


def alloc_quantized(fmt: int, g: int, N: int, K: int, device) -> QuantizedWeight:
    torch = _torch()
    nc, ns, nz = codes_bytes(N, K), scales_bytes(fmt, N, K, g), zeros_bytes(fmt, N, K, g)
    if nc == 0 or ns == 0:
        raise Q4Error(EINVAL, "alloc_quantized")
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device=device)
    zeros = torch.zeros((nz,), dtype=torch.uint8, device=device)[: (N * (K // g) + 1) // 2] if nz else None
    if fmt == NF4_DQ:
        # uint8 qc[N*G], zero bytes to a multiple of 16, float32 s2[runs]
        scales = torch.zeros((ns,), dtype=torch.uint8, device=device)[: dq_scales_size(N * (K // g))]
        return QuantizedWeight(fmt, g, N, K, codes, scales, zeros)
    sdt = torch.float32 if fmt in (NF4, FP4) else torch.float16
    # scale and zero-point storage carries the ABI's padding to 16 bytes;
    # the tensors handed out are views of the meaningful leading part
    es = 4 if fmt in (NF4, FP4) else 2
    scales = torch.zeros((ns // es,), dtype=sdt, device=device)[: N * (K // g)].view(N, K // g)
    return QuantizedWeight(fmt, g, N, K, codes, scales, zeros)


def dq_s2_offset(n_groups: int) -> int:
    """Byte offset of the second-level constants in an NF4_DQ scales buffer."""
    return (n_groups + 15) // 16 * 16


def dq_scales_size(n_groups: int) -> int:
    """Meaningful bytes of an NF4_DQ scales buffer (without the padding)."""
    return dq_s2_offset(n_groups) + 4 * ((n_groups + DQ_RUN - 1) // DQ_RUN)


def dq_parts(q: QuantizedWeight):
    """(qc uint8 [N, K/g], s2 float32 [runs]) views of an NF4_DQ weight."""
    ng = q.N * (q.K // q.g)
    off = dq_s2_offset(ng)
    runs = (ng + DQ_RUN - 1) // DQ_RUN
    return (q.scales[:ng].view(q.N, q.K // q.g),
            q.scales[off:off + 4 * runs].view(_torch().float32))


def quantize(w, fmt: int, g: int, out: QuantizedWeight | None = None) -> QuantizedWeight:
    """Quantize an fp16 [N, K] CUDA tensor (q4_quantize)."""
    torch = _torch()
    _cuda(w, "w")
    if w.dtype != torch.float16 or w.dim() != 2:
        raise TypeError("w must be a 2-D float16 tensor")
    N, K = w.shape
    q = out if out is not None else alloc_quantized(fmt, g, N, K, w.device)
    st = lib().q4_quantize(fmt, g, _ptr(w), N, K, _ptr(q.codes), _ptr(q.scales), _ptr(q.zeros),
                           _stream_ptr(w))
    _check(st, "q4_quantize")
    return q


def dequantize(q: QuantizedWeight, dtype=None, out=None):
    """Dequantize to float16 (default) or bfloat16 (q4_dequantize)."""
    torch = _torch()
    dtype = dtype or torch.float16
    out_t = _act_code(dtype)
    if out is None:
        out = torch.empty((q.N, q.K), dtype=dtype, device=q.codes.device)
    _cuda(out, "out")
    st = lib().q4_dequantize(q.fmt, q.g, _ptr(q.codes), _ptr(q.scales), _ptr(q.zeros), q.N, q.K,
                             out_t, _ptr(out), _stream_ptr(out))
    _check(st, "q4_dequantize")
    return out


def _product(name: str, x, q: QuantizedWeight, out):
    torch = _torch()
    _cuda(x, "x")
    if x.dim() != 2 or x.shape[1] != q.K:
        raise ValueError("x must be [M, K]")
    act = _act_code(x.dtype)
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, q.N), dtype=x.dtype, device=x.device)
    _cuda(out, "out")
    fn = getattr(lib(), name)
    st = fn(q.fmt, q.g, act, _ptr(x), M, _ptr(q.codes), _ptr(q.scales), _ptr(q.zeros), q.N, q.K,
            _ptr(out), _stream_ptr(x))
    _check(st, name)
    return out


def gemv(x, q: QuantizedWeight, out=None):
    """y = x . What^T for 1 <= M <= 16 (q4_gemv)."""
    return _product("q4_gemv", x, q, out)


def gemm(x, q: QuantizedWeight, out=None):
    """y = x . What^T for any M (q4_gemm, matrix cores)."""
    return _product("q4_gemm", x, q, out)


def gemm_dx(dy, q: QuantizedWeight, out=None):
    """dX = dY . What for dY [M, N] (q4_gemm_dx): the gradient through the
    frozen quantized weight, on the matrix cores."""
    torch = _torch()
    _cuda(dy, "dy")
    if dy.dim() != 2 or dy.shape[1] != q.N:
        raise ValueError("dy must be [M, N]")
    act = _act_code(dy.dtype)
    M = dy.shape[0]
    if out is None:
        out = torch.empty((M, q.K), dtype=dy.dtype, device=dy.device)
    _cuda(out, "out")
    st = lib().q4_gemm_dx(q.fmt, q.g, act, _ptr(dy), M, _ptr(q.codes), _ptr(q.scales),
                          _ptr(q.zeros), q.N, q.K, _ptr(out), _stream_ptr(dy))
    _check(st, "q4_gemm_dx")
    return out


def chain_sync(device):
    """A zeroed sync buffer for gemv_chain (words 0-1 counters, word 2 the
    timeout flag); reusable by later chains on the same stream."""
    torch = _torch()
    return torch.zeros((CHAIN_SYNC_BYTES // 4,), dtype=torch.int32, device=device)


def _chain_tasks(tasks):
    """The q4_gemv_task array of a chain, its outputs, format, group size
    and activation code."""
    torch = _torch()
    if not tasks:
        raise ValueError("empty chain")
    q0 = tasks[0][1]
    act = _act_code(tasks[0][0].dtype)
    arr = (GemvTask * len(tasks))()
    outs = []
    for i, t in enumerate(tasks):
        x, q, y = t[0], t[1], t[2]
        flags = t[3] if len(t) > 3 else 0
        _cuda(x, "x")
        if (q.fmt, q.g) != (q0.fmt, q0.g) or _act_code(x.dtype) != act:
            raise ValueError("chain tasks must share format, group size and activation dtype")
        if x.dim() != 2 or x.shape != (1, q.K):
            raise ValueError("x must be [1, K]")
        if y is None:
            y = torch.empty((1, q.N), dtype=x.dtype, device=x.device)
        _cuda(y, "y")
        arr[i] = GemvTask(_ptr(x), _ptr(q.codes), _ptr(q.scales), _ptr(q.zeros), _ptr(y),
                          q.N, q.K, flags)
        outs.append(y)
    return arr, outs, q0.fmt, q0.g, act


def gemv_chain(tasks, sync=None):
    """Run M = 1 GEMVs in order in one launch (q4_gemv_chain).

    tasks: sequence of (x [1, K], QuantizedWeight, y [1, N] or None[, flags]);
    every weight shares one format and group size, every x one dtype.
    Returns the list of outputs."""
    arr, outs, fmt, g, act = _chain_tasks(tasks)
    if sync is None:
        sync = chain_sync(tasks[0][0].device)
    _cuda(sync, "sync")
    st = lib().q4_gemv_chain(fmt, g, act, ctypes.addressof(arr), len(tasks), _ptr(sync),
                             _stream_ptr(tasks[0][0]))
    _check(st, "q4_gemv_chain")
    return outs


def gemv_chain_static(tasks):
    """q4_gemv_chain_static: the same chain with the library's static sync
    words (no sync buffer; the outputs are allocated here unless given)."""
    arr, outs, fmt, g, act = _chain_tasks(tasks)
    st = lib().q4_gemv_chain_static(fmt, g, act, ctypes.addressof(arr), len(tasks),
                                    _stream_ptr(tasks[0][0]))
    _check(st, "q4_gemv_chain_static")
    return outs
