"""FP64 CPU oracle for C = alpha*A*B + beta*C (test infrastructure only).

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package.  The GPU product never imports it; this package
imports nothing from the product.

`liboracle.so` (built from oracle.c with gcc) walks each operand's byte-strided
view itself, decodes FP16/BF16/FP32/E4M3FN with its own decoders, and sums the
naive triple loop in FP64 with k ascending.  `compare.py` turns the result into
the per-element tolerance bound and a report.

Citations for what is computed are in oracle.c's header.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# Oracle's own dtype codes (match the enum in oracle.c).
OR_F32, OR_F16, OR_BF16, OR_E4M3 = 0, 1, 2, 3
_TORCH_CODE = {
    torch.float32: OR_F32,
    torch.float16: OR_F16,
    torch.bfloat16: OR_BF16,
    torch.float8_e4m3fn: OR_E4M3,
}


def build(verbose: bool = False) -> str:
    """Compile liboracle.so with gcc (FP64, no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O3", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
           "-shared", "-std=c11", "-Wall", "-o", _LIB + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class _View(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4),
                ("dtype", ctypes.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.POINTER(_View)
        L.or_gemm.argtypes = [P, P, P, P, P, ctypes.c_double, ctypes.c_double,
                              ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]
        L.or_gemm.restype = ctypes.c_int
        L.or_decode.argtypes = [ctypes.c_int32, ctypes.c_uint32]
        L.or_decode.restype = ctypes.c_double
        L.or_gather.argtypes = [P, ctypes.c_void_p]
        L.or_gather.restype = ctypes.c_int
        L.or_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


@dataclass
class HostView:
    """A byte-strided view into a host copy of an operand's whole storage."""
    storage: np.ndarray      # uint8, the whole underlying storage
    offset: int              # byte offset of element (0,..,0)
    shape: tuple
    stride: tuple            # bytes
    dtype: int               # OR_* code

    def c(self) -> _View:
        v = _View()
        v.base = self.storage.ctypes.data + self.offset
        v.ndim = len(self.shape)
        for d in range(len(self.shape)):
            v.shape[d] = int(self.shape[d])
            v.stride[d] = int(self.stride[d])
        v.dtype = self.dtype
        return v


def host_view(t: torch.Tensor) -> HostView:
    """Describe tensor `t` (any device) by a host copy of its whole storage plus
    its byte offset, shape and byte strides.  Nothing is re-laid-out: the oracle
    walks the original strides."""
    es = t.element_size()
    st = t.untyped_storage()
    raw = torch.empty(0, dtype=torch.uint8).set_(st.cpu() if st.device.type != "cpu" else st)
    arr = raw.numpy().copy()
    shape = tuple(t.shape) if t.dim() > 0 else (1,)
    stride = tuple(s * es for s in t.stride()) if t.dim() > 0 else (es,)
    return HostView(arr, t.storage_offset() * es, shape, stride, _TORCH_CODE[t.dtype])


def _rows_cols(v: HostView):
    r = 1
    for s in v.shape[:-1]:
        r *= s
    return r, v.shape[-1]


def gather(v: HostView) -> np.ndarray:
    """Row-major FP64 copy of a view's logical matrix (the oracle's view walk)."""
    r, c = _rows_cols(v)
    out = np.empty((r, c), dtype=np.float64)
    cv = v.c()
    rc = lib().or_gather(ctypes.byref(cv), out.ctypes.data)
    if rc != 0:
        raise ValueError(f"or_gather failed: {rc}")
    return out


def decode(dtype_code: int, bits: int) -> float:
    return lib().or_decode(dtype_code, bits)


@dataclass
class RefResult:
    C: np.ndarray        # [rows, N] float64 reference
    S: np.ndarray        # [rows, N] sum_k |a*b|
    Cin: np.ndarray      # [rows, N] decoded C_in (zeros if beta == 0)
    rows: np.ndarray     # row indices computed
    alpha: float
    beta: float


def ref_gemm(A, B, C_in=None, alpha: float = 1.0, beta: float = 0.0, rows=None,
             A_scale=None, B_scale=None, nthreads: int = 0) -> RefResult:
    """Reference C = alpha*A*B + beta*C_in over the given rows (default: all).

    A, B, C_in, A_scale, B_scale are torch tensors (any device, any strides) or
    HostViews.  alpha and beta are rounded to FP32 first, because the GPU entry
    points take FP32 scalars.
    """
    hv = lambda x: None if x is None else (x if isinstance(x, HostView) else host_view(x))
    a, b, c, sa, sb = hv(A), hv(B), hv(C_in), hv(A_scale), hv(B_scale)
    alpha = float(np.float32(alpha))
    beta = float(np.float32(beta))
    M, K = _rows_cols(a)
    Kb, N = _rows_cols(b)
    if K != Kb:
        raise ValueError(f"K mismatch {K} vs {Kb}")
    if rows is None:
        rows_arr = np.arange(M, dtype=np.int64)
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    n = len(rows_arr)
    out = np.zeros((n, N), dtype=np.float64)
    S = np.zeros((n, N), dtype=np.float64)
    cin = np.zeros((n, N), dtype=np.float64)
    ca, cb = a.c(), b.c()
    cc = c.c() if c is not None else None
    csa = sa.c() if sa is not None else None
    csb = sb.c() if sb is not None else None
    ref = lambda x: ctypes.byref(x) if x is not None else None
    rc = lib().or_gemm(ref(ca), ref(csa), ref(cb), ref(csb), ref(cc), alpha, beta,
                       rows_arr.ctypes.data, n, out.ctypes.data, S.ctypes.data,
                       cin.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError(f"or_gemm rejected the call: {rc}")
    return RefResult(out, S, cin, rows_arr, alpha, beta)


def num_threads() -> int:
    return lib().or_num_threads()


from .compare import bound, compare, CompareReport, ulp, fmt_of  # noqa: E402,F401
