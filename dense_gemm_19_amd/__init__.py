"""Python binding of the gfx950 dense GEMM library (libdg.so, C ABI in include/dg.h).

Argument marshalling only: every step of the computation runs in the library's
HIP kernels.  PyTorch provides the device memory and the current stream.

    import dense_gemm_19_amd as dg
    dg.gemm(A, B, C, alpha=1.0, beta=0.0)                     # C <- alpha*A@B + beta*C
    dg.gemm_fp8(qA, sA, qB, sB, C, alpha=1.0, beta=0.0)       # block-scaled E4M3
    dg.gemm_epilogue(A, B, C, bias, dg.DG_ACT_GELU_TANH)       # C <- gelu(A@B + bias)
    print(dg.plan(A, B, C))                                    # the chosen plan, no launch

Tensors may have any strides (transposes, padded rows, up to 4-D views whose
leading dims merge into one row stride); views are passed as pointer + shape +
byte strides, nothing is copied or made contiguous.  The library is loaded from
this directory; if it is missing, every call raises (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdg.so")

# dg_dtype codes
DG_F32, DG_F16, DG_BF16, DG_F8E4M3 = 0, 1, 2, 3
# dg_act codes (fused epilogue activation)
DG_ACT_NONE, DG_ACT_RELU, DG_ACT_GELU_TANH = 0, 1, 2
_DTYPE = {torch.float32: DG_F32, torch.float16: DG_F16, torch.bfloat16: DG_BF16,
          torch.float8_e4m3fn: DG_F8E4M3}

STATUS = ["DG_SUCCESS", "DG_ERR_NULL", "DG_ERR_NDIM", "DG_ERR_STRIDE", "DG_ERR_SHAPE_MISMATCH",
          "DG_ERR_DTYPE", "DG_ERR_MISALIGNED", "DG_ERR_ALIAS", "DG_ERR_NONFINITE_SCALAR",
          "DG_ERR_OVERFLOW", "DG_ERR_UNSUPPORTED_VIEW", "DG_ERR_POINTER", "DG_ERR_ARCH",
          "DG_ERR_HIP", "DG_ERR_INVALID_ARG", "DG_ERR_SCRATCH"]


class DGError(RuntimeError):
    def __init__(self, status: int, where: str = ""):
        self.status = status
        name = STATUS[status] if 0 <= status < len(STATUS) else f"status {status}"
        super().__init__(f"{where}: {name}" if where else name)


class View(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4),
                ("dtype", ctypes.c_int32)]


class PlanChoice(ctypes.Structure):
    """dg_plan_choice: path (0 built-in, 1 streaming, 2 matrix-core), tile (-1 or a
    tile index), splits (0 built-in), tail (-1 built-in, 0 no tail split)."""
    _fields_ = [("path", ctypes.c_int32), ("tile", ctypes.c_int32), ("splits", ctypes.c_int32),
                ("tail", ctypes.c_int32)]

    def astuple(self):
        return (self.path, self.tile, self.splits, self.tail)


class TuneResult(ctypes.Structure):
    _fields_ = [("default_us", ctypes.c_double), ("best_us", ctypes.c_double), ("tune_ms", ctypes.c_double),
                ("candidates", ctypes.c_int32), ("chosen", ctypes.c_int32), ("sets", ctypes.c_int32),
                ("plan", ctypes.c_char * 512)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libdg.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m dense_gemm_19_amd.build` (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(View)
        L.dg_gemm.argtypes = [P, P, P, ctypes.c_float, ctypes.c_float, ctypes.c_void_p]
        L.dg_gemm_fp8.argtypes = [P, P, P, P, P, ctypes.c_float, ctypes.c_float, ctypes.c_void_p]
        L.dg_gemm_plan.argtypes = [P, P, P, ctypes.c_float, ctypes.c_float, ctypes.c_char_p,
                                   ctypes.c_size_t]
        L.dg_gemm_fp8_plan.argtypes = [P, P, P, P, P, ctypes.c_float, ctypes.c_float,
                                       ctypes.c_char_p, ctypes.c_size_t]
        L.dg_gemm_epilogue.argtypes = [P, P, P, P, ctypes.c_int, ctypes.c_float, ctypes.c_float,
                                       ctypes.c_void_p]
        L.dg_gemm_fp8_epilogue.argtypes = [P, P, P, P, P, P, ctypes.c_int, ctypes.c_float,
                                           ctypes.c_float, ctypes.c_void_p]
        PC = ctypes.POINTER(PlanChoice)
        L.dg_gemm_candidates.argtypes = [P, P, P, P, P, PC, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]
        L.dg_gemm_with_choice.argtypes = [P, P, P, P, P, PC, ctypes.c_float, ctypes.c_float, ctypes.c_void_p]
        L.dg_gemm_tune.argtypes = [P, P, P, P, P, ctypes.c_int32, ctypes.POINTER(TuneResult), ctypes.c_void_p]
        L.dg_gemm_noalloc.argtypes = [P, P, P, P, P, ctypes.c_float, ctypes.c_float, ctypes.c_void_p]
        L.dg_gemm_noalloc.restype = ctypes.c_int
        L.dg_tune_save.argtypes = [ctypes.c_char_p]
        L.dg_tune_load.argtypes = [ctypes.c_char_p]
        for f in ("dg_gemm_candidates", "dg_gemm_with_choice", "dg_gemm_tune", "dg_tune_save", "dg_tune_load"):
            getattr(L, f).restype = ctypes.c_int
        L.dg_tune_clear.restype = None
        L.dg_tune_count.restype = ctypes.c_int32
        L.dg_gemm_grouped.argtypes = [ctypes.c_int32, P, P, P, ctypes.c_float, ctypes.c_float, ctypes.c_void_p]
        L.dg_gemm_grouped_plan.argtypes = [ctypes.c_int32, P, P, P, ctypes.c_float, ctypes.c_float,
                                           ctypes.c_char_p, ctypes.c_size_t]
        for f in ("dg_gemm", "dg_gemm_fp8", "dg_gemm_plan", "dg_gemm_fp8_plan", "dg_gemm_epilogue",
                  "dg_gemm_fp8_epilogue", "dg_gemm_grouped", "dg_gemm_grouped_plan"):
            getattr(L, f).restype = ctypes.c_int
        L.dg_quant_fp8.argtypes = [P, P, P, ctypes.c_int, ctypes.c_void_p]
        L.dg_quant_fp8.restype = ctypes.c_int
        D = ctypes.POINTER(ctypes.c_double)
        L.dg_calib_mfma.argtypes = [ctypes.c_int, D, ctypes.c_void_p]
        L.dg_calib_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, D, ctypes.c_void_p]
        L.dg_calib_launch.argtypes = [D, ctypes.c_void_p]
        for f in ("dg_calib_mfma", "dg_calib_read", "dg_calib_launch"):
            getattr(L, f).restype = ctypes.c_int
        L.dg_status_str.argtypes = [ctypes.c_int]
        L.dg_status_str.restype = ctypes.c_char_p
        L.dg_version.restype = ctypes.c_int
        _lib = L
    return _lib


def make_view(ptr: int, shape, byte_strides, dtype_code: int) -> View:
    """A dg_view from raw geometry (pointer value, extents, byte strides)."""
    if len(shape) != len(byte_strides):
        raise ValueError("shape and strides differ in length")
    v = View()
    v.ptr = ptr
    v.ndim = len(shape)
    for d in range(min(len(shape), 4)):
        v.shape[d] = int(shape[d])
        v.stride[d] = int(byte_strides[d])
    v.dtype = dtype_code
    return v


def view_of(t: torch.Tensor) -> View:
    """A dg_view of a tensor: data_ptr, shape, strides * element size, dtype."""
    if t.dtype not in _DTYPE:
        raise TypeError(f"unsupported dtype {t.dtype}")
    if t.dim() == 0:
        t = t.reshape(1)
    es = t.element_size()
    return make_view(t.data_ptr(), tuple(t.shape), tuple(s * es for s in t.stride()), _DTYPE[t.dtype])


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(st: int, where: str):
    if st != 0:
        raise DGError(st, where)


def gemm(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, alpha: float = 1.0, beta: float = 0.0,
         stream=None) -> torch.Tensor:
    """C <- alpha * A @ B + beta * C on the current (or given) stream; returns C."""
    va, vb, vc = view_of(A), view_of(B), view_of(C)
    _check(lib().dg_gemm(ctypes.byref(va), ctypes.byref(vb), ctypes.byref(vc), alpha, beta,
                         _stream(stream)), "dg_gemm")
    return C


def gemm_fp8(A: torch.Tensor, A_scale: torch.Tensor, B: torch.Tensor, B_scale: torch.Tensor,
             C: torch.Tensor, alpha: float = 1.0, beta: float = 0.0, stream=None) -> torch.Tensor:
    """C <- alpha * (qA*sA) @ (qB*sB) + beta * C with 1x128 / 128x128 block scales; returns C."""
    vs = [view_of(t) for t in (A, A_scale, B, B_scale, C)]
    _check(lib().dg_gemm_fp8(*[ctypes.byref(v) for v in vs], alpha, beta, _stream(stream)),
           "dg_gemm_fp8")
    return C


def gemm_epilogue(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, bias: torch.Tensor | None = None,
                  act: int = DG_ACT_NONE, alpha: float = 1.0, beta: float = 0.0,
                  stream=None) -> torch.Tensor:
    """C <- act(alpha * A @ B + beta * C + bias[None, :]) in one kernel; returns C."""
    va, vb, vc = view_of(A), view_of(B), view_of(C)
    vbias = view_of(bias) if bias is not None else None
    _check(lib().dg_gemm_epilogue(ctypes.byref(va), ctypes.byref(vb), ctypes.byref(vc),
                                  ctypes.byref(vbias) if vbias is not None else None, int(act),
                                  alpha, beta, _stream(stream)), "dg_gemm_epilogue")
    return C


def gemm_fp8_epilogue(A: torch.Tensor, A_scale: torch.Tensor, B: torch.Tensor, B_scale: torch.Tensor,
                      C: torch.Tensor, bias: torch.Tensor | None = None, act: int = DG_ACT_NONE,
                      alpha: float = 1.0, beta: float = 0.0, stream=None) -> torch.Tensor:
    """gemm_fp8 followed in the same kernel by + bias and the activation; returns C."""
    vs = [view_of(t) for t in (A, A_scale, B, B_scale, C)]
    vbias = view_of(bias) if bias is not None else None
    _check(lib().dg_gemm_fp8_epilogue(*[ctypes.byref(v) for v in vs],
                                      ctypes.byref(vbias) if vbias is not None else None, int(act),
                                      alpha, beta, _stream(stream)), "dg_gemm_fp8_epilogue")
    return C


def _view_array(ts):
    arr = (View * max(len(ts), 1))()
    for i, t in enumerate(ts):
        arr[i] = view_of(t)
    return arr


def gemm_grouped(As, Bs, Cs, alpha: float = 1.0, beta: float = 0.0, stream=None):
    """C[g] <- alpha * A[g] @ B[g] + beta * C[g] for every g, in as few launches as
    the shapes allow (lists of tensors of equal length); returns Cs."""
    if not (len(As) == len(Bs) == len(Cs)):
        raise ValueError("A, B and C lists differ in length")
    a, b, c = _view_array(As), _view_array(Bs), _view_array(Cs)
    _check(lib().dg_gemm_grouped(len(As), a, b, c, alpha, beta, _stream(stream)), "dg_gemm_grouped")
    return Cs


def grouped_plan_views(G: int, a, b, c, alpha: float = 1.0, beta: float = 0.0):
    """(status, description) of dg_gemm_grouped_plan for view arrays a, b, c."""
    buf = ctypes.create_string_buffer(4096)
    st = lib().dg_gemm_grouped_plan(G, a, b, c, alpha, beta, buf, len(buf))
    return st, buf.value.decode()


def grouped_plan(As, Bs, Cs, alpha: float = 1.0, beta: float = 0.0) -> str:
    """Describe the launches dg_gemm_grouped would make for these tensors."""
    st, text = grouped_plan_views(len(As), _view_array(As), _view_array(Bs), _view_array(Cs), alpha, beta)
    _check(st, "dg_gemm_grouped_plan")
    return text


def _opt_views(A, A_scale, B, B_scale, C):
    vs = [view_of(A), None if A_scale is None else view_of(A_scale), view_of(B),
          None if B_scale is None else view_of(B_scale), view_of(C)]
    return vs, [ctypes.byref(v) if v is not None else None for v in vs]


def candidates(A, B, C, A_scale=None, B_scale=None) -> list:
    """The candidate plan choices the tuner would time, as (path, tile, splits, tail)."""
    _, refs = _opt_views(A, A_scale, B, B_scale, C)
    arr = (PlanChoice * 64)()
    n = ctypes.c_int32(0)
    _check(lib().dg_gemm_candidates(*refs, arr, 64, ctypes.byref(n)), "dg_gemm_candidates")
    return [arr[i].astuple() for i in range(min(n.value, 64))]


def gemm_with_choice(A, B, C, choice, alpha: float = 1.0, beta: float = 0.0, A_scale=None, B_scale=None,
                     stream=None):
    """dg_gemm / dg_gemm_fp8 with an explicit (path, tile, splits, tail) plan choice; returns C."""
    vs, refs = _opt_views(A, A_scale, B, B_scale, C)
    c = PlanChoice(*choice)
    _check(lib().dg_gemm_with_choice(*refs, ctypes.byref(c), alpha, beta, _stream(stream)), "dg_gemm_with_choice")
    return C


def gemm_noalloc(A, B, C, alpha: float = 1.0, beta: float = 0.0, A_scale=None, B_scale=None, stream=None):
    """dg_gemm / dg_gemm_fp8 on the library's fixed split-K scratch (allocates nothing); returns C."""
    vs, refs = _opt_views(A, A_scale, B, B_scale, C)
    _check(lib().dg_gemm_noalloc(*refs, alpha, beta, _stream(stream)), "dg_gemm_noalloc")
    return C


def tune(A, B, C, A_scale=None, B_scale=None, reps: int = 0, stream=None) -> dict:
    """Time the candidate plans of this problem (C is overwritten), keep the fastest."""
    vs, refs = _opt_views(A, A_scale, B, B_scale, C)
    r = TuneResult()
    _check(lib().dg_gemm_tune(*refs, reps, ctypes.byref(r), _stream(stream)), "dg_gemm_tune")
    return {"default_us": r.default_us, "best_us": r.best_us, "tune_ms": r.tune_ms,
            "candidates": r.candidates, "chosen": r.chosen, "sets": r.sets, "plan": r.plan.decode()}


def tune_save(path: str):
    _check(lib().dg_tune_save(os.fsencode(path)), "dg_tune_save")


def tune_load(path: str):
    _check(lib().dg_tune_load(os.fsencode(path)), "dg_tune_load")


def tune_clear():
    lib().dg_tune_clear()


def tune_count() -> int:
    return lib().dg_tune_count()


def plan_views(A: View, B: View, C: View, alpha: float = 1.0, beta: float = 0.0,
               A_scale: View | None = None, B_scale: View | None = None) -> tuple[int, str]:
    """(status, plan text) for raw views, without launching anything."""
    buf = ctypes.create_string_buffer(1024)
    if A_scale is None and B_scale is None:
        st = lib().dg_gemm_plan(ctypes.byref(A), ctypes.byref(B), ctypes.byref(C), alpha, beta,
                                buf, len(buf))
    else:
        st = lib().dg_gemm_fp8_plan(ctypes.byref(A), ctypes.byref(A_scale), ctypes.byref(B),
                                    ctypes.byref(B_scale), ctypes.byref(C), alpha, beta, buf, len(buf))
    return st, buf.value.decode()


def plan(A, B, C, alpha: float = 1.0, beta: float = 0.0, A_scale=None, B_scale=None) -> str:
    """Describe the plan dg_gemm / dg_gemm_fp8 would run for these tensors."""
    st, text = plan_views(view_of(A), view_of(B), view_of(C), alpha, beta,
                          None if A_scale is None else view_of(A_scale),
                          None if B_scale is None else view_of(B_scale))
    _check(st, "dg_gemm_plan")
    return text


DG_QUANT_TOKEN, DG_QUANT_BLOCK = 0, 1


def quant_fp8(X: torch.Tensor, Q: torch.Tensor, S: torch.Tensor, mode: int = DG_QUANT_TOKEN,
              stream=None) -> None:
    """Q, S <- FP8 E4M3 codes and FP32 scales of X (dg_quant_fp8)."""
    vx, vq, vs = view_of(X), view_of(Q), view_of(S)
    _check(lib().dg_quant_fp8(ctypes.byref(vx), ctypes.byref(vq), ctypes.byref(vs), mode, _stream(stream)),
           "dg_quant_fp8")


# ---- measured roofline denominators (include/dg_calib.h)

def calib_mfma(dtype: int, stream=None) -> float:
    """Sustained dense matrix-instruction TFLOP/s (DG_BF16 or DG_F8E4M3)."""
    out = ctypes.c_double(0.0)
    _check(lib().dg_calib_mfma(dtype, ctypes.byref(out), _stream(stream)), "dg_calib_mfma")
    return out.value


def calib_read(buf: torch.Tensor, stream=None) -> float:
    """Streaming read GB/s over a device tensor's bytes."""
    out = ctypes.c_double(0.0)
    _check(lib().dg_calib_read(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                               ctypes.byref(out), _stream(stream)), "dg_calib_read")
    return out.value


def calib_launch(stream=None) -> float:
    """Back-to-back empty-kernel launch floor in microseconds."""
    out = ctypes.c_double(0.0)
    _check(lib().dg_calib_launch(ctypes.byref(out), _stream(stream)), "dg_calib_launch")
    return out.value


def status_str(st: int) -> str:
    return lib().dg_status_str(st).decode()


def version() -> int:
    return lib().dg_version()
