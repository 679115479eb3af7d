"""FP64 reference of the fused GEMM epilogue (test infrastructure only).

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this module; it imports nothing from the GPU product.

What it computes, per output element:

    out[m, n] = act(alpha * (A*B)[m, n] + beta * C_in[m, n] + bias[n])

The GEMM part is the FP64 oracle (`ref_gemm`, oracle.c); this module adds the
bias row to every row and applies the activation, all in FP64:
  - GEMM + BiasAdd + GeLU fused in one kernel: "DeepGEMM is not a new model"
    article (cf-1.com), section 3.3 (bias broadcast along the rows, then the
    tanh-approximated GeLU, then one store).  The pages do not say where beta*C
    goes; here the bias and the activation act on the finished GEMM value,
    beta*C included.
  - GELU, tanh form: Hendrycks and Gimpel, "Gaussian Error Linear Units"
    (2016): 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))).
  - ReLU: x < 0 -> 0, else x (NaN stays NaN).

Tolerance (`bound_epilogue`): the pre-activation value carries the GEMM bound
of compare.py plus one more FP32 rounding for the bias add; the activation
moves that error by at most its Lipschitz constant L (1 for identity and
ReLU, 1.13 for GELU: max |d/dx GELU| = 1.1289 for the tanh form, pinned in the
tests); its FP32 evaluation adds at most 8 * 2^-24 * |y| (a handful of
roundings and two hardware approximations of about 1 ulp each, and |GELU(y)|
<= |y|); the result is then rounded once to the output format.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from . import RefResult, gather, host_view
from .compare import U32, CompareReport, _report, ulp

ACT_NONE, ACT_RELU, ACT_GELU_TANH = "none", "relu", "gelu_tanh"
ACTS = (ACT_NONE, ACT_RELU, ACT_GELU_TANH)

SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)
GELU_CUBIC = 0.044715

# max |act'(x)| over the reals (GELU: pinned by tests/test_epilogue_oracle.py)
LIPSCHITZ = {ACT_NONE: 1.0, ACT_RELU: 1.0, ACT_GELU_TANH: 1.13}
# FP32 evaluation error of the activation, in units of 2^-24 * |y|
EVAL_ULPS = {ACT_NONE: 0.0, ACT_RELU: 0.0, ACT_GELU_TANH: 8.0}


def relu(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return np.where(x < 0.0, 0.0, x)


def gelu_tanh(x) -> np.ndarray:
    """0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) in FP64 (Hendrycks and Gimpel)."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        inner = SQRT_2_OVER_PI * (x + GELU_CUBIC * x * x * x)
        return 0.5 * x * (1.0 + np.tanh(inner))


def activate(act: str, x) -> np.ndarray:
    if act == ACT_NONE:
        return np.asarray(x, dtype=np.float64)
    if act == ACT_RELU:
        return relu(x)
    if act == ACT_GELU_TANH:
        return gelu_tanh(x)
    raise ValueError(act)


@dataclass
class EpiRef:
    C: np.ndarray        # [rows, N] act(Y)
    Y: np.ndarray        # [rows, N] pre-activation alpha*AB + beta*C_in + bias
    bias: np.ndarray     # [N] decoded bias (zeros when there is none)
    gemm: RefResult      # the GEMM part (S, C_in, rows, alpha, beta)
    act: str

    @property
    def rows(self):
        return self.gemm.rows


def ref_epilogue(ref: RefResult, bias=None, act: str = ACT_NONE) -> EpiRef:
    """Apply bias[n] and the activation to the GEMM reference `ref` (FP64).

    bias: None, or a tensor / HostView of N elements (any strides, F32, F16
    or BF16), decoded by the oracle's own view walk."""
    if act not in ACTS:
        raise ValueError(act)
    N = ref.C.shape[1]
    if bias is None:
        b = np.zeros(N, dtype=np.float64)
    else:
        hv = bias if not hasattr(bias, "untyped_storage") else host_view(bias)
        b = gather(hv).reshape(-1)
        if b.shape[0] != N:
            raise ValueError(f"bias has {b.shape[0]} elements, N = {N}")
    Y = ref.C + b[None, :]
    return EpiRef(activate(act, Y), Y, b, ref, act)


def bound_epilogue(e: EpiRef, out_fmt: str, rtol: float) -> np.ndarray:
    """Per-element tolerance of the fused epilogue (see the module docstring)."""
    g = e.gemm
    a = abs(g.alpha)
    pre = rtol * a * g.S + 4.0 * U32 * (a * g.S + np.abs(g.beta * g.Cin) + np.abs(e.bias)[None, :])
    L = LIPSCHITZ[e.act]
    ev = EVAL_ULPS[e.act] * U32 * np.abs(e.Y)
    tol = L * pre + ev
    return tol + 0.5 * ulp(np.abs(e.C) + tol, out_fmt)


def compare_epilogue(C_gpu, e: EpiRef, out_fmt: str, rtol: float) -> CompareReport:
    """Element-wise comparison of GPU rows `e.rows` against the epilogue reference."""
    return _report(C_gpu, e.C, bound_epilogue(e, out_fmt, rtol), e.rows, out_fmt)
