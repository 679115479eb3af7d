"""Tolerance bound and element-wise comparison against the FP64 reference.

Test infrastructure only (see the package docstring).

The stated tolerance is |C - C_ref| <= rtol * sum_k |a_ik * b_kj| with
rtol = 1e-4 for FP16/BF16 inputs and 1e-3 for FP8 (the kwkr.cn view-native
GEMM article, section 4.3, uses 1e-4 as its CPU-reference tolerance; its
troubleshooting table in section 5.1 names 1e-3).  That factor bounds the FP32
accumulation.  Two terms are added because the stored result is rounded once
more after accumulation:

  bound = rtol*|alpha|*S
        + 4*u32*(|alpha|*S + |beta*C_in|)          (FP32 epilogue arithmetic)
        + 0.5*ulp_out(|C_ref| + rtol*|alpha|*S)    (rounding to the C dtype)

with u32 = 2^-24 and ulp_out the spacing of the output format at that
magnitude (with its subnormal floor).  `literal=True` drops the two extra
terms, for results stored as FP32 where the stated factor alone must hold.

The report gives the worst err/bound and where, RMSE and mean signed error
(the sheratonhq.com deep dive, section 4.2, asks for error distribution, not
only the maximum), the failure count, NaN agreement and whether the result is
bitwise equal to the reference rounded to the output format.  NaN and Inf in
the data propagate per IEEE (the cf-1.com article, section 5.3, tells of a
NaN that a kernel must not hide): a NaN reference needs a NaN result, and an
infinite one the same infinity.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

U32 = 2.0 ** -24
# (mantissa bits, smallest subnormal spacing) per output format
_FMT = {
    "f32": (23, 2.0 ** -149),
    "bf16": (7, 2.0 ** -133),
    "f16": (10, 2.0 ** -24),
}
_TORCH_FMT = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}


def fmt_of(dtype) -> str:
    return _TORCH_FMT[dtype] if not isinstance(dtype, str) else dtype


def ulp(x: np.ndarray, fmt: str) -> np.ndarray:
    """Spacing of format `fmt` at magnitude |x| (2^(e-p), e = floor(log2|x|))."""
    p, tiny = _FMT[fmt]
    ax = np.abs(np.asarray(x, dtype=np.float64))
    _, E = np.frexp(ax)           # ax = f * 2^E, f in [0.5, 1)
    u = np.ldexp(1.0, (E - 1 - p).astype(np.int64))
    return np.where(ax > 0, np.maximum(u, tiny), tiny)


def bound(ref, out_fmt: str, rtol: float, literal: bool = False) -> np.ndarray:
    a = abs(ref.alpha)
    acc = rtol * a * ref.S
    if literal:
        return acc
    epi = 4.0 * U32 * (a * ref.S + np.abs(ref.beta * ref.Cin))
    rnd = 0.5 * ulp(np.abs(ref.C) + acc, out_fmt)
    return acc + epi + rnd


@dataclass
class CompareReport:
    ok: bool
    max_ratio: float
    argmax: tuple
    rmse: float
    mean_err: float
    fails: int
    nan_mismatch: int
    bitwise: bool
    n: int

    def __str__(self):
        return (f"ok={self.ok} max(err/bound)={self.max_ratio:.3g} at {self.argmax} "
                f"rmse={self.rmse:.3g} mean_err={self.mean_err:.3g} fails={self.fails}/{self.n} "
                f"nan_mismatch={self.nan_mismatch} bitwise={self.bitwise}")


def _round_to(x: np.ndarray, fmt: str) -> np.ndarray:
    """Reference rounded to the output format (RNE), as FP64 again."""
    t = torch.from_numpy(np.ascontiguousarray(x))
    if fmt == "f32":
        return t.to(torch.float32).double().numpy()
    dt = torch.bfloat16 if fmt == "bf16" else torch.float16
    # FP64 -> FP32 is exact for the integer-valued cases where bitwise equality
    # is asked for; the FP32 -> 16-bit step is the RNE the GPU epilogue does.
    return t.to(torch.float32).to(dt).double().numpy()


def compare(C_gpu, ref, out_fmt: str, rtol: float, literal: bool = False) -> CompareReport:
    """Compare GPU rows `ref.rows` of C against the reference element by element."""
    return _report(C_gpu, ref.C, bound(ref, out_fmt, rtol, literal), ref.rows, out_fmt)


def _report(C_gpu, want: np.ndarray, b: np.ndarray, rows, out_fmt: str) -> CompareReport:
    """Report of |C_gpu - want| against the per-element bound b (rows: row ids of want)."""
    if isinstance(C_gpu, torch.Tensor):
        C_gpu = C_gpu.detach().to("cpu", torch.float64).numpy()
    got = np.asarray(C_gpu, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    nan_g, nan_w = np.isnan(got), np.isnan(want)
    nan_mismatch = int(np.count_nonzero(nan_g != nan_w))
    # An infinite reference (an Inf operand propagated per IEEE) is matched only
    # by the same infinity; it takes no part in the error statistics.
    inf_w = np.isinf(want) & ~nan_g
    inf_mismatch = int(np.count_nonzero(inf_w & (got != want)))
    both = ~(nan_g | nan_w | inf_w)
    err = np.where(both, got - want, 0.0)
    aerr = np.abs(err)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(both, np.where(b > 0, aerr / b, np.where(aerr > 0, np.inf, 0.0)), 0.0)
    ratio = np.where(np.isnan(ratio), np.inf, ratio)
    fails = int(np.count_nonzero(ratio > 1.0)) + nan_mismatch + inf_mismatch
    if ratio.size:
        idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        mx = float(ratio[idx])
        argmax = (int(rows[idx[0]]), int(idx[1]))
    else:
        mx, argmax = 0.0, (-1, -1)
    nb = max(int(np.count_nonzero(both)), 1)
    rmse = float(np.sqrt(np.sum(err * err) / nb))
    mean_err = float(np.sum(err) / nb)
    rounded = _round_to(want, out_fmt)
    bitwise = bool(np.array_equal(got[both], rounded[both]) and nan_mismatch == 0 and inf_mismatch == 0)
    return CompareReport(fails == 0, mx, argmax, rmse, mean_err, fails, nan_mismatch, bitwise,
                         int(got.size))
