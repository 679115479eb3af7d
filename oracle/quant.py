"""FP8 E4M3 quantizer oracle (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU leg may import
this module; it imports nothing from the GPU product.

What is computed (the operation include/dg.h states for dg_quant_fp8: FP8
GEMM needs per-token or per-block FP32 scales that squeeze each block into the
representable range, sheratonhq.com deep dive, sections 2.4 and 5.4):

  for each block (1 x 128 of a row, or 128 x 128), in FP32:
      amax = max |x| over the block's elements inside X
      s    = max(amax, 1e-12) / 448
      q    = the E4M3 code nearest to min(max(x / s, -448), 448),
             ties to the even code; -0 keeps its sign

The code is found by nearest-value search over the 127 non-negative finite
E4M3FN values, each decoded from the OCP format definition (bias 7, 3
mantissa bits, subnormals m * 2^-9, largest finite 448); the GPU kernel
encodes arithmetically instead, so the two share no method.
"""
from __future__ import annotations

import numpy as np
import torch

E4M3_MAX = np.float32(448.0)
TINY = np.float32(1e-12)


def e4m3_value(code: int) -> float:
    """Value of a non-negative finite E4M3FN code (0x00..0x7E), from the format definition."""
    e, m = code >> 3, code & 7
    if e == 0:
        return m * 2.0 ** -9
    return (1.0 + m / 8.0) * 2.0 ** (e - 7)


_POS = np.array([e4m3_value(c) for c in range(0x7F)], dtype=np.float64)   # ascending


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Codes (uint8) of float32 values with |v| <= 448: nearest, ties to the even code."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 1, len(_POS) - 1)
    lo = hi - 1
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return code | (np.signbit(v).astype(np.uint8) << 7)


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    """float32 values of finite codes."""
    code = np.asarray(code, dtype=np.uint8)
    mag = _POS[np.minimum(code & 0x7F, 0x7E)].astype(np.float32)
    return np.where(code & 0x80, -mag, mag).astype(np.float32)


def _as_f32(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu").float().numpy()   # exact widening of FP16/BF16/FP32
    return np.asarray(x, dtype=np.float32)


def _scale(amax: np.ndarray) -> np.ndarray:
    return (np.maximum(amax.astype(np.float32), TINY) / E4M3_MAX).astype(np.float32)


def _codes(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    v = np.clip((x / s).astype(np.float32), -E4M3_MAX, E4M3_MAX)
    return e4m3_encode(v)


def quant_tokens(x) -> tuple[np.ndarray, np.ndarray]:
    """Per (row, 128-wide K block): codes [M][K] uint8 and scales [M][ceil(K/128)] float32."""
    x = _as_f32(x)
    M, K = x.shape
    KB = (K + 127) // 128
    q = np.zeros((M, K), dtype=np.uint8)
    s = np.zeros((M, KB), dtype=np.float32)
    for kb in range(KB):
        blk = x[:, kb * 128:(kb + 1) * 128]
        sc = _scale(np.abs(blk).max(axis=1) if blk.size else np.zeros(M, np.float32))
        s[:, kb] = sc
        q[:, kb * 128:(kb + 1) * 128] = _codes(blk, sc[:, None])
    return q, s


def quant_blocks(x) -> tuple[np.ndarray, np.ndarray]:
    """Per 128 x 128 block: codes [M][K] uint8 and scales [ceil(M/128)][ceil(K/128)] float32."""
    x = _as_f32(x)
    M, K = x.shape
    MB, KB = (M + 127) // 128, (K + 127) // 128
    q = np.zeros((M, K), dtype=np.uint8)
    s = np.zeros((MB, KB), dtype=np.float32)
    for mb in range(MB):
        for kb in range(KB):
            blk = x[mb * 128:(mb + 1) * 128, kb * 128:(kb + 1) * 128]
            sc = _scale(np.abs(blk).max())
            s[mb, kb] = sc
            q[mb * 128:(mb + 1) * 128, kb * 128:(kb + 1) * 128] = _codes(blk, sc)
    return q, s
