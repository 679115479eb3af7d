"""Seeded synthetic inputs for the GEMM workloads (shared by tests and bench).

This module only draws numbers and lays them out in memory.  It holds none of
the GEMM arithmetic: it imports neither the GPU library nor the oracle, and
both sides consume exactly the tensors it returns.

Recipe (every draw is seeded and reproducible):
  * numpy PCG64 `default_rng(seed)`; float64 draws -> float32 -> torch cast to
    the input dtype (round-to-nearest-even).
  * Draw order: A, then B, then C_in; each in row-major order of the matrix
    that owns the storage (for a transposed view, the stored matrix).
  * Distributions and shapes are those of the workloads the pages describe:
      c1   FP16 64x512x512, U[-1,1], FP32 C, beta=0
      c2a  BF16 x.W1, M=1, K=4096, N=14336, W1 row-major [K,N], N(0,1), BF16 C
      c2b  BF16 q.K_cache^T, M=1, K=4096, N=128, B = K_cache[128,4096]^T, BF16 C
      c3   FP16 64x4096x4096, N(0,0.02), FP32 C preloaded N(0,1), alpha=beta=1
      c4   BF16 4096^3, N(0,1), A a strided view of a (1,64,64,4160) tensor
           (row pitch padded by 64 elements, pad filled with NaN), BF16 C
      c5_128 / c5_4096  FP8 E4M3, M in {128, 4096}, N=7168, K=4096, sources
           N(0,1), quantized per (row, 128-wide K block) for A and per 128x128
           block for B, BF16 C
      moe8 8 MoE experts, x[1,512] . W_e[512,4096] (cf-1.com article, section 1),
           BF16, x shared (one token routed to all 8), N(0,1), seed 108
      <config>_gelu  the same operands with a fused epilogue: BF16 bias
           N(0,1) of N elements drawn from rng(201), then GELU (tanh form)
  * The FP8 quantizer stands in for the producer of quantized activations and
    weights: s = max(amax, 1e-12) / 448 in FP32, q = clamp(x / s, -448, 448)
    cast to float8_e4m3fn with torch (RNE).  The GEMM consumes (q, s) as given,
    so the result does not depend on these choices.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

E4M3_MAX = 448.0


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(np.random.PCG64(seed))


def draw(g: np.random.Generator, shape, dist: str, scale: float = 1.0) -> np.ndarray:
    """float64 draws of the given distribution, rounded to float32."""
    if dist == "normal":
        x = g.standard_normal(size=shape) * scale
    elif dist == "uniform":
        x = g.uniform(-scale, scale, size=shape)
    elif dist == "int":  # integers in [-scale, scale]
        x = g.integers(-int(scale), int(scale) + 1, size=shape).astype(np.float64)
    else:
        raise ValueError(dist)
    return x.astype(np.float32)


def to_dtype(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype)


def quantize_rows_k128(x: torch.Tensor):
    """Per-token quantization: one FP32 scale per (row, 128-wide K block)."""
    M, K = x.shape
    KB = (K + 127) // 128
    xp = torch.zeros(M, KB * 128, dtype=torch.float32)
    xp[:, :K] = x.float()
    blk = xp.view(M, KB, 128)
    amax = blk.abs().amax(dim=2)
    s = (torch.clamp(amax, min=1e-12) / E4M3_MAX).float()
    q = torch.clamp(blk / s[:, :, None], -E4M3_MAX, E4M3_MAX).view(M, KB * 128)[:, :K]
    return q.contiguous().to(torch.float8_e4m3fn), s.contiguous()


def quantize_blocks_128(x: torch.Tensor):
    """Per-block quantization: one FP32 scale per 128x128 block of a [K, N] matrix."""
    K, N = x.shape
    KB, NB = (K + 127) // 128, (N + 127) // 128
    xp = torch.zeros(KB * 128, NB * 128, dtype=torch.float32)
    xp[:K, :N] = x.float()
    blk = xp.view(KB, 128, NB, 128)
    amax = blk.abs().amax(dim=(1, 3))
    s = (torch.clamp(amax, min=1e-12) / E4M3_MAX).float()
    q = torch.clamp(blk / s[:, None, :, None], -E4M3_MAX, E4M3_MAX).view(KB * 128, NB * 128)
    return q[:K, :N].contiguous().to(torch.float8_e4m3fn), s.contiguous()


# ---------------------------------------------------------------- layouts

def place(x: torch.Tensor, layout: str, pad: int = 0, fill=0.0) -> torch.Tensor:
    """Return a view with the logical values of the 2-D tensor `x` laid out as:
      'row'  row-major contiguous;
      'col'  column-major (a transposed view of a contiguous [cols, rows]);
      'pad'  row-major with the row pitch padded by `pad` elements (filled with `fill`).
    """
    R, C = x.shape
    if layout == "row":
        return x.contiguous()
    if layout == "col":
        return x.t().contiguous().t()
    if layout == "pad":
        st = torch.full((R, C + pad), fill, dtype=x.dtype) if x.dtype != torch.float8_e4m3fn \
            else torch.zeros((R, C + pad), dtype=torch.uint8).view(torch.float8_e4m3fn)
        st[:, :C] = x
        return st[:, :C]
    raise ValueError(layout)


@dataclass
class Case:
    """One GEMM problem: tensors on the host (move with .to(device))."""
    name: str
    A: torch.Tensor
    B: torch.Tensor
    C: torch.Tensor               # output view (holds C_in when beta != 0)
    alpha: float = 1.0
    beta: float = 0.0
    A_scale: torch.Tensor | None = None
    B_scale: torch.Tensor | None = None
    rtol: float = 1e-4
    extra: dict = field(default_factory=dict)
    bias: torch.Tensor | None = None   # fused epilogue: N-vector added to every row
    act: str = "none"                  # fused epilogue: "none", "relu" or "gelu_tanh"

    @property
    def fp8(self) -> bool:
        return self.A_scale is not None

    @property
    def mnk(self):
        M = int(np.prod(self.A.shape[:-1])) if self.A.dim() > 1 else 1
        return M, self.B.shape[-1], self.A.shape[-1]

    def to(self, device) -> "Case":
        """Copy every tensor to `device`, keeping strides and storage geometry."""
        def mv(t):
            if t is None:
                return None
            st = t.untyped_storage()
            base = torch.empty(0, dtype=t.dtype, device=device)
            dev_st = torch.empty(st.nbytes(), dtype=torch.uint8).set_(st).to(device).untyped_storage()
            return base.set_(dev_st, t.storage_offset(), t.shape, t.stride())
        return Case(self.name, mv(self.A), mv(self.B), mv(self.C), self.alpha, self.beta,
                    mv(self.A_scale), mv(self.B_scale), self.rtol, dict(self.extra), mv(self.bias),
                    self.act)

    @property
    def fused(self) -> bool:
        return self.bias is not None or self.act != "none"


def gemm_case(M, N, K, in_dtype=torch.bfloat16, out_dtype=torch.float32, seed=0,
              dist="normal", scale=1.0, a_layout="row", b_layout="row", c_layout="row",
              alpha=1.0, beta=0.0, pad=64, cin_dist="normal", cin_scale=1.0,
              name=None) -> Case:
    """A 16-bit-input GEMM case with the given layouts (values drawn logically)."""
    g = rng(seed)
    a = to_dtype(draw(g, (M, K), dist, scale), in_dtype)
    if b_layout == "col":   # stored matrix is B^T [N, K]: draw it in its own row-major order
        b = to_dtype(draw(g, (N, K), dist, scale), in_dtype).t()
    else:
        b = to_dtype(draw(g, (K, N), dist, scale), in_dtype)
    if beta != 0.0:
        c = to_dtype(draw(g, (M, N), cin_dist, cin_scale), out_dtype)
    else:  # C is write-only: fill with NaN so any read of it shows up
        c = torch.full((M, N), float("nan"), dtype=out_dtype)
    nanfill = float("nan")
    A = place(a, a_layout, pad, nanfill)
    B = b if b_layout == "col" else place(b, b_layout, pad, nanfill)
    C = place(c, c_layout, pad, nanfill)
    return Case(name or f"{M}x{N}x{K}", A, B, C, alpha, beta, rtol=1e-4)


def fp8_case(M, N, K, seed=0, out_dtype=torch.bfloat16, alpha=1.0, beta=0.0, dist="normal",
             scale=1.0, b_layout="row", a_layout="row", name=None) -> Case:
    """An FP8 E4M3 case: sources drawn, then quantized per token and per block."""
    g = rng(seed)
    a_src = torch.from_numpy(draw(g, (M, K), dist, scale))
    if b_layout == "col":
        b_src = torch.from_numpy(draw(g, (N, K), dist, scale)).t()
    else:
        b_src = torch.from_numpy(draw(g, (K, N), dist, scale))
    qa, sa = quantize_rows_k128(a_src)
    qb, sb = quantize_blocks_128(b_src.contiguous())
    if b_layout == "col":
        qb = qb.t().contiguous().t()
    if a_layout == "col":   # same values, stored column-major
        qa = qa.t().contiguous().t()
    if beta != 0.0:
        c = to_dtype(draw(g, (M, N), "normal", 1.0), out_dtype)
    else:
        c = torch.full((M, N), float("nan"), dtype=out_dtype)
    return Case(name or f"fp8_{M}x{N}x{K}", qa, qb, c, alpha, beta, sa, sb, rtol=1e-3)


def bias_vector(N: int, dtype=torch.bfloat16, seed=0, layout="contig", scale=1.0) -> torch.Tensor:
    """The epilogue's bias: N(0, scale^2) draws from its own generator rng(seed).
    layout "contig": N adjacent elements; "strided": every other element of a
    2N buffer (the gaps hold NaN); "bcast": one drawn value seen through
    stride 0."""
    g = rng(seed)
    if layout == "bcast":
        return to_dtype(draw(g, (1,), "normal", scale), dtype).expand(N)
    v = to_dtype(draw(g, (N,), "normal", scale), dtype)
    if layout == "contig":
        return v
    if layout == "strided":
        st = torch.full((2 * max(N, 1),), float("nan"), dtype=dtype)
        st[0:2 * N:2] = v
        return st[0:2 * N:2]
    raise ValueError(layout)


def with_epilogue(case: Case, act: str, bias_dtype=torch.bfloat16, bias_layout="contig",
                  seed=0, bias_scale=1.0, name=None) -> Case:
    """The same operands with a fused bias (bias_dtype None: no bias) and activation."""
    N = case.mnk[1]
    bias = None if bias_dtype is None else bias_vector(N, bias_dtype, seed, bias_layout, bias_scale)
    return Case(name or f"{case.name}+{act}", case.A, case.B, case.C, case.alpha, case.beta,
                case.A_scale, case.B_scale, case.rtol, dict(case.extra), bias, act)


def moe_experts(E=8, M=1, K=512, N=4096, seed=108, dtype=torch.bfloat16, out_dtype=torch.bfloat16,
                shared_x=True) -> list:
    """E expert GEMMs x . W_e (the token rows routed to each expert times that
    expert's [K, N] row-major weight): x N(0,1) [M, K] (one tensor shared by all
    experts when shared_x, else one per expert, drawn first), then W_0 .. W_{E-1}
    N(0,1); C write-only (NaN-filled)."""
    g = rng(seed)
    xs = [to_dtype(draw(g, (M, K), "normal"), dtype)] if shared_x else \
        [to_dtype(draw(g, (M, K), "normal"), dtype) for _ in range(E)]
    cases = []
    for e in range(E):
        W = to_dtype(draw(g, (K, N), "normal"), dtype)
        C = torch.full((M, N), float("nan"), dtype=out_dtype)
        cases.append(Case(f"expert{e}", xs[0] if shared_x else xs[e], W, C))
    return cases


def c4_strided_a(g: np.random.Generator, dtype=torch.bfloat16) -> torch.Tensor:
    """A as a (1,64,64,4096) view of a (1,64,64,4160) tensor whose row pitch is
    padded by 64 elements; the pad holds NaN so a stray read shows up."""
    st = torch.full((1, 64, 64, 4160), float("nan"), dtype=dtype)
    st[..., :4096] = to_dtype(draw(g, (1, 64, 64, 4096), "normal"), dtype)
    return st[..., :4096]


def config(name: str) -> Case:
    """The seeded workload configurations (see the module docstring)."""
    if name == "c1":
        return gemm_case(64, 512, 512, torch.float16, torch.float32, seed=101, dist="uniform",
                         name="c1")
    if name == "c2a":
        return gemm_case(1, 14336, 4096, torch.bfloat16, torch.bfloat16, seed=102, name="c2a")
    if name == "c2b":
        return gemm_case(1, 128, 4096, torch.bfloat16, torch.bfloat16, seed=103, b_layout="col",
                         name="c2b")
    if name == "c3":
        return gemm_case(64, 4096, 4096, torch.float16, torch.float32, seed=104, scale=0.02,
                         beta=1.0, name="c3")
    if name == "c4":
        g = rng(105)
        A = c4_strided_a(g)
        B = to_dtype(draw(g, (4096, 4096), "normal"), torch.bfloat16)
        C = torch.full((4096, 4096), float("nan"), dtype=torch.bfloat16)
        return Case("c4", A, B, C, 1.0, 0.0, rtol=1e-4)
    if name == "c5_128":
        return fp8_case(128, 7168, 4096, seed=106, name="c5_128")
    if name == "c5_4096":
        return fp8_case(4096, 7168, 4096, seed=107, name="c5_4096")
    if name == "c5_tail":
        # FP8 4096 x 4224 x 4096: 1056 tiles of 128 x 128, two whole waves of 512
        # workgroup slots and 32 tiles over (a shape with a short last wave)
        return fp8_case(4096, 4224, 4096, seed=109, name="c5_tail")
    if name.endswith("_gelu") and name[:-5] in CONFIGS:
        # the same operands, then a BF16 bias N(0,1) from rng(seed 201) and GELU
        return with_epilogue(config(name[:-5]), "gelu_tanh", torch.bfloat16, "contig", seed=201,
                             name=name)
    raise KeyError(name)


CONFIGS = ["c1", "c2a", "c2b", "c3", "c4", "c5_128", "c5_4096"]
