"""GPU parity of the fused epilogue (dg_gemm_epilogue, dg_gemm_fp8_epilogue)
against the FP64 oracle: C <- act(alpha * A*B + beta * C + bias[n]).

Tolerance (written here and in oracle/epilogue.py): with the GEMM bound
E = rtol * |alpha| * S + 4 * 2^-24 * (|alpha| * S + |beta * C_in| + |bias|)
on the pre-activation value y, the result must lie within
L * E + c * 2^-24 * |y| + 0.5 * ulp_out of act(y), where L = 1 (none, ReLU)
or 1.13 (GELU, its largest slope) and c = 0 (none, ReLU) or 8 (GELU's FP32
evaluation).  Every kernel path is covered: the streaming kernels (B
N-contiguous, with and without split K; B K-contiguous), the register-staged
matrix-core kernel (with the split-K reduction kernel), the direct-to-LDS
matrix-core kernel (with its in-kernel split-K reduction), FP8, and the
alpha == 0 / K == 0 scaling kernel.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import epilogue as E

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
F16, BF16, F32 = torch.float16, torch.bfloat16, torch.float32


@pytest.fixture(scope="module")
def dg():
    import dense_gemm_19_amd as m
    m.lib()   # raises if the library is missing: there is no fallback
    return m


def act_code(dg, act):
    return {"none": dg.DG_ACT_NONE, "relu": dg.DG_ACT_RELU, "gelu_tanh": dg.DG_ACT_GELU_TANH}[act]


def run_epi(dg, case):
    d = case.to(DEV)
    a = act_code(dg, case.act)
    if case.fp8:
        dg.gemm_fp8_epilogue(d.A, d.A_scale, d.B, d.B_scale, d.C, d.bias, a, case.alpha, case.beta)
    else:
        dg.gemm_epilogue(d.A, d.B, d.C, d.bias, a, case.alpha, case.beta)
    torch.cuda.synchronize()
    return d


def plan_text(dg, case):
    d = case.to(DEV)
    return dg.plan(d.A, d.B, d.C, case.alpha, case.beta, d.A_scale, d.B_scale)


def check_epi(dg, case, rows=None, want_in_plan=()):
    text = plan_text(dg, case)
    print(f"[epilogue] {case.name} M,N,K={case.mnk} act={case.act} "
          f"bias={None if case.bias is None else (case.bias.dtype, tuple(case.bias.stride()))} "
          f"alpha={case.alpha} beta={case.beta} | {text.split(' | ')[0]}", flush=True)
    for w in want_in_plan:
        assert w in text, (w, text)
    ref = oracle.ref_gemm(case.A, case.B, case.C if case.beta != 0 else None, case.alpha, case.beta,
                          rows=rows, A_scale=case.A_scale, B_scale=case.B_scale)
    e = E.ref_epilogue(ref, case.bias, case.act)
    d = run_epi(dg, case)
    got = d.C.detach().cpu()
    if got.dim() > 2:
        got = got.reshape(-1, got.shape[-1])
    got = got[torch.as_tensor(ref.rows)]
    rep = E.compare_epilogue(got, e, oracle.fmt_of(case.C.dtype), case.rtol)
    print(f"[epilogue] {case.name}: {rep}", flush=True)
    assert rep.ok, str(rep)
    return rep, d


# ---------------------------------------------------------------- every kernel path

PATHS = [
    # (M, N, K, b_layout, a_layout, what the plan must say)
    (1, 1000, 777, "row", "row", ("path=skinny", "kind=BN", "splits=3")),
    (2, 14336, 4096, "row", "row", ("path=skinny", "kind=BN", "splits=8", "cols=448")),
    (8, 64, 8, "row", "row", ("path=skinny", "kind=BN", "splits=1")),
    (3, 129, 1000, "col", "row", ("path=skinny", "kind=BK")),
    (65, 129, 255, "row", "row", ("path=mfma", "dtl=0", "splits=1")),
    (300, 257, 192, "row", "pad", ("path=mfma", "dtl=0")),
    (65, 200, 1000, "row", "row", ("path=mfma", "dtl=0", "splits=8")),
    (512, 640, 512, "row", "row", ("path=mfma", "dtl=1", "splits=1")),
    (384, 384, 1024, "row", "row", ("path=mfma", "dtl=1", "splits=2")),
    (4096, 4160, 128, "row", "row", ("path=split_n", "n1=4096")),   # column split: bias of both parts
    (1000, 4104, 512, "col", "row", ("path=mfma", "dtl=1")),
]


@pytest.mark.parametrize("act", ["relu", "gelu_tanh"])
@pytest.mark.parametrize("p", PATHS, ids=lambda p: f"{p[0]}x{p[1]}x{p[2]}-B{p[3]}-A{p[4]}")
def test_paths(dg, p, act):
    M, N, K, bl, al, want = p
    c = synth.gemm_case(M, N, K, BF16, BF16, seed=M + 3 * N + 7 * K, a_layout=al, b_layout=bl)
    c = synth.with_epilogue(c, act, BF16, "contig", seed=M + N)
    check_epi(dg, c, want_in_plan=want)


# ---------------------------------------------------------------- dtypes and bias layouts

@pytest.mark.parametrize("bias_dtype", [F32, F16, BF16], ids=["bias_f32", "bias_f16", "bias_bf16"])
@pytest.mark.parametrize("out", [F32, F16, BF16], ids=["f32", "f16", "bf16"])
def test_output_and_bias_dtypes(dg, out, bias_dtype):
    for M, N, K in [(130, 200, 256), (4, 520, 4096)]:
        c = synth.gemm_case(M, N, K, F16 if out == F16 else BF16, out, seed=M + N + out.itemsize)
        check_epi(dg, synth.with_epilogue(c, "gelu_tanh", bias_dtype, "contig", seed=5))


@pytest.mark.parametrize("layout", ["strided", "bcast"])
@pytest.mark.parametrize("shape", [(1, 3000, 2048), (256, 384, 512), (77, 300, 333)],
                         ids=lambda s: "x".join(map(str, s)))
def test_bias_layouts(dg, shape, layout):
    M, N, K = shape
    c = synth.gemm_case(M, N, K, BF16, F32, seed=M * N + K)
    check_epi(dg, synth.with_epilogue(c, "relu", F32, layout, seed=9))


@pytest.mark.parametrize("act", ["none", "relu", "gelu_tanh"])
def test_activation_without_bias(dg, act):
    c = synth.gemm_case(256, 512, 512, BF16, BF16, seed=3)
    check_epi(dg, synth.with_epilogue(c, act, None))


# ---------------------------------------------------------------- alpha, beta, K = 0

@pytest.mark.parametrize("ab", [(1.0, 1.0), (-0.5, 2.0), (0.0, 1.5), (0.0, 0.0)])
@pytest.mark.parametrize("shape", [(1, 4096, 4096), (200, 300, 1024)], ids=lambda s: "x".join(map(str, s)))
def test_alpha_beta(dg, shape, ab):
    M, N, K = shape
    alpha, beta = ab
    c = synth.gemm_case(M, N, K, BF16, F32, seed=M + K, alpha=alpha, beta=beta)
    check_epi(dg, synth.with_epilogue(c, "gelu_tanh", BF16, "contig", seed=11))


def test_k_zero_is_act_of_beta_c_plus_bias(dg):
    c = synth.gemm_case(40, 70, 0, BF16, F32, seed=2, beta=0.5)
    check_epi(dg, synth.with_epilogue(c, "gelu_tanh", F16, "contig", seed=12), want_in_plan=("path=scale",))


def test_nan_in_c_propagates_through_relu(dg):
    c = synth.gemm_case(64, 256, 512, BF16, F32, seed=4, beta=1.0)
    c.C[3, 7] = float("nan")
    c.C[60, 200] = float("nan")
    check_epi(dg, synth.with_epilogue(c, "relu", BF16, "contig", seed=13))


def test_empty_problems(dg):
    for M, N in [(0, 64), (64, 0)]:
        A = torch.zeros(M, 32, dtype=BF16, device=DEV)
        B = torch.zeros(32, N, dtype=BF16, device=DEV)
        C = torch.zeros(M, N, dtype=BF16, device=DEV)
        bias = torch.zeros(N, dtype=BF16, device=DEV)
        dg.gemm_epilogue(A, B, C, bias, dg.DG_ACT_GELU_TANH)
    torch.cuda.synchronize()


# ---------------------------------------------------------------- identity with the plain entry point

@pytest.mark.parametrize("shape", [(1, 1000, 777), (3, 129, 1000), (65, 200, 1000), (512, 640, 512),
                                   (384, 384, 1024), (300, 257, 192)], ids=lambda s: "x".join(map(str, s)))
def test_no_bias_no_act_is_bitwise_dg_gemm(dg, shape):
    M, N, K = shape
    c = synth.gemm_case(M, N, K, BF16, F32, seed=K, beta=0.5, b_layout="col" if M == 3 else "row")
    d1 = c.to(DEV)
    dg.gemm(d1.A, d1.B, d1.C, c.alpha, c.beta)
    d2 = c.to(DEV)
    dg.gemm_epilogue(d2.A, d2.B, d2.C, None, dg.DG_ACT_NONE, c.alpha, c.beta)
    torch.cuda.synchronize()
    assert torch.equal(d1.C.cpu(), d2.C.cpu())


# ---------------------------------------------------------------- FP8

@pytest.mark.parametrize("shape", [(100, 260, 384), (256, 512, 1024), (1008, 4112, 256), (1, 7168, 4096)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("act", ["relu", "gelu_tanh"])
def test_fp8(dg, shape, act):
    M, N, K = shape
    c = synth.fp8_case(M, N, K, seed=M + N, beta=0.25 if M == 100 else 0.0)
    check_epi(dg, synth.with_epilogue(c, act, BF16, "contig", seed=14))


# ---------------------------------------------------------------- the workloads at full size

@pytest.mark.parametrize("name", ["c2a_gelu", "c3_gelu", "c4_gelu", "c5_128_gelu", "c5_4096_gelu"])
def test_workload_full_size(dg, name):
    case = synth.config(name)
    _, d = check_epi(dg, case)     # every element of C
    assert torch.isfinite(d.C.float()).all()
