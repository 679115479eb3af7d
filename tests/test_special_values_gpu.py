"""GPU parity on special values: NaN and Inf in the operands, subnormal inputs.

Every kernel path (both streaming kernels, the direct-to-LDS matrix-core kernel
with and without split K, its 256x256 tile, the register-staged kernel, FP8)
gets operands holding NaN and +-Inf (E4M3FN: its NaN codes 0x7F and 0xFF; it
has no infinity), and operands made of subnormal numbers.  The FP64 oracle
decides: NaN results must sit exactly where the oracle's are, infinite results
must be the same infinity, everything else within the stated bound.

Data conventions under test: NaN/Inf in the data propagate per IEEE (the
cf-1.com article, section 5.3, tells of a NaN that a kernel must not hide);
subnormal FP16/BF16/E4M3 inputs are not flushed to zero.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
F16, BF16, E4M3 = torch.float16, torch.bfloat16, torch.float8_e4m3fn


@pytest.fixture(scope="module")
def dg():
    import dense_gemm_19_amd as m
    m.lib()
    return m


def _plan(dg, c):
    d = c.to(DEV)
    return dg.plan(d.A, d.B, d.C, c.alpha, c.beta, d.A_scale, d.B_scale)


def _run_and_check(dg, c, plan_has):
    text = _plan(dg, c)
    for s in plan_has:
        assert s in text, (s, text)
    print(f"[special] {c.name} M,N,K={c.mnk} plan: {text}", flush=True)
    ref = oracle.ref_gemm(c.A, c.B, c.C if c.beta != 0 else None, c.alpha, c.beta,
                          A_scale=c.A_scale, B_scale=c.B_scale)
    d = c.to(DEV)
    if c.fp8:
        dg.gemm_fp8(d.A, d.A_scale, d.B, d.B_scale, d.C, c.alpha, c.beta)
    else:
        dg.gemm(d.A, d.B, d.C, c.alpha, c.beta)
    torch.cuda.synchronize()
    rep = oracle.compare(d.C.cpu(), ref, oracle.fmt_of(c.C.dtype), c.rtol)
    print(f"[special] {c.name}: {rep}", flush=True)
    assert rep.ok, str(rep)
    return ref


# (name, M, N, K, input, B layout, what the plan must say)
PATHS = [
    ("skinny_bn", 4, 1000, 4096, BF16, "row", ["path=skinny", "kind=BN"]),
    ("skinny_bn_split", 1, 304, 4096, F16, "row", ["path=skinny", "kind=BN", "splits=16"]),
    ("skinny_bk", 3, 129, 1000, BF16, "col", ["path=skinny", "kind=BK"]),
    ("dtl_64_splitk", 64, 512, 4096, F16, "row", ["dtl=1", "tile=64x64", "splits=4"]),
    ("dtl_128", 1000, 4104, 512, BF16, "row", ["dtl=1", "tile=128x128"]),
    ("dtl_256", 4096, 4096, 256, BF16, "row", ["dtl=1", "tile=256x256"]),
    ("general", 300, 257, 1000, F16, "row", ["dtl=0"]),
    ("fp8_64x128_splitk", 128, 7168, 4096, E4M3, "row", ["dtl=1", "tile=64x128", "splits=2"]),
    ("fp8_128", 2048, 2048, 1024, E4M3, "col", ["dtl=1", "tile=128x128"]),
    ("fp8_256", 4096, 4096, 256, E4M3, "row", ["dtl=1", "tile=256x256"]),
]


def _base(name, M, N, K, kind, bl, seed):
    if kind == E4M3:
        return synth.fp8_case(M, N, K, seed=seed, b_layout=bl, out_dtype=torch.float32, name=name)
    return synth.gemm_case(M, N, K, kind, torch.float32, seed=seed, b_layout=bl, name=name)


def _poke(t, i, j, value):
    """t[i, j] = value in place (a view: the stored element changes)."""
    if t.dtype == E4M3:
        t.view(torch.uint8)[i, j] = value
    else:
        t[i, j] = value


@pytest.mark.parametrize("path", PATHS, ids=lambda p: p[0])
def test_nan_inf_propagate(dg, path):
    name, M, N, K, kind, bl, has = path
    c = _base(name + "_naninf", M, N, K, kind, bl, seed=M + N + K)
    r_nan, r_inf = M - 1, min(1, M - 1)
    c_nan, c_inf = 0, N // 2
    if kind == E4M3:
        _poke(c.A, r_nan, K // 3, 0x7F)          # E4M3FN NaN codes
        _poke(c.B, (2 * K) // 3, c_nan, 0xFF)
    else:
        _poke(c.A, r_nan, K // 3, float("nan"))
        _poke(c.B, (2 * K) // 3, c_nan, float("nan"))
        if M > 2:
            _poke(c.A, r_inf, K - 1, float("inf"))
        _poke(c.B, 1, c_inf, float("-inf"))
    ref = _run_and_check(dg, c, has)
    assert np.isnan(ref.C[r_nan]).all() and np.isnan(ref.C[:, c_nan]).all()
    if kind != E4M3 and M > 2:       # (with one row, the NaN row is the only row)
        assert np.isinf(ref.C).any()


@pytest.mark.parametrize("path", [p for p in PATHS if p[4] != E4M3], ids=lambda p: p[0])
def test_fp16_subnormal_inputs(dg, path):
    # Every element of A and B an FP16 subnormal (|x| in [2^-24, 2^-14)): their
    # products are normal FP32 numbers, so a kernel that flushed subnormal
    # inputs would return zeros.
    name, M, N, K, _, bl, has = path
    g = synth.rng(M * 3 + N + K)

    def sub(shape):
        m = g.integers(1, 1024, size=shape) * g.choice([-1.0, 1.0], size=shape)
        return torch.from_numpy(m * 2.0 ** -24).to(F16)
    A = sub((M, K))
    B = sub((N, K)).t() if bl == "col" else sub((K, N))
    assert (A.float().abs() < 2.0 ** -14).all() and (A != 0).all()
    c = synth.Case(name + "_f16sub", A, B, torch.full((M, N), float("nan")), 1.0, 0.0)
    ref = _run_and_check(dg, c, has)
    assert (np.abs(ref.C) > 0).mean() > 0.99


@pytest.mark.parametrize("path", [p for p in PATHS if p[4] == BF16], ids=lambda p: p[0])
def test_bf16_subnormal_inputs(dg, path):
    # A made of BF16 subnormals (|a| < 2^-126), B of large BF16 values (~2^100):
    # the products are normal FP32 numbers, zeros if A were flushed.
    name, M, N, K, _, bl, has = path
    g = synth.rng(M * 5 + N + K)
    m = g.integers(1, 128, size=(M, K)) * g.choice([-1.0, 1.0], size=(M, K))
    A = torch.from_numpy(m * 2.0 ** -133).to(BF16)
    assert (A.float().abs() < 2.0 ** -126).all() and (A != 0).all()
    b = synth.draw(g, (N, K) if bl == "col" else (K, N), "normal", 2.0 ** 100)
    B = synth.to_dtype(b, BF16)
    B = B.t() if bl == "col" else B
    c = synth.Case(name + "_bf16sub", A, B, torch.full((M, N), float("nan")), 1.0, 0.0)
    ref = _run_and_check(dg, c, has)
    assert (np.abs(ref.C) > 0).mean() > 0.99


@pytest.mark.parametrize("path", [p for p in PATHS if p[4] == E4M3], ids=lambda p: p[0])
def test_fp8_subnormal_codes(dg, path):
    # E4M3FN subnormals (exponent field 0: m * 2^-9, codes 0x01-0x07 and 0x81-0x87)
    # in A, ordinary codes in B, unit scales.
    name, M, N, K, _, bl, has = path
    c = _base(name + "_f8sub", M, N, K, E4M3, bl, seed=M + 2 * N + K)
    g = synth.rng(M + N)
    codes = g.integers(1, 8, size=(M, K)) | (g.integers(0, 2, size=(M, K)) << 7)
    c.A.view(torch.uint8).copy_(torch.from_numpy(codes.astype(np.uint8)))
    c.A_scale.fill_(1.0)
    assert (c.A.float().abs() < 2.0 ** -6).all()
    ref = _run_and_check(dg, c, has)
    assert (np.abs(ref.C) > 0).mean() > 0.99
