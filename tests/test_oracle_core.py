"""Pins for the oracle's GEMM: exact arithmetic, independent loops, closed
forms, alpha/beta algebra, integer exactness, the view walk, and the power of
the comparator to reject known-wrong results.

Nothing here retypes oracle.c's loop: the exact reference is built from
fractions.Fraction, the independent loop is pure Python, and the closed forms
are mathematical identities of C = alpha*A*B + beta*C.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

F16, BF16, E4M3 = torch.float16, torch.bfloat16, torch.float8_e4m3fn


def _vals(t: torch.Tensor):
    """Logical values of a (possibly strided) tensor as Python floats, via torch."""
    return t.double().tolist()


# ----------------------------------------------------------------- exact brute force

@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("seed", range(6))
def test_fraction_brute_force_16bit(dtype, seed):
    g = np.random.default_rng(seed)
    M, N, K = (int(x) for x in g.integers(1, 9, size=3))
    c = synth.gemm_case(M, N, K, dtype, torch.float32, seed=seed + 100, beta=0.75, alpha=-1.5,
                        a_layout=["row", "col", "pad"][seed % 3], b_layout=["row", "col"][seed % 2])
    r = oracle.ref_gemm(c.A, c.B, c.C, c.alpha, c.beta)
    a, b, cin = _vals(c.A), _vals(c.B), _vals(c.C)
    al, be = Fraction(r.alpha), Fraction(r.beta)
    for m in range(M):
        for n in range(N):
            p = sum((Fraction(a[m][k]) * Fraction(b[k][n]) for k in range(K)), Fraction(0))
            s = sum(abs(Fraction(a[m][k]) * Fraction(b[k][n])) for k in range(K))
            exact = al * p + be * Fraction(cin[m][n])
            assert r.S[m, n] == float(s) or abs(Fraction(r.S[m, n]) - s) <= K * Fraction(2) ** -52 * s
            err = abs(Fraction(r.C[m, n]) - exact)
            tol = (K + 2) * Fraction(2) ** -52 * (abs(al) * s + abs(be * Fraction(cin[m][n])))
            assert err <= tol, (m, n, float(err), float(tol))


@pytest.mark.parametrize("seed", range(4))
def test_fraction_brute_force_fp8(seed):
    g = np.random.default_rng(seed + 50)
    M, N = (int(x) for x in g.integers(1, 9, size=2))
    K = int(g.integers(129, 300))        # spans more than one 128-wide scale block
    c = synth.fp8_case(M, N, K, seed=seed + 200, out_dtype=torch.float32)
    r = oracle.ref_gemm(c.A, c.B, None, 1.0, 0.0, A_scale=c.A_scale, B_scale=c.B_scale)
    qa, qb = _vals(c.A), _vals(c.B)
    sa, sb = _vals(c.A_scale), _vals(c.B_scale)
    for m in range(M):
        for n in range(N):
            terms = [Fraction(qa[m][k]) * Fraction(sa[m][k // 128]) *
                     Fraction(qb[k][n]) * Fraction(sb[k // 128][n // 128]) for k in range(K)]
            exact, s = sum(terms, Fraction(0)), sum(abs(t) for t in terms)
            assert abs(Fraction(r.C[m, n]) - exact) <= (K + 2) * Fraction(2) ** -52 * s


# ----------------------------------------------------------------- independent loop

@pytest.mark.parametrize("seed", range(5))
def test_bitwise_equal_to_python_triple_loop(seed):
    g = np.random.default_rng(seed + 1000)
    M, N, K = (int(x) for x in g.integers(1, 34, size=3))
    dtype = [F16, BF16][seed % 2]
    alpha, beta = [(1.0, 0.0), (0.5, -2.0), (-1.25, 1.0)][seed % 3]
    c = synth.gemm_case(M, N, K, dtype, torch.float32, seed=seed, alpha=alpha, beta=beta,
                        a_layout=["row", "pad", "col"][seed % 3],
                        b_layout=["col", "row", "pad"][seed % 3])
    r = oracle.ref_gemm(c.A, c.B, c.C, alpha, beta)
    a, b = _vals(c.A), _vals(c.B)
    cin = _vals(c.C) if beta != 0 else None
    for m in range(M):
        for n in range(N):
            p = 0.0
            for k in range(K):
                p += a[m][k] * b[k][n]
            t = alpha * p if alpha != 0 else 0.0
            want = t if beta == 0 else t + beta * cin[m][n]
            assert r.C[m, n] == want


# ----------------------------------------------------------------- closed forms

def _int_case(M, N, K, dtype=BF16, seed=0, lim=8):
    g = synth.rng(seed)
    A = synth.to_dtype(synth.draw(g, (M, K), "int", lim), dtype)
    B = synth.to_dtype(synth.draw(g, (K, N), "int", lim), dtype)
    return A, B


def test_identity_left_and_right():
    g = synth.rng(3)
    B = synth.to_dtype(synth.draw(g, (24, 17), "normal"), BF16)
    Cin = synth.to_dtype(synth.draw(g, (24, 17), "normal"), torch.float32)
    I = torch.eye(24, dtype=BF16)
    r = oracle.ref_gemm(I, B, Cin, 2.0, 0.5)
    assert np.array_equal(r.C, 2.0 * B.double().numpy() + 0.5 * Cin.double().numpy())
    A = synth.to_dtype(synth.draw(g, (9, 17), "normal"), F16)
    I2 = torch.eye(17, dtype=F16)
    r2 = oracle.ref_gemm(A, I2)
    assert np.array_equal(r2.C, A.double().numpy())


def test_rank_one_closed_form():
    # A = u 1^T, B = 1 z^T with dyadic u, z => C[m,n] = K * u_m * z_n exactly.
    M, N, K = 13, 11, 96
    u = torch.tensor([(-1) ** i * 2.0 ** (i % 5 - 2) for i in range(M)])
    z = torch.tensor([(i % 7 - 3) * 0.25 for i in range(N)])
    A = u[:, None].expand(M, K).to(BF16)
    B = z[None, :].expand(K, N).to(BF16)                   # stride-0 views are walked as given
    r = oracle.ref_gemm(A, B)
    assert np.array_equal(r.C, K * np.outer(u.double().numpy(), z.double().numpy()))


def test_k1_outer_product_and_zeros():
    g = synth.rng(4)
    a = synth.to_dtype(synth.draw(g, (7, 1), "normal"), F16)
    b = synth.to_dtype(synth.draw(g, (1, 5), "normal"), F16)
    r = oracle.ref_gemm(a, b, alpha=-3.0)
    assert np.array_equal(r.C, -3.0 * (a.double().numpy() * b.double().numpy()))
    Z = torch.zeros(7, 6, dtype=F16)
    Cin = synth.to_dtype(synth.draw(g, (7, 5), "normal"), torch.float32)
    r0 = oracle.ref_gemm(Z, torch.zeros(6, 5, dtype=F16), Cin, 1.0, -0.25)
    assert np.array_equal(r0.C, -0.25 * Cin.double().numpy())


def test_all_ones_gives_column_sums():
    _, B = _int_case(3, 19, 257, seed=5)
    A = torch.ones(4, 257, dtype=BF16)
    r = oracle.ref_gemm(A, B)
    colsum = B.double().numpy().sum(axis=0)
    assert np.array_equal(r.C, np.tile(colsum, (4, 1)))


def test_k_zero_is_beta_c():
    Cin = torch.arange(12, dtype=torch.float32).view(3, 4)
    r = oracle.ref_gemm(torch.zeros(3, 0, dtype=F16), torch.zeros(0, 4, dtype=F16), Cin, 1.0, 2.0)
    assert np.array_equal(r.C, 2.0 * Cin.double().numpy())


def test_fp8_power_of_two_scales_exact():
    c = synth.fp8_case(6, 140, 260, seed=9, out_dtype=torch.float32)
    sa = torch.full_like(c.A_scale, 0.5)
    sb = torch.full_like(c.B_scale, 4.0)
    r = oracle.ref_gemm(c.A, c.B, None, A_scale=sa, B_scale=sb)
    r1 = oracle.ref_gemm(c.A, c.B, None, A_scale=torch.ones_like(sa), B_scale=torch.ones_like(sb))
    assert np.array_equal(r.C, 2.0 * r1.C)
    # E4M3 codes times 1 are small dyadics: the unscaled sum is exact vs an FP64 matmul
    ref = c.A.double().numpy() @ c.B.double().numpy()
    assert np.allclose(r1.C, ref, rtol=0, atol=1e-9 * np.abs(ref).max())


# ----------------------------------------------------------------- alpha / beta algebra

@pytest.mark.parametrize("alpha", [0.0, 0.5, -0.5, 1.0, -1.0, 2.0])
@pytest.mark.parametrize("beta", [0.0, 0.25, -0.25, 1.0, -1.0])
def test_alpha_beta_algebra(alpha, beta):
    A, B = _int_case(9, 10, 70, F16, seed=12)
    Cin = synth.to_dtype(synth.draw(synth.rng(13), (9, 10), "normal"), torch.float32)
    base = oracle.ref_gemm(A, B).C                      # exact integers
    r = oracle.ref_gemm(A, B, Cin, alpha, beta)
    assert np.array_equal(r.C, alpha * base + beta * Cin.double().numpy() if beta != 0 else alpha * base)


def test_alpha_zero_ignores_nan_operands_and_beta_zero_ignores_nan_c():
    A = torch.full((4, 8), float("nan"), dtype=BF16)
    B = torch.full((8, 3), float("nan"), dtype=BF16)
    Cin = torch.arange(12, dtype=torch.float32).view(4, 3)
    r = oracle.ref_gemm(A, B, Cin, 0.0, 3.0)
    assert np.array_equal(r.C, 3.0 * Cin.double().numpy())
    A2, B2 = _int_case(4, 3, 8, seed=2)
    r2 = oracle.ref_gemm(A2, B2, torch.full((4, 3), float("nan")), 1.0, 0.0)
    assert not np.isnan(r2.C).any()


def test_sign_and_power_of_two_scaling():
    c = synth.gemm_case(11, 9, 77, BF16, torch.float32, seed=21)
    r = oracle.ref_gemm(c.A, c.B).C
    assert np.array_equal(oracle.ref_gemm(-c.A, c.B).C, -r)
    assert np.array_equal(oracle.ref_gemm(c.A * 4, c.B).C, 4 * r)


def test_fp8_scale_applied_once():
    c = synth.fp8_case(5, 130, 300, seed=22, out_dtype=torch.float32)
    r = oracle.ref_gemm(c.A, c.B, None, A_scale=c.A_scale, B_scale=c.B_scale).C
    r2 = oracle.ref_gemm(c.A, c.B, None, A_scale=c.A_scale * 2, B_scale=c.B_scale).C
    assert np.array_equal(r2, 2 * r)
    # Per-block independence: doubling only K-block 1's scales doubles only its share.
    sa = c.A_scale.clone(); sa[:, 1] *= 2
    r3 = oracle.ref_gemm(c.A, c.B, None, A_scale=sa, B_scale=c.B_scale).C
    qa, qb = c.A.double().numpy(), c.B.double().numpy()
    deq_a = qa * np.repeat(c.A_scale.double().numpy(), 128, axis=1)[:, :300]
    deq_b = qb * np.repeat(np.repeat(c.B_scale.double().numpy(), 128, axis=0), 128, axis=1)[:300, :130]
    blk1 = deq_a[:, 128:256] @ deq_b[128:256, :]
    assert np.allclose(r3 - r, blk1, rtol=1e-12, atol=1e-12 * np.abs(blk1).max())


# ----------------------------------------------------------------- integer exactness

@pytest.mark.parametrize("dtype", [F16, BF16, E4M3])
def test_integer_inputs_exact(dtype):
    K = 4096 if dtype != E4M3 else 1024
    g = synth.rng(31)
    A = synth.to_dtype(synth.draw(g, (6, K), "int", 8), torch.float32)
    B = synth.to_dtype(synth.draw(g, (K, 7), "int", 8), torch.float32)
    want = A.numpy().astype(np.int64) @ B.numpy().astype(np.int64)
    if dtype == E4M3:
        sa = torch.ones(6, K // 128); sb = torch.ones(K // 128, 1)
        r = oracle.ref_gemm(A.to(dtype), B.to(dtype), None, A_scale=sa, B_scale=sb)
    else:
        r = oracle.ref_gemm(A.to(dtype), B.to(dtype))
    assert np.array_equal(r.C, want.astype(np.float64))


# ----------------------------------------------------------------- the view walk

def _golden_views():
    rows = []
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "views.txt")
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        name, dt, shape, stride, unit, cite = [x.strip() for x in line.split("|")]
        rows.append((name, dt, tuple(map(int, shape.split(","))), tuple(map(int, stride.split(","))),
                     unit, cite))
    return rows


_DT = {"f32": torch.float32, "bf16": BF16, "f16": F16, "e4m3": E4M3}


@pytest.mark.parametrize("g", _golden_views(), ids=lambda g: g[0])
def test_golden_view_walk_matches_torch(g):
    name, dt, shape, stride, unit, _ = g
    dtype = _DT[dt]
    es = torch.empty(0, dtype=dtype).element_size()
    el_stride = stride if unit == "elements" else tuple(s // es for s in stride)
    assert unit == "elements" or all(s % es == 0 for s in stride)
    span = 1 + sum((n - 1) * s for n, s in zip(shape, el_stride))
    base = synth.to_dtype(synth.draw(synth.rng(77), (span,), "normal"), dtype if dtype != E4M3 else torch.float32)
    base = base.to(dtype)
    t = base.as_strided(shape, el_stride)
    got = oracle.gather(oracle.host_view(t))
    rows = math.prod(shape[:-1])
    assert got.shape == (rows, shape[-1])
    assert np.array_equal(got, t.reshape(rows, shape[-1]).double().numpy(), equal_nan=True)


@pytest.mark.parametrize("layout", [("pad", "row"), ("col", "col"), ("row", "pad")])
def test_strided_equals_contiguous(layout):
    c = synth.gemm_case(37, 29, 131, F16, torch.float32, seed=40, a_layout=layout[0],
                        b_layout=layout[1], beta=1.0, c_layout="pad")
    r1 = oracle.ref_gemm(c.A, c.B, c.C, 1.0, 1.0)
    r2 = oracle.ref_gemm(c.A.contiguous(), c.B.contiguous(), c.C.contiguous(), 1.0, 1.0)
    assert np.array_equal(r1.C, r2.C) and np.array_equal(r1.S, r2.S)


def test_four_d_padded_view_and_row_subset():
    # A scaled-down copy of the square workload's A geometry: (1,4,8,64) over pitch 72.
    st = torch.full((1, 4, 8, 72), float("nan"), dtype=BF16)
    st[..., :64] = synth.to_dtype(synth.draw(synth.rng(41), (1, 4, 8, 64), "normal"), BF16)
    A = st[..., :64]
    B = synth.to_dtype(synth.draw(synth.rng(42), (64, 10), "normal"), BF16)
    full = oracle.ref_gemm(A, B)
    assert not np.isnan(full.C).any()
    assert np.array_equal(full.C, oracle.ref_gemm(A.reshape(32, 64).contiguous(), B).C)
    sub = oracle.ref_gemm(A, B, rows=[31, 0, 17])
    assert np.array_equal(sub.C, full.C[[31, 0, 17]])


# ----------------------------------------------------------------- comparator power

def _truth(M=48, N=40, K=512, seed=60):
    c = synth.gemm_case(M, N, K, BF16, torch.float32, seed=seed)
    return c, oracle.ref_gemm(c.A, c.B)


def test_comparator_accepts_fp32_gemm_in_another_order():
    c, ref = _truth()
    got = torch.matmul(c.A.float(), c.B.float())           # library FP32 GEMM, its own order
    assert oracle.compare(got, ref, "f32", 1e-4).ok
    assert oracle.compare(got.to(BF16), ref, "bf16", 1e-4).ok


def test_comparator_rejects_dropped_k_block():
    c, ref = _truth()
    wrong = oracle.ref_gemm(c.A[:, :384], c.B[:384]).C
    assert not oracle.compare(wrong, ref, "f32", 1e-4).ok


def test_comparator_rejects_swapped_columns():
    c, ref = _truth()
    wrong = ref.C.copy(); wrong[:, [3, 4]] = wrong[:, [4, 3]]
    assert not oracle.compare(wrong, ref, "f32", 1e-4).ok


def test_comparator_rejects_reading_c_when_beta_zero():
    c, ref = _truth()
    junk = synth.to_dtype(synth.draw(synth.rng(61), ref.C.shape, "normal"), torch.float32)
    wrong = oracle.ref_gemm(c.A, c.B, junk, 1.0, 1.0).C
    assert not oracle.compare(wrong, ref, "f32", 1e-4).ok


def test_comparator_rejects_element_strides_taken_as_bytes():
    c = synth.gemm_case(32, 24, 256, BF16, torch.float32, seed=62, a_layout="pad")
    ref = oracle.ref_gemm(c.A, c.B)
    hv = oracle.host_view(c.A)
    es = c.A.element_size()
    bad = oracle.HostView(hv.storage, hv.offset, hv.shape, tuple(s // es for s in hv.stride), hv.dtype)
    wrong = oracle.ref_gemm(bad, c.B).C
    assert not oracle.compare(wrong, ref, "f32", 1e-4).ok


def test_comparator_rejects_fp8_scale_applied_twice():
    c = synth.fp8_case(16, 256, 512, seed=63, out_dtype=torch.float32)
    ref = oracle.ref_gemm(c.A, c.B, None, A_scale=c.A_scale, B_scale=c.B_scale)
    wrong = oracle.ref_gemm(c.A, c.B, None, A_scale=c.A_scale * c.A_scale, B_scale=c.B_scale).C
    assert not oracle.compare(wrong, ref, "f32", 1e-3).ok
    ok = oracle.ref_gemm(c.A, c.B, None, A_scale=c.A_scale, B_scale=c.B_scale).C
    assert oracle.compare(ok, ref, "f32", 1e-3).ok


def test_comparator_flags_nan_mismatch_and_reports_stats():
    c, ref = _truth(8, 8, 64)
    wrong = ref.C.copy(); wrong[2, 5] = np.nan
    rep = oracle.compare(wrong, ref, "f32", 1e-4)
    assert not rep.ok and rep.nan_mismatch == 1
    rep2 = oracle.compare(ref.C, ref, "f32", 1e-4)
    assert rep2.ok and rep2.rmse == 0.0 and rep2.max_ratio == 0.0
    # "bitwise" means equal to the reference rounded (RNE) to the output format
    rep3 = oracle.compare(ref.C.astype(np.float32), ref, "f32", 1e-4)
    assert rep3.ok and rep3.bitwise


# ----------------------------------------------------------------- special values (IEEE propagation)

@pytest.mark.parametrize("dtype", [F16, BF16])
def test_nan_and_inf_propagate_like_a_python_loop(dtype):
    # A NaN or an infinity in one operand reaches exactly the outputs it
    # touches, as IEEE arithmetic says (the cf-1.com article, section 5.3: a
    # NaN must show up, not vanish): checked against a pure-Python loop, whose
    # floats are IEEE binary64.
    M, N, K = 5, 6, 7
    g = synth.rng(5)
    A = synth.to_dtype(synth.draw(g, (M, K), "normal"), dtype)
    B = synth.to_dtype(synth.draw(g, (K, N), "normal"), dtype)
    A[1, 2] = float("nan")
    A[3, 4] = float("inf")
    B[0, 1] = float("-inf")
    B[5, 4] = float("inf")
    r = oracle.ref_gemm(A, B, None)
    a, b = _vals(A), _vals(B)
    for m in range(M):
        for n in range(N):
            p = 0.0
            for k in range(K):
                p += a[m][k] * b[k][n]
            got = r.C[m, n]
            assert (math.isnan(p) and math.isnan(got)) or got == p, (m, n, got, p)
    assert np.isnan(r.C[1]).all()            # the NaN row
    assert np.isinf(r.C[3, [0, 2, 3, 5]]).all()


def test_fp8_nan_codes_propagate():
    # E4M3FN has no infinity: 0x7F and 0xFF are its NaNs.
    qa = torch.zeros(3, 128, dtype=torch.uint8)
    qa[:] = 0x38          # 1.0
    qa[1, 7] = 0x7F
    qb = torch.full((128, 4), 0x38, dtype=torch.uint8)
    qb[9, 2] = 0xFF
    A, B = qa.view(E4M3), qb.view(E4M3)
    r = oracle.ref_gemm(A, B, None, A_scale=torch.ones(3, 1), B_scale=torch.ones(1, 1))
    want = np.full((3, 4), 128.0)
    want[1, :] = np.nan
    want[:, 2] = np.nan
    assert np.array_equal(r.C, want, equal_nan=True)


def test_fp16_subnormal_inputs_are_not_flushed():
    # products of FP16 subnormals are exact in FP64: 2^-24 * 2^-24 summed K times
    M, N, K = 2, 3, 16
    A = torch.full((M, K), 2.0 ** -24, dtype=F16)
    B = torch.full((K, N), 2.0 ** -24, dtype=F16)
    B[:, 1] = 2.0 ** -15          # the largest binary exponent of the subnormal range
    r = oracle.ref_gemm(A, B, None)
    assert np.array_equal(r.C[:, 0], np.full(M, K * 2.0 ** -48))
    assert np.array_equal(r.C[:, 1], np.full(M, K * 2.0 ** -39))


def test_comparator_requires_the_same_infinity():
    A = torch.ones(2, 4, dtype=BF16)
    B = torch.ones(4, 3, dtype=BF16)
    A[0, 1] = float("inf")
    B[2, 2] = float("-inf")
    ref = oracle.ref_gemm(A, B, None)
    assert np.isinf(ref.C[0, 0]) and np.isnan(ref.C[0, 2]) and ref.C[1, 2] == -np.inf
    assert oracle.compare(ref.C.copy(), ref, "f32", 1e-4).ok
    for (i, j, v) in [(0, 0, -np.inf), (0, 0, 1e30), (1, 2, np.nan), (1, 2, np.inf), (0, 2, np.inf)]:
        wrong = ref.C.copy()
        wrong[i, j] = v
        assert not oracle.compare(wrong, ref, "f32", 1e-4).ok, (i, j, v)
