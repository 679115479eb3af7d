"""GPU parity of the grouped GEMM (dg_gemm_grouped) against the FP64 oracle,
group by group: C[g] <- alpha * A[g] * B[g] + beta * C[g].

Each group's result must meet the dg_gemm bound (oracle/compare.py):
|C - C_ref| <= 1e-4 * |alpha| * S + 4 * 2^-24 * (|alpha| * S + |beta * C_in|)
+ 0.5 * ulp_out, S = sum_k |a_ik * b_kj|.  Covered: the MoE experts of the
pages (8 x [1,512] x [512,4096], one shared token row), every M class of the
grouped streaming kernel, ragged N and K, groups that run alone (K-contiguous
or unaligned B, K = 0, alpha = 0, a lone matrix-core configuration), empty
groups, more than 16 groups (several launches), the grouped matrix-core launch
(experts with 17-256 tokens each, two operand layouts, more than 16 groups),
and run-to-run bitwise reproducibility.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
F16, BF16, F32 = torch.float16, torch.bfloat16, torch.float32


@pytest.fixture(scope="module")
def dg():
    import dense_gemm_19_amd as m
    m.lib()   # raises if the library is missing: there is no fallback
    return m


def to_dev(t):
    return synth.Case("x", t, t, t).to(DEV).A


def run_grouped(dg, cases, alpha=1.0, beta=0.0):
    As = [to_dev(c.A) for c in cases]
    Bs = [to_dev(c.B) for c in cases]
    Cs = [to_dev(c.C) for c in cases]
    text = dg.grouped_plan(As, Bs, Cs, alpha, beta)
    print(f"[grouped] G={len(cases)} alpha={alpha} beta={beta} | {text}", flush=True)
    dg.gemm_grouped(As, Bs, Cs, alpha, beta)
    torch.cuda.synchronize()
    return [c.cpu() for c in Cs], text


def check_grouped(dg, cases, alpha=1.0, beta=0.0, rows_cap=None):
    got, text = run_grouped(dg, cases, alpha, beta)
    worst = 0.0
    for c, C in zip(cases, got):
        M = c.mnk[0]
        rows = None if rows_cap is None or M <= rows_cap else list(range(0, M, max(1, M // rows_cap)))
        ref = oracle.ref_gemm(c.A, c.B, c.C if beta != 0 else None, alpha, beta, rows=rows)
        sel = C if rows is None else C[torch.as_tensor(ref.rows)]
        rep = oracle.compare(sel, ref, oracle.fmt_of(c.C.dtype), 1e-4)
        worst = max(worst, rep.max_ratio)
        assert rep.ok, f"{c.name} {c.mnk}: {rep}"
    print(f"[grouped] worst err/bound {worst:.3g}", flush=True)
    return got, text


def test_moe_experts(dg):
    cases = synth.moe_experts()
    got, text = check_grouped(dg, cases)
    assert "batch mmax=1 units=256" in text and text.endswith("solo="), text


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8])
def test_each_m_class(dg, M):
    cases = synth.moe_experts(E=5, M=M, K=700, N=1000, seed=M, shared_x=False, out_dtype=F32)
    _, text = check_grouped(dg, cases)
    assert "batch" in text and text.endswith("solo="), text


def test_mixed_shapes_and_solo_groups(dg):
    g = synth.rng(21)
    cases = []
    shapes = [(1, 4096, 512, "row"), (3, 1000, 777, "row"), (8, 300, 1000, "row"), (20, 512, 256, "row"),
              (2, 128, 4096, "col"), (1, 14336, 4096, "row"), (6, 8, 33, "row"), (1, 1, 1, "row")]
    for i, (M, N, K, bl) in enumerate(shapes):
        c = synth.gemm_case(M, N, K, BF16, F32 if i % 2 else BF16, seed=100 + i, b_layout=bl, beta=0.5)
        cases.append(c)
    _, text = check_grouped(dg, cases, alpha=1.5, beta=0.5)
    assert "solo=" in text and "batch" in text, text


def test_shared_input_and_f16(dg):
    x = synth.to_dtype(synth.draw(synth.rng(3), (4, 2048), "normal"), F16)
    cases = []
    for e, N in enumerate([256, 1024, 2000, 4096]):
        W = synth.to_dtype(synth.draw(synth.rng(10 + e), (2048, N), "uniform"), F16)
        cases.append(synth.Case(f"e{e}", x, W, torch.full((4, N), float("nan"), dtype=F16)))
    check_grouped(dg, cases)


def test_more_than_sixteen_groups(dg):
    g = np.random.default_rng(5)
    cases = []
    for i in range(40):
        M = int(g.integers(1, 9))
        N = int(g.integers(1, 375)) * 8 if i % 5 else int(g.integers(1, 3000))   # mostly 16-byte rows
        K = int(g.integers(1, 2000))
        cases.append(synth.gemm_case(M, N, K, BF16, BF16, seed=1000 + i, name=f"g{i}"))
    _, text = check_grouped(dg, cases)
    assert text.count("batch") >= 3, text


def test_empty_and_degenerate_groups(dg):
    cases = [synth.gemm_case(1, 512, 256, BF16, F32, seed=1, beta=1.0),
             synth.gemm_case(0, 512, 256, BF16, F32, seed=2, beta=1.0),
             synth.gemm_case(2, 0, 256, BF16, F32, seed=3, beta=1.0),
             synth.gemm_case(2, 300, 0, BF16, F32, seed=4, beta=1.0),     # K = 0: C <- beta * C
             synth.gemm_case(4, 700, 900, BF16, F32, seed=5, beta=1.0)]
    check_grouped(dg, cases, alpha=-1.0, beta=1.0)
    check_grouped(dg, cases[:1] + cases[4:], alpha=0.0, beta=2.0)      # alpha = 0: scaling only
    # G = 0 is a no-op
    dg.gemm_grouped([], [], [])


def test_run_twice_bitwise(dg):
    cases = synth.moe_experts(E=8, M=2, K=1536, N=3000, seed=9, shared_x=False)
    a, _ = run_grouped(dg, cases)
    b, _ = run_grouped(dg, cases)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_wide_and_narrow_slab_batches(dg):
    # Streaming groups whose planned slabs are wider than 256 columns run in a
    # launch of their own (the 64-lane row layout) beside the 32-lane batch of the
    # same M class; one wide group has N = 9003 with B rows padded by NaN, so its
    # last slab has a lane straddling N.
    cases = [synth.gemm_case(1, 14336, 2048, BF16, BF16, seed=801, name="w0"),
             synth.gemm_case(2, 1000, 700, BF16, F32, seed=802, name="n1"),
             synth.gemm_case(1, 9003, 1024, BF16, BF16, seed=803, b_layout="pad", pad=13, name="w2"),
             synth.gemm_case(3, 12000, 512, BF16, F32, seed=804, name="w3")]
    _, text = check_grouped(dg, cases)
    widths = [int(g.split("c")[-1]) for g in text.replace(" |", "").split("groups=")[1:] for g in g.split()[0].split(",")]
    assert any(w > 256 for w in widths) and any(w <= 256 for w in widths), text


def test_moe_full_precision_output(dg):
    cases = synth.moe_experts(E=8, M=1, K=512, N=4096, seed=108, out_dtype=F32)
    got, _ = check_grouped(dg, cases)
    # literal bound on the FP32 result: the accumulation alone within 1e-4 * S
    for c, C in zip(cases, got):
        ref = oracle.ref_gemm(c.A, c.B)
        assert oracle.compare(C, ref, "f32", 1e-4, literal=True).ok


# ---------------------------------------------------------------- the grouped matrix-core launch

def _prefill_experts(tokens, K=512, N=4096, seed=300, b_layout="row", dtype=BF16, out=BF16):
    """One token block [M_e, K] and one weight [K, N] per expert (an MoE layer
    after routing, with M_e tokens sent to expert e)."""
    return [synth.gemm_case(M, N, K, dtype, out, seed=seed + e, b_layout=b_layout, name=f"e{e}")
            for e, M in enumerate(tokens)]


def test_moe_prefill_experts_in_one_launch(dg):
    cases = _prefill_experts([64, 32, 128, 17, 64, 96, 40, 64])
    _, text = check_grouped(dg, cases)
    assert text.count("| mfma tile=") == 1 and "groups=0,1,2,3,4,5,6,7" in text and text.endswith("solo="), text


def test_mfma_batches_by_configuration_and_count(dg):
    # two B storage orders (two launches), 20 groups of one order (two launches
    # of at most 16), a K that the direct kernel cannot take (alone), FP32 C,
    # alpha and beta
    cases = _prefill_experts([48] * 20, K=256, N=1024, seed=400, out=F32)
    cases += _prefill_experts([96, 33, 70], K=384, N=640, seed=500, b_layout="col", out=F32)
    cases += [synth.gemm_case(40, 512, 200, BF16, F32, seed=600, name="k200")]
    for c in cases:
        c.C.copy_(synth.to_dtype(synth.draw(synth.rng(7), tuple(c.C.shape), "normal"), F32))
    _, text = check_grouped(dg, cases, alpha=0.75, beta=-0.5)
    assert text.count("| mfma tile=") == 3 and "b=KMAJ" in text and "b=MNMAJ" in text, text
    assert text.endswith("solo=23"), text


def test_mfma_batch_f16_and_bitwise_repeat(dg):
    cases = _prefill_experts([16, 200, 64, 129], K=1024, N=2048, seed=700, dtype=F16, out=F32)
    a, text = run_grouped(dg, cases)
    b, _ = run_grouped(dg, cases)
    assert "| mfma tile=" in text, text
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    check_grouped(dg, cases)
