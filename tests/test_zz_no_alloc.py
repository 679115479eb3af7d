"""GPU: dg_gemm_noalloc, the entry point for callers that cannot allocate.

It runs the plan dg_gemm / dg_gemm_fp8 would run, on the library's fixed
split-K scratch instead of the stream's workspace.  Through the C ABI, on two
calls in a row (the second smaller, so stale partials and counters of the first
would show), its output must equal dg_gemm's bit for bit and the oracle's
within the stated bound; a problem whose plan needs more scratch than the fixed
buffer holds is refused with DG_ERR_SCRATCH and C is left untouched.
"""
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
F16, BF16 = torch.float16, torch.bfloat16


@pytest.fixture(scope="module")
def dg():
    import dense_gemm_19_amd as m
    m.lib()
    return m


def _both(dg, c):
    """(noalloc result, dg_gemm result) of case c, each into a fresh copy of C."""
    d = c.to(DEV)
    c1, c2 = d.C.clone(), d.C.clone()
    print(f"[noalloc] {c.name}: {dg.plan(d.A, d.B, d.C, c.alpha, c.beta, d.A_scale, d.B_scale)}", flush=True)
    dg.gemm_noalloc(d.A, d.B, c1, c.alpha, c.beta, d.A_scale, d.B_scale)
    if c.fp8:
        dg.gemm_fp8(d.A, d.A_scale, d.B, d.B_scale, c2, c.alpha, c.beta)
    else:
        dg.gemm(d.A, d.B, c2, c.alpha, c.beta)
    torch.cuda.synchronize()
    return c1.cpu(), c2.cpu()


def _check(dg, c):
    got, want = _both(dg, c)
    ref = oracle.ref_gemm(c.A, c.B, c.C if c.beta != 0 else None, c.alpha, c.beta,
                          A_scale=c.A_scale, B_scale=c.B_scale)
    rep = oracle.compare(got, ref, oracle.fmt_of(c.C.dtype), c.rtol)
    print(f"[noalloc] {c.name}: {rep}", flush=True)
    assert rep.ok, str(rep)
    assert torch.equal(got, want), c.name


# Pairs (first, second smaller), each on a path that uses split-K scratch.
PAIRS = [
    ("mfma_splitk", lambda: synth.gemm_case(64, 4096, 4096, F16, torch.float32, seed=104, dist="normal",
                                            scale=0.02, beta=1.0, name="64x4096x4096 beta=1"),
     lambda: synth.gemm_case(64, 512, 512, F16, torch.float32, seed=101, name="64x512x512")),
    ("skinny_bn", lambda: synth.gemm_case(1, 14336, 4096, BF16, BF16, seed=102, name="1x14336x4096"),
     lambda: synth.gemm_case(3, 2048, 1024, BF16, BF16, seed=5, name="3x2048x1024")),
    ("fp8_splitk", lambda: synth.fp8_case(128, 7168, 4096, seed=106, name="fp8 128x7168x4096"),
     lambda: synth.fp8_case(64, 1024, 2048, seed=7, name="fp8 64x1024x2048")),
    ("general_splitk", lambda: synth.gemm_case(64, 2000, 4104, BF16, torch.float32, seed=9, name="64x2000x4104"),
     lambda: synth.gemm_case(20, 304, 1000, BF16, torch.float32, seed=10, name="20x304x1000")),
]


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: p[0])
def test_noalloc_matches_dg_gemm_twice(dg, pair):
    _, first, second = pair
    for make in (first, second):
        c = make()
        text = dg.plan(c.A, c.B, c.C, c.alpha, c.beta, c.A_scale, c.B_scale)
        assert "splits=1 " not in text, text     # the scratch is used
        _check(dg, c)


def test_noalloc_refuses_more_scratch_than_it_holds(dg, tmp_path):
    # A tuned plan may split K further than the fixed buffer allows: tune the
    # problem, rewrite its saved entry to ask for 64 K splits of the
    # register-staged kernel (33 pieces of 2 K tiles: 33 * 256 * 1024 * 4 bytes
    # of partials, more than the 16 MiB the buffer holds) and load it back.  dg_gemm_noalloc must refuse the call
    # with DG_ERR_SCRATCH and leave C untouched.
    c = synth.gemm_case(256, 1024, 4104, BF16, torch.float32, seed=11, name="256x1024x4104")
    d = c.to(DEV)
    dg.tune_clear()
    try:
        dg.tune(d.A, d.B, d.C)
        f = tmp_path / "tuned.txt"
        dg.tune_save(str(f))
        lines = [l for l in f.read_text().splitlines() if l.startswith("dgtune1")]
        assert len(lines) == 1, lines
        fields = lines[0].split()
        fields[-4:] = ["2", "-1", "64", "-1"]
        f.write_text(" ".join(fields) + "\n")
        dg.tune_clear()
        dg.tune_load(str(f))
        text = dg.plan(d.A, d.B, d.C)
        ws = int(text.split(" ws=")[1].split(" ")[0])
        assert ws > 16 << 20, text
        d.C.fill_(float("nan"))
        with pytest.raises(dg.DGError) as e:
            dg.gemm_noalloc(d.A, d.B, d.C)
        assert "DG_ERR_SCRATCH" in str(e.value)
        torch.cuda.synchronize()
        assert torch.isnan(d.C).all()      # untouched
    finally:
        dg.tune_clear()
