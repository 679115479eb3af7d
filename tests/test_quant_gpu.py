"""GPU parity of the FP8 quantizer (dg_quant_fp8) against the oracle
(oracle/quant.py): codes and scales must match bit for bit (the kernel and the
oracle take every rounding decision in FP32 with IEEE operations, then the same
round-to-nearest-even onto E4M3)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import quant as oq
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOKEN, BLOCK = 0, 1


@pytest.fixture(scope="module")
def dg():
    import dense_gemm_19_amd as m
    m.lib()   # raises if the library is missing: there is no fallback
    return m


def run(dg, x: torch.Tensor, mode: int, q_layout="row", s_layout="row"):
    M, K = x.shape
    srows = M if mode == TOKEN else (M + 127) // 128
    scols = (K + 127) // 128
    xd = x.to(DEV)
    q = torch.empty((K, M) if q_layout == "col" else (M, K), dtype=torch.float8_e4m3fn, device=DEV)
    s = torch.empty((scols, srows) if s_layout == "col" else (srows, scols), dtype=torch.float32, device=DEV)
    q = q.t() if q_layout == "col" else q
    s = s.t() if s_layout == "col" else s
    q.view(torch.uint8).fill_(0x7F)   # NaN codes: anything left unwritten shows up
    s.fill_(float("nan"))
    dg.quant_fp8(xd, q, s, mode)
    torch.cuda.synchronize()
    return q.cpu().contiguous().view(torch.uint8).numpy(), s.cpu().contiguous().numpy()


def check(dg, x, mode, **kw):
    print(f"[quant] shape={tuple(x.shape)} dtype={x.dtype} mode={mode} {kw}", flush=True)
    q, s = run(dg, x, mode, **kw)
    rq, rs = oq.quant_tokens(x) if mode == TOKEN else oq.quant_blocks(x)
    sbad = np.argwhere(s.view(np.uint32) != rs.view(np.uint32))
    assert sbad.size == 0, (f"{len(sbad)} scales differ, first at {sbad[0]}: {s[tuple(sbad[0])]!r} vs "
                            f"{rs[tuple(sbad[0])]!r}")
    bad = np.argwhere(q != rq)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[0]}: {q[tuple(bad[0])]:#x} vs {rq[tuple(bad[0])]:#x}"


SHAPES = [(1, 1), (1, 4096), (3, 130), (7, 127), (128, 128), (129, 257), (300, 1000), (1000, 4104)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16], ids=["f32", "f16", "bf16"])
@pytest.mark.parametrize("mode", [TOKEN, BLOCK], ids=["token", "block"])
def test_shapes(dg, shape, dtype, mode):
    g = synth.rng(shape[0] * 31 + shape[1] + mode)
    x = synth.to_dtype(synth.draw(g, shape, "normal", 3.0), dtype)
    check(dg, x, mode)


@pytest.mark.parametrize("mode", [TOKEN, BLOCK], ids=["token", "block"])
def test_strided_views(dg, mode):
    # X column-major, Q column-major, S transposed: every access through byte strides
    g = synth.rng(11 + mode)
    x = synth.place(synth.to_dtype(synth.draw(g, (200, 300), "normal", 1.0), torch.bfloat16), "col")
    check(dg, x, mode, q_layout="col", s_layout="col")
    # X with a padded row pitch (odd element offset: the element path)
    xp = synth.place(synth.to_dtype(synth.draw(g, (130, 260), "normal", 1.0), torch.float16), "pad", pad=3)
    check(dg, xp, mode)
    # K >= 512 (token scales: 512-column tiles) through the same strided views
    x = synth.place(synth.to_dtype(synth.draw(g, (40, 1100), "normal", 1.0), torch.bfloat16), "col")
    check(dg, x, mode, q_layout="col", s_layout="col")
    xp = synth.place(synth.to_dtype(synth.draw(g, (37, 1031), "normal", 1.0), torch.float16), "pad", pad=3)
    check(dg, xp, mode)


def test_special_values(dg):
    # zero blocks, a lone peak, tiny values in the subnormal range of E4M3, -0
    x = torch.zeros(130, 260, dtype=torch.float32)
    x[1, 5] = -3.0
    x[2, 0:128] = torch.linspace(-1e-6, 1e-6, 128)
    x[3, 130:258] = torch.logspace(-30, 3, 128)
    x[4, 7] = -0.0
    for mode in (TOKEN, BLOCK):
        check(dg, x, mode)


def test_every_e4m3_midpoint(dg):
    # a block holding 448 has s = 448 / 448 = 1 exactly, so x / s = x: put every
    # midpoint between adjacent E4M3 values, and the FP32 values on either side
    # of it, through the kernel's rounding (ties go to the even code)
    vals = [oq.e4m3_value(c) for c in range(0x7F)]
    mids = np.array([(a + b) / 2 for a, b in zip(vals[:-1], vals[1:])], dtype=np.float32)
    pts = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(448))])
    pts = np.concatenate([pts, -pts]).astype(np.float32)
    rows = -(-pts.size // 127)
    body = np.zeros(rows * 127, dtype=np.float32)
    body[: pts.size] = pts
    x = np.zeros((rows, 128), dtype=np.float32)
    x[:, :127] = body.reshape(rows, 127)
    x[:, 127] = 448.0   # every row block holds 448: s = 1 per token and per block
    assert np.isin(pts, x).all()
    check(dg, torch.from_numpy(x), TOKEN)
    check(dg, torch.from_numpy(x), BLOCK)


@pytest.mark.parametrize("which", ["a_token_4096x4096", "b_block_4096x7168"])
def test_workload_sizes(dg, which):
    # the producers of the 4096x7168x4096 FP8 GEMM's operands, at full size
    g = synth.rng(106 if which.startswith("a") else 107)
    shape = (4096, 4096) if which.startswith("a") else (4096, 7168)
    x = synth.to_dtype(synth.draw(g, shape, "normal", 1.0), torch.bfloat16)
    check(dg, x, TOKEN if which.startswith("a") else BLOCK)


def test_quantize_then_gemm(dg):
    # device-quantized operands feed dg_gemm_fp8; the result is checked against
    # the FP64 oracle on the oracle's own codes and scales (equal by the tests above)
    M, N, K = 256, 384, 512
    g = synth.rng(5)
    a = synth.to_dtype(synth.draw(g, (M, K), "normal", 1.0), torch.bfloat16)
    b = synth.to_dtype(synth.draw(g, (K, N), "normal", 1.0), torch.bfloat16)
    qa, sa = run(dg, a, TOKEN)
    qb, sb = run(dg, b, BLOCK)
    qa_t = torch.from_numpy(qa).view(torch.float8_e4m3fn)
    qb_t = torch.from_numpy(qb).view(torch.float8_e4m3fn)
    c = torch.empty(M, N, dtype=torch.float32, device=DEV)
    dg.gemm_fp8(qa_t.to(DEV), torch.from_numpy(sa).to(DEV), qb_t.to(DEV), torch.from_numpy(sb).to(DEV), c)
    torch.cuda.synchronize()
    ra, rsa = oq.quant_tokens(a)
    rb, rsb = oq.quant_blocks(b)
    ref = oracle.ref_gemm(torch.from_numpy(ra).view(torch.float8_e4m3fn), torch.from_numpy(rb).view(torch.float8_e4m3fn),
                          None, 1.0, 0.0, A_scale=torch.from_numpy(rsa), B_scale=torch.from_numpy(rsb))
    rep = oracle.compare(c.cpu(), ref, "f32", 1e-3)
    assert rep.ok, str(rep)
