"""GPU parity: the HIP library (through its C ABI) against the FP64 oracle.

Tolerance (written here and in oracle/compare.py): |C - C_ref| <= rtol * S
+ 4*2^-24*(|alpha|*S + |beta*C_in|) + 0.5*ulp_out(|C_ref| + rtol*S), with
S = sum_k |a_ik * b_kj|, rtol = 1e-4 for FP16/BF16 and 1e-3 for FP8.  Results
stored as FP32 are also checked against the bare rtol * S.  Integer-valued
inputs must match bitwise.
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
    m.lib()   # raises if the library is missing: there is no fallback
    return m


def run_case(dg, case: synth.Case) -> synth.Case:
    d = case.to(DEV)
    if case.fp8:
        dg.gemm_fp8(d.A, d.A_scale, d.B, d.B_scale, d.C, case.alpha, case.beta)
    else:
        dg.gemm(d.A, d.B, d.C, case.alpha, case.beta)
    torch.cuda.synchronize()
    return d


def check(dg, case: synth.Case, rows=None, literal=False, expect_bitwise=False):
    print(f"[parity] {case.name} M,N,K={case.mnk} fp8={case.fp8} alpha={case.alpha} beta={case.beta}",
          flush=True)
    ref = oracle.ref_gemm(case.A, case.B, case.C if case.beta != 0 else None, case.alpha, case.beta,
                          rows=rows, A_scale=case.A_scale, B_scale=case.B_scale)
    d = run_case(dg, case)
    got = d.C.detach().cpu()
    if got.dim() > 2:
        got = got.reshape(-1, got.shape[-1])
    got = got[torch.as_tensor(ref.rows)]
    fmt = oracle.fmt_of(case.C.dtype)
    rep = oracle.compare(got, ref, fmt, case.rtol, literal=literal)
    print(f"[parity] {case.name}: {rep}", flush=True)
    assert rep.ok, str(rep)
    if expect_bitwise:
        assert rep.bitwise, str(rep)
    return rep, d


# ---------------------------------------------------------------- small shapes, every path

SHAPES = [(1, 1, 1), (2, 3, 7), (7, 17, 33), (16, 16, 16), (17, 31, 63), (33, 65, 127),
          (64, 64, 64), (65, 129, 255), (128, 128, 256), (129, 257, 129), (255, 200, 320),
          (8, 1000, 777), (1, 300, 4096), (5, 129, 1000)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", [F16, BF16], ids=["f16", "bf16"])
def test_small_row_major(dg, shape, dtype):
    M, N, K = shape
    c = synth.gemm_case(M, N, K, dtype, torch.float32, seed=M * 7 + N * 3 + K)
    check(dg, c)


@pytest.mark.parametrize("layouts", [("row", "col"), ("col", "row"), ("col", "col"), ("pad", "pad")],
                         ids=lambda l: "-".join(l))
@pytest.mark.parametrize("shape", [(3, 70, 130), (96, 160, 200), (300, 257, 192), (256, 512, 512)],
                         ids=lambda s: "x".join(map(str, s)))
def test_layouts(dg, layouts, shape):
    M, N, K = shape
    c = synth.gemm_case(M, N, K, BF16, torch.bfloat16, seed=11 + M, a_layout=layouts[0],
                        b_layout=layouts[1])
    check(dg, c)


@pytest.mark.parametrize("out", [torch.float32, F16, BF16], ids=["f32", "f16", "bf16"])
@pytest.mark.parametrize("ab", [(1.0, 0.0), (-0.5, 2.0), (2.0, -1.0), (0.0, 0.75), (0.0, 0.0)])
def test_alpha_beta_and_output_dtypes(dg, out, ab):
    alpha, beta = ab
    c = synth.gemm_case(70, 90, 150, F16, out, seed=5, alpha=alpha, beta=beta, c_layout="pad")
    if alpha == 0.0:   # A and B must not be read at all
        c.A.fill_(float("nan"))
        c.B.fill_(float("nan"))
    check(dg, c)


def test_k_zero_is_beta_c(dg):
    C = synth.to_dtype(synth.draw(synth.rng(3), (20, 30), "normal"), torch.float32)
    c = synth.Case("k0", torch.zeros(20, 0, dtype=BF16), torch.zeros(0, 30, dtype=BF16), C, 1.0, 0.5)
    check(dg, c)


@pytest.mark.parametrize("shape", [(1, 16, 128), (3, 200, 300), (64, 256, 512), (130, 300, 260),
                                   (256, 256, 1024)], ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("b_layout", ["row", "col"])
def test_fp8_small(dg, shape, b_layout):
    M, N, K = shape
    c = synth.fp8_case(M, N, K, seed=M + N + K, b_layout=b_layout, out_dtype=torch.float32)
    check(dg, c, literal=True)


def test_fp8_alpha_beta_bf16_out(dg):
    c = synth.fp8_case(100, 260, 384, seed=9, alpha=0.5, beta=-1.0)
    check(dg, c)


# ---------------------------------------------------------------- exactness, determinism, canaries

@pytest.mark.parametrize("kind", ["skinny", "mfma16", "fp8", "splitk"])
def test_integer_inputs_bitwise(dg, kind):
    g = synth.rng(77)
    if kind == "fp8":
        M, N, K = 130, 256, 1024
        A = synth.to_dtype(synth.draw(g, (M, K), "int", 8), torch.float32).to(E4M3)
        B = synth.to_dtype(synth.draw(g, (K, N), "int", 8), torch.float32).to(E4M3)
        c = synth.Case("int_fp8", A, B, torch.zeros(M, N), 1.0, 0.0,
                       torch.ones(M, K // 128), torch.ones(K // 128, N // 128), rtol=1e-3)
    else:
        M, N, K = {"skinny": (4, 1000, 4096), "mfma16": (256, 256, 4096), "splitk": (64, 512, 4096)}[kind]
        A = synth.to_dtype(synth.draw(g, (M, K), "int", 8), BF16)
        B = synth.to_dtype(synth.draw(g, (K, N), "int", 8), BF16)
        c = synth.Case("int_" + kind, A, B, torch.zeros(M, N), 1.0, 0.0)
    check(dg, c, expect_bitwise=True)
    # BF16 output must equal RNE_bf16 of the exact integer result
    cb = synth.Case(c.name + "_bf16", c.A, c.B, torch.zeros(M, N, dtype=BF16), 1.0, 0.0, c.A_scale,
                    c.B_scale, c.rtol)
    check(dg, cb, expect_bitwise=True)


@pytest.mark.parametrize("k_sa", [(512, "row"), (1536, "row"), (640, "row"), (1536, "col")],
                         ids=lambda v: f"K{v[0]}-SA{v[1]}")
def test_fp8_256x256_integer_bitwise(dg, k_sa):
    # The FP8 256x256 tile (loader waves, promotion in registers): integer-valued
    # codes with power-of-two scales, drawn per row and K block, give exact sums,
    # so every element of C is bitwise the oracle's and a scale taken from the
    # wrong row or K block shows.  Row scales are loaded 4 K blocks per load
    # where each row's scales are contiguous and K is a multiple of 4 blocks
    # (K 512: one group of 4 blocks; 1536: three, the two buffers reused), else
    # one block per tile: K 640 (5 blocks), or column-major scales.
    K, sa_layout = k_sa
    g = synth.rng(79)
    M, N = 4096, 4096
    A = synth.to_dtype(synth.draw(g, (M, K), "int", 8), torch.float32).to(E4M3)
    B = synth.to_dtype(synth.draw(g, (K, N), "int", 8), torch.float32).to(E4M3)
    sa = torch.from_numpy(np.exp2(g.integers(-2, 3, size=(M, K // 128)))).float()
    sb = torch.from_numpy(np.exp2(g.integers(-2, 3, size=(K // 128, N // 128)))).float()
    if sa_layout == "col":
        sa = sa.t().contiguous().t()
    c = synth.Case("int_fp8_256", A, B, torch.zeros(M, N), 1.0, 0.0, sa, sb, rtol=1e-3)
    tile, text = _plan_field(dg, c, "tile")
    assert tile == "256x256", text
    check(dg, c, expect_bitwise=True)     # the whole C


def test_fp8_256x256_ragged_m_grouped_scales(dg):
    # The FP8 256x256 tile with an M edge inside its last tile row (4000 = 15 x 256
    # + 160) and row scales loaded 4 K blocks at a time (K 1024: two groups): the
    # rows past M load the last row's scales, and their products are never stored.
    c = synth.fp8_case(4000, 7168, 1024, seed=4001, out_dtype=torch.float32, beta=0.5)
    tile, text = _plan_field(dg, c, "tile")
    assert tile == "256x256", text
    check(dg, c, literal=True)


@pytest.mark.parametrize("mnk", [(128, 1024, 1536), (4096, 128, 2560), (128, 1024, 640)],
                         ids=lambda v: "x".join(map(str, v)))
def test_fp8_64x128_integer_bitwise(dg, mnk):
    # The FP8 64x128 tile (six-stage ring) with its K split: integer-valued codes
    # and power-of-two scales per row and K block, so every element of C is
    # bitwise the oracle's.  128 x 1024 x 1536: 12 K blocks in 4 pieces of 3,
    # most starting inside a group of 4 blocks, whose row scales the fills of
    # the group before load a quarter at a time; 4096 x 128 x 2560 (a tall strip):
    # 20 blocks in 2 pieces of 10; 128 x 1024 x 640: 5 blocks, one row scale per
    # tile.
    M, N, K = mnk
    g = synth.rng(83 + K)
    A = synth.to_dtype(synth.draw(g, (M, K), "int", 8), torch.float32).to(E4M3)
    B = synth.to_dtype(synth.draw(g, (K, N), "int", 8), torch.float32).to(E4M3)
    sa = torch.from_numpy(np.exp2(g.integers(-3, 4, size=(M, K // 128)))).float()
    sb = torch.from_numpy(np.exp2(g.integers(-2, 3, size=(K // 128, N // 128)))).float()
    c = synth.Case("int_fp8_64x128", A, B, torch.full((M, N), float("nan")), 1.0, 0.0, sa, sb, rtol=1e-3)
    tile, text = _plan_field(dg, c, "tile")
    assert tile == "64x128" and "splits=1 " not in text, text
    check(dg, c, expect_bitwise=True)


@pytest.mark.parametrize("kind", ["fp8", "bf16"])
def test_column_split_integer_bitwise(dg, kind):
    # A column split: the first 4096 columns on 256x256 tiles (one whole wave of
    # 256 CUs), the last 128 (FP8) or 64 (BF16) columns as a strip of their own,
    # launched after it on the same workspace.  Integer-valued inputs (with
    # power-of-two scales per block for FP8) give exact sums: every element of C
    # bitwise the oracle's, so a column of either part computed, scaled or
    # stored in the wrong place would show.
    g = synth.rng(91 + len(kind))
    M, K = 4096, 512
    N = 4224 if kind == "fp8" else 4160
    if kind == "fp8":
        A = synth.to_dtype(synth.draw(g, (M, K), "int", 8), torch.float32).to(E4M3)
        B = synth.to_dtype(synth.draw(g, (K, N), "int", 8), torch.float32).to(E4M3)
        sa = torch.from_numpy(np.exp2(g.integers(-2, 3, size=(M, K // 128)))).float()
        sb = torch.from_numpy(np.exp2(g.integers(-2, 3, size=(K // 128, -(-N // 128))))).float()
        c = synth.Case("int_split_fp8", A, B, torch.full((M, N), float("nan")), 1.0, 0.0, sa, sb, rtol=1e-3)
    else:
        A = synth.to_dtype(synth.draw(g, (M, K), "int", 8), BF16)
        B = synth.to_dtype(synth.draw(g, (K, N), "int", 8), BF16)
        c = synth.Case("int_split_bf16", A, B, torch.full((M, N), float("nan")), 1.0, 0.0)
    path, text = _plan_field(dg, c, "path")
    assert path == "split_n" and "n1=4096" in text, text
    check(dg, c, expect_bitwise=True)


def test_column_split_alpha_beta(dg):
    # The same split with alpha, beta and a strided C (every part reads and
    # writes its own columns of C_in / C through the view's strides).
    c = synth.gemm_case(4096, 4160, 128, BF16, torch.float32, seed=93, alpha=0.5, beta=-1.5, c_layout="pad")
    path, text = _plan_field(dg, c, "path")
    assert path == "split_n", text
    check(dg, c, literal=True)


def test_bf16_256x256_integer_bitwise_whole_c(dg):
    # The BF16 256x256 tile (loader waves): integer-valued inputs, every element
    # of C compared, FP32 and BF16 outputs bitwise equal to the oracle's.
    g = synth.rng(80)
    M, N, K = 4096, 4096, 512
    A = synth.to_dtype(synth.draw(g, (M, K), "int", 8), BF16)
    B = synth.to_dtype(synth.draw(g, (K, N), "int", 8), BF16)
    for out in (torch.float32, BF16):
        c = synth.Case("int_bf16_256", A, B, torch.full((M, N), float("nan"), dtype=out), 1.0, 0.0)
        tile, text = _plan_field(dg, c, "tile")
        assert tile == "256x256", text
        check(dg, c, expect_bitwise=True)


def test_run_twice_bitwise(dg):
    for case in [synth.gemm_case(64, 512, 2048, F16, torch.float32, seed=1),      # split-K
                 synth.gemm_case(1, 4096, 4096, BF16, BF16, seed=2),              # skinny
                 synth.fp8_case(256, 512, 1024, seed=3)]:
        d1 = run_case(dg, case).C.cpu()
        d2 = run_case(dg, case).C.cpu()
        assert torch.equal(d1.view(torch.uint8) if d1.dtype == E4M3 else d1, d2), case.name


def test_output_canaries_untouched(dg):
    # C is a window of a larger buffer; everything outside the window must keep its bits.
    M, N, K = 100, 150, 200
    big = torch.full((M + 8, N + 40), 12345.0, dtype=torch.float32)
    Cwin = big[4:4 + M, 16:16 + N]
    c = synth.gemm_case(M, N, K, BF16, torch.float32, seed=8)
    c = synth.Case("canary", c.A, c.B, Cwin, 1.0, 0.0)
    d = c.to(DEV)
    dg.gemm(d.A, d.B, d.C)
    torch.cuda.synchronize()
    full = torch.empty(0, dtype=torch.float32, device=DEV).set_(d.C.untyped_storage()).view(M + 8, N + 40).cpu()
    mask = torch.ones_like(full, dtype=torch.bool)
    mask[4:4 + M, 16:16 + N] = False
    assert (full[mask] == 12345.0).all()


# ---------------------------------------------------------------- the workloads at full size

@pytest.mark.parametrize("name", synth.CONFIGS)
def test_workload_full_size(dg, name):
    # Every element of C against the oracle.  The workloads that already store
    # FP32 (the FP16 64x512x512 and 64x4096x4096 problems) must also meet the
    # bare rtol * sum|a*b| bound.
    case = synth.config(name)
    rep, d = check(dg, case, literal=case.C.dtype == torch.float32)
    C = d.C.float()
    assert torch.isfinite(C).all(), "non-finite output (NaN padding or garbage read?)"


@pytest.mark.parametrize("name", ["c2a", "c2b", "c4", "c5_128", "c5_4096"])
def test_workload_fp32_c_literal_bound(dg, name):
    # The same kernels with an FP32 C view: the bare rtol * sum|a*b| bound must
    # hold on every element.
    case = synth.config(name)
    M, N, _ = case.mnk
    c = synth.Case(name + "_f32", case.A, case.B, torch.full((M, N), float("nan")), case.alpha,
                   case.beta, case.A_scale, case.B_scale, case.rtol)
    check(dg, c, literal=True)


# ---------------------------------------------------------------- the streaming (skinny) kernels

def _plan_field(dg, case, name):
    import re
    d = case.to(DEV)
    text = dg.plan(d.A, d.B, d.C, case.alpha, case.beta, d.A_scale, d.B_scale)
    m = re.search(r"\b" + name + r"=(\S+)", text)
    return m.group(1) if m else None, text


@pytest.mark.parametrize("nk", [(64, 8), (1000, 777), (4104, 4096), (200, 17000), (14336, 520), (96, 4096)],
                         ids=lambda t: f"N{t[0]}K{t[1]}")
@pytest.mark.parametrize("M", [1, 2, 3, 5, 8])
def test_skinny_bn(dg, M, nk):
    # B row-major (N-contiguous): ragged slabs, K tails, several LDS chunks of A,
    # and the split-K fallback when there are few column slabs.
    N, K = nk
    dtype = BF16 if (M + N) % 2 else F16
    c = synth.gemm_case(M, N, K, dtype, BF16 if M % 2 else torch.float32, seed=M * 31 + N + K,
                        alpha=1.0 if M != 3 else -0.5, beta=0.0 if M != 5 else 1.0)
    kind, text = _plan_field(dg, c, "kind")
    assert "path=skinny" in text and kind == "BN", text
    # A is staged with 16-byte loads exactly when its rows allow it (K % 8 == 0)
    assert _plan_field(dg, c, "a_vec")[0] == ("1" if K % 8 == 0 else "0"), text
    check(dg, c)


@pytest.mark.parametrize("mnk", [(1, 14003, 2048), (1, 20003, 4096), (4, 14003, 4096), (4, 9003, 1000), (8, 5003, 1000),
                                 (2, 1003, 4096), (3, 301, 777)],
                         ids=lambda t: "x".join(map(str, t)))
def test_skinny_bn_ragged_slabs(dg, mnk):
    # N not a multiple of 8, B rows padded to a 16-byte pitch with NaN: in the
    # last column slab one lane's 8 columns straddle N (element loads), the lanes
    # past N and past the slab width read nothing of B, and any read of the
    # padding would surface as NaN.  Slab widths from 64 to 512 columns, the
    # 32-lane and the 64-lane row layouts (320 and 512 columns), with and
    # without K splits.
    M, N, K = mnk
    c = synth.gemm_case(M, N, K, BF16, torch.float32, seed=M + N + K, b_layout="pad", pad=(8 - N % 8) % 8 + 8)
    kind, text = _plan_field(dg, c, "kind")
    assert "path=skinny" in text and kind == "BN", text
    cols = int(_plan_field(dg, c, "cols")[0])
    assert 64 <= cols <= 512 and cols % 8 == 0, text
    print(f"[skinny] {M}x{N}x{K} cols={cols} splits={_plan_field(dg, c, 'splits')[0]}", flush=True)
    check(dg, c)


@pytest.mark.parametrize("nk", [(1, 8), (128, 4096), (129, 1000), (1500, 4104), (7, 9000)],
                         ids=lambda t: f"N{t[0]}K{t[1]}")
@pytest.mark.parametrize("M", [1, 3, 8])
def test_skinny_bk(dg, M, nk):
    # B = K_cache^T (K-contiguous columns), as in the query x key-cache product.
    N, K = nk
    c = synth.gemm_case(M, N, K, BF16, BF16, seed=M * 7 + N + K, b_layout="col")
    kind, text = _plan_field(dg, c, "kind")
    assert "path=skinny" in text and kind == "BK", text
    check(dg, c)


# ---------------------------------------------------------------- the direct-to-LDS matrix-core kernels

@pytest.mark.parametrize("shape", [(1000, 4104, 512), (4000, 4096, 256)], ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("layouts", [("row", "row"), ("row", "col"), ("col", "row"), ("col", "col")],
                         ids=lambda l: "A" + l[0] + "-B" + l[1])
@pytest.mark.parametrize("kind", ["f16", "bf16", "fp8"])
def test_dtl_tiles(dg, kind, layouts, shape):
    # 128x128 and 256x256 macro tiles with M and N edges that cut through a tile,
    # every operand storage order, every input type; K a whole number of tiles.
    M, N, K = shape
    if kind == "fp8" and M == 1000:   # 1-byte elements: 16-element chunks need M, N multiples of 16
        M, N = 1008, 4112
    seed = M + N + K + len(kind) + 3 * len(layouts[0]) + len(layouts[1])
    if kind == "fp8":
        c = synth.fp8_case(M, N, K, seed=seed, a_layout=layouts[0], b_layout=layouts[1],
                           out_dtype=torch.float32, beta=0.5)
    else:
        c = synth.gemm_case(M, N, K, F16 if kind == "f16" else BF16, BF16, seed=seed,
                            a_layout=layouts[0], b_layout=layouts[1], alpha=1.5)
    dtl, text = _plan_field(dg, c, "dtl")
    assert dtl == "1", text
    check(dg, c)


@pytest.mark.parametrize("out", [BF16, torch.float32, F16], ids=["bf16", "f32", "f16"])
def test_dtl_256_row_stores(dg, out):
    # The 256x256 tile's epilogue: an M edge that cuts a tile, an N edge,
    # beta != 0 (C_in read), every output type.
    M, N, K = 4000, 4360, 256
    c = synth.gemm_case(M, N, K, F16 if out == F16 else BF16, out, seed=811 + out.itemsize,
                        alpha=1.25, beta=0.5)
    tile, text = _plan_field(dg, c, "tile")
    assert tile == "256x256", text
    check(dg, c)


def test_dtl_256_row_stores_misaligned_window(dg):
    # C is a window at column offset 1 of a wider buffer (no row is 8-byte
    # aligned): every element lands in the window, nothing outside it is touched.
    M, N, K = 4096, 4096, 256
    big = torch.full((M + 2, N + 8), 777.0, dtype=BF16)
    Cwin = big[1:1 + M, 1:1 + N]
    c0 = synth.gemm_case(M, N, K, BF16, BF16, seed=812)
    c = synth.Case("win256", c0.A, c0.B, Cwin, 1.0, 0.0)
    tile, text = _plan_field(dg, c, "tile")
    assert tile == "256x256", text
    rep, d = check(dg, c)
    full = torch.empty(0, dtype=BF16, device=DEV).set_(d.C.untyped_storage()).view(M + 2, N + 8).cpu()
    mask = torch.ones_like(full, dtype=torch.bool)
    mask[1:1 + M, 1:1 + N] = False
    assert (full[mask] == 777.0).all()


# ---------------------------------------------------------------- the split tail of the last wave

TAIL_CASES = [
    ("fp8", 2512, 3312, 2048, "row"),      # 520 tiles of 128x128: 512 whole, 8 split in 2
    ("fp8", 2512, 3312, 2048, "col"),
    ("fp8", 2512, 3312, 2560, "row"),      # 8 split in 2 of 10 K blocks: the second piece starts mid-group
    ("bf16", 2900, 2904, 2048, "row"),     # 529 tiles: 512 whole, 17 split in 4, ragged edges
    ("f16", 2900, 2904, 1024, "row"),      # 17 split in 2, beta = 1 and an FP32 C
]


@pytest.mark.parametrize("tc", TAIL_CASES, ids=lambda t: f"{t[0]}-{t[1]}x{t[2]}x{t[3]}-B{t[4]}")
def test_tail_split(dg, tc):
    kind, M, N, K, bl = tc
    if kind == "fp8":
        c = synth.fp8_case(M, N, K, seed=M + K, b_layout=bl, out_dtype=torch.float32, beta=0.5)
    else:
        c = synth.gemm_case(M, N, K, F16 if kind == "f16" else BF16, torch.float32 if kind == "f16" else BF16,
                            seed=N + K, b_layout=bl, beta=1.0 if kind == "f16" else 0.0)
    dp, text = _plan_field(dg, c, "dp_tiles")
    assert int(dp) == 512 and "splits=1 " not in text, text
    check(dg, c)     # the whole C: the whole tiles and the split ones


def test_tail_split_integer_bitwise_and_repeatable(dg):
    g = synth.rng(91)
    M, N, K = 2512, 3312, 2048
    A = synth.to_dtype(synth.draw(g, (M, K), "int", 8), torch.float32).to(E4M3)
    B = synth.to_dtype(synth.draw(g, (K, N), "int", 8), torch.float32).to(E4M3)
    c = synth.Case("int_tail", A, B, torch.zeros(M, N), 1.0, 0.0, torch.ones(M, K // 128),
                   torch.ones(K // 128, -(-N // 128)), rtol=1e-3)
    assert int(_plan_field(dg, c, "dp_tiles")[0]) == 512
    check(dg, c, expect_bitwise=True)
    d1 = run_case(dg, c).C.cpu()
    d2 = run_case(dg, c).C.cpu()
    assert torch.equal(d1, d2)


def test_workload_c5_tail(dg):
    # FP8 4096 x 4224 x 4096: a column split, 256 whole 256x256 tiles (one wave),
    # then the 4096 x 128 strip with its K split
    case = synth.config("c5_tail")
    path, text = _plan_field(dg, case, "path")
    assert path == "split_n" and "n1=4096" in text, text
    check(dg, case)     # the whole C: both parts
