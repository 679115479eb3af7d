"""The C-ABI boundary on the CPU: the library loads, exports every declared
symbol, and validates views exactly as include/dg.h documents (dg_gemm_plan
needs no GPU).  Fake pointer values are fine: nothing is dereferenced."""
import math
import os
import re

import pytest
import torch

import dense_gemm_19_amd as dg
from dense_gemm_19_amd import DG_BF16, DG_F16, DG_F32, DG_F8E4M3, make_view

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BASE = 0x7F0000000000   # a fake, 256-byte aligned device address


def declared_symbols():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        text = open(os.path.join(ROOT, "include", h)).read()
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(dg_\w+)\s*\(", text, re.M))
    return sorted(names)


def test_exports_every_declared_symbol():
    names = declared_symbols()
    assert {"dg_gemm", "dg_gemm_fp8", "dg_gemm_plan", "dg_gemm_fp8_plan", "dg_status_str",
            "dg_gemm_epilogue", "dg_gemm_fp8_epilogue",
            "dg_version", "dg_calib_mfma", "dg_calib_read", "dg_calib_launch"} <= set(names)
    L = dg.lib()
    for n in names:
        assert hasattr(L, n), n
    assert dg.version() == 10000
    assert dg.status_str(7) == "DG_ERR_ALIAS"
    assert dg.status_str(15) == "DG_ERR_SCRATCH"


def mat(ptr, rows, cols, rs, cs, dt=DG_BF16):
    return make_view(ptr, (rows, cols), (rs, cs), dt)


def plan(A, B, C, alpha=1.0, beta=0.0, SA=None, SB=None):
    return dg.plan_views(A, B, C, alpha, beta, SA, SB)


def ok_triplet(M=64, N=64, K=64):
    A = mat(BASE, M, K, 2 * K, 2)
    B = mat(BASE + 0x10000000, K, N, 2 * N, 2)
    C = mat(BASE + 0x20000000, M, N, 4 * N, 4, DG_F32)
    return A, B, C


def field(text, name):
    m = re.search(r"\b" + name + r"=(\S+)", text)
    return m.group(1) if m else None


def test_valid_plan():
    st, text = plan(*ok_triplet())
    assert st == 0, text
    assert "path=" in text


@pytest.mark.parametrize("case,expect", [
    ("ndim0", "DG_ERR_NDIM"), ("ndim5", "DG_ERR_NDIM"), ("neg_stride", "DG_ERR_STRIDE"),
    ("odd_stride", "DG_ERR_STRIDE"), ("null_ptr", "DG_ERR_NULL"), ("misaligned", "DG_ERR_MISALIGNED"),
    ("k_mismatch", "DG_ERR_SHAPE_MISMATCH"), ("m_mismatch", "DG_ERR_SHAPE_MISMATCH"),
    ("dtype_mix", "DG_ERR_DTYPE"), ("dtype_f32_in", "DG_ERR_DTYPE"), ("nan_alpha", "DG_ERR_NONFINITE_SCALAR"),
    ("inf_beta", "DG_ERR_NONFINITE_SCALAR"), ("alias", "DG_ERR_ALIAS"), ("c_stride0", "DG_ERR_STRIDE"),
    ("c_overlap_rows", "DG_ERR_STRIDE"), ("overflow", "DG_ERR_OVERFLOW"),
    ("unmergeable", "DG_ERR_UNSUPPORTED_VIEW"), ("null_view", "DG_ERR_NULL"),
])
def test_error_codes(case, expect):
    A, B, C = ok_triplet()
    alpha, beta = 1.0, 0.0
    if case == "ndim0":
        A = make_view(BASE, (), (), DG_BF16)
    elif case == "ndim5":
        A = make_view(BASE, (1, 1, 1, 64, 64), (2, 2, 2, 128, 2), DG_BF16)
        A.ndim = 5
    elif case == "neg_stride":
        A = mat(BASE, 64, 64, -128, 2)
    elif case == "odd_stride":
        A = mat(BASE, 64, 64, 129, 2)
    elif case == "null_ptr":
        A = mat(0, 64, 64, 128, 2)
    elif case == "misaligned":
        A = mat(BASE + 1, 64, 64, 128, 2)
    elif case == "k_mismatch":
        B = mat(BASE + 0x10000000, 65, 64, 128, 2)
    elif case == "m_mismatch":
        C = mat(BASE + 0x20000000, 63, 64, 256, 4, DG_F32)
    elif case == "dtype_mix":
        B = mat(BASE + 0x10000000, 64, 64, 128, 2, DG_F16)
    elif case == "dtype_f32_in":
        A = mat(BASE, 64, 64, 256, 4, DG_F32)
        B = mat(BASE + 0x10000000, 64, 64, 256, 4, DG_F32)
    elif case == "nan_alpha":
        alpha = math.nan
    elif case == "inf_beta":
        beta = math.inf
    elif case == "alias":
        C = mat(BASE + 64, 64, 64, 256, 4, DG_F32)
    elif case == "c_stride0":
        C = mat(BASE + 0x20000000, 64, 64, 0, 4, DG_F32)
    elif case == "c_overlap_rows":
        C = mat(BASE + 0x20000000, 64, 64, 8, 4, DG_F32)
    elif case == "overflow":
        A = mat(BASE, 2 ** 40, 64, 2 ** 40, 2)
    elif case == "unmergeable":
        A = make_view(BASE, (4, 16, 64), (4096, 128, 2), DG_BF16)   # 4*16 rows, pitch gap between dim 0 steps
    if case == "null_view":
        import ctypes
        buf = ctypes.create_string_buffer(256)
        st = dg.lib().dg_gemm_plan(None, ctypes.byref(B), ctypes.byref(C), 1.0, 0.0, buf, 256)
    else:
        st, _ = plan(A, B, C, alpha, beta)
    assert dg.STATUS[st] == expect


def test_fp8_scale_shapes_and_dtypes():
    M, N, K = 256, 384, 300
    A = mat(BASE, M, K, K, 1, DG_F8E4M3)
    B = mat(BASE + 0x1000000, K, N, N, 1, DG_F8E4M3)
    C = mat(BASE + 0x2000000, M, N, 2 * N, 2, DG_BF16)
    SA = mat(BASE + 0x3000000, M, 3, 12, 4, DG_F32)
    SB = mat(BASE + 0x4000000, 3, 3, 12, 4, DG_F32)
    assert plan(A, B, C, SA=SA, SB=SB)[0] == 0
    bad = mat(BASE + 0x3000000, M, 2, 8, 4, DG_F32)
    assert dg.STATUS[plan(A, B, C, SA=bad, SB=SB)[0]] == "DG_ERR_SHAPE_MISMATCH"
    bad16 = mat(BASE + 0x3000000, M, 3, 6, 2, DG_BF16)
    assert dg.STATUS[plan(A, B, C, SA=bad16, SB=SB)[0]] == "DG_ERR_DTYPE"
    alias = mat(BASE + 0x2000000 + 64, 3, 3, 12, 4, DG_F32)
    assert dg.STATUS[plan(A, B, C, SA=SA, SB=alias)[0]] == "DG_ERR_ALIAS"


def test_beyond_32bit_strides_are_accepted():
    # byte strides above 2^32 are legal (64-bit offsets throughout)
    A = mat(BASE, 4, 64, 2 ** 33, 2)
    B = mat(BASE + 2 ** 36, 64, 8, 16, 2)
    C = mat(BASE + 2 ** 37, 4, 8, 32, 4, DG_F32)
    st, text = plan(A, B, C)
    assert st == 0, text
    assert field(text, "rs") == str(2 ** 33)


def _golden():
    rows = []
    for line in open(os.path.join(ROOT, "tests", "golden", "views.txt")):
        if line.startswith("#") or not line.strip():
            continue
        name, dt, shape, stride, unit, _ = [x.strip() for x in line.split("|")]
        rows.append((name, dt, tuple(map(int, shape.split(","))), tuple(map(int, stride.split(","))), unit))
    return rows


_ES = {"f32": 4, "bf16": 2, "f16": 2, "e4m3": 1}
_CODE = {"f32": DG_F32, "bf16": DG_BF16, "f16": DG_F16, "e4m3": DG_F8E4M3}


@pytest.mark.parametrize("g", _golden(), ids=lambda g: g[0])
def test_golden_views_canonicalize(g):
    """The pages' view geometries become the matrix the definition says:
    rows = product of leading dims, cols = last dim, one row stride."""
    name, dt, shape, stride, unit = g
    es = _ES[dt]
    bstride = stride if unit == "bytes" else tuple(s * es for s in stride)
    rows, cols = math.prod(shape[:-1]), shape[-1]
    # the row stride after merging is the stride of the innermost leading dim > 1
    lead = [(n, s) for n, s in zip(shape[:-1], bstride[:-1]) if n > 1]
    want_rs = lead[-1][1]
    if dt in ("f32", "e4m3"):
        # use the view as A of a plan whose other operands fit it
        if dt == "f32":
            pytest.skip("FP32 inputs are not a supported GEMM input; geometry checked with T3h")
        A = make_view(BASE, shape, bstride, _CODE[dt])
        B = mat(BASE + 2 ** 36, cols, 128, 128, 1, DG_F8E4M3)
        C = mat(BASE + 2 ** 37, rows, 128, 256, 2, DG_BF16)
        SA = mat(BASE + 2 ** 38, rows, (cols + 127) // 128, 4 * ((cols + 127) // 128), 4, DG_F32)
        SB = mat(BASE + 2 ** 38 + 2 ** 30, (cols + 127) // 128, 1, 4, 4, DG_F32)
        st, text = plan(A, B, C, SA=SA, SB=SB)
    else:
        A = make_view(BASE, shape, bstride, _CODE[dt])
        B = mat(BASE + 2 ** 36, cols, 16, 32, 2, _CODE[dt])
        C = mat(BASE + 2 ** 37, rows, 16, 64, 4, DG_F32)
        st, text = plan(A, B, C)
    assert st == 0, text
    a = text.split("| A ")[1].split("|")[0].split()
    assert a[0] == f"{rows}x{cols}"
    assert a[1] == f"rs={want_rs}" and a[2] == f"cs={bstride[-1]}"


def test_plans_for_the_workloads():
    """Which path each workload takes (the selector's contract for these shapes)."""
    t = lambda *s, dt=torch.bfloat16: torch.empty(*s, dtype=dt)
    p = dg.plan(t(4096, 4096), t(4096, 4096), t(4096, 4096))
    assert field(p, "path") == "mfma" and field(p, "tile") == "256x256" and field(p, "splits") == "1"
    p = dg.plan(t(1, 4096), t(4096, 14336), t(1, 14336))
    assert field(p, "path") == "skinny" and field(p, "kind") == "BN"
    p = dg.plan(t(1, 4096), t(128, 4096).t(), t(1, 128))
    assert field(p, "path") == "skinny" and field(p, "kind") == "BK"
    p = dg.plan(t(64, 4096, dt=torch.half), t(4096, 4096, dt=torch.half), t(64, 4096, dt=torch.float32), 1.0, 1.0)
    assert field(p, "path") == "mfma" and int(field(p, "splits")) > 1
    p = dg.plan(t(4, 4, dt=torch.half), t(4, 4, dt=torch.half), t(4, 4, dt=torch.float32), 0.0, 1.0)
    assert field(p, "path") == "scale"


def test_few_tile_k_split():
    """Few-row problems with very few tiles split K into up to 4 pieces of at
    least 2 K tiles; larger ones keep at least 16 K tiles per piece."""
    t = lambda *s, dt=torch.half: torch.empty(*s, dtype=dt)
    p = dg.plan(t(64, 512), t(512, 512), t(64, 512, dt=torch.float32))        # 8 tiles, 8 K tiles
    assert field(p, "tile") == "64x64" and field(p, "splits") == "4", p
    p = dg.plan(t(64, 4096), t(4096, 4096), t(64, 4096, dt=torch.float32))    # 64 tiles, 64 K tiles
    assert field(p, "splits") == "4", p
    p = dg.plan(t(16, 64), t(64, 256), t(16, 256, dt=torch.float32))          # 1 K tile: nothing to split
    assert field(p, "splits") == "1", p


def test_fp8_tile_choice():
    """FP8 takes the 256x256 tile where its tiles fill at least 3/4 of the CU waves,
    else 128x128 (with the split tail where the last wave is short), or a column
    split where the columns up to the last multiple of 256 fill whole waves."""
    E4 = torch.float8_e4m3fn

    def fp8_plan(M, N, K):
        sa, sb = torch.ones(M, -(-K // 128)), torch.ones(-(-K // 128), -(-N // 128))
        return dg.plan(torch.empty(M, K, dtype=E4), torch.empty(K, N, dtype=E4),
                       torch.empty(M, N, dtype=torch.bfloat16), 1.0, 0.0, sa, sb)
    p = fp8_plan(4096, 7168, 4096)     # 448 tiles over 256 CUs: 7/8 of two waves
    assert field(p, "tile") == "256x256" and field(p, "splits") == "1", p
    p = fp8_plan(4096, 4224, 4096)     # 272 tiles: the second wave would hold 16; the first
    # 4096 columns fill one wave of 256x256 tiles, the last 128 run as a strip of their own
    assert field(p, "path") == "split_n" and field(p, "n1") == "4096" and field(p, "tile") == "256x256", p
    part2 = p.split("part2 {")[1].split("}")[0]
    assert "tile=64x128" in part2 and "splits=4 " in part2, p   # the 4096 x 128 strip: A read once
    p = fp8_plan(2048, 2048, 2048)     # 64 tiles of 256x256: too few
    assert field(p, "tile") == "128x128", p


def test_calib_argument_errors():
    """The calibration entry points reject bad arguments before touching a device."""
    import ctypes
    L = dg.lib()
    out = ctypes.c_double(0.0)
    assert dg.STATUS[L.dg_calib_mfma(DG_F32, ctypes.byref(out), None)] == "DG_ERR_DTYPE"
    assert dg.STATUS[L.dg_calib_mfma(DG_BF16, None, None)] == "DG_ERR_NULL"
    assert dg.STATUS[L.dg_calib_read(None, 1024, ctypes.byref(out), None)] == "DG_ERR_NULL"
    assert dg.STATUS[L.dg_calib_read(ctypes.c_void_p(BASE), 1000, ctypes.byref(out), None)] == "DG_ERR_MISALIGNED"
    assert dg.STATUS[L.dg_calib_read(ctypes.c_void_p(BASE + 8), 1024, ctypes.byref(out), None)] == "DG_ERR_MISALIGNED"
    assert dg.STATUS[L.dg_calib_read(ctypes.c_void_p(BASE), 0, ctypes.byref(out), None)] == "DG_ERR_MISALIGNED"
    assert dg.STATUS[L.dg_calib_launch(None, None)] == "DG_ERR_NULL"


def test_quant_validation():
    """dg_quant_fp8 rejects bad views before touching a device (include/dg.h)."""
    import ctypes
    L = dg.lib()
    M, K = 200, 300
    X = mat(BASE, M, K, 2 * K, 2, DG_BF16)
    Q = mat(BASE + 0x1000000, M, K, K, 1, DG_F8E4M3)
    S_tok = mat(BASE + 0x2000000, M, 3, 12, 4, DG_F32)
    S_blk = mat(BASE + 0x2000000, 2, 3, 12, 4, DG_F32)
    q = lambda x, qq, ss, mode: dg.STATUS[L.dg_quant_fp8(ctypes.byref(x), ctypes.byref(qq), ctypes.byref(ss), mode, None)]
    assert q(X, Q, S_blk, 0) == "DG_ERR_SHAPE_MISMATCH"          # token mode wants [M][3]
    assert q(X, Q, S_tok, 1) == "DG_ERR_SHAPE_MISMATCH"          # block mode wants [2][3]
    assert q(X, Q, S_tok, 2) == "DG_ERR_INVALID_ARG"
    assert q(X, mat(BASE + 0x1000000, M, K, 2 * K, 2, DG_BF16), S_tok, 0) == "DG_ERR_DTYPE"
    assert q(X, Q, mat(BASE + 0x2000000, M, 3, 6, 2, DG_BF16), 0) == "DG_ERR_DTYPE"
    assert q(mat(BASE, M, K, K, 1, DG_F8E4M3), Q, S_tok, 0) == "DG_ERR_DTYPE"
    assert q(X, mat(BASE + 0x1000000, M, K + 1, K + 1, 1, DG_F8E4M3), S_tok, 0) == "DG_ERR_SHAPE_MISMATCH"
    assert q(X, mat(BASE + 64, M, K, K, 1, DG_F8E4M3), S_tok, 0) == "DG_ERR_ALIAS"          # Q inside X
    assert q(X, Q, mat(BASE + 0x1000000 + 64, M, 3, 12, 4, DG_F32), 0) == "DG_ERR_ALIAS"   # S inside Q
    assert q(X, mat(BASE + 0x1000000, M, K, 0, 1, DG_F8E4M3), S_tok, 0) == "DG_ERR_STRIDE"   # Q rows collide
    Xe = mat(BASE, 0, K, 2 * K, 2, DG_BF16)
    assert q(Xe, mat(BASE + 0x1000000, 0, K, K, 1, DG_F8E4M3), mat(BASE + 0x2000000, 0, 3, 12, 4, DG_F32), 0) == "DG_SUCCESS"


def test_epilogue_validation():
    """dg_gemm_epilogue / dg_gemm_fp8_epilogue reject a bad bias or activation
    before touching a device (include/dg.h); a valid call gets past validation
    (on a machine without a GPU it then stops at the device query)."""
    import ctypes
    L = dg.lib()
    A, B, C = ok_triplet(64, 96, 64)
    bias = lambda ptr, n, es, dt: make_view(ptr, (n,), (es,), dt)
    good = bias(BASE + 0x30000000, 96, 2, DG_BF16)
    e = lambda bb, act: dg.STATUS[L.dg_gemm_epilogue(ctypes.byref(A), ctypes.byref(B), ctypes.byref(C),
                                                     ctypes.byref(bb) if bb is not None else None, act,
                                                     1.0, 0.0, None)]
    assert e(good, 3) == "DG_ERR_INVALID_ARG"
    assert e(good, -1) == "DG_ERR_INVALID_ARG"
    assert e(bias(BASE + 0x30000000, 96, 1, DG_F8E4M3), 2) == "DG_ERR_DTYPE"
    assert e(bias(BASE + 0x30000000, 95, 2, DG_BF16), 2) == "DG_ERR_SHAPE_MISMATCH"
    assert e(make_view(BASE + 0x30000000, (96, 1), (2, 2), DG_BF16), 2) == "DG_ERR_SHAPE_MISMATCH"   # a column
    assert e(bias(BASE + 0x20000000 + 4 * 96 * 10, 96, 4, DG_F32), 2) == "DG_ERR_ALIAS"   # a row of C
    assert e(bias(BASE + 0x30000001, 96, 2, DG_BF16), 2) == "DG_ERR_MISALIGNED"
    assert e(bias(0, 96, 2, DG_BF16), 2) == "DG_ERR_NULL"
    for bb in (good, bias(BASE + 0x30000000, 96, 0, DG_F32), make_view(BASE + 0x30000000, (1, 96), (192, 2), DG_F16),
               None):
        for act in (0, 1, 2):
            assert e(bb, act) in ("DG_ERR_HIP", "DG_ERR_ARCH", "DG_SUCCESS"), (bb, act)
    # FP8 form: the same checks after the scale views
    M, N, K = 64, 256, 256
    qa = mat(BASE, M, K, K, 1, DG_F8E4M3)
    sa = mat(BASE + 0x1000000, M, 2, 8, 4, DG_F32)
    qb = mat(BASE + 0x2000000, K, N, N, 1, DG_F8E4M3)
    sb = mat(BASE + 0x3000000, 2, 2, 8, 4, DG_F32)
    c = mat(BASE + 0x4000000, M, N, 2 * N, 2, DG_BF16)
    f = lambda bb, act: dg.STATUS[L.dg_gemm_fp8_epilogue(*[ctypes.byref(v) for v in (qa, sa, qb, sb, c)],
                                                         ctypes.byref(bb), act, 1.0, 0.0, None)]
    assert f(bias(BASE + 0x5000000, N, 2, DG_BF16), 7) == "DG_ERR_INVALID_ARG"
    assert f(bias(BASE + 0x5000000, N - 1, 2, DG_BF16), 2) == "DG_ERR_SHAPE_MISMATCH"
    assert f(bias(BASE + 0x4000000, N, 2, DG_BF16), 2) == "DG_ERR_ALIAS"
    assert f(bias(BASE + 0x5000000, N, 2, DG_BF16), 2) in ("DG_ERR_HIP", "DG_ERR_ARCH", "DG_SUCCESS")


def test_grouped_validation_and_plan():
    """dg_gemm_grouped_plan validates every group and batches the thin
    N-contiguous groups (include/dg.h)."""
    import ctypes
    V = dg.View
    def arr(vs):
        a = (V * max(len(vs), 1))()
        for i, v in enumerate(vs):
            a[i] = v
        return a
    def gp(As, Bs, Cs, alpha=1.0, beta=0.0):
        st, text = dg.grouped_plan_views(len(As), arr(As), arr(Bs), arr(Cs), alpha, beta)
        return dg.STATUS[st], text
    E = 8
    x = mat(BASE, 1, 512, 1024, 2)
    Ws = [mat(BASE + (1 + e) * 0x1000000, 512, 4096, 8192, 2) for e in range(E)]
    Cs = [mat(BASE + (20 + e) * 0x1000000, 1, 4096, 8192, 2) for e in range(E)]
    st, text = gp([x] * E, Ws, Cs)
    assert st == "DG_SUCCESS", text
    assert "batch mmax=1 units=256" in text and "solo= " not in text and text.endswith("solo="), text
    # 40 groups: three batches of at most 16
    st, text = gp([x] * 40, [Ws[0]] * 40, [mat(BASE + (40 + e) * 0x1000000, 1, 4096, 8192, 2) for e in range(40)])
    assert st == "DG_SUCCESS" and text.count("batch mmax=1") == 3, text
    # a group with M = 20 runs alone; a K-contiguous B runs alone
    A20 = mat(BASE, 20, 512, 1024, 2)
    Bk = mat(BASE + 0x3000000, 512, 128, 2, 1024)
    st, text = gp([x, A20, x], [Ws[0], Ws[1], Bk], [Cs[0], mat(BASE + 0x30000000, 20, 4096, 8192, 2),
                                                    mat(BASE + 0x31000000, 1, 128, 256, 2)])
    assert st == "DG_SUCCESS" and text.endswith("solo=1,2"), text
    assert gp([], [], [])[0] == "DG_SUCCESS"
    L = dg.lib()
    assert dg.STATUS[L.dg_gemm_grouped_plan(-1, None, None, None, 1.0, 0.0, None, 0)] == "DG_ERR_INVALID_ARG"
    assert dg.STATUS[L.dg_gemm_grouped_plan(2, None, None, None, 1.0, 0.0, None, 0)] == "DG_ERR_NULL"
    assert dg.STATUS[L.dg_gemm_grouped(-1, None, None, None, 1.0, 0.0, None)] == "DG_ERR_INVALID_ARG"
    # two groups writing one C, or one C inside another group's input
    assert gp([x, x], Ws[:2], [Cs[0], Cs[0]])[0] == "DG_ERR_ALIAS"
    x_in_c0 = mat(BASE + (20 + 0) * 0x1000000, 1, 512, 1024, 2)   # group 1 reads what group 0 writes
    assert gp([x, x_in_c0], Ws[:2], Cs[:2])[0] == "DG_ERR_ALIAS"
    assert gp([x, x], [Ws[0], Ws[1]], [Cs[0], mat(BASE + 0x1000000 + 64, 1, 4096, 8192, 2)])[0] == "DG_ERR_ALIAS"
    # dtype mix across groups; a bad group reports its own error
    x16 = mat(BASE, 1, 512, 1024, 2, DG_F16)
    W16 = mat(BASE + 0x1000000, 512, 4096, 8192, 2, DG_F16)
    assert gp([x, x16], [Ws[0], W16], Cs[:2])[0] == "DG_ERR_DTYPE"
    assert gp([x, x], [Ws[0], mat(BASE + 0x2000000, 511, 4096, 8192, 2)], Cs[:2])[0] == "DG_ERR_SHAPE_MISMATCH"
    assert gp([x, x], Ws[:2], Cs[:2], alpha=float("nan"))[0] == "DG_ERR_NONFINITE_SCALAR"


def test_candidates_and_tuned_plan_files(tmp_path):
    """dg_gemm_candidates lists distinct plans, built-in first; dg_tune_load /
    dg_tune_save / dg_tune_clear manage the tuned table, which dg_gemm_plan
    consults (all without a GPU: plans for a 256-CU gfx950)."""
    import ctypes
    L = dg.lib()
    A, B, C = ok_triplet(64, 4096, 4096)
    arr = (dg.PlanChoice * 64)()
    n = ctypes.c_int32(0)
    assert L.dg_gemm_candidates(ctypes.byref(A), None, ctypes.byref(B), None, ctypes.byref(C), arr, 64,
                                ctypes.byref(n)) == 0
    cands = [arr[i].astuple() for i in range(n.value)]
    assert cands[0] == (0, -1, 0, -1) and len(set(cands)) == len(cands) and 2 <= len(cands) <= 24, cands
    # argument errors
    assert dg.STATUS[L.dg_gemm_candidates(ctypes.byref(A), None, ctypes.byref(B), None, ctypes.byref(C), arr, 64,
                                          None)] == "DG_ERR_NULL"
    assert dg.STATUS[L.dg_gemm_candidates(ctypes.byref(A), ctypes.byref(A), ctypes.byref(B), None, ctypes.byref(C),
                                          arr, 64, ctypes.byref(n))] == "DG_ERR_NULL"
    bad = dg.PlanChoice(3, -1, 0, -1)
    assert dg.STATUS[L.dg_gemm_with_choice(ctypes.byref(A), None, ctypes.byref(B), None, ctypes.byref(C),
                                           ctypes.byref(bad), 1.0, 0.0, None)] == "DG_ERR_INVALID_ARG"
    assert dg.STATUS[L.dg_gemm_with_choice(ctypes.byref(A), None, ctypes.byref(B), None, ctypes.byref(C),
                                           None, 1.0, 0.0, None)] == "DG_ERR_NULL"
    assert dg.STATUS[L.dg_gemm_tune(ctypes.byref(A), None, ctypes.byref(B), None, ctypes.byref(C), 5, None,
                                    None)] == "DG_ERR_NULL"
    r = dg.TuneResult()
    assert dg.STATUS[L.dg_gemm_tune(ctypes.byref(A), None, ctypes.byref(B), None, ctypes.byref(C), -1,
                                    ctypes.byref(r), None)] == "DG_ERR_INVALID_ARG"
    # a tuned entry for this key (the plan's own view of the default device)
    dg.tune_clear()
    before = plan(A, B, C)[1]
    assert field(before, "tile") == "64x64"
    line = ("dgtune1 gfx950 256 64 4096 4096 8192 2 8192 2 0 0 0 1 0 0 16 16 16 2 16 2 "
            "2 1 2 0\n")   # path 2, tile 128x128, 2 splits, no tail split
    f = tmp_path / "tuned.txt"
    f.write_text("# handmade\n" + line)
    dg.tune_load(str(f))
    assert dg.tune_count() == 1
    after = plan(A, B, C)[1]
    assert field(after, "tile") == "128x128" and field(after, "splits") == "2", after
    out = tmp_path / "saved.txt"
    dg.tune_save(str(out))
    assert line.split() == [l for l in out.read_text().splitlines() if l.startswith("dgtune1")][0].split()
    dg.tune_clear()
    assert dg.tune_count() == 0 and plan(A, B, C)[1] == before
    dg.tune_load(str(out))
    assert plan(A, B, C)[1] == after
    dg.tune_clear()
    # a malformed file adds nothing; a missing one is an error
    (tmp_path / "bad.txt").write_text(line + "dgtune1 gfx950 256 1 2 3\n")
    with pytest.raises(dg.DGError):
        dg.tune_load(str(tmp_path / "bad.txt"))
    assert dg.tune_count() == 0
    with pytest.raises(dg.DGError):
        dg.tune_load(str(tmp_path / "missing.txt"))
