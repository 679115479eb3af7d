"""Pins for the oracle's own number decoders and for the rounding the comparator uses.

Each decoder is checked exhaustively (every FP16, BF16 and E4M3FN bit
pattern) against torch's conversions, a library routine written
independently of oracle.c.  FP32 is checked on specials and 10^6 random
patterns against numpy.  The FP32 -> BF16/FP16 round-to-nearest-even that the
comparator applies to the reference is checked against an integer RNE
written here from the definition.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import OR_BF16, OR_E4M3, OR_F16, OR_F32, HostView


def _decode_all(code, bits: np.ndarray, esize: int) -> np.ndarray:
    """Decode a 1-D array of bit patterns through the oracle's view walk."""
    raw = bits.astype({1: np.uint8, 2: np.uint16, 4: np.uint32}[esize]).view(np.uint8).copy()
    v = HostView(raw, 0, (1, len(bits)), (len(bits) * esize, esize), code)
    return oracle.gather(v)[0]


def _same(a: np.ndarray, b: np.ndarray) -> bool:
    return np.array_equal(a, b, equal_nan=True) and np.array_equal(np.signbit(a), np.signbit(b))


def test_f16_exhaustive():
    bits = np.arange(65536, dtype=np.uint32)
    got = _decode_all(OR_F16, bits, 2)
    want = torch.from_numpy(bits.astype(np.uint16).view(np.int16)).view(torch.float16).double().numpy()
    assert _same(got, want)


def test_bf16_exhaustive():
    bits = np.arange(65536, dtype=np.uint32)
    got = _decode_all(OR_BF16, bits, 2)
    want = torch.from_numpy(bits.astype(np.uint16).view(np.int16)).view(torch.bfloat16).double().numpy()
    assert _same(got, want)


def test_e4m3fn_exhaustive():
    bits = np.arange(256, dtype=np.uint32)
    got = _decode_all(OR_E4M3, bits, 1)
    want = torch.from_numpy(bits.astype(np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    assert _same(got, want)
    # Facts of the format itself: no infinities, max 448, smallest subnormal 2^-9.
    assert not np.isinf(got).any()
    assert np.nanmax(got) == 448.0 and np.nanmin(got) == -448.0
    assert np.count_nonzero(np.isnan(got)) == 2          # 0x7F and 0xFF
    assert got[1] == 2.0 ** -9


def test_f32_random_and_specials():
    g = np.random.default_rng(7)
    bits = g.integers(0, 2 ** 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    specials = np.array([0, 0x80000000, 1, 0x807fffff, 0x7f7fffff, 0xff7fffff, 0x7f800000,
                         0xff800000, 0x7fc00000, 0x00800000, 0x3f800000], dtype=np.uint32)
    bits = np.concatenate([specials, bits])
    got = _decode_all(OR_F32, bits, 4)
    want = bits.view(np.float32).astype(np.float64)
    assert _same(got, want)


def test_scalar_decode_entry():
    assert oracle.decode(OR_F16, 0x3C00) == 1.0
    assert oracle.decode(OR_BF16, 0xC040) == -3.0
    assert oracle.decode(OR_E4M3, 0x7E) == 448.0
    assert oracle.decode(OR_F32, 0x40490FDB) == float(np.float32(np.pi))


def _rne_16(bits32: np.ndarray, fmt: str) -> np.ndarray:
    """FP32 -> BF16 by integer round-to-nearest-even on the bit pattern (the
    definition), NaN kept quiet.  Only used for BF16 here."""
    assert fmt == "bf16"
    b = bits32.astype(np.uint64)
    lsb = (b >> 16) & 1
    r = (b + 0x7FFF + lsb) >> 16
    nan = ((b & 0x7F800000) == 0x7F800000) & ((b & 0x7FFFFF) != 0)
    r = np.where(nan, (b >> 16) | 0x40, r)
    return (r & 0xFFFF).astype(np.uint16)


def test_bf16_rne_matches_definition():
    g = np.random.default_rng(11)
    rnd = g.integers(0, 2 ** 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x00008000, 0x00018000,
                     0x7F7F8000, 0x7F7FFFFF, 0x7F800000, 0xFF800000, 0x00000001,
                     0x80000001, 0x007FFFFF], dtype=np.uint32)
    bits = np.concatenate([ties, rnd])
    f = torch.from_numpy(bits.view(np.float32).copy())
    got = f.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    want = _rne_16(bits, "bf16")
    nan = np.isnan(bits.view(np.float32))
    assert np.array_equal(got[~nan], want[~nan])
    assert np.isnan(f[nan].to(torch.bfloat16).float().numpy()).all()


@pytest.mark.parametrize("x,expect", [
    (1.0, 2.0 ** -23), (1.5, 2.0 ** -23), (2.0, 2.0 ** -22), (0.75, 2.0 ** -24), (0.0, 2.0 ** -149),
])
def test_ulp_f32(x, expect):
    assert oracle.ulp(np.array([x]), "f32")[0] == expect


def test_ulp_16bit():
    assert oracle.ulp(np.array([1.0]), "bf16")[0] == 2.0 ** -7
    assert oracle.ulp(np.array([128.0]), "bf16")[0] == 1.0
    assert oracle.ulp(np.array([1.0]), "f16")[0] == 2.0 ** -10
    assert oracle.ulp(np.array([1e-9]), "f16")[0] == 2.0 ** -24
