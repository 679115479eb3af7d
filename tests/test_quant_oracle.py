"""Pins of the FP8 quantizer oracle (oracle/quant.py) against the E4M3 format
definition, a library cast, closed forms and the harness's torch quantizer."""
import numpy as np
import pytest
import torch

import synth
from oracle import quant as oq


def _torch_codes(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = oq.e4m3_decode(codes)
    assert (oq.e4m3_encode(vals) == codes).all()
    # the format's landmarks: 448 = 0x7E, 2^-6 = 0x08 (smallest normal), 2^-9 = 0x01, -0 = 0x80
    assert oq.e4m3_value(0x7E) == 448.0 and oq.e4m3_value(0x08) == 2.0 ** -6 and oq.e4m3_value(0x01) == 2.0 ** -9
    assert oq.e4m3_encode(np.float32(-0.0)) == 0x80


def test_midpoints_tie_to_the_even_code():
    for c in range(0x7E):
        mid = np.float32((oq.e4m3_value(c) + oq.e4m3_value(c + 1)) / 2)   # exact in FP32
        want = c if c % 2 == 0 else c + 1
        assert oq.e4m3_encode(mid) == want, (c, mid)
        assert oq.e4m3_encode(-mid) == (want | 0x80)


@pytest.mark.parametrize("scale", [1e-3, 0.05, 1.0, 60.0, 400.0])
def test_matches_torch_cast(scale):
    g = np.random.default_rng(7)
    x = np.clip((g.standard_normal(200000) * scale).astype(np.float32), -448, 448)
    assert (oq.e4m3_encode(x) == _torch_codes(x)).all()


def test_zero_block_and_single_peak():
    x = np.zeros((3, 200), dtype=np.float32)
    x[1, 5] = -3.0
    q, s = oq.quant_tokens(x)
    tiny = np.float32(np.float32(1e-12) / np.float32(448))
    assert s[0, 0] == tiny and s[0, 1] == tiny and s[1, 1] == tiny
    assert s[1, 0] == np.float32(np.float32(3.0) / np.float32(448))
    assert q[1, 5] == 0xFE                      # -448
    assert (np.delete(q.ravel(), 1 * 200 + 5) == 0).all()


def test_power_of_two_scaling_leaves_codes_alone():
    g = np.random.default_rng(3)
    x = (g.standard_normal((130, 300)) * 3).astype(np.float32)
    q1, s1 = oq.quant_blocks(x)
    q2, s2 = oq.quant_blocks(x * np.float32(8.0))
    assert (q1 == q2).all() and (s2 == s1 * np.float32(8.0)).all()


@pytest.mark.parametrize("shape", [(1, 1), (5, 127), (3, 129), (130, 300), (256, 512)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
def test_agrees_with_the_harness_quantizer(shape, dtype):
    g = synth.rng(sum(shape) + len(str(dtype)))
    x = synth.to_dtype(synth.draw(g, shape, "normal", 2.0), dtype)
    q, s = oq.quant_tokens(x)
    tq, ts = synth.quantize_rows_k128(x)
    assert (q == tq.view(torch.uint8).numpy()).all() and (s == ts.numpy()).all()
    q, s = oq.quant_blocks(x)
    tq, ts = synth.quantize_blocks_128(x)
    assert (q == tq.view(torch.uint8).numpy()).all() and (s == ts.numpy()).all()
