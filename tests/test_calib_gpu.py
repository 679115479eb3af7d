"""The measured roofline denominators (include/dg_calib.h) on the GPU: each
returns a rate inside what the part can physically do, so a report that
divides by them is not dividing by garbage."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_gemm_19_amd as dg
    dg.lib()
    return dg


def test_mfma_rates(dg):
    bf16 = dg.calib_mfma(dg.DG_BF16)
    fp8 = dg.calib_mfma(dg.DG_F8E4M3)
    # dense peaks 2516.6 (BF16) and 5033.2 (FP8) TFLOP/s at the boost clock
    assert 300.0 < bf16 < 2600.0, bf16
    assert 600.0 < fp8 < 5200.0, fp8
    assert fp8 > 1.3 * bf16


def test_read_rate(dg):
    buf = torch.empty(256 << 20, dtype=torch.uint8, device="cuda:0").fill_(1)
    gbs = dg.calib_read(buf)
    assert 500.0 < gbs < 20000.0, gbs   # above the 8 TB/s HBM peak only if cache-resident


def test_launch_floor(dg):
    us = dg.calib_launch()
    assert 0.05 < us < 100.0, us
