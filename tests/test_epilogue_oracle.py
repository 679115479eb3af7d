"""Pins of the fused-epilogue oracle (oracle/epilogue.py) against facts that do
not come from the oracle's own formula: the exact GELU x * Phi(x) (SciPy's
normal CDF), textbook values of Phi, symmetry and limits, the curvature at 0,
a brute-force composition on a tiny integer problem, and planted mistakes that
the comparator must reject."""
import numpy as np
import pytest
import torch
from scipy.stats import norm

import oracle
from oracle import epilogue as E


X = np.linspace(-12.0, 12.0, 480001)


def test_gelu_tanh_close_to_exact_gelu():
    # Hendrycks and Gimpel's tanh form approximates x * Phi(x); its largest
    # deviation on the real line is 4.73e-4 (near x = -2.70).  A wrong
    # constant (sqrt(pi/2), a mistyped cubic coefficient, a missing 0.5) moves
    # it far outside [4.6e-4, 4.8e-4].
    err = np.abs(E.gelu_tanh(X) - X * norm.cdf(X))
    assert 4.6e-4 < err.max() < 4.8e-4
    assert abs(X[np.argmax(err)] + 2.70) < 0.05


def test_gelu_tanh_textbook_points():
    # Phi(1) = 0.841345, Phi(2) = 0.977250, Phi(-1) = 0.158655 (normal tables):
    # x * Phi(x) within the approximation error above.
    for x, phi in [(1.0, 0.8413447460685429), (2.0, 0.9772498680518208), (-1.0, 0.15865525393145707),
                   (0.5, 0.6914624612740131)]:
        assert abs(float(E.gelu_tanh(x)) - x * phi) < 5e-4
    assert float(E.gelu_tanh(0.0)) == 0.0


def test_gelu_tanh_odd_part_is_identity():
    # tanh is odd, so GELU(x) - GELU(-x) = x exactly in real arithmetic.
    d = E.gelu_tanh(X) - E.gelu_tanh(-X)
    assert np.max(np.abs(d - X)) < 1e-14 * 12


def test_gelu_tanh_derivatives_at_zero():
    # GELU'(0) = 1/2 and GELU''(0) = 2 phi(0) = sqrt(2/pi) (the tanh form is
    # built to match the exact curvature at 0).
    h = 1e-4
    g = lambda t: float(E.gelu_tanh(t))
    d1 = (g(h) - g(-h)) / (2 * h)
    d2 = (g(h) - 2 * g(0.0) + g(-h)) / (h * h)
    assert abs(d1 - 0.5) < 1e-8
    assert abs(d2 - 2 * norm.pdf(0.0)) < 1e-5


def test_gelu_tanh_limits():
    assert float(E.gelu_tanh(10.0)) == pytest.approx(10.0, rel=1e-15)
    assert abs(float(E.gelu_tanh(-10.0))) < 1e-30
    assert float(E.gelu_tanh(-1e20)) == 0.0
    assert float(E.gelu_tanh(1e20)) == 1e20


def test_lipschitz_constants_cover_the_slopes():
    for act, f in [(E.ACT_GELU_TANH, E.gelu_tanh), (E.ACT_RELU, E.relu)]:
        d = np.abs(np.gradient(f(X), X))
        assert d.max() <= E.LIPSCHITZ[act] * (1 + 1e-9)   # (finite-difference rounding)
    # and the GELU constant is tight (1.1290 at x = 1.5)
    assert np.abs(np.gradient(E.gelu_tanh(X), X)).max() > 1.128


def test_relu_matches_maximum_and_keeps_nan():
    x = np.array([-3.0, -0.0, 0.0, 1e-30, 5.0, np.nan, -np.inf, np.inf])
    r = E.relu(x)
    fin = ~np.isnan(x)
    assert np.array_equal(r[fin], np.maximum(x[fin], 0.0))
    assert np.isnan(r[5])


def _tiny_problem():
    # integer inputs: every sum is exact, so the brute force below is exact too
    g = np.random.default_rng(5)
    A = torch.tensor(g.integers(-3, 4, (3, 5)), dtype=torch.bfloat16)
    B = torch.tensor(g.integers(-3, 4, (5, 4)), dtype=torch.bfloat16)
    C = torch.tensor(g.integers(-3, 4, (3, 4)), dtype=torch.float32)
    bias = torch.tensor([0.5, -1.25, 2.0, -3.0], dtype=torch.float32)
    return A, B, C, bias


@pytest.mark.parametrize("act", E.ACTS)
def test_composition_brute_force(act):
    A, B, C, bias = _tiny_problem()
    alpha, beta = 0.5, -2.0
    ref = oracle.ref_gemm(A, B, C, alpha, beta)
    e = E.ref_epilogue(ref, bias, act)
    a, b, c, bb = (t.double().tolist() for t in (A, B, C, bias))
    for m in range(3):
        for n in range(4):
            y = alpha * sum(a[m][k] * b[k][n] for k in range(5)) + beta * c[m][n] + bb[n]
            want = y if act == E.ACT_NONE else (max(y, 0.0) if act == E.ACT_RELU else float(E.gelu_tanh(y)))
            assert e.Y[m, n] == y
            assert e.C[m, n] == pytest.approx(want, rel=1e-15, abs=1e-300)


def test_bias_strided_and_broadcast_views():
    A, B, C, _ = _tiny_problem()
    ref = oracle.ref_gemm(A, B)
    store = torch.arange(8, dtype=torch.float16)
    e = E.ref_epilogue(ref, store[::2], E.ACT_NONE)          # every other element
    assert np.array_equal(e.Y - ref.C, np.tile([0.0, 2.0, 4.0, 6.0], (3, 1)))
    one = torch.tensor([3.0], dtype=torch.bfloat16).expand(4)  # stride 0
    e = E.ref_epilogue(ref, one, E.ACT_NONE)
    assert np.array_equal(e.Y - ref.C, np.full((3, 4), 3.0))


def test_alpha_zero_is_act_of_beta_c_plus_bias():
    A, B, C, bias = _tiny_problem()
    ref = oracle.ref_gemm(A, B, C, 0.0, 1.5)
    e = E.ref_epilogue(ref, bias, E.ACT_RELU)
    want = np.maximum(1.5 * C.double().numpy() + bias.double().numpy()[None, :], 0.0)
    assert np.array_equal(e.C, want)


def _random_ref(act, seed=1):
    g = np.random.default_rng(seed)
    A = torch.tensor(g.standard_normal((40, 96)), dtype=torch.bfloat16)
    B = torch.tensor(g.standard_normal((96, 72)), dtype=torch.bfloat16)
    bias = torch.tensor(g.standard_normal(72), dtype=torch.bfloat16)
    return E.ref_epilogue(oracle.ref_gemm(A, B), bias, act), bias


@pytest.mark.parametrize("fmt", ["f32", "bf16"])
def test_comparator_accepts_the_rounded_reference(fmt):
    e, _ = _random_ref(E.ACT_GELU_TANH)
    dt = torch.float32 if fmt == "f32" else torch.bfloat16
    got = torch.from_numpy(e.C).to(torch.float32).to(dt)
    assert E.compare_epilogue(got, e, fmt, 1e-4).ok


@pytest.mark.parametrize("mistake", ["no_bias", "bias_by_row", "act_before_bias", "relu_for_gelu",
                                     "sign_flip"])
def test_comparator_rejects_planted_mistakes(mistake):
    # Each mistake is planted in a copy of the oracle's result on the CPU.
    e, bias = _random_ref(E.ACT_GELU_TANH)
    b = bias.double().numpy()
    pre = e.gemm.C
    if mistake == "no_bias":
        wrong = E.gelu_tanh(pre)
    elif mistake == "bias_by_row":
        wrong = E.gelu_tanh(pre + b[: pre.shape[0], None])
    elif mistake == "act_before_bias":
        wrong = E.gelu_tanh(pre) + b[None, :]
    elif mistake == "relu_for_gelu":
        wrong = E.relu(e.Y)
    else:
        wrong = 0.5 * e.Y * (1.0 - np.tanh(E.SQRT_2_OVER_PI * (e.Y + E.GELU_CUBIC * e.Y ** 3)))
    got = torch.from_numpy(wrong).to(torch.float32)
    assert not E.compare_epilogue(got, e, "f32", 1e-4).ok

