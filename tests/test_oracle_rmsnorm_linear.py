"""Pins for the oracle's RMSNorm + linear + scale.

Source: the TeleTron write-up (2kiu.com/news/5927820), section 4.2 (one fused
kernel: the row's RMS factor is computed in the block and used directly in the
linear layer's multiply-accumulate, bias and an elementwise scale follow, no
normalised tensor is stored) and section 3.1 (a norm followed by a projection
in every transformer block).

The section's kernel keeps the weighted input v * w in an fp32 array (for
16-bit inputs that product is exact), so the operand of the dot product is the
unrounded x * w. Its listing squares v * w for the mean square; the reading
here is RMSNorm's definition (the mean square of x), and a pin shows the two
coincide at w = 1 and differ otherwise.

Pins: torch in float64 on the unrounded product (library matmul), exact
rational arithmetic on tiny shapes (fp32 and bf16), a hand-worked case where
rounding the operand to the input type would change the result, the K = 1
closed form, the identity weight (the product reduces to the RMS-normalised
row), RMSNorm's scale invariance (2x with 4 eps), linearity in bias and scale,
the listing's form at w = 1, and hand-worked cases of the three-step unfused
form.
"""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import BF16, F16, F32
from tolerance import bf16_bits_to_f32, ulp_dist16

getcontext().prec = 60


def _bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _inputs(M, K, N, seed):
    x = synth.normal((M, K), seed, "bf16")
    w = synth.normal((K,), seed + 1, "bf16", mean=1.0, std=0.1)
    Wt = synth.normal((N, K), seed + 2, "bf16", std=K ** -0.5)
    b = synth.normal((N,), seed + 3, "bf16", std=0.1)
    return x, w, Wt, b


def test_against_torch_float64(orc):
    M, K, N = 24, 512, 96
    x, w, Wt, b = _inputs(M, K, N, 40)
    scale, eps = 0.7, 1e-6
    out = orc.rmsnorm_linear(x, w, Wt, b, eps, scale, BF16)
    xt = _bf16(x).double()
    a = xt * _bf16(w).double()  # the unrounded product (exact in float64)
    rstd = 1.0 / torch.sqrt((xt * xt).mean(dim=1, keepdim=True) + float(np.float32(eps)))
    ref = scale * (rstd * (a @ _bf16(Wt).double().t()) + _bf16(b).double())
    d = ulp_dist16(out, _bits(ref.to(torch.bfloat16)))
    assert d.max() <= 1 and (d == 0).mean() > 0.999


def test_exact_rationals(orc):
    rng = np.random.default_rng(1)
    M, K, N = 2, 5, 3
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(K)).astype(np.float32)
    Wt = rng.standard_normal((N, K)).astype(np.float32)
    b = rng.standard_normal(N).astype(np.float32)
    eps, scale = np.float32(1e-5), np.float32(0.375)
    out, exact, _ = orc.rmsnorm_linear(x, w, Wt, b, float(eps), float(scale), F32,
                                       want_exact=True)
    for m in range(M):
        ms = sum(Fraction(float(v)) ** 2 for v in x[m]) / K + Fraction(float(eps))
        rstd = 1 / (Decimal(ms.numerator) / Decimal(ms.denominator)).sqrt()
        a = [Fraction(float(np.float32(np.float64(x[m, k]) * np.float64(w[k])))) for k in range(K)]
        for n in range(N):
            acc = sum(a[k] * Fraction(float(Wt[n, k])) for k in range(K))
            want = Decimal(float(scale)) * (rstd * (Decimal(acc.numerator) / Decimal(acc.denominator))
                                            + Decimal(float(b[n])))
            assert abs(Decimal(exact[m, n]) - want) <= abs(want) * Decimal(1e-15) + Decimal(1e-300)
            assert out[m, n] == np.float32(float(want))


def test_exact_rationals_bf16_unrounded_operand(orc):
    """bf16 inputs: the operand is x * w exactly (16 significant bits, not a
    bf16); the exact value agrees with rational arithmetic on that product."""
    M, K, N = 3, 6, 4
    x, w, Wt, b = _inputs(M, K, N, 41)
    eps, scale = 1e-6, -0.625
    out, exact, _ = orc.rmsnorm_linear(x, w, Wt, b, eps, scale, BF16, want_exact=True)
    xv, wv = bf16_bits_to_f32(x), bf16_bits_to_f32(w)
    Wv, bv = bf16_bits_to_f32(Wt), bf16_bits_to_f32(b)
    e32 = Fraction(float(np.float32(eps)))
    for m in range(M):
        ms = sum(Fraction(float(v)) ** 2 for v in xv[m]) / K + e32
        rstd = 1 / (Decimal(ms.numerator) / Decimal(ms.denominator)).sqrt()
        for n in range(N):
            acc = sum(Fraction(float(xv[m, k])) * Fraction(float(wv[k])) *
                      Fraction(float(Wv[n, k])) for k in range(K))
            want = Decimal(scale) * (rstd * (Decimal(acc.numerator) / Decimal(acc.denominator))
                                     + Decimal(float(bv[n])))
            assert abs(Decimal(exact[m, n]) - want) <= abs(want) * Decimal(1e-15)
            assert out[m, n] == synth.to_bf16_bits(np.array([float(want)]))[0]


@pytest.mark.parametrize("dt,xw,want_bits", [
    # fp16: x = (1 + 2^-10, 1 + 2^-9), w = (1 + 2^-10, 1), Wt row (1, -1).
    # x1 w1 = 1 + 2^-9 + 2^-20 exactly and x2 w2 = 1 + 2^-9, so the dot
    # product is 2^-20; rstd = 1/sqrt(((1+2^-10)^2 + (1+2^-9)^2)/2 + eps)
    # = 0.998544..., out = 0.99854 * 2^-20 = 15.977 * 2^-24 -> the fp16
    # subnormal 16 * 2^-24 (bits 0x0010). Rounding x1 w1 to fp16 first
    # (-> 1 + 2^-9) would give exactly 0.
    (F16, ((1 + 2 ** -10, 1 + 2 ** -9), (1 + 2 ** -10, 1.0)), 0x0010),
    # bf16: x = (1 + 2^-7, 1 + 2^-6), w = (1 + 2^-7, 1): the products differ
    # by 2^-14; rstd = 0.988366..., out = 1.97682 * 2^-15 -> 1.9765625 * 2^-15
    # (bits 0x387D); with x1 w1 rounded to bf16 the result is 0.
    (BF16, ((1 + 2 ** -7, 1 + 2 ** -6), (1 + 2 ** -7, 1.0)), 0x387D),
])
def test_operand_is_not_rounded_hand_worked(orc, dt, xw, want_bits):
    (x1, x2), (w1, w2) = xw
    enc = (lambda a: np.asarray(a, np.float16).view(np.uint16)) if dt == F16 else \
        (lambda a: synth.to_bf16_bits(np.asarray(a, np.float32)))
    x = enc([[x1, x2]])
    w = enc([w1, w2])
    Wt = enc([[1.0, -1.0]])
    out = orc.rmsnorm_linear(x, w, Wt, None, 1e-6, 1.0, dt)
    assert int(out[0, 0]) == want_bits


def test_listing_form_at_unit_weight(orc):
    """The section's listing squares v * w (the weighted input) for the mean
    square. At w = 1 that is RMSNorm's mean square of x, so the two forms give
    the same bits; with w ~ N(1, 0.1) they differ, so the reading matters."""
    M, K, N = 6, 256, 24
    x, w, Wt, b = _inputs(M, K, N, 45)
    xv = bf16_bits_to_f32(x).astype(np.float64)
    Wv = bf16_bits_to_f32(Wt).astype(np.float64)
    bv = bf16_bits_to_f32(b).astype(np.float64)
    e32 = float(np.float32(1e-6))

    def listing_form(wv):
        s = xv * wv  # the weighted input, squared for the mean square as listed
        rstd = 1.0 / np.sqrt((s * s).mean(axis=1, keepdims=True) + e32)
        return synth.to_bf16_bits(0.5 * (rstd * (s @ Wv.T) + bv))

    ones = synth.to_bf16_bits(np.ones(K, np.float32))
    at_one = orc.rmsnorm_linear(x, ones, Wt, b, 1e-6, 0.5, BF16)
    assert ulp_dist16(at_one, listing_form(np.ones(K))).max() <= 1
    assert (at_one == listing_form(np.ones(K))).mean() > 0.99
    general = orc.rmsnorm_linear(x, w, Wt, b, 1e-6, 0.5, BF16)
    assert (ulp_dist16(general, listing_form(bf16_bits_to_f32(w).astype(np.float64))) > 0).mean() > 0.4


def test_k1_closed_form(orc):
    x = np.array([[3.0], [-0.5], [0.0]], np.float32)
    w = np.array([2.0], np.float32)
    Wt = np.array([[1.5], [-4.0]], np.float32)
    b = np.array([0.25, 1.0], np.float32)
    eps = 1e-3
    _, exact, _ = orc.rmsnorm_linear(x, w, Wt, b, eps, 2.0, F32, want_exact=True)
    e32 = float(np.float32(eps))
    for m in range(3):
        xv = float(x[m, 0])
        want = [2.0 * (xv * 2.0 * Wt[n, 0] / np.sqrt(xv * xv + e32) + b[n]) for n in range(2)]
        np.testing.assert_allclose(exact[m], want, rtol=1e-15, atol=1e-300)


def test_identity_weight_is_the_normalised_row(orc):
    M, K = 6, 64
    x, w, _, _ = _inputs(M, K, 1, 50)
    I = synth.to_bf16_bits(np.eye(K, dtype=np.float32))
    _, exact, _ = orc.rmsnorm_linear(x, w, I, None, 1e-6, 1.0, BF16, want_exact=True)
    xv = bf16_bits_to_f32(x).astype(np.float64)
    a = xv * bf16_bits_to_f32(w)  # the exact product
    rstd = 1.0 / np.sqrt((xv * xv).mean(axis=1, keepdims=True) + float(np.float32(1e-6)))
    np.testing.assert_allclose(exact, rstd * a, rtol=1e-14, atol=0)


def test_scale_invariance(orc):
    M, K, N = 8, 256, 40
    x, w, Wt, b = _inputs(M, K, N, 60)
    x2 = synth.to_bf16_bits(2.0 * bf16_bits_to_f32(x))  # exact in bf16
    o1 = orc.rmsnorm_linear(x, w, Wt, b, 1e-6, 0.5, BF16)
    o2 = orc.rmsnorm_linear(x2, w, Wt, b, 4e-6, 0.5, BF16)
    assert np.array_equal(o1, o2)


def test_linear_in_bias_and_scale(orc):
    M, K, N = 5, 128, 33
    x, w, Wt, b = _inputs(M, K, N, 70)
    _, e0, c0 = orc.rmsnorm_linear(x, w, Wt, None, 1e-6, 1.0, BF16, want_exact=True)
    _, e1, c1 = orc.rmsnorm_linear(x, w, Wt, b, 1e-6, -3.0, BF16, want_exact=True)
    bv = bf16_bits_to_f32(b).astype(np.float64)
    np.testing.assert_allclose(e1, -3.0 * (e0 + bv), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(c1, 3.0 * c0, rtol=1e-15)
    assert (c0 >= np.abs(e0) * (1 - 1e-12)).all()


@pytest.mark.parametrize("dt", [F16, F32])
def test_other_dtypes_against_torch(orc, dt):
    M, K, N = 7, 96, 20
    rng = np.random.default_rng(3)
    np_dt = np.float16 if dt == F16 else np.float32
    x = rng.standard_normal((M, K)).astype(np_dt)
    w = (1 + 0.1 * rng.standard_normal(K)).astype(np_dt)
    Wt = (rng.standard_normal((N, K)) / np.sqrt(K)).astype(np_dt)
    raw = (lambda a: a.view(np.uint16)) if dt == F16 else (lambda a: a)
    out = orc.rmsnorm_linear(raw(x), raw(w), raw(Wt), None, 1e-6, 1.0, dt)
    xt = torch.from_numpy(x.astype(np.float64))
    # fp16: the product is exact in fp32; fp32: the listing's fp32 array rounds it
    a = torch.from_numpy((x.astype(np.float64) * w.astype(np.float64)).astype(np.float32)
                         .astype(np.float64))
    rstd = 1.0 / torch.sqrt((xt * xt).mean(dim=1, keepdim=True) + float(np.float32(1e-6)))
    ref = (rstd * (a @ torch.from_numpy(Wt.astype(np.float64)).t())).numpy().astype(np_dt)
    got = out.view(np.float16) if dt == F16 else out
    assert (got == ref).mean() > 0.99
    np.testing.assert_allclose(got.astype(np.float64), ref.astype(np.float64),
                               rtol=2.0 ** -10 if dt == F16 else 1e-6, atol=1e-6)


def test_eager_close(orc):
    M, K, N = 4, 1024, 64
    x, w, Wt, b = _inputs(M, K, N, 80)
    f, fe, cond = orc.rmsnorm_linear(x, w, Wt, b, 1e-6, 0.5, BF16, want_exact=True)
    e, ee, _ = orc.rmsnorm_linear(x, w, Wt, b, 1e-6, 0.5, BF16, eager=True, want_exact=True)
    # the unfused form rounds each normalised operand (<= 2^-9 relative per
    # term), the GEMM result and the scaled output: the two definitions differ
    # by at most 2^-9 of the terms' total size plus two output roundings
    bv = np.abs(bf16_bits_to_f32(b).astype(np.float64)) * 0.5
    lim = 2.0 ** -9 * (cond + bv) + 2.0 ** -8 * np.abs(fe) + 2.0 ** -8 * bv
    assert (np.abs(fe - ee) <= lim).all()
    assert (ulp_dist16(f, e) <= 2).mean() > 0.8


def test_rejects(orc):
    x = np.zeros((2, 4), np.float32)
    with pytest.raises(ValueError):
        orc.rmsnorm_linear(x, None, np.zeros((3, 5), np.float32), None, 1e-6, 1.0, F32)
    with pytest.raises(ValueError):
        orc.rmsnorm_linear(x, None, np.zeros((3, 4), np.float32), None, 0.0, 1.0, F32)


def test_eager_hand_worked(orc):
    """The unfused form stores y = x rstd w (the RMSNorm kernel's output) and
    z = y Wt^T + bias (the GEMM's output) in bf16 before the scale kernel.
    K = 4, N = 2, scale 0.75, by hand:
      x = (1.21875, 0.58203125, 1.3984375, -1.375), mean x^2 = 1.417602539,
      rstd = 1/sqrt(1.417602539 + 1e-6) = 0.839893768
      w = (1.171875, 0.8125, 0.84765625, 0.83984375): x rstd w =
          (1.199555308, 0.397186091, 0.995605274, -0.969896856) -> bf16
          (1.203125, 0.396484375, 0.99609375, -0.96875)
      Wt = ((0.55078125, 0.00921630859375, 0.84375, 0.94921875),
            (0.90625, 0.228515625, -0.296875, 0.9140625)),
      bias = (0.09326171875, -0.12158203125):
      z = (0.680472970, -0.121860504) -> bf16 (0.6796875, -0.1220703125)
      out = 0.75 z = (0.509765625, -0.091552734375) -> bf16 (0.5078125,
          -0.091796875) (bits 0x3F02, 0xBDBC)
    Fused (one rounding of the exact value): 0x3F02, 0xBDC1. Skipping either
    intermediate rounding changes the eager result."""
    bf = lambda v: synth.to_bf16_bits(np.array(v, np.float32))
    x = bf([[1.21875, 0.58203125, 1.3984375, -1.375]])
    w = bf([1.171875, 0.8125, 0.84765625, 0.83984375])
    Wt = bf([[0.55078125, 0.00921630859375, 0.84375, 0.94921875],
             [0.90625, 0.228515625, -0.296875, 0.9140625]])
    b = bf([0.09326171875, -0.12158203125])
    e = orc.rmsnorm_linear(x, w, Wt, b, 1e-6, 0.75, BF16, eager=True)
    assert [int(v) for v in e[0]] == [0x3F02, 0xBDBC]
    f = orc.rmsnorm_linear(x, w, Wt, b, 1e-6, 0.75, BF16)
    assert [int(v) for v in f[0]] == [0x3F02, 0xBDC1]
