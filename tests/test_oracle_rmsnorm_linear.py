"""Pins for the oracle's RMSNorm + linear + scale.

Source: the TeleTron write-up (2kiu.com/news/5927820), section 4.2 (one fused
kernel: the row's RMS factor is computed in the block and used directly in the
linear layer's multiply-accumulate, bias and an elementwise scale follow, no
normalised tensor is stored) and section 3.1 (a norm followed by a projection
in every transformer block).

Pins: torch in float64 on the same rounded operand (library matmul), exact
rational arithmetic on tiny shapes, the K = 1 closed form, the identity
weight (the product reduces to the RMS-normalised row), RMSNorm's scale
invariance (2x with 4 eps), linearity in bias and scale, and closeness of the
three-step unfused form.
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
    a = (_bf16(x).float() * _bf16(w).float()).to(torch.bfloat16).double()  # one RNE rounding
    rstd = 1.0 / torch.sqrt((xt * xt).mean(dim=1, keepdim=True) + eps)
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
    a = bf16_bits_to_f32(synth.to_bf16_bits(xv * bf16_bits_to_f32(w)))  # RNE of the exact product
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
    a = torch.from_numpy((x.astype(np.float64) * w.astype(np.float64)).astype(np_dt).astype(np.float64))
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
