"""Pins for the oracle's residual-add + RMSNorm.

Source: the TeleTron write-up (2kiu.com/news/5927820), section 3.3 (residual
and normalisation fused: a per-row reduction, then elementwise scaling, with
float accumulation) and section 4.2 (the RMSNorm half of the fused
RMSNorm + linear + scale kernel: a per-row sum of squares, the reciprocal
square root of mean + 1e-6, half-precision data with fp32 accumulation).

Pins: exact rational arithmetic on tiny rows (fractions + 60-digit decimal
square root), the constant-row closed form (out = sign(c) * w), the zero row,
the stored h against torch's bfloat16 add, scale invariance, and the
mean-square invariant.
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


def _bf16_from_f64(v):
    return torch.tensor(np.asarray(v, np.float64)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_brute_force_exact_rationals(orc):
    rng = np.random.default_rng(0)
    rows, cols = 2, 8
    x = synth.to_bf16_bits(rng.standard_normal((rows, cols)).astype(np.float32))
    r = synth.to_bf16_bits(rng.standard_normal((rows, cols)).astype(np.float32))
    w = synth.to_bf16_bits((1 + 0.1 * rng.standard_normal(cols)).astype(np.float32))
    eps = np.float32(1e-6)
    h_got, out_got = orc.add_rmsnorm(x, r, w, float(eps), BF16)
    xv, rv, wv = (bf16_bits_to_f32(a).astype(np.float64) for a in (x, r, w))
    for i in range(rows):
        # x + r is exact in float64 for bf16 operands of these magnitudes
        h = _bf16_from_f64(xv[i] + rv[i])
        assert np.array_equal(h, h_got[i])
        hv = bf16_bits_to_f32(h).astype(np.float64)
        ms = sum(Fraction(float(t)) ** 2 for t in hv) / cols
        den = Decimal(ms.numerator) / Decimal(ms.denominator) + Decimal(float(eps))
        rstd = 1 / den.sqrt()
        want = [float(Decimal(float(hv[j])) * rstd * Decimal(float(wv[j]))) for j in range(cols)]
        assert np.array_equal(_bf16_from_f64(want), out_got[i])


def test_constant_row_gives_signed_weight(orc):
    cols = 4096
    w = synth.normal((cols,), 99, "bf16", mean=1.0, std=0.1)
    cs = [1.0, -1.0, 0.0625, -0.0625, 3.5, -100.0, 0.25]
    x = synth.to_bf16_bits(np.repeat(np.array(cs, np.float32)[:, None], cols, axis=1))
    _, out = orc.add_rmsnorm(x, None, w, 1e-6, BF16)
    for i, c in enumerate(cs):
        want = w if c > 0 else (w ^ np.uint16(0x8000))
        assert np.array_equal(out[i], want), c


def test_zero_row(orc):
    x = np.zeros((1, 64), np.uint16)
    _, out = orc.add_rmsnorm(x, None, None, 1e-6, BF16)
    assert not out.any()


def test_h_matches_torch_bf16_add(orc):
    x, r, w = synth.c3_inputs(rows=64, cols=512, seed=3)
    h, _ = orc.add_rmsnorm(x, r, w, 1e-6, BF16)
    tx = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    tr = torch.from_numpy(r.view(np.int16)).view(torch.bfloat16)
    ref = (tx + tr).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(h, ref)


def test_scale_invariance(orc):
    x, r, w = synth.c3_inputs(rows=32, cols=1024, seed=4)
    _, o1 = orc.add_rmsnorm(x, r, w, 1e-6, BF16)
    # doubling x and r (exact in bf16) and quadrupling eps leaves out unchanged
    x2 = synth.to_bf16_bits(bf16_bits_to_f32(x) * 2)
    r2 = synth.to_bf16_bits(bf16_bits_to_f32(r) * 2)
    _, o2 = orc.add_rmsnorm(x2, r2, w, float(np.float32(1e-6) * 4), BF16)
    assert np.array_equal(o1, o2)


def test_mean_square_invariant(orc):
    x, r, _ = synth.c3_inputs(rows=16, cols=2048, seed=5)
    h, out, exact = orc.add_rmsnorm(x, r, None, 1e-6, BF16, want_exact=True)
    hv = bf16_bits_to_f32(h).astype(np.float64)
    ms = (hv ** 2).mean(axis=1)
    got = (exact ** 2).mean(axis=1)
    np.testing.assert_allclose(got, ms / (ms + 1e-6), rtol=1e-12)


def test_unit_weight_equals_weight_inside_norm_form(orc):
    """With w = 1 the standard form equals TeleTron's sec. 4.2 form, which
    normalises v * w (not v): both are h / sqrt(mean(h^2) + eps)."""
    x, r, _ = synth.c3_inputs(rows=8, cols=256, seed=6)
    ones = synth.to_bf16_bits(np.ones(256, np.float32))
    _, a = orc.add_rmsnorm(x, r, ones, 1e-6, BF16)
    _, b = orc.add_rmsnorm(x, r, None, 1e-6, BF16)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("dt,np_dt", [(F16, np.float16), (F32, np.float32)])
def test_other_dtypes(orc, dt, np_dt):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((4, 96)).astype(np_dt)
    r = rng.standard_normal((4, 96)).astype(np_dt)
    h, out = orc.add_rmsnorm(x.view(np.uint16) if dt == F16 else x,
                             r.view(np.uint16) if dt == F16 else r, None, 1e-6, dt)
    hv = (x.astype(np.float64) + r.astype(np.float64)).astype(np_dt).astype(np.float64)
    got_h = (h.view(np.float16) if dt == F16 else h).astype(np.float64)
    assert np.array_equal(got_h, hv)
    ref = hv / np.sqrt((hv ** 2).mean(axis=1, keepdims=True) + float(np.float32(1e-6)))
    got = (out.view(np.float16) if dt == F16 else out).astype(np.float64)
    np.testing.assert_allclose(got, ref, rtol=2.0 ** -10 if dt == F16 else 1e-7)


def test_eager_close(orc):
    x, r, w = synth.c3_inputs(rows=8, cols=4096, seed=8)
    _, f = orc.add_rmsnorm(x, r, w, 1e-6, BF16)
    _, e = orc.add_rmsnorm(x, r, w, 1e-6, BF16, eager=True)
    assert ulp_dist16(f, e).max() <= 4


def test_rejects_bad_eps(orc):
    x = np.zeros((1, 8), np.uint16)
    with pytest.raises(ValueError):
        orc.add_rmsnorm(x, None, None, 0.0, BF16)


def test_eager_hand_worked(orc):
    """The six-kernel unfused form stores each step in bf16 (add; square; row
    mean; +eps and 1/sqrt; x rstd; x w). One row h = (-2.421875, 0.6640625,
    0.7109375) (r = NULL), w = (0.8671875, 1.1640625, 0.88671875), worked by
    hand:
      h^2 = 5.865478515625, 0.44097900390625, 0.505432128906 -> bf16 5.875,
            0.44140625, 0.50390625
      mean = 6.8203125 / 3 = 2.2734375 -> bf16 2.28125
      1/sqrt(2.28125 + 1e-6) = 0.662084566 -> bf16 0.66015625
      h rstd = -1.598815918, 0.438385010, 0.469329834 -> bf16 -1.6015625,
            0.4375, 0.46875
      x w = -1.388854980, 0.50927734375, 0.415649414 -> bf16 -1.390625,
            0.5078125, 0.416015625 (bits 0xBFB2, 0x3F02, 0x3ED5)
    The fused form (one rounding) gives 0xBFB2, 0x3F03, 0x3ED6; skipping any
    one of the four intermediate roundings changes the eager result."""
    h = synth.to_bf16_bits(np.array([[-2.421875, 0.6640625, 0.7109375]], np.float32))
    w = synth.to_bf16_bits(np.array([0.8671875, 1.1640625, 0.88671875], np.float32))
    _, e = orc.add_rmsnorm(h, None, w, 1e-6, BF16, eager=True)
    assert [int(v) for v in e[0]] == [0xBFB2, 0x3F02, 0x3ED5]
    _, f = orc.add_rmsnorm(h, None, w, 1e-6, BF16)
    assert [int(v) for v in f[0]] == [0xBFB2, 0x3F03, 0x3ED6]
