"""Pins for the oracle's residual-add + LayerNorm.

Source: the DeepJIT write-up (hotelren.com/news/5350627), section 4.3 (one
block per row: the row's mean and variance, then normalise and apply gamma and
beta), and the runtime page "CUDA算子与AI运行时" (gtnt.cn/news/145880), section
4.1 (LayerNorm = (x - mean) * rsqrt(var + eps) * gamma + beta).

Pins: torch.nn.functional.layer_norm in float64 on the same rounded h (a
library routine), exact rational arithmetic on tiny rows, the constant-row and
zero-gamma closed forms, and the normalised-moment identities.
"""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import BF16, F16, F32
from tolerance import bf16_bits_to_f32, ulp_dist16

getcontext().prec = 60


def _bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def _to_bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def test_against_torch_layer_norm(orc):
    x, r, g = synth.c3_inputs(rows=64, cols=1024, seed=21)
    b = synth.normal((1024,), 77, "bf16", std=0.1)
    h, out = orc.add_layernorm(x, r, g, b, 1e-5, BF16)
    th = _bf16(x) + _bf16(r)  # bf16 add: fp32 sum rounded once
    assert np.array_equal(_to_bits(th), h)
    ref = F.layer_norm(th.double(), (1024,), _bf16(g).double(), _bf16(b).double(), 1e-5)
    ref_bits = _to_bits(ref.to(torch.bfloat16))
    d = ulp_dist16(out, ref_bits)
    assert d.max() <= 1 and (d == 0).mean() > 0.9999


def test_brute_force_exact_rationals(orc):
    rng = np.random.default_rng(3)
    cols = 8
    x = rng.standard_normal((2, cols)).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(cols)).astype(np.float32)
    b = (0.1 * rng.standard_normal(cols)).astype(np.float32)
    eps = np.float32(1e-5)
    h, out, exact = orc.add_layernorm(x, None, g, b, float(eps), F32, want_exact=True)
    for i in range(2):
        hv = [Fraction(float(v)) for v in x[i]]
        mu = sum(hv) / cols
        var = sum((v - mu) ** 2 for v in hv) / cols
        den = (Decimal(var.numerator) / Decimal(var.denominator) + Decimal(float(eps))).sqrt()
        for j in range(cols):
            d = hv[j] - mu
            want = (Decimal(d.numerator) / Decimal(d.denominator)) / den * Decimal(float(g[j])) \
                + Decimal(float(b[j]))
            assert abs(Decimal(exact[i, j]) - want) <= abs(want) * Decimal(1e-15) + Decimal(1e-300)
            assert out[i, j] == np.float32(float(want))


def test_constant_row_gives_beta(orc):
    cols = 512
    g = synth.normal((cols,), 5, "bf16", mean=1.0, std=0.1)
    b = synth.normal((cols,), 6, "bf16", std=0.5)
    for c in (0.0, 1.0, -3.5, 100.0):
        x = synth.to_bf16_bits(np.full((1, cols), c, np.float32))
        _, out = orc.add_layernorm(x, None, g, b, 1e-5, BF16)
        assert np.array_equal(out[0], b), c  # h - mean is exactly 0


def test_zero_gamma_gives_beta(orc):
    x, r, _ = synth.c3_inputs(rows=4, cols=256, seed=8)
    zero = np.zeros(256, np.uint16)
    b = synth.normal((256,), 9, "bf16")
    _, out = orc.add_layernorm(x, r, zero, b, 1e-5, BF16)
    assert np.array_equal(out, np.broadcast_to(b, out.shape)) or \
        np.array_equal(out & 0x7FFF, np.broadcast_to(b & 0x7FFF, out.shape))


def test_normalised_moments(orc):
    x, r, _ = synth.c3_inputs(rows=16, cols=2048, seed=10)
    h, out, exact = orc.add_layernorm(x, r, None, None, 1e-5, BF16, want_exact=True)
    hv = bf16_bits_to_f32(h).astype(np.float64)
    var = hv.var(axis=1)
    np.testing.assert_allclose(exact.mean(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose((exact ** 2).mean(axis=1), var / (var + 1e-5), rtol=1e-9)


@pytest.mark.parametrize("dt,np_dt", [(F16, np.float16), (F32, np.float32)])
def test_other_dtypes_against_torch(orc, dt, np_dt):
    rng = np.random.default_rng(11)
    x = rng.standard_normal((5, 96)).astype(np_dt)
    g = (1 + 0.1 * rng.standard_normal(96)).astype(np_dt)
    b = (0.1 * rng.standard_normal(96)).astype(np_dt)
    raw = (lambda a: a.view(np.uint16)) if dt == F16 else (lambda a: a)
    _, out = orc.add_layernorm(raw(x), None, raw(g), raw(b), 1e-5, dt)
    ref = F.layer_norm(torch.from_numpy(x.astype(np.float64)), (96,),
                       torch.from_numpy(g.astype(np.float64)),
                       torch.from_numpy(b.astype(np.float64)), 1e-5).numpy().astype(np_dt)
    got = out.view(np.float16) if dt == F16 else out
    assert (got == ref).mean() > 0.999
    np.testing.assert_allclose(got.astype(np.float64), ref.astype(np.float64),
                               rtol=2.0 ** -10 if dt == F16 else 1e-6, atol=1e-6)


def test_eager_close(orc):
    x, r, g = synth.c3_inputs(rows=8, cols=4096, seed=12)
    b = synth.normal((4096,), 13, "bf16", std=0.1)
    _, f = orc.add_layernorm(x, r, g, b, 1e-5, BF16)
    _, e = orc.add_layernorm(x, r, g, b, 1e-5, BF16, eager=True)
    # rounding after every step moves values by a few ulps of the row's scale
    # (outputs near 0, where gamma * y and beta cancel, differ by many of their
    # own ulps)
    fv, ev = bf16_bits_to_f32(f), bf16_bits_to_f32(e)
    assert np.abs(fv - ev).max() < 0.05
    assert (ulp_dist16(f, e) <= 2).mean() > 0.98


def test_rejects_bad_eps(orc):
    with pytest.raises(ValueError):
        orc.add_layernorm(np.zeros((1, 8), np.uint16), None, None, None, -1.0, BF16)


def test_eager_hand_worked(orc):
    """The nine-kernel unfused form stores each step in bf16. One row h =
    (1.828125, 2.28125, -0.27734375), gamma = (1.1875, 0.82421875, 0.859375),
    beta = (-0.009765625, -0.255859375, 0.1845703125), eps 1e-5, by hand:
      mean = 3.83203125 / 3 = 1.27734375 -> bf16 1.28125
      h - mean = 0.546875, 1, -1.55859375 -> bf16 0.546875, 1, -1.5625
      squares = 0.299072265625, 1, 2.44140625 -> bf16 0.298828125, 1, 2.4375
      var = 3.736328125 / 3 = 1.245442708 -> bf16 1.2421875
      1/sqrt(1.2421875 + 1e-5) = 0.897231835 -> bf16 0.8984375
      x rstd = 0.491333008, 0.8984375, -1.403808594 -> bf16 0.4921875,
               0.8984375, -1.40625
      x gamma = 0.58447265625, 0.740509033, -1.20849609375 -> bf16 0.5859375,
               0.7421875, -1.2109375
      + beta = 0.576171875, 0.486328125, -1.0263671875 -> bf16 0.578125,
               0.486328125, -1.0234375 (bits 0x3F14, 0x3EF9, 0xBF83)
    Fused: 0x3F14, 0x3EF9, 0xBF82. Skipping any one of the seven intermediate
    roundings changes the eager result."""
    bf = lambda v: synth.to_bf16_bits(np.array(v, np.float32))
    h = bf([[1.828125, 2.28125, -0.27734375]])
    g = bf([1.1875, 0.82421875, 0.859375])
    b = bf([-0.009765625, -0.255859375, 0.1845703125])
    _, e = orc.add_layernorm(h, None, g, b, 1e-5, BF16, eager=True)
    assert [int(v) for v in e[0]] == [0x3F14, 0x3EF9, 0xBF83]
    _, f = orc.add_layernorm(h, None, g, b, 1e-5, BF16)
    assert [int(v) for v in f[0]] == [0x3F14, 0x3EF9, 0xBF82]
