"""Pins for the oracle's QKV split + RoPE + Q scale.

Source: the TeleTron write-up (2kiu.com/news/5927820), section 3.1 (the QKV
projection followed by multi-head split, rotary position encoding and scaling
as one fused group) and section 1.1 (RoPE among the hot small operators). The
pages name RoPE without defining it; the rotate-half form with pairs (d, d+64),
base 10000 and the fp32 angle is the plain reading.

Pins: the inverse-frequency table against 60-digit decimal arithmetic, the
rotation against Python complex multiplication (u + i w) * e^(i theta), the
position-0 identity, pair-norm preservation, the unit-vector angle table, and a
unique-value marker for the head-major layout.
"""
import cmath
import math
from decimal import Decimal, getcontext

import numpy as np
import pytest

import synth
from oracle import BF16, F32
from tolerance import bf16_bits_to_f32

getcontext().prec = 60
QS = float(np.float32(1.0 / math.sqrt(128.0)))


def test_inv_freq_correctly_rounded(orc):
    inv = orc.rope_inv_freq(10000.0, 128)
    ln = Decimal(10000).ln()
    for i, v in enumerate(inv):
        true = (-(Decimal(2 * i) / Decimal(128)) * ln).exp()
        half_ulp = Decimal(float(np.spacing(np.float32(v)))) / 2
        # nearest binary32 (spacing below a power of two is half as wide)
        assert abs(Decimal(float(v)) - true) <= half_ulp, i


def _qkv_f32(T, H, D, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, 3 * H * D)).astype(np.float32)


def test_rotation_against_complex_multiplication(orc):
    T, H, D = 5, 2, 8
    qkv = _qkv_f32(T, H, D, 1)
    pos = np.array([0, 1, 7, 1000, 16383], np.int32)
    q, k, v, eq, ek, _, _ = orc.qkv_rope(qkv, H, D, 10000.0, QS, F32, positions=pos,
                                         want_bound=True)
    inv = orc.rope_inv_freq(10000.0, D)
    P = qkv.reshape(T, 3, H, D).astype(np.float64)
    for t in range(T):
        for h in range(H):
            for i in range(D // 2):
                theta = float(np.float32(np.float32(pos[t]) * inv[i]))
                for s, ex, scale in ((0, eq, QS), (1, ek, 1.0)):
                    z = complex(P[t, s, h, i], P[t, s, h, i + D // 2]) * cmath.exp(1j * theta)
                    assert ex[h, t, i] == pytest.approx(z.real * scale, rel=1e-12, abs=1e-12)
                    assert ex[h, t, i + D // 2] == pytest.approx(z.imag * scale, rel=1e-12,
                                                                 abs=1e-12)
    assert np.array_equal(v, P[:, 2].transpose(1, 0, 2).astype(np.float32))


def test_position_zero_is_identity(orc):
    T, H, D = 1, 3, 128
    qkv = synth.c4_inputs(tokens=T, heads=H, head_dim=D, seed=2)
    q, k, v = orc.qkv_rope(qkv, H, D, 10000.0, QS, BF16)
    P = qkv.reshape(T, 3, H, D)
    assert np.array_equal(k[:, 0], P[0, 1])
    assert np.array_equal(v[:, 0], P[0, 2])
    want_q = synth.to_bf16_bits(bf16_bits_to_f32(P[0, 0]).astype(np.float64) * QS)
    # x * qs computed in float64 is exact for bf16 x; one rounding to bf16
    assert np.array_equal(q[:, 0], want_q)


def test_pair_norm_preserved(orc):
    T, H, D = 64, 2, 128
    qkv = synth.c4_inputs(tokens=T, heads=H, head_dim=D, seed=3)
    pos = np.arange(T, dtype=np.int32) * 257
    _, _, _, eq, ek, _, _ = orc.qkv_rope(qkv, H, D, 10000.0, QS, BF16, positions=pos,
                                         want_bound=True)
    P = bf16_bits_to_f32(qkv).astype(np.float64).reshape(T, 3, H, D)
    for s, ex, sc in ((0, eq, QS), (1, ek, 1.0)):
        u = P[:, s, :, :64].transpose(1, 0, 2)
        w = P[:, s, :, 64:].transpose(1, 0, 2)
        n_in = (u ** 2 + w ** 2) * sc * sc
        n_out = ex[..., :64] ** 2 + ex[..., 64:] ** 2
        np.testing.assert_allclose(n_out, n_in, rtol=1e-12, atol=1e-300)


def test_unit_vector_gives_angle_table(orc):
    T, H, D = 16384, 1, 128
    qkv = np.zeros((T, 3, H, D), np.float32)
    qkv[:, :2, :, :64] = 1.0
    sel = np.array([0, 1, 2, 3, 100, 4095, 8191, 12345, 16383], np.int32)
    qkvs = qkv[sel].reshape(len(sel), -1)
    q, k, v = orc.qkv_rope(qkvs, H, D, 10000.0, QS, F32, positions=sel)
    inv = orc.rope_inv_freq(10000.0, D)
    for j, t in enumerate(sel):
        theta = (np.float32(t) * inv).astype(np.float64)  # binary32 products
        want_c = np.array([math.cos(a) for a in theta]).astype(np.float32)
        want_s = np.array([math.sin(a) for a in theta]).astype(np.float32)
        assert np.array_equal(k[0, j, :64], want_c)
        assert np.array_equal(k[0, j, 64:], want_s)


def test_layout_marker(orc):
    T, H, D = 6, 3, 8
    vals = np.arange(T * 3 * H * D, dtype=np.float32) + 1.0  # unique, exact in fp32
    qkv = vals.reshape(T, 3 * H * D)
    pos = np.zeros(T, np.int32)  # identity rotation: values move without change
    q, k, v = orc.qkv_rope(qkv, H, D, 10000.0, 1.0, F32, positions=pos)
    P = vals.reshape(T, 3, H, D)
    for h in range(H):
        for t in range(T):
            assert np.array_equal(q[h, t], P[t, 0, h])
            assert np.array_equal(k[h, t], P[t, 1, h])
            assert np.array_equal(v[h, t], P[t, 2, h])


def test_eager_q_double_rounding_close(orc):
    qkv = synth.c4_inputs(tokens=32, heads=2, head_dim=128, seed=9)
    q1, k1, _ = orc.qkv_rope(qkv, 2, 128, 10000.0, QS, BF16)
    q2, k2, _ = orc.qkv_rope(qkv, 2, 128, 10000.0, QS, BF16, eager=True)
    assert np.array_equal(k1, k2)
    d = np.abs(q1.view(np.int16).astype(np.int32) - q2.view(np.int16).astype(np.int32))
    assert d.max() <= 1


def test_eager_hand_worked(orc):
    """The unfused form stores the rotated Q in bf16 before the scale kernel.
    T = 2, one head, head_dim 2 (one pair, inv_0 = 1), so token 1 has angle
    exactly 1 rad. With (u, w) = (2.546875, 0.005035400390625), by hand:
      o = (u cos 1 - w sin 1, w cos 1 + u sin 1) = (1.371845292, 2.145842053)
      eager Q: bf16(o) = (1.375, 2.140625); x fl32(1/sqrt 128) =
               (0.121533976, 0.189207...) -> bf16 (0.12158203125, 0.189453125)
               (bits 0x3DF9, 0x3E42)
      fused Q: o x q_scale = (0.121255137, ...) -> bf16 (0.12109375, ...)
               (bits 0x3DF8, 0x3E42)
    K carries no intermediate rounding, so both forms give bf16(o) = (1.375,
    2.140625) (bits 0x3FB0, 0x4009)."""
    u, w = 2.546875, 0.005035400390625
    qkv = synth.to_bf16_bits(np.array([[0, 0, 0, 0, 0, 0], [u, w, u, w, u, w]], np.float32))
    q, k, _ = orc.qkv_rope(qkv, 1, 2, 10000.0, QS, BF16, eager=True)
    assert [int(x) for x in q[0, 1]] == [0x3DF9, 0x3E42]
    assert [int(x) for x in k[0, 1]] == [0x3FB0, 0x4009]
    q2, k2, _ = orc.qkv_rope(qkv, 1, 2, 10000.0, QS, BF16)
    assert [int(x) for x in q2[0, 1]] == [0x3DF8, 0x3E42]
    assert [int(x) for x in k2[0, 1]] == [0x3FB0, 0x4009]
