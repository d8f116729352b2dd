"""Pins for the oracle's own IEEE binary16 / bfloat16 / binary32 converters.

The oracle writes its converters from the bit layouts; here they are checked
against independent library routines (numpy's half-precision casts, torch's
bfloat16 cast, the C cast to float) exhaustively over every 16-bit pattern and
on rounding ties, subnormals and the overflow boundary.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import F16, BF16, F32


def test_f16_decode_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint16)
    ours = orc.decode(bits, F16)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zero survives
    assert np.signbit(ours[0x8000]) and not np.signbit(ours[0])


def test_bf16_decode_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint16)
    ours = orc.decode(bits, BF16)
    ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def _f16_probe_values(rng):
    # every finite fp16 value, the midpoints between neighbours (ties), points a
    # hair either side of the midpoints, random doubles over the whole range
    fin = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (fin[:-1] + fin[1:]) / 2
    eps = np.abs(mids) * 2.0 ** -40 + 2.0 ** -60
    rnd = rng.standard_normal(200000) * np.exp(rng.uniform(-20, 11, 200000))
    v = np.concatenate([fin, mids, mids + eps, mids - eps, rnd,
                        [65504.0, 65519.99, 65520.0, 70000.0, 2.0 ** -25, 2.0 ** -26,
                         3 * 2.0 ** -26, 1e-30]])
    return np.concatenate([v, -v])


def test_f16_rounding_matches_numpy(orc):
    rng = np.random.default_rng(1)
    v = _f16_probe_values(rng)
    ours = orc.round_array(v, F16)
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_rounding_matches_torch(orc):
    rng = np.random.default_rng(2)
    # binary32 inputs (torch rounds float32 -> bfloat16 to nearest even)
    fin = (np.arange(0, 0x7F80, dtype=np.uint32) << 16).view(np.float32)
    mids = (fin[:-1].astype(np.float64) + fin[1:].astype(np.float64)) / 2  # exact in f32
    rnd = (rng.standard_normal(300000) * np.exp(rng.uniform(-80, 80, 300000))).astype(np.float32)
    sub = (rng.integers(1, 1 << 23, 20000).astype(np.uint32)).view(np.float32)
    v = np.concatenate([fin, mids.astype(np.float32), rnd, sub]).astype(np.float32)
    v = np.concatenate([v, -v])
    ours = orc.round_array(v.astype(np.float64), BF16)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f32_rounding_matches_c_cast(orc):
    rng = np.random.default_rng(3)
    v = rng.standard_normal(200000) * np.exp(rng.uniform(-100, 88, 200000))
    f = (np.arange(1, 1 << 16, dtype=np.uint32) * 65521).view(np.float32).astype(np.float64)
    f = f[np.isfinite(f)]
    ulp = np.abs(np.spacing(f.astype(np.float32))).astype(np.float64)
    ties = f + ulp / 2  # exact midpoints in double
    v = np.concatenate([v, ties, -ties, [2.0 ** -149, 1.5 * 2.0 ** -149, 2.5 * 2.0 ** -149]])
    ours = orc.round_array(v, F32)
    ref = v.astype(np.float32)
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("dt", [F16, BF16])
def test_round_trip(orc, dt):
    bits = np.arange(65536, dtype=np.uint16)
    vals = orc.decode(bits, dt)
    fin = np.isfinite(vals)
    back = orc.round_array(vals[fin], dt)
    assert np.array_equal(back, bits[fin])
