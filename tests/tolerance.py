"""Comparison helpers shared by the tests (test-side only; no chain arithmetic).

Tolerances are fixed numbers: fp32 outputs within 1e-6 relative of the oracle,
fp16 / bf16 outputs within 2 units in the last place of the output type,
layout and index work bit-exact. An element that misses the ulp bar may still
pass when it lies within the oracle's fp32 evaluation bound (beta) plus one
output ulp of the exact value -- an ill-conditioned element (cancellation, or a
cast decided by the last fp32 bit). Such exemptions are counted and must stay
below 1e-4 of the elements.
"""
import numpy as np

EXEMPT_FRACTION = 1e-4


def ordinal16(bits: np.ndarray) -> np.ndarray:
    """Map 16-bit float patterns monotonically onto integers (-0 and +0 -> 0)."""
    b = np.asarray(bits).view(np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ordinal32(x: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.int64)
    mag = b & 0x7FFFFFFF
    return np.where(b & 0x80000000, -mag, mag)


def ulp_dist16(a, b) -> np.ndarray:
    return np.abs(ordinal16(a) - ordinal16(b))


def ulp_of(values: np.ndarray, dt: str) -> np.ndarray:
    """Spacing of the output format at |values| (for the exemption bar)."""
    p, emin = {"f16": (11, -14), "bf16": (8, -126), "f32": (24, -126)}[dt]
    a = np.abs(np.asarray(values, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, emin)
    return np.ldexp(1.0, (e - (p - 1)).astype(np.int64))


def check_half(got_bits, ref_bits, dt: str, got_vals=None, exact=None, bound=None,
               max_ulp: int = 2, what: str = ""):
    """Assert fp16/bf16 outputs match: <= max_ulp, else within beta + 1 ulp (counted)."""
    got_bits = np.asarray(got_bits).view(np.uint16).ravel()
    ref_bits = np.asarray(ref_bits).view(np.uint16).ravel()
    assert got_bits.shape == ref_bits.shape
    nan_mask = _is_nan16(got_bits, dt)
    assert not nan_mask.any(), f"{what}: NaN in output"
    d = ulp_dist16(got_bits, ref_bits)
    bad = d > max_ulp
    n_bad = int(bad.sum())
    exempt = 0
    if n_bad:
        assert exact is not None and bound is not None and got_vals is not None, \
            f"{what}: {n_bad} elements beyond {max_ulp} ulp (max {int(d.max())})"
        gv = np.asarray(got_vals, np.float64).ravel()[bad]
        ex = np.asarray(exact, np.float64).ravel()[bad]
        bd = np.asarray(bound, np.float64).ravel()[bad]
        ok = np.abs(gv - ex) <= bd + ulp_of(ex, dt)
        assert ok.all(), (f"{what}: {int((~ok).sum())} elements beyond {max_ulp} ulp and "
                          f"outside the fp32 bound; worst ulp {int(d.max())}")
        exempt = n_bad
        assert exempt <= EXEMPT_FRACTION * got_bits.size + 0.5, \
            f"{what}: {exempt} exempted elements of {got_bits.size}"
    return {"max_ulp": int(d.max()) if d.size else 0, "exempt": exempt, "n": int(d.size)}


def _is_nan16(bits, dt):
    b = bits.astype(np.uint32)
    if dt == "f16":
        return ((b & 0x7C00) == 0x7C00) & ((b & 0x03FF) != 0)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)


def check_f32(got, ref, rel: float = 1e-6, what: str = ""):
    got = np.asarray(got, np.float32).ravel()
    ref = np.asarray(ref, np.float32).ravel()
    assert not np.isnan(got).any(), f"{what}: NaN in output"
    g = got.astype(np.float64)
    r = ref.astype(np.float64)
    err = np.abs(g - r)
    ok = np.where(r == 0, g == 0, err <= rel * np.abs(r))
    assert ok.all(), (f"{what}: {int((~ok).sum())} elements beyond {rel} relative; "
                      f"worst {float((err / np.maximum(np.abs(r), 1e-300)).max()):.3g}")
    return {"max_rel": float((err / np.where(r == 0, 1, np.abs(r))).max()) if g.size else 0.0}


def check_f32_counted(got, ref, exact, bound, rel: float = 1e-6, what: str = ""):
    """fp32 outputs: within rel of the oracle's value (zero only where it is
    zero), else within the oracle's fp32 evaluation bound beta plus one fp32
    ulp of the exact value -- an exemption, counted, at most 1e-4 of the
    elements."""
    got = np.asarray(got, np.float32).ravel()
    r = np.asarray(ref, np.float32).ravel().astype(np.float64)
    assert got.shape == r.shape
    assert not np.isnan(got).any(), f"{what}: NaN in output"
    g = got.astype(np.float64)
    ok = np.where(r == 0, g == 0, np.abs(g - r) <= rel * np.abs(r))
    exempt = 0
    if not ok.all():
        ex = np.asarray(exact, np.float64).ravel()[~ok]
        bd = np.asarray(bound, np.float64).ravel()[~ok]
        within = np.abs(g[~ok] - ex) <= bd + ulp_of(ex, "f32")
        assert within.all(), (f"{what}: {int((~within).sum())} elements beyond {rel} relative "
                              f"and outside the fp32 bound")
        exempt = int((~ok).sum())
        assert exempt <= EXEMPT_FRACTION * got.size + 0.5, \
            f"{what}: {exempt} exempted elements of {got.size}"
    rel_err = np.abs(g - r) / np.where(r == 0, 1.0, np.abs(r))
    return {"max_rel": float(rel_err.max()) if g.size else 0.0, "exempt": exempt, "n": int(g.size)}


def bf16_bits_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits).view(np.uint16).astype(np.uint32) << 16).view(np.float32)


def half_values(bits, dt: str) -> np.ndarray:
    if dt == "f16":
        return np.asarray(bits).view(np.float16).astype(np.float64)
    return bf16_bits_to_f32(bits).astype(np.float64)
