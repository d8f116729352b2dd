"""Pins for the oracle's elementwise chains (relu(a+b)*0.5 and the seeded 29-op chain).

Sources: the DeepJIT write-up (hotelren.com/news/5350627), sections 3.2-4.2,
give the fused add -> relu -> scale kernel (t = a + b; t > 0 ? t : 0; t *
scale); the NaiveRT write-up (zhaixingw.cn/coding/291.html) gives the
29-call layer. The pins below are hand-worked values, closed forms, exact
special cases, and exhaustive one-op chains over every fp16 input checked
against Python's math library in double precision rounded by numpy's
correctly rounded double -> half cast.
"""
import math

import numpy as np
import pytest

import synth
from oracle import F16, F32, BF16
from tolerance import ulp_dist16

LOAD, ADD_IN, MUL_IN, ADD_C, MUL_C, SCALE, RELU, SIGMOID, EXP, TANH, CAST_F16, CAST_BF16 = range(12)
C1 = synth.C1_CHAIN


def test_c1_hand_values(orc):
    a = np.array([1.0, -3.0, 2.5, -2.5, 2.0 ** -126, 0.0, -0.0, 1e30, 3 * 2.0 ** -149],
                 np.float32)
    b = np.array([2.0, 1.0, -2.5, 2.5, 2.0 ** -126, -0.0, -0.0, 1e30, 0.0], np.float32)
    y = orc.chain(C1, [a, b], F32)
    want = np.array([1.5, 0.0, 0.0, 0.0, 2.0 ** -126, 0.0, 0.0, 1e30, 2 * 2.0 ** -149],
                    np.float32)
    assert np.array_equal(y.view(np.uint32), want.view(np.uint32))  # never -0


def test_c1_running_value_has_binary32_range(orc):
    """t = a + b is held in a float register (DeepJIT write-up, section 3.2): a sum
    beyond the binary32 range is inf even though t * 0.5 would fit."""
    a = np.array([3e38, -3e38, 1.8e38, 1.7e38], np.float32)
    b = np.array([3e38, -3e38, 1.8e38, 1.7e38], np.float32)
    y = orc.chain(C1, [a, b], F32)
    assert np.isposinf(y[0]) and y[1] == 0 and np.isposinf(y[2])
    assert y[3] == np.float32(1.7e38)  # 3.4e38 still fits binary32


def test_c1_invariants(orc):
    a, b = synth.c1_inputs(1 << 16, seed=7)
    y = orc.chain(C1, [a, b], F32)
    s = a + b  # binary32 add, correctly rounded
    assert (y >= 0).all() and not np.signbit(y).any()
    assert np.array_equal(y == 0, s <= 0)
    pos = s > 0
    # scaling by 0.5 is exact outside the subnormal range
    assert np.array_equal((y[pos] * 2).view(np.uint32), s[pos].view(np.uint32))


def test_c1_eager_equals_fused(orc):
    a, b = synth.c1_inputs(1 << 14, seed=8)
    f = orc.chain(C1, [a, b], F32)
    e = orc.chain(C1, [a, b], F32, eager=True)
    assert np.array_equal(f.view(np.uint32), e.view(np.uint32))


def _all_f16():
    bits = np.arange(65536, dtype=np.uint16)
    v = bits.view(np.float16)
    return v[np.isfinite(v)]


def _round16(x):
    with np.errstate(over="ignore", invalid="ignore"):
        return np.asarray(x, np.float64).astype(np.float16)


def _math_sigmoid(t):
    # independent route: sigma(t) = (1 + tanh(t/2)) / 2
    return (1.0 + math.tanh(t / 2.0)) / 2.0


@pytest.mark.parametrize("kind,c,fn", [
    (EXP, 0.0, math.exp),
    (SIGMOID, 0.0, _math_sigmoid),
    (TANH, 0.0, math.tanh),
    (ADD_C, 0.883171, None),
    (MUL_C, -0.563752, None),
    (SCALE, 0.483334, None),
    (CAST_F16, 0.0, lambda t: t),
])
def test_c5_one_op_exhaustive(orc, kind, c, fn):
    """Every finite fp16 input through a one-op chain vs math-library double."""
    x = _all_f16()
    c32 = float(np.float32(c))
    y = orc.chain([(LOAD, 0, 0.0), (kind, 0, c)], [x], F16)
    xd = x.astype(np.float64)
    if kind == ADD_C:
        ref = xd + c32
    elif kind in (MUL_C, SCALE):
        ref = xd * c32
    else:
        ref = np.array([_safe(fn, t) for t in xd])
    r16 = _round16(ref)
    d = ulp_dist16(y.view(np.uint16), r16.view(np.uint16))
    # both are one rounding of the same real number computed in double; they
    # can only differ where the double values straddle an fp16 tie
    assert (d <= 1).all()
    assert (d == 0).mean() > 0.99999


def _safe(fn, t):
    try:
        return fn(t)
    except OverflowError:
        return math.inf


def test_c5_special_cases(orc):
    z = np.zeros(4, np.float16)
    assert orc.chain([(LOAD, 0, 0), (SIGMOID, 0, 0)], [z], F16)[0] == 0.5
    assert orc.chain([(LOAD, 0, 0), (TANH, 0, 0)], [z], F16)[0] == 0.0
    assert orc.chain([(LOAD, 0, 0), (EXP, 0, 0)], [z], F16)[0] == 1.0
    x = synth.c5_inputs(4096, seed=3)
    once = orc.chain([(LOAD, 0, 0), (CAST_F16, 0, 0)], [x], F16)
    twice = orc.chain([(LOAD, 0, 0), (CAST_F16, 0, 0), (CAST_F16, 0, 0)], [x], F16)
    assert np.array_equal(once.view(np.uint16), x.view(np.uint16))
    assert np.array_equal(once.view(np.uint16), twice.view(np.uint16))
    # add c then add -c is the identity before the single output rounding
    c = float(np.float32(0.3711))
    y = orc.chain([(LOAD, 0, 0), (ADD_C, 0, c), (ADD_C, 0, -c)], [x], F16)
    assert np.array_equal(y.view(np.uint16), x.view(np.uint16))


def test_c5_ranges(orc):
    x = synth.c5_inputs(1 << 14, seed=4)
    for kind, lo, hi in ((SIGMOID, 0.0, 1.0), (TANH, -1.0, 1.0), (EXP, 0.0, np.inf)):
        y = orc.chain([(LOAD, 0, 0), (MUL_C, 0, 3.0), (kind, 0, 0)], [x], F16).astype(np.float64)
        assert (y >= lo).all() and (y <= hi).all()


def test_c5_chain_is_finite_and_bounded(orc):
    ops = synth.c5_chain()
    assert len(ops) == 30 and ops[0][0] == LOAD
    x = synth.c5_inputs(1 << 16)
    y, exact, bound = orc.chain(ops, [x], F16, want_bound=True)
    assert np.isfinite(y.astype(np.float64)).all()
    assert np.isfinite(exact).all() and np.isfinite(bound).all()
    assert np.abs(exact).max() < 65504.0
    # the output still depends on the input (the generator's interval guard)
    assert len(np.unique(y.view(np.uint16))) > 100


def test_chain_bf16_cast_node(orc):
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 3 * 2.0 ** -9], np.float32)
    y = orc.chain([(LOAD, 0, 0), (CAST_BF16, 0, 0)], [x], F32)
    # bfloat16 keeps 8 significand bits: ties go to the even neighbour
    assert list(y) == [1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7]


def test_cast_node_bound(orc):
    """A cast whose input is decided by the last fp32 bit carries a one-ulp bound."""
    x = np.array([1.0, 0.25], np.float16)
    # 1 + 2^-11 is an exact fp16 tie; the fp32 evaluation bound straddles it
    ops = [(LOAD, 0, 0), (ADD_C, 0, 2.0 ** -11), (CAST_F16, 0, 0)]
    y, exact, bound = orc.chain(ops, [x], F16, want_bound=True)
    assert y[0] == 1.0 and bound[0] >= 2.0 ** -10
    assert bound[1] == 0.0


def test_chain_rejects_bad_arguments(orc):
    x = np.zeros(4, np.float32)
    with pytest.raises(ValueError):
        orc.chain([(RELU, 0, 0)], [x], F32)  # must start with a load
    with pytest.raises(ValueError):
        orc.chain([(LOAD, 1, 0)], [x], F32)  # input index out of range
    with pytest.raises(ValueError):
        orc.chain([(LOAD, 0, 0), (99, 0, 0)], [x], F32)


def test_c5_eager_differs_but_close(orc):
    ops = synth.c5_chain()
    x = synth.c5_inputs(1 << 14, seed=5)
    f = orc.chain(ops, [x], F16)
    e = orc.chain(ops, [x], F16, eager=True)
    d = ulp_dist16(f.view(np.uint16), e.view(np.uint16))
    assert d.max() > 0  # rounding after every op changes bits (NaiveRT pitfalls list)
    assert np.abs(f.astype(np.float64) - e.astype(np.float64)).max() < 0.05


# Hand-worked eager (unfused) cases. The unfused chain stores the running value
# in the storage type after every operator (each small kernel writes its
# tensor: DeepJIT write-up, section 1.1), the fused chain rounds once at the
# end. Each case is op, then "subtract the stored value", so the eager result
# is exactly 0 and the fused one is the rounding residual; an eager mode that
# skipped the rounding after that op would return the residual instead.
_EAGER_CASES = [
    # 1 + 2^-11 is the midpoint of 1 and 1 + 2^-10: ties-to-even gives 1;
    # the fused value 2^-11 is an fp16 normal (bits 0x1000)
    ("add_c", [(LOAD, 0, 0.0), (ADD_C, 0, 2.0 ** -11), (ADD_C, 0, -1.0)], [[1.0]], 0x1000),
    ("add_in", [(LOAD, 0, 0.0), (ADD_IN, 1, 0.0), (ADD_C, 0, -1.0)], [[1.0], [2.0 ** -11]], 0x1000),
    # (1 + 2^-10)^2 = 1 + 2^-9 + 2^-20 -> fp16 1 + 2^-9; fused residual 2^-20,
    # the fp16 subnormal 16 * 2^-24 (bits 0x0010)
    ("mul_c", [(LOAD, 0, 0.0), (MUL_C, 0, 1 + 2.0 ** -10), (ADD_C, 0, -(1 + 2.0 ** -9))],
     [[1 + 2.0 ** -10]], 0x0010),
    ("scale", [(LOAD, 0, 0.0), (SCALE, 0, 1 + 2.0 ** -10), (ADD_C, 0, -(1 + 2.0 ** -9))],
     [[1 + 2.0 ** -10]], 0x0010),
    ("mul_in", [(LOAD, 0, 0.0), (MUL_IN, 1, 0.0), (ADD_C, 0, -(1 + 2.0 ** -9))],
     [[1 + 2.0 ** -10], [1 + 2.0 ** -10]], 0x0010),
    # sigma(1) = 0.7310585786 -> fp16 0.73095703125 (1497 * 2^-11); residual
    # 1.015474e-4 -> 1704 * 2^-24 = 1.015663e-4 (bits 0x06A8)
    ("sigmoid", [(LOAD, 0, 0.0), (SIGMOID, 0, 0.0), (ADD_C, 0, -0.73095703125)], [[1.0]], 0x06A8),
    # e = 2.7182818285 -> fp16 2.71875 (1392 * 2^-9); residual -4.681715e-4
    # -> -1964 * 2^-22 (bits 0x8FAC)
    ("exp", [(LOAD, 0, 0.0), (EXP, 0, 0.0), (ADD_C, 0, -2.71875)], [[1.0]], 0x8FAC),
    # tanh(1/2) = 0.4621171573 -> fp16 0.462158203125 (1893 * 2^-12); residual
    # -4.104586e-5 -> -689 * 2^-24 (bits 0x82B1)
    ("tanh", [(LOAD, 0, 0.0), (TANH, 0, 0.0), (ADD_C, 0, -0.462158203125)], [[0.5]], 0x82B1),
]


@pytest.mark.parametrize("name,ops,ins,fused_bits", _EAGER_CASES, ids=[c[0] for c in _EAGER_CASES])
def test_eager_rounds_after_every_op_hand_worked(orc, name, ops, ins, fused_bits):
    arrays = [np.array(v, np.float16) for v in ins]
    e = orc.chain(ops, arrays, F16, eager=True).view(np.uint16)
    f = orc.chain(ops, arrays, F16).view(np.uint16)
    assert int(e[0]) == 0x0000, name
    assert int(f[0]) == fused_bits, name


def test_eager_bf16_storage_hand_worked(orc):
    """bf16 storage: 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7, stored as 1;
    the fused chain keeps 2^-8 (bf16 bits 0x3B80)."""
    x = synth.to_bf16_bits(np.array([1.0], np.float32))
    ops = [(LOAD, 0, 0.0), (ADD_C, 0, 2.0 ** -8), (ADD_C, 0, -1.0)]
    assert int(orc.chain(ops, [x], BF16, in_dt=BF16, eager=True)[0]) == 0x0000
    assert int(orc.chain(ops, [x], BF16, in_dt=BF16)[0]) == 0x3B80
