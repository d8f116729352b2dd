"""Value ranges of the fp16-output runtime specialiser (host only, no GPU).

For chains whose output is fp16 the specialiser works out, in front of every
tanh, an interval that holds the tanh's argument for every possible input, and
emits a cheaper tanh where the interval allows it (a short odd Taylor
polynomial for small arguments, no branch or sign handling for one-signed
ones). It writes each interval into the generated source as a comment. Here
every fp16 input that is not NaN (finite values, both zeros, both infinities)
is pushed through the chain prefix in front of each tanh by the oracle, and
the values must lie inside the interval written for that tanh.
"""
import re

import numpy as np
import pytest

import synth

F32, F16 = 0, 1
RANGE_RE = re.compile(r"// tanh argument in \[(\S+), (\S+)\]")


@pytest.fixture(scope="module")
def npa():
    import norm_pass_amd
    return norm_pass_amd


def every_fp16():
    x = np.arange(1 << 16, dtype=np.uint16).view(np.float16)
    return x[~np.isnan(x)]


def tanh_ranges(npa, ops):
    src = npa.np_chain_source(ops, 1, npa.NP_F16, npa.NP_F16, 0)
    return [(float.fromhex(lo), float.fromhex(hi)) for lo, hi in RANGE_RE.findall(src)], src


CHAINS = ([synth.c5_chain()] + [synth.c5_chain(n_ops=29, seed=s) for s in range(200, 216)]
          + [synth.c5_chain(n_ops=12, seed=s) for s in range(300, 316)])


@pytest.mark.parametrize("ci", range(len(CHAINS)))
def test_tanh_ranges_hold_every_input(npa, orc, ci):
    ops = CHAINS[ci]
    ranges, _ = tanh_ranges(npa, ops)
    at = [i for i, o in enumerate(ops) if o[0] == synth.TANH]
    assert len(ranges) == len(at)
    x = every_fp16()
    for (lo, hi), i in zip(ranges, at):
        v = orc.chain(ops[:i], [x], F32).astype(np.float64)  # the tanh's argument
        v = v[~np.isnan(v)]
        assert lo <= hi
        assert v.min() >= lo and v.max() <= hi, (ci, i, lo, hi, v.min(), v.max())


def test_seed29_tanh_forms(npa):
    """The workload chain: its first tanh sees only values <= 0, the other four
    small positive ones, so none needs the general two-sided form."""
    ranges, src = tanh_ranges(npa, synth.c5_chain())
    assert len(ranges) == 5
    body = src[src.index("float chain("):src.index("return v;")]
    assert "np_fast_tanh_k(" not in body
    assert ranges[0][1] == 0.0 and all(lo > 0 and hi < 0.625 for lo, hi in ranges[1:])
    assert body.count("np_fast_tanh_neg_k(") == 1 and body.count("np_fast_tanh_poly_k(") == 1


def test_general_tanh_when_the_range_is_unknown(npa):
    """A tanh straight after the load (any input) keeps the two-sided form; a
    tanh after an exp (argument >= 0) takes the one-signed one."""
    ops = [(synth.LOAD, 0, 0.0), (synth.TANH, 0, 0.0)]
    ranges, src = tanh_ranges(npa, ops)
    assert ranges == [(-np.inf, np.inf)] and "np_fast_tanh_k(v, " in src
    ops = [(synth.LOAD, 0, 0.0), (synth.EXP, 0, 0.0), (synth.TANH, 0, 0.0)]
    ranges, src = tanh_ranges(npa, ops)
    assert ranges[0][0] == 0.0 and "np_fast_tanh_pos_k(v, " in src


def test_identity_for_tiny_arguments(npa):
    """tanh x = x to 2^-26 once |x| <= 2^-13: nothing is emitted."""
    ops = [(synth.LOAD, 0, 0.0), (synth.TANH, 0, 0.0), (synth.MUL_C, 0, 2.0 ** -14),
           (synth.TANH, 0, 0.0)]
    ranges, src = tanh_ranges(npa, ops)
    assert ranges[1][1] <= 2.0 ** -13 and "(tanh x = x there)" in src


def test_pinned_tanh_coefficient_matches_fastmath(npa):
    """The specialiser passes the minimax polynomial's leading coefficient to
    np_fast_tanh_*_k from a pinned register: its value must be the one
    fastmath.h's own np_fast_tanh_poly uses (NP_TANH_P4)."""
    import os
    import struct
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "norm_pass_amd", "csrc", "fastmath.h")).read()
    m = re.search(r"#define NP_TANH_P4 (\S+)f", hdr)
    want = struct.unpack("f", struct.pack("f", float(m.group(1))))[0]
    ops = [(synth.LOAD, 0, 0.0), (synth.TANH, 0, 0.0)]
    src = npa.np_chain_source(ops, 1, npa.NP_F16, npa.NP_F16, 0)
    k = re.search(r"np_fast_tanh_k\(v, kp\[(\d+)\]\)", src)
    pins = re.search(r"const float kp\[\d+\] = \{([^}]*)\}", src).group(1)
    # np_pin(<hex float>f): the exponent is decimal, so the only trailing f is the suffix
    vals = [float.fromhex(p.strip()[len("np_pin("):-1].rstrip("f")) for p in pins.split(",")]
    assert vals[int(k.group(1))] == want
