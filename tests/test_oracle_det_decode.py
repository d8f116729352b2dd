"""Pins for the oracle's detection-head decode.

Source: the DeepJIT write-up (hotelren.com/news/5350627), sections 1.1, 2.2 and
5.2: the detector's tail is a run of sigmoid / exp / mul / add / slice / concat /
cast kernels producing the box tensor. The formula (sigmoid on x, y, objectness
and classes, exp(w, h) times the anchor, plus the grid cell, times the stride;
rows ordered level, anchor, y, x) is the plain reading of the workload.

Pins: a one-hot marker over every position of tiny grids (layout, bit-exact),
the exact values at logit 0 (sigmoid(0) = 1/2, exp(0) = 1), the identity
sigmoid(t) = (1 + tanh(t/2))/2 evaluated with Python's math library, and range
invariants.
"""
import math

import numpy as np
import pytest

import synth
from oracle import F16, F32

ANCH = np.array(synth.YOLO_ANCHORS, np.float32).reshape(3, 3, 2)


def _zero_levels(hw, n_anchors, n_ch, batch=1):
    return [np.zeros((batch, n_anchors * n_ch, h, w), np.float16) for h, w in hw]


def _baseline(hw, strides, anchors, n_anchors, n_ch):
    """Expected output when every logit is 0 (exact closed form)."""
    rows = []
    for l, (h, w) in enumerate(hw):
        for a in range(n_anchors):
            for y in range(h):
                for x in range(w):
                    r = [(0.5 + x) * strides[l], (0.5 + y) * strides[l],
                         anchors[l][a][0], anchors[l][a][1]] + [0.5] * (n_ch - 4)
                    rows.append(r)
    return np.array(rows, np.float32)[None]


@pytest.mark.parametrize("hw", [((1, 1), (2, 2)), ((3, 2), (1, 3)), ((2, 3),)])
def test_marker_layout(orc, hw):
    n_anchors, n_ch = 3, 7
    strides = [8.0, 16.0][:len(hw)]
    anchors = ANCH[:len(hw)]
    base = _baseline(hw, strides, anchors, n_anchors, n_ch)
    got0 = orc.det_decode(_zero_levels(hw, n_anchors, n_ch), hw, strides, anchors, n_anchors, n_ch)
    assert np.array_equal(got0, base)
    row_off = 0
    for l, (h, w) in enumerate(hw):
        for a in range(n_anchors):
            for k in range(n_ch):
                for y in range(h):
                    for x in range(w):
                        lv = _zero_levels(hw, n_anchors, n_ch)
                        lv[l][0, a * n_ch + k, y, x] = np.float16(1.0)
                        got = orc.det_decode(lv, hw, strides, anchors, n_anchors, n_ch)
                        diff = np.argwhere(got != base)
                        row = row_off + (a * h + y) * w + x
                        assert diff.tolist() == [[0, row, k]]
        row_off += n_anchors * h * w


def test_logit_zero_closed_form(orc):
    hw = [(h, w) for h, w, _ in synth.YOLO_LEVELS]
    strides = [s for _, _, s in synth.YOLO_LEVELS]
    lv = _zero_levels(hw, 3, 85)
    got = orc.det_decode(lv, hw, strides, ANCH, 3, 85)
    assert got.shape == (1, 25200, 85)
    assert np.array_equal(got, _baseline(hw, strides, ANCH, 3, 85))


def test_sigmoid_and_exp_against_math(orc):
    hw = [(4, 5)]
    lv = synth.c2_inputs(levels=((4, 5, 8.0),), seed=11)
    got = orc.det_decode(lv, hw, [8.0], ANCH[:1], 3, 85)[0]
    t = lv[0][0].astype(np.float64)  # [255, 4, 5]
    n_exact = n_tot = 0
    for a in range(3):
        for y in range(4):
            for x in range(5):
                row = (a * 4 + y) * 5 + x
                tt = t[a * 85:(a + 1) * 85, y, x]
                want = [(0.5 * (1 + math.tanh(tt[0] / 2)) + x) * 8.0,
                        (0.5 * (1 + math.tanh(tt[1] / 2)) + y) * 8.0,
                        math.exp(tt[2]) * float(ANCH[0, a, 0]),
                        math.exp(tt[3]) * float(ANCH[0, a, 1])]
                want += [0.5 * (1 + math.tanh(v / 2)) for v in tt[4:]]
                want = np.array(want, np.float64).astype(np.float32)
                d = np.abs(got[row].view(np.int32).astype(np.int64) - want.view(np.int32))
                assert d.max() <= 1
                n_exact += int((d == 0).sum())
                n_tot += d.size
    assert n_exact >= n_tot - 2


def test_invariants_full_size(orc):
    lv = synth.c2_inputs()
    hw = [(h, w) for h, w, _ in synth.YOLO_LEVELS]
    strides = [s for _, _, s in synth.YOLO_LEVELS]
    out = orc.det_decode(lv, hw, strides, ANCH, 3, 85)[0]
    assert np.isfinite(out).all()
    assert (out[:, 4:] > 0).all() and (out[:, 4:] <= 1).all()
    assert (out[:, 2:4] > 0).all()
    row = 0
    for l, (h, w) in enumerate(hw):
        s = strides[l]
        n = 3 * h * w
        cell = np.arange(n) % (h * w)
        x = cell % w
        y = cell // w
        blk = out[row:row + n]
        assert (blk[:, 0] >= x * s).all() and (blk[:, 0] <= (x + 1) * s).all()
        assert (blk[:, 1] >= y * s).all() and (blk[:, 1] <= (y + 1) * s).all()
        row += n


def test_eager_close_to_fused(orc):
    lv = synth.c2_inputs(levels=((8, 8, 8.0), (4, 4, 16.0)), seed=5)
    hw = [(8, 8), (4, 4)]
    f = orc.det_decode(lv, hw, [8.0, 16.0], ANCH[:2], 3, 85)
    e = orc.det_decode(lv, hw, [8.0, 16.0], ANCH[:2], 3, 85, eager=True)
    # every eager value is an fp16 number; relative gap within a few fp16 ulps
    assert np.array_equal(e.astype(np.float16).astype(np.float32), e)
    rel = np.abs(f.astype(np.float64) - e) / np.abs(f.astype(np.float64))
    assert rel.max() < 4 * 2.0 ** -11


def test_rejects_bad_arguments(orc):
    with pytest.raises(ValueError):
        orc.det_decode(_zero_levels([(2, 2)], 3, 4), [(2, 2)], [8.0], ANCH[:1], 3, 4)  # n_ch < 5


def test_eager_hand_worked(orc):
    """The unfused tail stores every step in fp16 (23 small kernels, each
    writing its tensor: DeepJIT write-up, section 1.1); only the final cast to
    fp32 is exact. One level of 8 x 8 cells, one anchor (30, 45), six channels,
    stride 12 (not a power of two, so the stride multiply rounds); the logits
    of cell (y, x) = (6, 6) as below, 0 elsewhere. Worked by hand:
    - x and y: sigma(3.638671875) = 0.9743860854 -> fp16 0.974609375; + 6 =
      6.974609375 -> fp16 6.9765625; x 12 = 83.71875 -> fp16 83.75. Fused:
      (0.9743860854 + 6) x 12 = 83.692633 in fp32.
    - w: e^1.2392578125 = 3.4530497032 -> fp16 3.453125; x 30 = 103.59375 ->
      fp16 103.625. Fused: 103.591491.
    - h: e^2.361328125 = 10.605026905 -> fp16 10.6015625; x 45 = 477.0703125
      -> fp16 477.0. Fused: 477.226211.
    - objectness and class: sigma(-0.07989501953125) = 0.4800368631 -> fp16
      0.47998046875.
    Skipping any one of the roundings (sigma, + cell, x stride on either
    coordinate, exp, x anchor on either size, the class sigma) changes the
    stored value. The other cells (logit 0) are exact in both forms."""
    lv = np.zeros((1, 6, 8, 8), np.float16)
    lv[0, :, 6, 6] = [3.638671875, 3.638671875, 1.2392578125, 2.361328125,
                      -0.07989501953125, -0.07989501953125]
    e = orc.det_decode([lv], [(8, 8)], [12.0], [[30.0, 45.0]], 1, 6, eager=True)
    assert e[0, 6 * 8 + 6].tolist() == [83.75, 83.75, 103.625, 477.0, 0.47998046875,
                                          0.47998046875]
    f = orc.det_decode([lv], [(8, 8)], [12.0], [[30.0, 45.0]], 1, 6)
    np.testing.assert_allclose(f[0, 6 * 8 + 6], [83.692633, 83.692633, 103.591491, 477.226211,
                                                 0.4800368631, 0.4800368631], rtol=2e-7)
    zero = np.zeros_like(lv)
    base = orc.det_decode([zero], [(8, 8)], [12.0], [[30.0, 45.0]], 1, 6, eager=True)
    others = np.ones(64, bool)
    others[6 * 8 + 6] = False
    assert np.array_equal(e[0, others], base[0, others])
