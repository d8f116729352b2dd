"""GPU parity of fuse_det_decode / unfused_det_decode against the oracle
(DeepJIT write-up, sections 1.1, 2.2 and 5.2: the detection-head tail).

Layout (row = level, anchor, y, x; column = channel) must be bit-exact: a
one-hot marker swept over tiny grids may change exactly one output element.
Values: fp32 within 1e-6 relative of the oracle. The unfused (fp16 storage)
tail must match the oracle's unfused definition within 2 fp16 ulps.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import ORACLE_DT, empty, misaligned, need_gpu, to_dev, to_host
from tolerance import check_f32

pytestmark = pytest.mark.gpu
ANCH = np.array(synth.YOLO_ANCHORS, np.float32).reshape(3, 3, 2)


@pytest.fixture(scope="module")
def npa():
    need_gpu()
    import norm_pass_amd
    norm_pass_amd.np_init(0)
    return norm_pass_amd


def _run(npa, levels_np, levels_hw, strides, anchors, n_anchors, n_ch, dt, fn="fuse",
         align=True):
    tl = [to_dev(a, dt) for a in levels_np]
    if not align:
        tl = [misaligned(t) for t in tl]
    batch = levels_np[0].shape[0]
    rows = npa.det_rows(tl, n_anchors)
    out = torch.full((batch, rows, n_ch), float("nan"), device="cuda")
    if fn == "fuse":
        npa.fuse_det_decode(tl, strides, anchors, out, n_anchors, n_ch)
    else:
        ws = torch.empty(npa.det_workspace_bytes(tl, n_anchors, n_ch), dtype=torch.uint8,
                         device="cuda")
        npa.unfused_det_decode(tl, strides, anchors, out, ws, n_anchors, n_ch)
    torch.cuda.synchronize()
    return to_host(out)


def test_full_config(npa, orc):
    lv = synth.c2_inputs()
    hw = [(h, w) for h, w, _ in synth.YOLO_LEVELS]
    st = [s for _, _, s in synth.YOLO_LEVELS]
    got = _run(npa, lv, hw, st, ANCH, 3, 85, "f16")
    ref = orc.det_decode(lv, hw, st, ANCH, 3, 85, in_dt=1)
    assert got.shape == (1, 25200, 85)
    check_f32(got, ref, what="det decode full")


def test_full_config_unfused(npa, orc):
    lv = synth.c2_inputs()
    hw = [(h, w) for h, w, _ in synth.YOLO_LEVELS]
    st = [s for _, _, s in synth.YOLO_LEVELS]
    got = _run(npa, lv, hw, st, ANCH, 3, 85, "f16", fn="unfused")
    ref = orc.det_decode(lv, hw, st, ANCH, 3, 85, in_dt=1, eager=True)
    g16 = got.astype(np.float16)
    assert np.array_equal(g16.astype(np.float32), got)  # values are fp16 numbers
    d = np.abs(g16.view(np.int16).astype(np.int32) - ref.astype(np.float16).view(np.int16))
    assert d.max() <= 2


@pytest.mark.parametrize("levels,batch,n_ch,dt,align", [
    (((7, 5, 8.0), (3, 3, 16.0)), 2, 85, "f16", True),     # ragged: H*W not a multiple of 8
    (((16, 8, 8.0), (8, 4, 16.0), (4, 2, 32.0)), 1, 85, "f16", True),
    (((13, 13, 32.0),), 3, 7, "bf16", True),
    (((8, 8, 8.0), (9, 7, 4.0)), 2, 12, "f32", True),
    (((16, 16, 8.0),), 1, 85, "f16", False),               # misaligned level pointers
    (((1, 1, 8.0), (2, 1, 16.0)), 1, 5, "f16", True),
    (((64, 80, 8.0),), 1, 600, "f16", True),               # wide rows: smaller tiles
    # W not a multiple of the vector: a vector's cells cross into the next grid row
    (((8, 12, 8.0), (4, 10, 16.0)), 2, 85, "f16", True),
    (((6, 6, 8.0), (8, 2, 16.0)), 1, 9, "f32", True),       # fp32 vectors; W = 2 < 4 per cell
])
def test_shapes(npa, orc, levels, batch, n_ch, dt, align):
    lv = synth.c2_inputs(levels=levels, n_ch=n_ch, batch=batch, dtype=dt, seed=7)
    hw = [(h, w) for h, w, _ in levels]
    st = [s for _, _, s in levels]
    anchors = np.tile(ANCH[:1], (len(levels), 1, 1))
    got = _run(npa, lv, hw, st, anchors, 3, n_ch, dt, align=align)
    ref = orc.det_decode(lv, hw, st, anchors, 3, n_ch, in_dt=ORACLE_DT[dt])
    check_f32(got, ref, what=str(levels))
    got = _run(npa, lv, hw, st, anchors, 3, n_ch, dt, fn="unfused")
    ref = orc.det_decode(lv, hw, st, anchors, 3, n_ch, in_dt=ORACLE_DT[dt], eager=True)
    if dt == "f32":
        check_f32(got, ref, rel=1e-6, what="unfused f32")
    else:
        rel = np.abs(got.astype(np.float64) - ref) / np.maximum(np.abs(ref), 1e-30)
        assert rel.max() <= 2 * (2.0 ** -10 if dt == "f16" else 2.0 ** -7)


@pytest.mark.parametrize("hw", [
    [(3, 2), (1, 3)],    # per-cell path (H*W not a multiple of 8)
    [(2, 12), (1, 8)],   # 16-byte vectors; with W = 12 some vectors cross a grid row
])
def test_marker_layout_bit_exact(npa, orc, hw):
    """One logit = 1, all others 0: exactly the predicted output element changes."""
    n_anchors, n_ch = 3, 6
    levels = tuple((h, w, s) for (h, w), s in zip(hw, (8.0, 16.0)))
    zero = [np.zeros((1, n_anchors * n_ch, h, w), np.float16) for h, w in hw]
    base = _run(npa, zero, hw, [8.0, 16.0], ANCH[:2], n_anchors, n_ch, "f16")
    assert np.array_equal(base, orc.det_decode(zero, hw, [8.0, 16.0], ANCH[:2], n_anchors, n_ch))
    row_off = 0
    for l, (h, w) in enumerate(hw):
        for a in range(n_anchors):
            for k in range(n_ch):
                for y in range(h):
                    for x in range(w):
                        lv = [z.copy() for z in zero]
                        lv[l][0, a * n_ch + k, y, x] = np.float16(1.0)
                        got = _run(npa, lv, hw, [8.0, 16.0], ANCH[:2], n_anchors, n_ch, "f16")
                        diff = np.argwhere(got != base)
                        assert diff.tolist() == [[0, row_off + (a * h + y) * w + x, k]]
        row_off += n_anchors * h * w
    assert levels  # shapes used above


def test_deterministic(npa):
    lv = synth.c2_inputs()
    hw = [(h, w) for h, w, _ in synth.YOLO_LEVELS]
    st = [s for _, _, s in synth.YOLO_LEVELS]
    a = _run(npa, lv, hw, st, ANCH, 3, 85, "f16")
    b = _run(npa, lv, hw, st, ANCH, 3, 85, "f16")
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
