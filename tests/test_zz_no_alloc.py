"""unfused_det_decode_noalloc (no workspace, no allocation: the library's own
device scratch array) against unfused_det_decode (the caller's workspace),
through the C ABI: two calls in a row, the second with a smaller input, each
output bit-identical to the existing entry point's; the outputs also
against the oracle's unfused (eager) decode: every value an fp16 number,
within 2 fp16 ulps (the bar of the unfused tail's own parity test)."""
import ctypes as C

import numpy as np
import pytest
import torch

import synth
from gpu_util import need_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def npa():
    need_gpu()
    import norm_pass_amd
    norm_pass_amd.np_init(0)
    return norm_pass_amd


def _call(npa, name, levels, strides, anchors, out, ws=None):
    a = list(npa._a_fuse_det_decode(levels, strides, anchors, out))
    if ws is not None:
        a = a[:-1] + [C.c_void_p(ws.data_ptr()), ws.numel(), a[-1]]
    rc = getattr(npa.lib(), name)(*a)
    assert rc == 0, npa.lib().np_last_error().decode()


def _case(npa, orc, levels_hw, seed, check_oracle):
    lv_np = synth.c2_inputs(levels=levels_hw, seed=seed)
    lv = [to_dev(a, "f16") for a in lv_np]
    strides = [s for _, _, s in levels_hw]
    an = np.array(synth.YOLO_ANCHORS, np.float32).reshape(3, 3, 2)[:len(levels_hw)]
    rows = sum(3 * h * w for h, w, _ in levels_hw)
    print(f"noalloc case: levels {levels_hw}, rows {rows}", flush=True)
    ref = torch.full((1, rows, 85), float("nan"), device="cuda")
    ws = torch.empty(npa.det_workspace_bytes(lv), dtype=torch.uint8, device="cuda")
    _call(npa, "unfused_det_decode", lv, strides, an.tolist(), ref, ws)
    out = torch.full((1, rows, 85), float("nan"), device="cuda")
    _call(npa, "unfused_det_decode_noalloc", lv, strides, an.tolist(), out)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
    if check_oracle:
        want = orc.det_decode(lv_np, [(h, w) for h, w, _ in levels_hw], strides, an, 3, 85,
                              eager=True)
        got = out.cpu().numpy()
        g16 = got.astype(np.float16)
        assert np.array_equal(g16.astype(np.float32), got)  # values are fp16 numbers
        d = np.abs(g16.view(np.int16).astype(np.int32) - want.astype(np.float16).view(np.int16))
        assert d.max() <= 2


def test_noalloc_matches_workspace_call_twice(npa, orc):
    # the full 3-level head (8,568,000 staged bytes), then a smaller 2-level one
    _case(npa, orc, ((80, 80, 8.0), (40, 40, 16.0), (20, 20, 32.0)), 1002, True)
    _case(npa, orc, ((13, 11, 8.0), (7, 5, 16.0)), 77, True)


def test_noalloc_rejects_oversized(npa):
    # 3 images of one 80 x 80 level stage 2 x 3 x 19,200 x 85 x 2 = 19,584,000 bytes
    lv = [torch.zeros((3, 255, 80, 80), dtype=torch.float16, device="cuda")]
    out = torch.empty((3, 3 * 6400, 85), device="cuda")
    a = npa._a_fuse_det_decode(lv, [8.0], [[(10, 13), (16, 30), (33, 23)]], out)
    assert npa.lib().unfused_det_decode_noalloc(*a) == npa.NP_EINVAL
    assert "scratch array" in npa.lib().np_last_error().decode()
