"""The unfused N-launch chains captured in a HIP graph (the DeepJIT write-up,
sections 3.1 and 6.1: a graph removes launch cost but keeps every kernel's
HBM round trip). Each replay must reproduce the eager result bit for bit; the
replays are interleaved with eager work and synchronisations."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import need_gpu, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def npa():
    need_gpu()
    import norm_pass_amd
    norm_pass_amd.np_init(0)
    return norm_pass_amd


def _replays_match(call, out, eager_ref, side_work):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for _ in range(3):
        out.fill_(0)
        side_work()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_ref)


def test_graph_unfused_chain(npa):
    x = to_dev(synth.c5_inputs(1 << 16), "f16")
    out = torch.empty_like(x)
    ops = synth.c5_chain()
    npa.unfused_chain(ops, [x], out)
    torch.cuda.synchronize()
    ref = out.clone()
    junk = torch.empty_like(x)
    _replays_match(lambda: npa.unfused_chain(ops, [x], out), out, ref,
                   lambda: npa.fuse_chain(ops, [x], junk))


def test_graph_unfused_rmsnorm(npa):
    x, r, w = (to_dev(a, "bf16") for a in synth.c3_inputs(rows=64, cols=4096))
    h = torch.empty_like(x)
    out = torch.empty_like(x)
    ws = torch.empty(npa.rmsnorm_workspace_bytes(64, 4096, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    npa.unfused_add_rmsnorm(x, r, w, h, out, ws)
    torch.cuda.synchronize()
    ref = out.clone()
    _replays_match(lambda: npa.unfused_add_rmsnorm(x, r, w, h, out, ws), out, ref,
                   lambda: npa.fuse_add_rmsnorm(x, r, w, None, torch.empty_like(x)))


def test_graph_unfused_det_decode(npa):
    levels = ((16, 16, 8.0), (8, 8, 16.0))
    lv = [to_dev(a, "f16") for a in synth.c2_inputs(levels=levels)]
    an = np.array(synth.YOLO_ANCHORS, np.float32).reshape(3, 3, 2)[:2].tolist()
    out = torch.empty((1, 3 * (256 + 64), 85), device="cuda")
    ws = torch.empty(npa.det_workspace_bytes(lv), dtype=torch.uint8, device="cuda")
    npa.unfused_det_decode(lv, [8.0, 16.0], an, out, ws)
    torch.cuda.synchronize()
    ref = out.clone()
    _replays_match(lambda: npa.unfused_det_decode(lv, [8.0, 16.0], an, out, ws), out, ref,
                   lambda: None)


def test_bind_keeps_its_tensors_alive(npa):
    """bind() marshals device pointers once; the tensors behind them must live as
    long as the returned callable (no launch here: only the references)."""
    import gc
    import weakref

    def make():
        x = torch.zeros(1 << 10, dtype=torch.float16, device="cuda")
        y = torch.empty_like(x)
        return npa.bind("fuse_chain", [(synth.LOAD, 0, 0.0)], [x], y), weakref.ref(x), \
            weakref.ref(y)

    call, wx, wy = make()
    gc.collect()
    assert wx() is not None and wy() is not None
    del call
    gc.collect()
    assert wx() is None and wy() is None
