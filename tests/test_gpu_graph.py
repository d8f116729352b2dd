"""The unfused N-launch chains captured in a HIP graph (the DeepJIT write-up,
sections 3.1 and 6.1: a graph removes launch cost but keeps every kernel's
HBM round trip). Every replay is compared with the oracle's unfused (eager)
definition, to the bar of the unfused parity tests, and with the eager HIP
result bit for bit; the replays are interleaved with eager work and
synchronisations. A graph may hold several calls back to back, as the bench
captures them to amortise the graph launch itself."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import need_gpu, to_dev, to_host
from tolerance import check_f32, check_half, half_values

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def npa():
    need_gpu()
    import norm_pass_amd
    norm_pass_amd.np_init(0)
    return norm_pass_amd


def _replays(call, out, side_work, check, copies=1):
    """Capture `copies` calls in one graph; replay three times, each replay's
    output checked by `check` (against the oracle) and against the eager
    result."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = out.clone()
    check(eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(copies):
            call()
    for _ in range(3):
        out.fill_(0)
        side_work()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(out)
        assert torch.equal(out, eager)


@pytest.mark.parametrize("copies", [1, 8])
def test_graph_unfused_chain(npa, orc, copies):
    xs = synth.c5_inputs(1 << 16)
    x = to_dev(xs, "f16")
    out = torch.empty_like(x)
    ops = synth.c5_chain()
    ref, exact, bound = orc.chain(ops, [xs], 1, eager=True, want_bound=True)

    def check(t):
        got = to_host(t)
        check_half(got, ref.view(np.uint16), "f16", half_values(got, "f16"), exact, bound,
                   what="graph unfused chain")

    junk = torch.empty_like(x)
    _replays(lambda: npa.unfused_chain(ops, [x], out), out,
             lambda: npa.fuse_chain(ops, [x], junk), check, copies)


def test_graph_unfused_rmsnorm(npa, orc):
    xn, rn, wn = synth.c3_inputs(rows=64, cols=4096)
    x, r, w = (to_dev(a, "bf16") for a in (xn, rn, wn))
    h = torch.empty_like(x)
    out = torch.empty_like(x)
    ws = torch.empty(npa.rmsnorm_workspace_bytes(64, 4096, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    rh, ro = orc.add_rmsnorm(xn, rn, wn, 1e-6, 2, eager=True)

    def check(t):
        assert np.array_equal(to_host(h), rh)
        check_half(to_host(t), ro, "bf16", what="graph unfused rmsnorm")

    _replays(lambda: npa.unfused_add_rmsnorm(x, r, w, h, out, ws), out,
             lambda: npa.fuse_add_rmsnorm(x, r, w, None, torch.empty_like(x)), check, 4)


def test_graph_unfused_det_decode(npa, orc):
    levels = ((16, 16, 8.0), (8, 8, 16.0))
    lvn = synth.c2_inputs(levels=levels)
    lv = [to_dev(a, "f16") for a in lvn]
    an = np.array(synth.YOLO_ANCHORS, np.float32).reshape(3, 3, 2)[:2]
    out = torch.empty((1, 3 * (256 + 64), 85), device="cuda")
    ws = torch.empty(npa.det_workspace_bytes(lv), dtype=torch.uint8, device="cuda")
    want = orc.det_decode(lvn, [(16, 16), (8, 8)], [8.0, 16.0], an, 3, 85, eager=True)

    def check(t):
        got = t.cpu().numpy()
        g16 = got.astype(np.float16)
        assert np.array_equal(g16.astype(np.float32), got)  # values are fp16 numbers
        d = np.abs(g16.view(np.int16).astype(np.int32) - want.astype(np.float16).view(np.int16))
        assert d.max() <= 2

    _replays(lambda: npa.unfused_det_decode(lv, [8.0, 16.0], an.tolist(), out, ws), out,
             lambda: None, check, 3)


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


# The fused calls captured the same way (the bench times the small ones as
# graphs of 64 back-to-back calls, so that the host's launch rate does not set
# the figure); each replay is checked against the oracle's fused definition.
@pytest.mark.parametrize("copies", [1, 64])
def test_graph_fused_chain(npa, orc, copies):
    xs = synth.c5_inputs(1 << 16)
    x = to_dev(xs, "f16")
    out = torch.empty_like(x)
    ops = synth.c5_chain()
    ref, exact, bound = orc.chain(ops, [xs], 1, want_bound=True)

    def check(t):
        got = to_host(t)
        check_half(got, ref.view(np.uint16), "f16", half_values(got, "f16"), exact, bound,
                   what="graph fused chain")

    junk = torch.empty_like(x)
    _replays(lambda: npa.fuse_chain(ops, [x], out), out,
             lambda: npa.unfused_chain(ops, [x], junk), check, copies)


@pytest.mark.parametrize("copies", [1, 64])
def test_graph_fused_c1_chain(npa, orc, copies):
    a, b = synth.c1_inputs(1 << 16)
    ta, tb = to_dev(a, "f32"), to_dev(b, "f32")
    out = torch.empty_like(ta)
    ref = orc.chain(synth.C1_CHAIN, [a, b], 0)  # fp32 output

    def check(t):
        assert np.array_equal(to_host(t).view(np.uint32), np.asarray(ref).view(np.uint32))

    _replays(lambda: npa.fuse_chain(synth.C1_CHAIN, [ta, tb], out), out, lambda: None, check,
             copies)


@pytest.mark.parametrize("copies", [1, 64])
def test_graph_fused_det_decode(npa, orc, copies):
    lvn = synth.c2_inputs()
    lv = [to_dev(a, "f16") for a in lvn]
    hw = [(h, w) for h, w, _ in synth.YOLO_LEVELS]
    st = [s for _, _, s in synth.YOLO_LEVELS]
    an = np.array(synth.YOLO_ANCHORS, np.float32).reshape(3, 3, 2)
    out = torch.empty((1, 25200, 85), device="cuda")
    want = orc.det_decode(lvn, hw, st, an, 3, 85, in_dt=1)

    def check(t):
        check_f32(t.cpu().numpy(), want, what="graph fused det decode")

    _replays(lambda: npa.fuse_det_decode(lv, st, an.tolist(), out), out, lambda: None, check,
             copies)
