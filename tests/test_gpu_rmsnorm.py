"""GPU parity of fuse_add_rmsnorm / unfused_add_rmsnorm against the oracle
(TeleTron write-up, sections 3.3 and 4.2).

h = x + r must be bit-exact (one correctly rounded sum); out must be within
2 ulps of the output type (1e-6 relative for fp32). Shapes cover the register
path (several vector counts per thread), ragged and very long rows (generic
path), misaligned buffers, optional r / w / h, and the full [16384, 4096]
bf16 workload.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import ORACLE_DT, empty, misaligned, need_gpu, to_dev, to_host
from tolerance import check_f32, check_half

pytestmark = pytest.mark.gpu
EPS = 1e-6


@pytest.fixture(scope="module")
def npa():
    need_gpu()
    import norm_pass_amd
    norm_pass_amd.np_init(0)
    return norm_pass_amd


def _run(npa, x, r, w, dt, with_h=True, fn="fuse", align=True):
    tx = to_dev(x, dt)
    tr = None if r is None else to_dev(r, dt)
    tw = None if w is None else to_dev(w, dt)
    if not align:
        tx = misaligned(tx)
        tr = None if tr is None else misaligned(tr)
    rows, cols = x.shape
    h = empty((rows, cols), dt) if with_h else None
    out = empty((rows, cols), dt)
    if fn == "fuse":
        npa.fuse_add_rmsnorm(tx, tr, tw, h, out, EPS)
    else:
        ws = torch.empty(npa.rmsnorm_workspace_bytes(rows, cols, out.dtype, with_h),
                         dtype=torch.uint8, device="cuda")
        npa.unfused_add_rmsnorm(tx, tr, tw, h, out, ws, EPS)
    torch.cuda.synchronize()
    return (None if h is None else to_host(h)), to_host(out)


def _check(npa, orc, x, r, w, dt, with_h=True, fn="fuse", align=True):
    gh, go = _run(npa, x, r, w, dt, with_h, fn, align)
    rh, ro = orc.add_rmsnorm(x, r, w, EPS, ORACLE_DT[dt], eager=(fn != "fuse"))
    if with_h:
        assert np.array_equal(gh.view(np.uint8), rh.view(np.uint8))
    if dt == "f32":
        check_f32(go, ro, rel=1e-6 if fn == "fuse" else 2e-6, what=f"{x.shape} {fn}")
    else:
        check_half(go, ro, dt, max_ulp=2, what=f"{x.shape} {dt} {fn}")


@pytest.mark.parametrize("rows,cols", [(1, 8), (3, 96), (17, 2048), (5, 4096), (4, 4104),
                                       (2, 8192), (3, 16384), (3, 777), (2, 20000), (1, 1)])
@pytest.mark.parametrize("fn", ["fuse", "unfused"])
def test_shapes_bf16(npa, orc, rows, cols, fn):
    x, r, w = synth.c3_inputs(rows=rows, cols=cols, seed=rows * 31 + cols)
    _check(npa, orc, x, r, w, "bf16", fn=fn)


@pytest.mark.parametrize("dt", ["f16", "f32"])
@pytest.mark.parametrize("cols", [64, 4096, 1000])
def test_other_dtypes(npa, orc, dt, cols):
    x, r, w = synth.c3_inputs(rows=9, cols=cols, seed=cols, dtype=dt)
    _check(npa, orc, x, r, w, dt)
    _check(npa, orc, x, r, w, dt, fn="unfused")


@pytest.mark.parametrize("use_r,use_w,with_h", [(False, True, True), (True, False, True),
                                                (True, True, False), (False, False, False)])
def test_optional_operands(npa, orc, use_r, use_w, with_h):
    x, r, w = synth.c3_inputs(rows=6, cols=4096, seed=11)
    _check(npa, orc, x, r if use_r else None, w if use_w else None, "bf16", with_h=with_h)
    _check(npa, orc, x, r if use_r else None, w if use_w else None, "bf16", with_h=with_h,
           fn="unfused")


def test_misaligned(npa, orc):
    x, r, w = synth.c3_inputs(rows=5, cols=4096, seed=12)
    _check(npa, orc, x, r, w, "bf16", align=False)


def test_constant_rows_give_signed_weight(npa):
    cols = 4096
    w = synth.normal((cols,), 99, "bf16", mean=1.0, std=0.1)
    cs = [1.0, -1.0, 0.0625, -0.0625, 3.5, -100.0, 0.25, 0.0]
    x = synth.to_bf16_bits(np.repeat(np.array(cs, np.float32)[:, None], cols, axis=1))
    _, out = _run(npa, x, None, w, "bf16")
    for i, c in enumerate(cs):
        want = np.zeros_like(w) if c == 0 else (w if c > 0 else w ^ np.uint16(0x8000))
        assert np.array_equal(out[i], want), c


def test_in_place(npa, orc):
    """out may alias x exactly."""
    x, r, w = synth.c3_inputs(rows=4, cols=4096, seed=13)
    tx, tr, tw = to_dev(x, "bf16"), to_dev(r, "bf16"), to_dev(w, "bf16")
    h = empty(tx.shape, "bf16")
    npa.fuse_add_rmsnorm(tx, tr, tw, h, tx, EPS)
    torch.cuda.synchronize()
    rh, ro = orc.add_rmsnorm(x, r, w, EPS, 2)
    assert np.array_equal(to_host(h), rh)
    check_half(to_host(tx), ro, "bf16")


def test_full_size(npa, orc):
    x, r, w = synth.c3_inputs()
    gh, go = _run(npa, x, r, w, "bf16")
    rh, ro = orc.add_rmsnorm(x, r, w, EPS, 2)
    assert np.array_equal(gh, rh)
    st = check_half(go, ro, "bf16", what="16384x4096")
    assert st["exempt"] == 0


def test_deterministic(npa):
    x, r, w = synth.c3_inputs(rows=256, cols=4096, seed=14)
    a = _run(npa, x, r, w, "bf16")[1]
    b = _run(npa, x, r, w, "bf16")[1]
    assert np.array_equal(a, b)
