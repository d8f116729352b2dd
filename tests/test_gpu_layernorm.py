"""GPU parity of fuse_add_layernorm / unfused_add_layernorm against the oracle
(DeepJIT write-up, section 4.3: fused LayerNorm with gamma / beta).

h = x + r is bit-exact; out within 2 ulps of the output type (outputs where
gamma * y and beta cancel are judged against the oracle's exact value with one
row-scale ulp, see _check); shapes cover the register path and the generic
path, optional operands, misaligned buffers, fp16 / fp32, and the full
[16384, 4096] bf16 size."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import ORACLE_DT, empty, misaligned, need_gpu, to_dev, to_host
from tolerance import check_f32, half_values, ulp_dist16

pytestmark = pytest.mark.gpu
EPS = 1e-5


@pytest.fixture(scope="module")
def npa():
    need_gpu()
    import norm_pass_amd
    norm_pass_amd.np_init(0)
    return norm_pass_amd


def _inputs(rows, cols, dt, seed):
    x, r, g = synth.c3_inputs(rows=rows, cols=cols, seed=seed, dtype=dt)
    b = synth.normal((cols,), seed + 5, dt, std=0.1)
    return x, r, g, b


def _run(npa, x, r, g, b, dt, with_h=True, fn="fuse", align=True):
    tx = to_dev(x, dt)
    if not align:
        tx = misaligned(tx)
    tr, tg, tb = (None if a is None else to_dev(a, dt) for a in (r, g, b))
    rows, cols = x.shape
    h = empty((rows, cols), dt) if with_h else None
    out = empty((rows, cols), dt)
    if fn == "fuse":
        npa.fuse_add_layernorm(tx, tr, tg, tb, h, out, EPS)
    else:
        ws = torch.empty(npa.layernorm_workspace_bytes(rows, cols, out.dtype, with_h),
                         dtype=torch.uint8, device="cuda")
        npa.unfused_add_layernorm(tx, tr, tg, tb, h, out, ws, EPS)
    torch.cuda.synchronize()
    return (None if h is None else to_host(h)), to_host(out)


def _check(npa, orc, x, r, g, b, dt, with_h=True, fn="fuse", align=True):
    gh, go = _run(npa, x, r, g, b, dt, with_h, fn, align)
    rh, ro, ex = orc.add_layernorm(x, r, g, b, EPS, ORACLE_DT[dt], eager=(fn != "fuse"),
                                   want_exact=True)
    if with_h:
        assert np.array_equal(gh.view(np.uint8), rh.view(np.uint8))
    if dt == "f32":
        # beta added to gamma * y can cancel: judge against the row's scale
        gv = go.astype(np.float64)
        scale = np.abs(ex).max(axis=1, keepdims=True) + 1e-30
        err = np.abs(gv - ex)
        assert (err <= 1e-6 * np.maximum(np.abs(ex), 1e-3 * scale) + 4e-7 * scale).all()
        return
    d = ulp_dist16(go, ro)
    bad = d > 2
    if bad.any():
        # the few elements near 0 (gamma * y ~ -beta) may miss by their own
        # ulps; they must be within one output ulp of the row scale
        gv = half_values(go, dt)
        scale = np.abs(ex).max(axis=1, keepdims=True) * np.ones_like(ex)
        ulp_scale = scale * (2.0 ** -10 if dt == "f16" else 2.0 ** -7)
        ok = np.abs(gv - ex)[bad] <= (ulp_scale[bad] if fn == "fuse" else 4 * ulp_scale[bad])
        assert ok.all(), f"{int((~ok).sum())} elements off; worst {int(d.max())} ulp"
        assert bad.mean() < (1e-3 if fn == "fuse" else 3e-2)


@pytest.mark.parametrize("rows,cols", [(1, 8), (3, 96), (17, 2048), (5, 4096), (4, 4104),
                                       (2, 8192), (3, 16384), (3, 777), (2, 20000), (1, 1)])
@pytest.mark.parametrize("fn", ["fuse", "unfused"])
def test_shapes_bf16(npa, orc, rows, cols, fn):
    _check(npa, orc, *_inputs(rows, cols, "bf16", rows * 31 + cols), "bf16", fn=fn)


@pytest.mark.parametrize("dt", ["f16", "f32"])
@pytest.mark.parametrize("cols", [64, 4096, 1000])
def test_other_dtypes(npa, orc, dt, cols):
    args = _inputs(9, cols, dt, cols)
    _check(npa, orc, *args, dt)
    _check(npa, orc, *args, dt, fn="unfused")


@pytest.mark.parametrize("use_r,use_g,use_b,with_h", [(False, True, True, True),
                                                      (True, False, True, True),
                                                      (True, True, False, False),
                                                      (False, False, False, False)])
def test_optional_operands(npa, orc, use_r, use_g, use_b, with_h):
    x, r, g, b = _inputs(6, 4096, "bf16", 11)
    args = (x, r if use_r else None, g if use_g else None, b if use_b else None)
    _check(npa, orc, *args, "bf16", with_h=with_h)
    _check(npa, orc, *args, "bf16", with_h=with_h, fn="unfused")


def test_misaligned(npa, orc):
    _check(npa, orc, *_inputs(5, 4096, "bf16", 12), "bf16", align=False)


def test_constant_rows_give_beta(npa):
    cols = 4096
    _, _, g, b = _inputs(1, cols, "bf16", 13)
    cs = [0.0, 1.0, -3.5, 100.0]
    x = synth.to_bf16_bits(np.repeat(np.array(cs, np.float32)[:, None], cols, axis=1))
    _, out = _run(npa, x, None, g, b, "bf16")
    for i in range(len(cs)):
        assert np.array_equal(out[i], b), cs[i]


def test_full_size(npa, orc):
    _check(npa, orc, *_inputs(16384, 4096, "bf16", 14), "bf16")


def test_deterministic(npa):
    args = _inputs(256, 4096, "bf16", 15)
    a = _run(npa, *args, "bf16")[1]
    b = _run(npa, *args, "bf16")[1]
    assert np.array_equal(a, b)
