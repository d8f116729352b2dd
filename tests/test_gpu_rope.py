"""GPU parity of fuse_qkv_rope / unfused_qkv_rope against the oracle (TeleTron
write-up, section 3.1: QKV split + RoPE + scale).

The head-major placement and V are bit-exact; Q and K are within 2 bf16 ulps
of the oracle, except rotated values that nearly cancel (u cos - w sin close to
0), which must lie within the oracle's fp32 evaluation bound and stay below
1e-4 of the elements.
"""
import math

import numpy as np
import pytest
import torch

import synth
from gpu_util import ORACLE_DT, empty, misaligned, need_gpu, to_dev, to_host
from tolerance import check_f32_counted, check_half, half_values

pytestmark = pytest.mark.gpu
QS = float(np.float32(1.0 / math.sqrt(128.0)))


@pytest.fixture(scope="module")
def npa():
    need_gpu()
    import norm_pass_amd
    norm_pass_amd.np_init(0)
    return norm_pass_amd


def _run(npa, qkv, H, D, dt, qs, pos=None, fn="fuse", align=True):
    t = to_dev(qkv, dt)
    if not align:
        t = misaligned(t)
    T = qkv.shape[0]
    q, k, v = (empty((H, T, D), dt) for _ in range(3))
    tp = None if pos is None else torch.from_numpy(pos).cuda()
    getattr(npa, f"{fn}_qkv_rope")(t, q, k, v, H, D, tp, 10000.0, qs)
    torch.cuda.synchronize()
    return to_host(q), to_host(k), to_host(v)


def _check(npa, orc, qkv, H, D, dt, qs=QS, pos=None, fn="fuse", align=True):
    gq, gk, gv = _run(npa, qkv, H, D, dt, qs, pos, fn, align)
    rq, rk, rv, eq, ek, bq, bk = orc.qkv_rope(qkv, H, D, 10000.0, qs, ORACLE_DT[dt], positions=pos,
                                              eager=(fn != "fuse"), want_bound=True)
    assert np.array_equal(gv.view(np.uint8), rv.view(np.uint8))
    if dt == "f32":
        return tuple(check_f32_counted(g, r, e, b, what=f"{name} {qkv.shape} {fn}")
                     for name, g, r, e, b in (("Q", gq, rq, eq, bq), ("K", gk, rk, ek, bk)))
    s1 = check_half(gq, rq, dt, half_values(gq, dt), eq, bq, what=f"Q {qkv.shape} {fn}")
    s2 = check_half(gk, rk, dt, half_values(gk, dt), ek, bk, what=f"K {qkv.shape} {fn}")
    return s1, s2


@pytest.mark.parametrize("T,H,D", [(1, 1, 128), (5, 3, 128), (33, 2, 64), (7, 2, 16),
                                   (9, 1, 130), (4, 3, 8), (300, 24, 128)])
@pytest.mark.parametrize("fn", ["fuse", "unfused"])
def test_shapes_bf16(npa, orc, T, H, D, fn):
    qkv = synth.c4_inputs(tokens=T, heads=H, head_dim=D, seed=T * 7 + D)
    _check(npa, orc, qkv, H, D, "bf16", qs=float(np.float32(1 / math.sqrt(D))), fn=fn)


@pytest.mark.parametrize("dt,D", [("f16", 128), ("f32", 128), ("f32", 64), ("bf16", 64)])
def test_other_dtypes(npa, orc, dt, D):
    qkv = synth.c4_inputs(tokens=40, heads=3, head_dim=D, seed=5, dtype=dt)
    qs = float(np.float32(1 / math.sqrt(D)))
    _check(npa, orc, qkv, 3, D, dt, qs=qs)
    _check(npa, orc, qkv, 3, D, dt, qs=qs, fn="unfused")


@pytest.mark.parametrize("H", [1, 5, 8, 64, 65])
def test_head_counts(npa, orc, H):
    """Whole-token path for 1..64 heads (partial last chunk batch), generic beyond."""
    qkv = synth.c4_inputs(tokens=9, heads=H, head_dim=128, seed=H)
    _check(npa, orc, qkv, H, 128, "bf16")


def test_positions_array_and_misaligned(npa, orc):
    qkv = synth.c4_inputs(tokens=64, heads=4, head_dim=128, seed=6)
    pos = (np.arange(64, dtype=np.int32) * 257) % 16384
    _check(npa, orc, qkv, 4, 128, "bf16", pos=pos)
    _check(npa, orc, qkv, 4, 128, "bf16", pos=pos, align=False)
    _check(npa, orc, qkv, 4, 128, "bf16", pos=pos, fn="unfused")


def test_position_zero_identity(npa):
    qkv = synth.c4_inputs(tokens=1, heads=24, head_dim=128, seed=8)
    q, k, v = _run(npa, qkv, 24, 128, "bf16", QS)
    P = qkv.reshape(1, 3, 24, 128)
    assert np.array_equal(k[:, 0], P[0, 1])
    assert np.array_equal(v[:, 0], P[0, 2])


def test_layout_marker(npa, orc):
    """Unique values at every (t, s, h, d); position 0 everywhere and scale 1, so
    every value must land unchanged at [h][t][d]."""
    T, H, D = 12, 3, 128
    vals = (np.arange(T * 3 * H * D) % 2000 + 1).astype(np.float32)  # exact in fp32
    qkv = vals.reshape(T, 3 * H * D)
    pos = np.zeros(T, np.int32)
    q, k, v = _run(npa, qkv, H, D, "f32", 1.0, pos=pos)
    P = vals.reshape(T, 3, H, D)
    assert np.array_equal(q, P[:, 0].transpose(1, 0, 2))
    assert np.array_equal(k, P[:, 1].transpose(1, 0, 2))
    assert np.array_equal(v, P[:, 2].transpose(1, 0, 2))


def test_full_size(npa, orc):
    qkv = synth.c4_inputs()
    s1, s2 = _check(npa, orc, qkv, 24, 128, "bf16")
    print("full-size exemptions", s1, s2)


def test_deterministic(npa):
    qkv = synth.c4_inputs(tokens=512, heads=24, head_dim=128, seed=10)
    a = _run(npa, qkv, 24, 128, "bf16", QS)
    b = _run(npa, qkv, 24, 128, "bf16", QS)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
