"""Pins for the oracle's ChannelShuffle and batched transpose.

Source: the runtime page "CUDA算子与AI运行时" (gtnt.cn/news/145880), sections 2
and 2.1: ChannelShuffle views the C channels of [N, C, H, W] as [groups,
C/groups], swaps those two axes and views the result as C channels again; done
as a strided transpose it moves every element once.

Pins: channel orders worked by hand from that definition (golden fixture),
numpy's reshape / swapaxes (a library routine) on NCHW and NHWC tensors of
1- to 16-byte elements, and the group-theoretic invariants (groups 1 and C
are the identity, groups C/g undoes groups g, a transpose applied twice is the
identity).
"""
import os

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _orders():
    rows = []
    for line in open(os.path.join(HERE, "golden", "channel_shuffle_orders.txt")):
        if line.startswith("#") or not line.strip():
            continue
        head, tail = line.split("|")
        c, g = map(int, head.split())
        rows.append((c, g, [int(v) for v in tail.split()]))
    return rows


@pytest.mark.parametrize("C,g,order", _orders())
@pytest.mark.parametrize("layout", [0, 1])
def test_hand_worked_orders(orc, C, g, order, layout):
    N, H, W = 2, 3, 2
    if layout == 0:
        x = np.zeros((N, C, H, W), np.int32)
        x[:] = np.arange(C)[None, :, None, None]
        got = orc.channel_shuffle(x, g, 0)[:, :, :, :]
        assert (got == np.array(order)[None, :, None, None]).all()
    else:
        x = np.zeros((N, H, W, C), np.int32)
        x[:] = np.arange(C)
        got = orc.channel_shuffle(x, g, 1)
        assert (got == np.array(order)).all()


def _np_shuffle(x, g, layout):
    if layout == 0:
        n, c, h, w = x.shape
        return x.reshape(n, g, c // g, h, w).swapaxes(1, 2).reshape(n, c, h, w)
    n, h, w, c = x.shape
    return x.reshape(n, h, w, g, c // g).swapaxes(3, 4).reshape(n, h, w, c)


_DT = [np.uint8, np.float16, np.float32, np.float64, np.dtype("V3"), np.dtype("V16")]


def _rand(shape, dt, seed):
    rng = np.random.default_rng(seed)
    dt = np.dtype(dt)
    raw = rng.integers(0, 256, size=int(np.prod(shape)) * dt.itemsize, dtype=np.uint8)
    return raw.view(dt).reshape(shape)


@pytest.mark.parametrize("dt", _DT, ids=lambda d: np.dtype(d).name)
@pytest.mark.parametrize("shape,g", [((2, 12, 5, 7), 3), ((1, 116, 4, 4), 2), ((3, 8, 1, 1), 8),
                                     ((2, 6, 2, 3), 1)])
@pytest.mark.parametrize("layout", [0, 1])
def test_against_numpy(orc, dt, shape, g, layout):
    n, c, h, w = shape
    x = _rand(shape if layout == 0 else (n, h, w, c), dt, seed=c * 7 + g)
    got = orc.channel_shuffle(x, g, layout)
    assert got.tobytes() == np.ascontiguousarray(_np_shuffle(x, g, layout)).tobytes()


@pytest.mark.parametrize("dt", _DT, ids=lambda d: np.dtype(d).name)
@pytest.mark.parametrize("shape", [(1, 5, 7, 1), (3, 4, 4, 2), (2, 1, 9, 3), (1, 17, 1, 5),
                                   (0, 3, 3, 1), (2, 0, 4, 1)])
def test_transpose_against_numpy(orc, dt, shape):
    x = _rand(shape, dt, seed=sum(shape))
    got = orc.transpose021(x)
    assert got.shape == (shape[0], shape[2], shape[1], shape[3])
    assert got.tobytes() == np.ascontiguousarray(x.swapaxes(1, 2)).tobytes()


def test_invariants(orc):
    x = _rand((2, 24, 3, 5), np.float16, 1)
    assert orc.channel_shuffle(x, 1).tobytes() == x.tobytes()
    assert orc.channel_shuffle(x, 24).tobytes() == x.tobytes()
    for g in (2, 3, 4, 6, 8, 12):
        y = orc.channel_shuffle(x, g)
        assert y.tobytes() != x.tobytes()
        assert orc.channel_shuffle(y, 24 // g).tobytes() == x.tobytes()
        assert sorted(y.reshape(-1).view(np.uint16)) == sorted(x.reshape(-1).view(np.uint16))
    t = _rand((3, 7, 11, 2), np.float32, 2)
    assert orc.transpose021(orc.transpose021(t)).tobytes() == t.tobytes()


def test_nchw_shuffle_is_a_transpose_of_planes(orc):
    # the NCHW shuffle equals transpose021 of [N, groups, C/groups, H*W]
    x = _rand((2, 12, 3, 4), np.float16, 3)
    a = orc.channel_shuffle(x, 3, 0)
    b = orc.transpose021(x.reshape(2, 3, 4, 12))
    assert a.tobytes() == b.tobytes()


def test_rejects(orc):
    x = np.zeros((1, 6, 2, 2), np.float32)
    with pytest.raises(ValueError):
        orc.channel_shuffle(x, 4)
    with pytest.raises(ValueError):
        orc.channel_shuffle(x, 0)
    with pytest.raises(ValueError):
        orc.channel_shuffle(np.zeros((1, 6, 2, 2), np.dtype("V17")), 2)
