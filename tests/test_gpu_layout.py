"""GPU parity of the layout calls (fuse_/naive_transpose021,
fuse_/naive_channel_shuffle) against the oracle: bit-exact.

Source: the runtime page "CUDA算子与AI运行时" (gtnt.cn/news/145880), sections 2
and 2.1 (ChannelShuffle as a reshape + transpose; a strided transpose done
element by element versus one staged through on-chip memory).

Every kernel the planner can pick (LDS tiles with and without 16-byte vectors
for units of 1..16 bytes, whole matrices through LDS, item-by-item copies of
1..16-byte items, the contiguous-copy case) is run on ragged shapes and
misaligned pointers, at the workload sizes the bench times, and on tensors
large enough that the host splits the batch axis over several launches
(checked on sampled matrices).
"""
import ctypes as C

import numpy as np
import pytest
import torch

import synth
from gpu_util import need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def npa():
    need_gpu()
    import norm_pass_amd
    norm_pass_amd.np_init(0)
    return norm_pass_amd


def _vdt(es):
    return np.dtype(f"V{es}")


def _dev_buf(nbytes, offset):
    """A uint8 device buffer whose view starts `offset` bytes past a 256-byte boundary."""
    buf = torch.empty(nbytes + offset + 256, dtype=torch.uint8, device="cuda")
    base = (-buf.data_ptr()) % 256
    return buf, buf[base + offset: base + offset + nbytes]


def _run_tr(npa, x_bytes, shape, es, naive=False, off_in=0, off_out=0, expect=None):
    B, R, S, E = shape
    nbytes = x_bytes.size
    keep_i, xi = _dev_buf(nbytes, off_in)
    keep_o, xo = _dev_buf(nbytes, off_out)
    xi.copy_(torch.from_numpy(x_bytes))
    xo.fill_(0xA5)
    plan = npa.np_transpose_plan(xi.data_ptr(), xo.data_ptr(), shape, es, naive)
    if expect is not None:
        assert plan == expect, plan
    fn = npa.lib().naive_transpose021 if naive else npa.lib().fuse_transpose021
    rc = fn(C.c_void_p(xi.data_ptr()), C.c_void_p(xo.data_ptr()), B, R, S, E, es,
            C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, npa.lib().np_last_error()
    torch.cuda.synchronize()
    return xo.cpu().numpy(), plan


def _oracle_tr(orc, x_bytes, shape, es):
    return orc.transpose021(x_bytes.view(_vdt(es)).reshape(shape)).view(np.uint8).reshape(-1)


TILE = lambda item, vec, diag=False: {"kernel": "tile", "item": item, "vec": vec,  # noqa: E731
                                      "diag": diag}
SMALL = lambda item, vec: {"kernel": "small", "item": item, "vec": vec, "diag": False}  # noqa: E731
ITEMS = lambda item: {"kernel": "items", "item": item, "vec": False, "diag": False}  # noqa: E731

# (shape [B, R, S, E], elem_bytes, pointer offsets, expected plan of the fused call)
CASES = [
    ((2, 200, 300, 1), 4, (0, 0), TILE(4, True)),       # ragged both ways, 16-byte pitches
    ((1, 130, 75, 1), 4, (0, 0), TILE(4, False)),       # S * 4 not a multiple of 16
    ((3, 136, 264, 1), 2, (0, 0), TILE(2, True)),       # ragged against T = 128
    ((1, 257, 129, 1), 2, (0, 0), TILE(2, False)),
    ((1, 272, 400, 1), 1, (0, 0), TILE(1, True)),
    ((1, 300, 200, 1), 1, (0, 0), TILE(1, False)),
    ((2, 50, 70, 1), 8, (0, 0), TILE(8, True)),
    ((1, 45, 65, 1), 8, (0, 0), TILE(8, False)),
    ((1, 40, 33, 1), 16, (0, 0), TILE(16, True)),
    ((2, 100, 96, 2), 2, (0, 0), TILE(4, True)),        # unit of two fp16 elements
    ((1, 128, 160, 1), 4, (4, 0), TILE(4, False)),      # input off 16-byte alignment
    ((2, 1024, 300, 1), 4, (0, 0), TILE(4, True, True)),  # 4 KiB output pitch: diagonal order
    ((1, 2048, 200, 1), 2, (0, 0), TILE(2, True, True)),
    ((1, 520, 1024, 1), 4, (0, 0), TILE(4, True, True)),  # 4 KiB input pitch, ragged R
    ((1, 1000, 2048, 1), 1, (0, 4), TILE(1, False, False)),  # 2 KiB pitch: row order
    ((105, 2, 116, 1), 2, (0, 0), SMALL(2, True)),      # NHWC shuffle of 116 channels
    ((37, 3, 2, 1), 4, (0, 0), SMALL(4, True)),         # 24-byte matrices
    ((1000, 5, 3, 1), 1, (0, 0), SMALL(1, True)),       # 15-byte matrices
    ((7, 3, 5, 3), 2, (0, 0), SMALL(2, True)),          # 3-element units
    ((13, 7, 9, 1), 4, (4, 0), SMALL(4, False)),        # misaligned input
    ((5, 9, 11, 1), 1, (0, 3), SMALL(1, False)),        # misaligned output
    ((1, 100, 100, 3), 16, (0, 0), ITEMS(16)),          # 48-byte units, large matrix
    ((4, 2, 58, 784), 2, (0, 0), ITEMS(16)),            # NCHW shuffle, 28 x 28 planes
    ((2, 2, 232, 49), 2, (0, 0), ITEMS(2)),             # NCHW shuffle, 7 x 7 planes
    ((3, 150, 170, 3), 2, (0, 0), ITEMS(2)),            # 6-byte units
    ((2, 90, 100, 5), 3, (0, 0), ITEMS(1)),             # 3-byte elements
    ((3, 1, 700, 5), 2, (0, 0), ITEMS(8)),              # R = 1: a contiguous copy
    ((2, 60, 1, 8), 4, (0, 0), ITEMS(16)),              # S = 1: a contiguous copy
]


@pytest.mark.parametrize("shape,es,off,plan", CASES, ids=[f"{c[0]}x{c[1]}B" for c in CASES])
@pytest.mark.parametrize("naive", [False, True], ids=["fused", "naive"])
def test_transpose_matches_oracle(npa, orc, shape, es, off, plan, naive):
    n = int(np.prod(shape)) * es
    x = synth.random_bytes(n, seed=sum(shape) * 31 + es)
    got, p = _run_tr(npa, x, shape, es, naive, off[0], off[1], None if naive else plan)
    if naive:
        assert p["kernel"] == "items"
    want = _oracle_tr(orc, x, shape, es)
    assert np.array_equal(got, want)


def test_empty_is_a_no_op(npa):
    for shape in [(0, 5, 5, 1), (3, 0, 5, 1), (3, 5, 0, 1), (3, 5, 5, 0)]:
        assert npa.lib().fuse_transpose021(None, None, *shape, 4, None) == 0
        assert npa.lib().naive_transpose021(None, None, *shape, 4, None) == 0
        assert npa.np_transpose_plan(0, 0, shape, 4) is None


@pytest.mark.parametrize("layout", [0, 1], ids=["nchw", "nhwc"])
@pytest.mark.parametrize("es,shape,groups", [
    (2, (3, 116, 28, 28), 2), (2, (2, 464, 7, 7), 2), (4, (2, 24, 5, 3), 3),
    (1, (4, 12, 6, 6), 4), (8, (2, 10, 3, 3), 5), (2, (1, 6, 1, 1), 6), (2, (2, 8, 4, 4), 1),
    (4, (3, 22, 5, 7), 2), (8, (2, 14, 3, 5), 2), (1, (5, 18, 3, 3), 2), (2, (7, 6, 2, 3), 2),
])
@pytest.mark.parametrize("fn", ["fuse", "naive"])
def test_channel_shuffle_matches_oracle(npa, orc, layout, es, shape, groups, fn):
    N, Cc, H, W = shape
    dims = (N, Cc, H, W) if layout == 0 else (N, H, W, Cc)
    x = synth.random_bytes(int(np.prod(dims)) * es, seed=Cc + groups + es)
    tdt = {1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[es]
    xt = torch.from_numpy(x).cuda().view(tdt).view(dims)
    out = torch.empty_like(xt)
    getattr(npa, f"{fn}_channel_shuffle")(xt, out, groups, layout)
    torch.cuda.synchronize()
    got = out.cpu().view(torch.uint8).numpy().reshape(-1)
    want = orc.channel_shuffle(x.view(_vdt(es)).reshape(dims), groups, layout)
    assert np.array_equal(got, want.view(np.uint8).reshape(-1))


def test_transpose_2d_fp32_8192(npa, orc):
    """The bench's transpose workload, whole tensor against the oracle."""
    x = synth.transpose_inputs()
    xt = torch.from_numpy(x).cuda()
    for fn in ("fuse", "naive"):
        out = torch.empty_like(xt)
        getattr(npa, f"{fn}_transpose021")(xt, out)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().reshape(-1).view(np.uint32),
                              orc.transpose021(x).reshape(-1).view(np.uint32)), fn
    assert npa.np_transpose_plan(xt.data_ptr(), out.data_ptr(), synth.TRANSPOSE_2D, 4) == \
        TILE(4, True, True)


@pytest.mark.parametrize("layout", [0, 1], ids=["nchw", "nhwc"])
def test_channel_shuffle_workload(npa, orc, layout):
    """The bench's ShuffleNet-V2 stage-2 shuffle (fp16 [1024, 116, 28, 28],
    two groups), whole tensor against the oracle."""
    x = synth.shuffle_inputs(layout=layout)
    xt = torch.from_numpy(x).cuda()
    want = orc.channel_shuffle(x.view(np.uint16), synth.SHUFFLE_GROUPS, layout)
    for fn in ("fuse", "naive"):
        out = torch.empty_like(xt)
        getattr(npa, f"{fn}_channel_shuffle")(xt, out, synth.SHUFFLE_GROUPS, layout)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint16), want), fn


def _fill_pattern(t_u8, mult=151, add=7, chunk=1 << 28):
    """Structured bytes (i * mult + add) mod 256 written chunk by chunk on the GPU."""
    n = t_u8.numel()
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        idx = torch.arange(lo, hi, device="cuda", dtype=torch.int64)
        t_u8[lo:hi] = ((idx * mult + add) & 255).to(torch.uint8)
        del idx


def test_small_kernel_over_2_31_matrices(npa, orc):
    """More than 2^31 matrices: the host splits the batch over launches
    (whole-matrix kernel, 2 x 2 bytes per matrix); sampled matrices against
    the oracle."""
    B = (1 << 31) + 67
    shape = (B, 2, 2, 1)
    x = torch.empty(B * 4, dtype=torch.uint8, device="cuda")
    _fill_pattern(x)
    out = torch.empty_like(x)
    assert npa.np_transpose_plan(x.data_ptr(), out.data_ptr(), shape, 1)["kernel"] == "small"
    npa.fuse_transpose021(x, out, shape)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    idx = np.unique(np.concatenate([[0, 1, (1 << 31) - 1, 1 << 31, (1 << 31) + 1, B - 1],
                                    rng.integers(0, B, 2000)]))
    ti = torch.from_numpy(idx).cuda()
    xs = x.view(B, 4)[ti].cpu().numpy()
    os_ = out.view(B, 4)[ti].cpu().numpy()
    want = orc.transpose021(xs.reshape(len(idx), 2, 2, 1))
    assert np.array_equal(os_.reshape(-1), want.reshape(-1))
    del x, out
    torch.cuda.empty_cache()


def test_items_kernel_over_2_31_items(npa, orc):
    """3 x 2^30 four-byte elements: the naive kernel runs one launch per matrix
    (the host keeps each launch below 2^31 items); the tiled kernel runs one.
    Sampled 64 x 64 blocks against the oracle."""
    shape = (3, 1 << 15, 1 << 15, 1)
    B, R, S, _ = shape
    x = torch.empty(B * R * S * 4, dtype=torch.uint8, device="cuda")
    _fill_pattern(x, mult=40503, add=11)
    out = torch.empty_like(x)
    xv = x.view(torch.int32).view(B, R, S)
    rng = np.random.default_rng(9)
    blocks = [(0, 0, 0), (B - 1, R - 64, S - 64), (1, 4096, 8192 + 32)] + \
        [(int(rng.integers(B)), int(rng.integers(R - 64)), int(rng.integers(S - 64)))
         for _ in range(24)]
    for fn in ("naive", "fuse"):
        out.fill_(0)
        getattr(npa, f"{fn}_transpose021")(x.view(torch.int32), out.view(torch.int32),
                                           shape=shape)
        torch.cuda.synchronize()
        ov = out.view(torch.int32).view(B, S, R)
        for b, r0, s0 in blocks:
            src = xv[b, r0:r0 + 64, s0:s0 + 64].cpu().numpy()
            want = orc.transpose021(src.reshape(1, 64, 64, 1)).reshape(64, 64)
            got = ov[b, s0:s0 + 64, r0:r0 + 64].cpu().numpy()
            assert np.array_equal(got, want), (fn, b, r0, s0)
    del x, out, xv
    torch.cuda.empty_cache()


def test_python_wrapper_rejects(npa):
    x = torch.zeros(4, 6, 2, 2, dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        npa.fuse_transpose021(x.transpose(1, 2), torch.empty_like(x))
    with pytest.raises(npa.NPError):
        npa.fuse_channel_shuffle(x, torch.empty_like(x), 4)
    with pytest.raises(npa.NPError):
        npa.fuse_transpose021(x, x)  # in place
