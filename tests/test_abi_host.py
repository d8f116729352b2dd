"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every entry point that include/norm_pass.h
declares, reject bad arguments with NP_EINVAL and a message before touching any
device, and its runtime specialiser must generate source that hipRTC compiles
for gfx950 (compilation needs no GPU).
"""
import ctypes as C
import os
import re

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def npa():
    import norm_pass_amd
    return norm_pass_amd


def declared_functions():
    src = open(os.path.join(ROOT, "include", "norm_pass.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|int64_t|void|const char\*)\s+(\w+)\s*\(", src,
                                 flags=re.M)))


def test_library_exports_every_declared_symbol(npa):
    names = declared_functions()
    assert len(names) >= 18 and "np_chain_source" in names
    for n in names:
        assert hasattr(npa.lib(), n), n


def test_version(npa):
    assert npa.np_version() == 1


NULL = None


def _err(npa):
    return npa.lib().np_last_error().decode()


@pytest.mark.parametrize("ops,n_inputs,n,msg", [
    ([(synth.RELU, 0, 0)], 1, 4, "NP_LOAD"),
    ([(synth.LOAD, 2, 0)], 2, 4, "input index"),
    ([(synth.LOAD, 0, 0), (42, 0, 0)], 1, 4, "unknown kind"),
    ([(synth.LOAD, 0, 0)], 0, 4, "n_inputs"),
    ([(synth.LOAD, 0, 0)], 5, 4, "n_inputs"),
    ([(synth.LOAD, 0, 0)] * 33, 1, 4, "n_ops"),
    ([(synth.LOAD, 0, 0)], 1, -1, "n = -1"),
    ([(synth.LOAD, 0, 0)], 1, 1 << 40, "not below 2^40"),
])
def test_fuse_chain_rejects(npa, ops, n_inputs, n, msg):
    arr, k = npa._ops(ops)
    for fn in (npa.lib().fuse_chain, npa.lib().unfused_chain):
        rc = fn(arr, k, NULL, n_inputs, 0, NULL, 0, n, NULL)
        assert rc == npa.NP_EINVAL
        assert msg in _err(npa)


def test_fuse_chain_null_buffers(npa):
    arr, k = npa._ops(synth.C1_CHAIN)
    ptrs = (C.c_void_p * 2)(0x1000, 0)
    assert npa.lib().fuse_chain(arr, k, ptrs, 2, 0, C.c_void_p(0x2000), 0, 8, NULL) == -1
    assert "inputs[1] is NULL" in _err(npa)
    ptrs = (C.c_void_p * 2)(0x1000, 0x3000)
    assert npa.lib().fuse_chain(arr, k, ptrs, 2, 0, NULL, 0, 8, NULL) == -1
    assert "out is NULL" in _err(npa)
    assert npa.lib().fuse_chain(arr, k, ptrs, 2, 7, C.c_void_p(0x2000), 0, 8, NULL) == -1


def test_unfused_chain_requires_storage_type(npa):
    arr, k = npa._ops(synth.C1_CHAIN)
    ptrs = (C.c_void_p * 2)(0x1000, 0x3000)
    assert npa.lib().unfused_chain(arr, k, ptrs, 2, 1, C.c_void_p(0x2000), 0, 8, NULL) == -1
    assert "in_dt == out_dt" in _err(npa)


def test_zero_length_is_a_no_op(npa):
    # n == 0 needs no buffers and no device
    arr, k = npa._ops(synth.C1_CHAIN)
    assert npa.lib().fuse_chain(arr, k, NULL, 2, 0, NULL, 0, 0, NULL) == 0


def _det_call(npa, fn, n_levels=1, H=4, W=4, n_anchors=3, n_ch=85, batch=1, dt=1, out=0x4000,
              lv=0x1000, extra=()):
    ptrs = (C.c_void_p * max(n_levels, 1))(*([lv] * max(n_levels, 1)))
    Hs = (C.c_int32 * max(n_levels, 1))(*([H] * max(n_levels, 1)))
    Ws = (C.c_int32 * max(n_levels, 1))(*([W] * max(n_levels, 1)))
    st = (C.c_float * max(n_levels, 1))(*([8.0] * max(n_levels, 1)))
    an = (C.c_float * 256)()
    return fn(ptrs, n_levels, Hs, Ws, st, an, n_anchors, n_ch, batch, dt,
              C.c_void_p(out) if out else NULL, *extra)


@pytest.mark.parametrize("kw,msg", [
    (dict(n_levels=0), "n_levels"),
    (dict(n_levels=9), "n_levels"),
    (dict(n_anchors=0), "n_anchors"),
    (dict(n_anchors=17), "n_anchors"),
    (dict(n_ch=4), "n_ch"),
    (dict(n_ch=1025), "n_ch"),
    (dict(batch=0), "batch"),
    (dict(H=0), "bad H x W"),
    (dict(out=0), "NULL"),
    (dict(lv=0), "NULL"),
    (dict(dt=3), "dtype"),
])
def test_det_decode_rejects(npa, kw, msg):
    assert _det_call(npa, npa.lib().fuse_det_decode, extra=(NULL,), **kw) == -1
    assert msg in _err(npa)


def test_unfused_det_decode_needs_workspace(npa):
    rc = _det_call(npa, npa.lib().unfused_det_decode, extra=(C.c_void_p(0x8000), 100, NULL))
    assert rc == -1 and "workspace needs" in _err(npa)


@pytest.mark.parametrize("args,msg", [
    ((NULL, NULL, NULL, NULL, 0x2000, 4, 8, 1e-6, 2), "NULL"),
    ((0x1000, NULL, NULL, NULL, 0x2000, -1, 8, 1e-6, 2), "rows"),
    ((0x1000, NULL, NULL, NULL, 0x2000, 4, 0, 1e-6, 2), "cols"),
    ((0x1000, NULL, NULL, NULL, 0x2000, 4, (1 << 24) + 1, 1e-6, 2), "cols"),
    ((0x1000, NULL, NULL, NULL, 0x2000, 4, 8, 0.0, 2), "eps"),
    ((0x1000, NULL, NULL, NULL, 0x2000, 4, 8, float("inf"), 2), "eps"),
    ((0x1000, NULL, NULL, NULL, 0x2000, 4, 8, float("nan"), 2), "eps"),
    ((0x1000, NULL, NULL, 0x2000, 0x2000, 4, 8, 1e-6, 2), "differ"),
    ((0x1000, NULL, NULL, NULL, 0x2000, 4, 8, 1e-6, 5), "dtype"),
])
def test_add_rmsnorm_rejects(npa, args, msg):
    a = [C.c_void_p(v) if isinstance(v, int) and i < 5 else v for i, v in enumerate(args)]
    assert npa.lib().fuse_add_rmsnorm(*a, NULL) == -1
    assert msg in _err(npa)


@pytest.mark.parametrize("T,H,D,base,qs,msg", [
    (-1, 24, 128, 1e4, 0.1, "T out of range"),
    (4, 0, 128, 1e4, 0.1, "n_heads"),
    (4, 2, 7, 1e4, 0.1, "head_dim"),
    (4, 2, 514, 1e4, 0.1, "head_dim"),
    (4, 2, 128, 0.0, 0.1, "base"),
    (4, 2, 128, 1e4, float("inf"), "q_scale"),
])
def test_qkv_rope_rejects(npa, T, H, D, base, qs, msg):
    p = [C.c_void_p(0x1000 * (i + 1)) for i in range(4)]
    for fn in (npa.lib().fuse_qkv_rope, npa.lib().unfused_qkv_rope):
        assert fn(*p, T, H, D, NULL, base, qs, 2, NULL) == -1
        assert msg in _err(npa)


def test_qkv_rope_rejects_aliasing(npa):
    p = [C.c_void_p(0x1000), C.c_void_p(0x2000), C.c_void_p(0x2000), C.c_void_p(0x3000)]
    assert npa.lib().fuse_qkv_rope(*p, 4, 2, 8, NULL, 1e4, 0.5, 2, NULL) == -1
    assert "alias" in _err(npa)


def test_runtime_specialisation_compiles(npa):
    """The generated source compiles with hipRTC for gfx950 (DeepJIT write-up,
    sections 3.3 and 6.2: tens to hundreds of ms per runtime compile)."""
    ms1, b1 = npa.np_chain_compile(synth.C1_CHAIN, 2, npa.NP_F32, npa.NP_F32, 1 << 20)
    ms2, b2 = npa.np_chain_compile(synth.c5_chain(), 1, npa.NP_F16, npa.NP_F16, 0)
    assert b1 > 0 and b2 > 0 and ms1 > 0 and ms2 > 0
    with pytest.raises(npa.NPError):
        npa.np_chain_compile([(synth.LOAD, 0, 0), (77, 0, 0)], 1, 0, 0, 0)


def test_add_layernorm_rejects(npa):
    p = [C.c_void_p(0x1000), None, None, None, None, C.c_void_p(0x2000)]
    assert npa.lib().fuse_add_layernorm(*p, 4, 8, 0.0, 2, NULL) == -1
    assert "eps" in _err(npa)
    assert npa.lib().unfused_add_layernorm(*p, 4, 8, 1e-5, 2, NULL, 0, NULL) == -1
    assert "workspace" in _err(npa)


# ---- layout calls: validation and kernel choice (host only) ----------------

_LAY = [(1 << 40), (1 << 42)]


@pytest.mark.parametrize("args,msg", [
    ((-1, 4, 4, 1, 4), "negative"),
    ((1, 4, 4, 1, 0), "elem_bytes"),
    ((1, 4, 4, 1, 17), "elem_bytes"),
    ((1, 1 << 31, 4, 1, 4), "out of range"),
    ((1 << 20, 1 << 20, 1 << 20, 1, 4), "2^46"),
])
def test_transpose_rejects(npa, args, msg):
    B, R, S, E, es = args
    for fn in (npa.lib().fuse_transpose021, npa.lib().naive_transpose021):
        assert fn(C.c_void_p(_LAY[0]), C.c_void_p(_LAY[1]), B, R, S, E, es, NULL) == -1
        assert msg in _err(npa)


def test_transpose_rejects_null_and_overlap(npa):
    f = npa.lib().fuse_transpose021
    assert f(NULL, C.c_void_p(0x1000), 1, 4, 4, 1, 4, NULL) == -1 and "NULL" in _err(npa)
    # [0x1000, 0x1040) and [0x1020, 0x1060) overlap
    assert f(C.c_void_p(0x1000), C.c_void_p(0x1020), 1, 4, 4, 1, 4, NULL) == -1
    assert "overlap" in _err(npa)
    assert f(C.c_void_p(0x1000), C.c_void_p(0x1040), 1, 4, 4, 1, 4, NULL) != -1 or \
        "overlap" not in _err(npa)


@pytest.mark.parametrize("args,msg", [
    ((2, 6, 4, 4, 4, 0), "divide"),
    ((2, 6, 4, 4, 0, 0), "groups"),
    ((2, 6, 4, 4, 2, 7), "layout"),
    ((2, -6, 4, 4, 2, 0), "negative"),
])
def test_channel_shuffle_rejects(npa, args, msg):
    for fn in (npa.lib().fuse_channel_shuffle, npa.lib().naive_channel_shuffle):
        assert fn(C.c_void_p(_LAY[0]), C.c_void_p(_LAY[1]), *args, 2, NULL) == -1
        assert msg in _err(npa)


def test_transpose_plans(npa):
    """The kernel the planner picks for each case the GPU parity tests run."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "layout_cases", os.path.join(ROOT, "tests", "test_gpu_layout.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    for shape, es, off, plan in mod.CASES:
        got = npa.np_transpose_plan(_LAY[0] + off[0], _LAY[1] + off[1], shape, es)
        assert got == plan, (shape, es, got)
        naive = npa.np_transpose_plan(_LAY[0] + off[0], _LAY[1] + off[1], shape, es, True)
        assert naive["kernel"] == "items"
    assert npa.np_transpose_plan(_LAY[0], _LAY[1], (0, 3, 3, 1), 4) is None


@pytest.mark.parametrize("args,msg", [
    ((4, 32, 60, 1e-6, 1.0, 2), "multiple of 8"),
    ((4, 32, 64, 1e-6, 1.0, 0), "fp16 or bf16"),
    ((4, 0, 64, 1e-6, 1.0, 2), "N ="),
    ((-1, 32, 64, 1e-6, 1.0, 2), "M ="),
    ((4, 32, 64, 0.0, 1.0, 2), "eps"),
    ((4, 32, 64, 1e-6, float("inf"), 2), "scale"),
    (((1 << 31) - 1, (1 << 31) - 1, 64, 1e-6, 1.0, 2), "2^31 output tiles"),
])
def test_rmsnorm_linear_rejects(npa, args, msg):
    M, N, K, eps, scale, dt = args
    p = [C.c_void_p(1 << 40), None, C.c_void_p(1 << 42), None, C.c_void_p(1 << 44)]
    for fn in (npa.lib().fuse_rmsnorm_linear,):
        assert fn(*p, M, N, K, eps, scale, dt, NULL) == -1
        assert msg in _err(npa)
    assert npa.lib().unfused_rmsnorm_linear(*p, 4, 32, 64, 1e-6, 1.0, 2, NULL, 0, NULL) == -1
    assert "workspace" in _err(npa)


def test_rmsnorm_linear_rejects_overlap_and_alignment(npa):
    base = 1 << 40
    # out overlaps x
    assert npa.lib().fuse_rmsnorm_linear(C.c_void_p(base), None, C.c_void_p(1 << 42), None,
                                         C.c_void_p(base + 64), 4, 32, 64, 1e-6, 1.0, 2,
                                         NULL) == -1
    assert "overlaps" in _err(npa)
    assert npa.lib().fuse_rmsnorm_linear(C.c_void_p(base + 2), None, C.c_void_p(1 << 42), None,
                                         C.c_void_p(1 << 44), 4, 32, 64, 1e-6, 1.0, 2,
                                         NULL) == -1
    assert "aligned" in _err(npa)


def test_zero_rows_tokens_and_elements_are_no_ops(npa):
    """Every entry point with an empty leading size returns NP_OK before it
    looks for a device: the buffers (addresses that are never dereferenced
    here) are not touched and nothing is launched."""
    L = npa.lib()
    x, r, w, h, out, ws = (C.c_void_p(0x1000 * (i + 1)) for i in range(6))
    for dt in (0, 1, 2):
        assert L.fuse_add_rmsnorm(x, r, w, h, out, 0, 4096, 1e-6, dt, NULL) == 0
        assert L.fuse_add_rmsnorm(x, NULL, NULL, NULL, out, 0, 8, 1e-6, dt, NULL) == 0
        assert L.unfused_add_rmsnorm(x, r, w, h, out, 0, 4096, 1e-6, dt, ws, 1 << 20, NULL) == 0
        assert L.fuse_add_layernorm(x, r, w, w, h, out, 0, 4096, 1e-5, dt, NULL) == 0
        assert L.unfused_add_layernorm(x, r, w, w, h, out, 0, 4096, 1e-5, dt, ws, 1 << 20,
                                       NULL) == 0
        p = [C.c_void_p(0x1000 * (i + 1)) for i in range(4)]
        assert L.fuse_qkv_rope(*p, 0, 24, 128, NULL, 1e4, 0.125, dt, NULL) == 0
        assert L.unfused_qkv_rope(*p, 0, 24, 128, NULL, 1e4, 0.125, dt, NULL) == 0
    arr, k = npa._ops(synth.C1_CHAIN)
    ptrs = (C.c_void_p * 2)(0x1000, 0x3000)
    assert L.fuse_chain(arr, k, ptrs, 2, 0, out, 0, 0, NULL) == 0
    assert L.unfused_chain(arr, k, ptrs, 2, 0, out, 0, 0, NULL) == 0
    for bf in (1, 2):
        assert L.fuse_rmsnorm_linear(C.c_void_p(1 << 40), None, C.c_void_p(1 << 42), None,
                                     C.c_void_p(1 << 44), 0, 32, 64, 1e-6, 1.0, bf, NULL) == 0


def test_zero_size_rejects_still_apply(npa):
    """An empty call is still checked: a NULL required buffer or a bad
    dtype, width or head_dim is NP_EINVAL even when there is nothing to do."""
    L = npa.lib()
    out = C.c_void_p(0x2000)
    assert L.fuse_add_rmsnorm(NULL, NULL, NULL, NULL, out, 0, 8, 1e-6, 2, NULL) == -1
    assert L.fuse_add_rmsnorm(C.c_void_p(0x1000), NULL, NULL, NULL, out, 0, 0, 1e-6, 2,
                              NULL) == -1
    p = [C.c_void_p(0x1000 * (i + 1)) for i in range(4)]
    assert L.fuse_qkv_rope(*p, 0, 24, 7, NULL, 1e4, 0.125, 2, NULL) == -1
    assert L.fuse_add_layernorm(C.c_void_p(0x1000), NULL, NULL, NULL, NULL, out, 0, 8, 1e-5, 9,
                                NULL) == -1


def test_unfused_chain_rejects_alias_read_again(npa):
    """out may alias the first loaded input only while no later op reads that
    input again: the first launch has overwritten it by then."""
    ops = (npa.np_op * 3)()
    for i, (k, a, c) in enumerate([(synth.LOAD, 0, 0.0), (synth.MUL_C, 0, 2.0),
                                   (synth.ADD_IN, 0, 0.0)]):
        ops[i].kind, ops[i].arg, ops[i].c = k, a, c
    buf = C.c_void_p(0x10000)
    ins = (C.c_void_p * 1)(buf)
    assert npa.lib().unfused_chain(ops, 3, ins, 1, 1, buf, 1, 64, NULL) == -1
    assert "reads after the first launch" in _err(npa)


# ---- the Python binding checks its tensors before any C call -------------

import torch  # noqa: E402


def _t(shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


@pytest.mark.parametrize("case,msg", [
    (lambda n: n._a_fuse_chain([(synth.LOAD, 0, 0.0)], [_t(8, torch.float16)], _t(8)),
     "every tensor must be on a GPU"),
    (lambda n: n._a_fuse_chain([(synth.LOAD, 0, 0.0), (synth.ADD_IN, 1, 0.0)],
                               [_t(8), _t(8, torch.float16)], _t(8)), "expected torch.bfloat16"),
    (lambda n: n._a_fuse_chain([(synth.LOAD, 0, 0.0)], [_t(7)], _t(8)), "has 7 elements"),
    (lambda n: n._a_fuse_chain([(synth.LOAD, 0, 0.0)], [_t((4, 4)).t()], _t(16)),
     "must be contiguous"),
    (lambda n: n._a_fuse_chain([(synth.LOAD, 0, 0.0)], [_t(8)] * 5, _t(8)), "1..4 inputs"),
    (lambda n: n._a_fuse_add_rmsnorm(_t((2, 3, 8)), _t((2, 3, 8)), _t(7), None, _t((2, 3, 8))),
     "w has 7 elements, expected 8"),
    (lambda n: n._a_fuse_add_rmsnorm(_t((2, 3, 8)), _t((2, 3, 8)), _t(8), _t((2, 8)),
                                     _t((2, 3, 8))), "h_out has 16 elements, expected 48"),
    (lambda n: n._a_fuse_add_layernorm(_t((4, 8)), None, _t(8), _t(8, torch.float16), None,
                                       _t((4, 8))), "beta is torch.float16"),
    (lambda n: n._a_fuse_qkv_rope(_t((4, 3 * 2 * 8)), _t((2, 4, 8)), _t((2, 4, 8)),
                                  _t((2, 4, 8)), 2, 8, torch.arange(4)), "expected torch.int32"),
    (lambda n: n._a_fuse_qkv_rope(_t((4, 3 * 2 * 8)), _t((2, 4, 8)), _t((2, 3, 8)),
                                  _t((2, 4, 8)), 2, 8), "k has 48 elements, expected 64"),
    (lambda n: n._a_fuse_qkv_rope(_t((4, 40)), _t((2, 4, 8)), _t((2, 4, 8)), _t((2, 4, 8)), 2,
                                  8), "qkv has 160 elements, expected 192"),
    (lambda n: n._a_fuse_rmsnorm_linear(_t((4, 64)), None, _t((32, 48)), None, _t((4, 32))),
     "x must be [M, K] and Wt [N, K]"),
    (lambda n: n._a_fuse_rmsnorm_linear(_t((4, 64)), None, _t((32, 64)), _t(31), _t((4, 32))),
     "bias has 31 elements"),
    (lambda n: n._a_fuse_det_decode([_t((1, 255, 4, 4), torch.float16)], [8.0],
                                    [[(1, 1)] * 3], _t((1, 48, 84), torch.float32)),
     "out has 4032 elements, expected 4080"),
    (lambda n: n._a_fuse_det_decode([_t((1, 254, 4, 4), torch.float16)], [8.0],
                                    [[(1, 1)] * 3], _t((1, 48, 85), torch.float32)),
     "[batch, n_anchors * n_ch, H, W]"),
    (lambda n: n._a_unfused_add_rmsnorm(_t((4, 8)), None, None, None, _t((4, 8)), None),
     "a workspace tensor is required"),
    (lambda n: n._a_fuse_transpose021(_t((2, 3, 4, 5)), _t(120)), "need GPU tensors"),
])
def test_binding_rejects_bad_tensors(npa, case, msg):
    with pytest.raises(ValueError, match=re.escape(msg)):
        case(npa)


def test_binding_norm_rows_span_leading_axes(npa):
    """A [B, T, C] tensor is B * T rows of C (every leading axis is a row)."""
    assert npa._rows_cols("f", _t((2, 3, 8))) == (6, 8)
    assert npa._rows_cols("f", _t(8)) == (1, 8)


def test_unfused_baselines_reject_oversized_calls(npa):
    """One thread per element: the unfused baselines take fewer than 2^31
    elements (and row reductions fewer than 2^23 rows) per call; nothing is
    launched then."""
    ops = (npa.np_op * 2)()
    ops[0].kind, ops[1].kind = synth.LOAD, synth.RELU
    buf = (C.c_void_p * 1)(C.c_void_p(0x10000))
    assert npa.lib().unfused_chain(ops, 2, buf, 1, 1, C.c_void_p(0x20000), 1, 1 << 31, NULL) == -1
    assert "2^31" in _err(npa)
    p = [C.c_void_p(0x1000 * (i + 1)) for i in range(6)]
    assert npa.lib().unfused_add_rmsnorm(p[0], NULL, NULL, p[1], p[2], 1 << 23, 1, 1e-6, 2,
                                         p[3], 1 << 40, NULL) == -1
    assert "2^23 rows" in _err(npa)
    assert npa.lib().unfused_qkv_rope(p[0], p[1], p[2], p[3], 1 << 22, 24, 128, NULL, 1e4, 0.5,
                                      2, NULL) == -1
    assert "2^31" in _err(npa)


def test_det_decode_rejects_more_tiles_than_one_launch(npa):
    """One 256-thread workgroup per 24-cell tile: at most 2^23 tiles."""
    lv = (C.c_void_p * 1)(C.c_void_p(0x10000))
    H = (C.c_int32 * 1)(2048)
    W = (C.c_int32 * 1)(2048)
    st = (C.c_float * 1)(8.0)
    an = (C.c_float * 2)(10.0, 13.0)
    # 2048 x 2048 cells = 174,763 tiles per (image, anchor); 48 images: 8.4e6 tiles
    assert npa.lib().fuse_det_decode(lv, 1, H, W, st, an, 1, 85, 48, 1, C.c_void_p(0x20000),
                                     NULL) == -1
    assert "tiles" in _err(npa)
