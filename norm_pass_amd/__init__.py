"""Python binding of libnorm_pass_amd.so (ctypes; argument marshalling only).

Every function here has the name of the C entry point it calls (declared in
``include/norm_pass.h``) and takes torch tensors on the GPU for the device
buffers: it passes ``data_ptr()``s, sizes and the current HIP stream, and
raises :class:`NPError` with the library's message when the call fails. All
computation happens in the library's HIP kernels; torch only owns memory and
streams. Importing this module fails loudly when the library is not built.
"""
from __future__ import annotations

import ctypes as C
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnorm_pass_amd.so")

NP_OK, NP_EINVAL, NP_ELAUNCH, NP_ECOMPILE, NP_EDEVICE = 0, -1, -3, -4, -5
NP_F32, NP_F16, NP_BF16 = 0, 1, 2
(NP_LOAD, NP_ADD_IN, NP_MUL_IN, NP_ADD_C, NP_MUL_C, NP_SCALE, NP_RELU, NP_SIGMOID, NP_EXP,
 NP_TANH, NP_CAST_F16, NP_CAST_BF16) = range(12)
MAX_OPS, MAX_INPUTS = 32, 4

_DT = {torch.float32: NP_F32, torch.float16: NP_F16, torch.bfloat16: NP_BF16}
_SIZE = {NP_F32: 4, NP_F16: 2, NP_BF16: 2}


class NPError(RuntimeError):
    def __init__(self, code: int, fn: str, msg: str):
        super().__init__(f"{fn} failed ({code}): {msg}")
        self.code = code


class np_op(C.Structure):
    _fields_ = [("kind", C.c_int32), ("arg", C.c_int32), ("c", C.c_float)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950)")
    L = C.CDLL(LIB_PATH)
    P, I, I64, F, S = C.c_void_p, C.c_int, C.c_int64, C.c_float, C.c_size_t
    OPS = C.POINTER(np_op)
    sig = {
        "np_init": [I],
        "np_version": [],
        "np_shutdown": [],
        "np_chain_compile": [OPS, I, I, I, I, I64, C.POINTER(C.c_double), C.POINTER(S)],
        "np_chain_source": [OPS, I, I, I, I, I64, C.c_char_p, S],
        "fuse_chain": [OPS, I, P, I, I, P, I, I64, P],
        "fuse_chain_prepare": [OPS, I, I, I, I, I64],
        "fuse_det_decode": [P, I, P, P, P, P, I, I, I, I, P, P],
        "fuse_add_rmsnorm": [P, P, P, P, P, I64, I64, F, I, P],
        "fuse_qkv_rope": [P, P, P, P, I64, I, I, P, F, F, I, P],
        "fuse_add_layernorm": [P, P, P, P, P, P, I64, I64, F, I, P],
        "unfused_add_layernorm": [P, P, P, P, P, P, I64, I64, F, I, P, S, P],
        "unfused_chain": [OPS, I, P, I, I, P, I, I64, P],
        "unfused_det_decode": [P, I, P, P, P, P, I, I, I, I, P, P, S, P],
        "unfused_det_decode_noalloc": [P, I, P, P, P, P, I, I, I, I, P, P],
        "unfused_add_rmsnorm": [P, P, P, P, P, I64, I64, F, I, P, S, P],
        "unfused_qkv_rope": [P, P, P, P, I64, I, I, P, F, F, I, P],
        "np_empty_launches": [I, P],
        "fuse_rmsnorm_linear": [P, P, P, P, P, I64, I64, I64, F, F, I, P],
        "unfused_rmsnorm_linear": [P, P, P, P, P, I64, I64, I64, F, F, I, P, S, P],
        "np_fold_norm_weight": [P, P, P, I64, I64, I, P],
        "fuse_transpose021": [P, P, I64, I64, I64, I64, I, P],
        "naive_transpose021": [P, P, I64, I64, I64, I64, I, P],
        "fuse_channel_shuffle": [P, P, I64, I64, I64, I64, I64, I, I, P],
        "naive_channel_shuffle": [P, P, I64, I64, I64, I64, I64, I, I, P],
        "np_transpose_plan": [P, P, I64, I64, I64, I64, I, I],
        "np_set_chain_table_min": [I64],
        "np_chain_cache_stats": [C.POINTER(I64)] * 3,
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = (None if name in ("np_shutdown", "np_chain_cache_stats") else
                      C.c_int64 if name in ("np_chain_source", "np_set_chain_table_min")
                      else C.c_int)
    L.np_last_error.restype = C.c_char_p
    L.np_last_error.argtypes = []
    return L


_lib = _load()


def lib():
    return _lib


def _check(rc: int, fn: str):
    if rc != NP_OK:
        raise NPError(rc, fn, _lib.np_last_error().decode(errors="replace"))


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _keep(stream, *tensors):
    """Tie tensor lifetimes to a non-current stream (caching-allocator safety)."""
    if stream is None or stream == torch.cuda.current_stream():
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _need(cond: bool, fn: str, msg: str):
    if not cond:
        raise ValueError(f"{fn}: {msg}")


def _dev(fn: str, name: str, t, dtype=None, numel=None):
    """A device buffer argument: a contiguous tensor, of `dtype` and with
    `numel` elements when those are given. Returns t (None passes)."""
    if t is None:
        return None
    _need(isinstance(t, torch.Tensor), fn, f"{name} must be a torch tensor")
    _need(t.is_contiguous(), fn, f"{name} must be contiguous")
    if dtype is not None:
        _need(t.dtype == dtype, fn, f"{name} is {t.dtype}, expected {dtype}")
    if numel is not None:
        _need(t.numel() == numel, fn, f"{name} has {t.numel()} elements, expected {numel}")
    return t


def _on_gpu(fn: str, *tensors):
    """Last check of a builder (after every shape and type check): all device
    buffers live on a GPU."""
    for t in tensors:
        if isinstance(t, (list, tuple)):
            _on_gpu(fn, *t)
        elif t is not None:
            _need(t.is_cuda, fn, "every tensor must be on a GPU")


def _float_dtype(fn: str, t):
    _need(isinstance(t, torch.Tensor) and t.dtype in _DT, fn,
          "tensors must be float32, float16 or bfloat16")
    return t.dtype


def _rows_cols(fn: str, x):
    """[..., cols] viewed as rows of cols (every leading axis is a row index)."""
    _need(x.dim() >= 1 and x.shape[-1] >= 1, fn, "x needs a last axis of at least one element")
    cols = x.shape[-1]
    return x.numel() // cols, cols


def _ops(ops):
    arr = (np_op * len(ops))()
    for i, (k, a, c) in enumerate(ops):
        arr[i].kind, arr[i].arg, arr[i].c = int(k), int(a), float(c)
    return arr, len(ops)


def dtype_code(t) -> int:
    return _DT[t.dtype if isinstance(t, torch.Tensor) else t]


# ------------------------------------------------------------------ helpers

def np_init(device: int = 0):
    _check(_lib.np_init(device), "np_init")


def np_version() -> int:
    return _lib.np_version()


def np_shutdown():
    _lib.np_shutdown()


def np_chain_compile(ops, n_inputs: int, in_dt: int, out_dt: int, n: int = 0):
    """Compile (not load) the specialised source; returns (compile_ms, code_bytes)."""
    arr, k = _ops(ops)
    ms = C.c_double(0)
    nb = C.c_size_t(0)
    _check(_lib.np_chain_compile(arr, k, n_inputs, in_dt, out_dt, n, C.byref(ms), C.byref(nb)),
           "np_chain_compile")
    return ms.value, nb.value


def np_chain_source(ops, n_inputs: int, in_dt: int, out_dt: int, n: int = 0) -> str:
    """The generated kernel source fuse_chain_prepare would compile."""
    arr, k = _ops(ops)
    size = _lib.np_chain_source(arr, k, n_inputs, in_dt, out_dt, n, None, 0)
    if size < 0:
        _check(int(size), "np_chain_source")
    buf = C.create_string_buffer(int(size))
    _lib.np_chain_source(arr, k, n_inputs, in_dt, out_dt, n, buf, size)
    return buf.value.decode()


def np_empty_launches(count: int, stream=None):
    _check(_lib.np_empty_launches(count, _stream(stream)), "np_empty_launches")


# -------------------------------------------------------------- fused calls
# Each call is split into an argument builder (_a_<name>: torch tensors ->
# ctypes arguments) and the C call itself, so that `bind` can marshal once and
# hand back a zero-argument callable for tight launch loops.

def _a_fuse_chain(ops, inputs, out, stream=None):
    fn = "fuse_chain"
    _need(1 <= len(inputs) <= MAX_INPUTS, fn, f"1..{MAX_INPUTS} inputs")
    dt = _float_dtype(fn, inputs[0])
    _float_dtype(fn, out)
    for j, t in enumerate(inputs):
        _dev(fn, f"inputs[{j}]", t, dt, out.numel())
    _dev(fn, "out", out)
    _on_gpu(fn, inputs, out)
    arr, k = _ops(ops)
    ptrs = (C.c_void_p * len(inputs))(*[t.data_ptr() for t in inputs])
    _keep(stream, out, *inputs)
    return (arr, k, ptrs, len(inputs), dtype_code(inputs[0]), _ptr(out), dtype_code(out),
            out.numel(), _stream(stream))


def _det_args(levels, strides, anchors):
    n_levels = len(levels)
    H = (C.c_int32 * n_levels)(*[t.shape[2] for t in levels])
    W = (C.c_int32 * n_levels)(*[t.shape[3] for t in levels])
    st = (C.c_float * n_levels)(*[float(s) for s in strides])
    flat = [float(v) for lvl in anchors for pair in lvl for v in pair]
    an = (C.c_float * len(flat))(*flat)
    ptrs = (C.c_void_p * n_levels)(*[t.data_ptr() for t in levels])
    return ptrs, n_levels, H, W, st, an


def det_rows(levels, n_anchors: int) -> int:
    return sum(n_anchors * t.shape[2] * t.shape[3] for t in levels)


def _a_fuse_det_decode(levels, strides, anchors, out, n_anchors: int = 3, n_ch: int = 85,
                       stream=None):
    fn = "fuse_det_decode"
    _need(len(levels) >= 1 and len(strides) == len(levels) and len(anchors) == len(levels), fn,
          "one stride and one anchor list per level")
    dt = _float_dtype(fn, levels[0])
    batch = levels[0].shape[0] if levels[0].dim() == 4 else 0
    for l, t in enumerate(levels):
        _need(t.dim() == 4 and t.shape[0] == batch and t.shape[1] == n_anchors * n_ch, fn,
              f"levels[{l}] must be [batch, n_anchors * n_ch, H, W] with one batch size")
        _dev(fn, f"levels[{l}]", t, dt)
        _need(len(anchors[l]) == n_anchors and all(len(p) == 2 for p in anchors[l]), fn,
              f"anchors[{l}] must hold n_anchors (w, h) pairs")
    _dev(fn, "out", out, torch.float32, batch * det_rows(levels, n_anchors) * n_ch)
    _on_gpu(fn, levels, out)
    ptrs, nl, H, W, st, an = _det_args(levels, strides, anchors)
    _keep(stream, out, *levels)
    return (ptrs, nl, H, W, st, an, n_anchors, n_ch, levels[0].shape[0], dtype_code(levels[0]),
            _ptr(out), _stream(stream))


def _norm_checks(fn, x, r, weights, h_out, out):
    dt = _float_dtype(fn, x)
    rows, cols = _rows_cols(fn, x)
    _dev(fn, "x", x, dt)
    for name, t in (("r", r), ("h_out", h_out), ("out", out)):
        _dev(fn, name, t, dt, x.numel())
    for name, t in weights:
        _dev(fn, name, t, dt, cols)
    _on_gpu(fn, x, r, h_out, out, [t for _, t in weights])
    return rows, cols


def _a_fuse_add_rmsnorm(x, r, w, h_out, out, eps: float = 1e-6, stream=None):
    rows, cols = _norm_checks("fuse_add_rmsnorm", x, r, (("w", w),), h_out, out)
    _keep(stream, x, r, w, h_out, out)
    return (_ptr(x), _ptr(r), _ptr(w), _ptr(h_out), _ptr(out), rows, cols, eps,
            dtype_code(x), _stream(stream))


def _a_fuse_qkv_rope(qkv, q, k, v, n_heads: int, head_dim: int, positions=None,
                     base: float = 10000.0, q_scale: float | None = None, stream=None):
    fn = "fuse_qkv_rope"
    if q_scale is None:
        q_scale = 1.0 / math.sqrt(head_dim)
    dt = _float_dtype(fn, qkv)
    _need(qkv.dim() >= 1, fn, "qkv must be [T, 3 * n_heads * head_dim]")
    T = qkv.shape[0]
    _dev(fn, "qkv", qkv, dt, T * 3 * n_heads * head_dim)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t is not None, fn, f"{name} is required")
        _dev(fn, name, t, dt, n_heads * T * head_dim)
    _dev(fn, "positions", positions, torch.int32, T)
    _on_gpu(fn, qkv, q, k, v, positions)
    _keep(stream, qkv, q, k, v, positions)
    return (_ptr(qkv), _ptr(q), _ptr(k), _ptr(v), T, n_heads, head_dim,
            _ptr(positions), base, q_scale, dtype_code(qkv), _stream(stream))


def _a_fuse_add_layernorm(x, r, gamma, beta, h_out, out, eps: float = 1e-5, stream=None):
    rows, cols = _norm_checks("fuse_add_layernorm", x, r, (("gamma", gamma), ("beta", beta)),
                              h_out, out)
    _keep(stream, x, r, gamma, beta, h_out, out)
    return (_ptr(x), _ptr(r), _ptr(gamma), _ptr(beta), _ptr(h_out), _ptr(out), rows, cols, eps,
            dtype_code(x), _stream(stream))


def _workspace(fn, t):
    _need(t is not None, fn, "a workspace tensor is required")
    _dev(fn, "workspace", t)
    _on_gpu(fn, t)
    return t


def _a_unfused_add_layernorm(x, r, gamma, beta, h_out, out, workspace, eps: float = 1e-5,
                             stream=None):
    _workspace("unfused_add_layernorm", workspace)
    a = _a_fuse_add_layernorm(x, r, gamma, beta, h_out, out, eps, stream)
    _keep(stream, workspace)
    return a[:-1] + (_ptr(workspace), workspace.numel() * workspace.element_size(), a[-1])


_a_unfused_chain = _a_fuse_chain
_a_unfused_qkv_rope = _a_fuse_qkv_rope


def _a_fuse_rmsnorm_linear(x, w_norm, Wt, bias, out, eps: float = 1e-6, scale: float = 1.0,
                           stream=None):
    fn = "fuse_rmsnorm_linear"
    dt = _float_dtype(fn, x)
    _need(x.dim() == 2 and Wt.dim() == 2 and Wt.shape[1] == x.shape[1], fn,
          "x must be [M, K] and Wt [N, K]")
    M, K = x.shape
    N = Wt.shape[0]
    _dev(fn, "x", x, dt)
    _dev(fn, "Wt", Wt, dt)
    _dev(fn, "w_norm", w_norm, dt, K)
    _dev(fn, "bias", bias, dt, N)
    _dev(fn, "out", out, dt, M * N)
    _on_gpu(fn, x, Wt, w_norm, bias, out)
    _keep(stream, x, w_norm, Wt, bias, out)
    return (_ptr(x), _ptr(w_norm), _ptr(Wt), _ptr(bias), _ptr(out), x.shape[0], Wt.shape[0],
            x.shape[-1], eps, scale, dtype_code(x), _stream(stream))


def _a_unfused_rmsnorm_linear(x, w_norm, Wt, bias, out, workspace, eps: float = 1e-6,
                              scale: float = 1.0, stream=None):
    _workspace("unfused_rmsnorm_linear", workspace)
    a = _a_fuse_rmsnorm_linear(x, w_norm, Wt, bias, out, eps, scale, stream)
    _keep(stream, workspace)
    return a[:-1] + (_ptr(workspace), workspace.numel() * workspace.element_size(), a[-1])


def _dense(*ts):
    for t in ts:
        if not t.is_contiguous():
            raise ValueError("layout calls need contiguous (dense row-major) tensors")
        if not t.is_cuda:
            raise ValueError("layout calls need GPU tensors")


def _tr_shape(x, shape):
    if shape is None:
        if x.dim() != 4:
            raise ValueError("pass shape=(B, R, S, E) for a tensor that is not 4-D")
        shape = tuple(x.shape)
    B, R, S, E = shape
    if B * R * S * E != x.numel():
        raise ValueError(f"shape {shape} does not match {x.numel()} elements")
    return B, R, S, E


def _a_fuse_transpose021(x, out, shape=None, stream=None):
    _dense(x, out)
    B, R, S, E = _tr_shape(x, shape)
    if out.numel() != x.numel() or out.element_size() != x.element_size():
        raise ValueError("out must hold as many elements of the same size as x")
    _keep(stream, x, out)
    return (_ptr(x), _ptr(out), B, R, S, E, x.element_size(), _stream(stream))


_a_naive_transpose021 = _a_fuse_transpose021

_LAYOUTS = {"nchw": 0, "nhwc": 1, 0: 0, 1: 1}


def _a_fuse_channel_shuffle(x, out, groups: int, layout="nchw", stream=None):
    _dense(x, out)
    if x.dim() != 4:
        raise ValueError("channel_shuffle needs a 4-D tensor")
    lay = _LAYOUTS[layout]
    if lay == 0:
        N, Cc, H, W = x.shape
    else:
        N, H, W, Cc = x.shape
    if out.numel() != x.numel() or out.element_size() != x.element_size():
        raise ValueError("out must hold as many elements of the same size as x")
    _keep(stream, x, out)
    return (_ptr(x), _ptr(out), N, Cc, H, W, groups, lay, x.element_size(), _stream(stream))


_a_naive_channel_shuffle = _a_fuse_channel_shuffle


def _a_unfused_det_decode(levels, strides, anchors, out, workspace, n_anchors: int = 3,
                          n_ch: int = 85, stream=None):
    _workspace("unfused_det_decode", workspace)
    a = _a_fuse_det_decode(levels, strides, anchors, out, n_anchors, n_ch, stream)
    _keep(stream, workspace)
    return a[:-1] + (_ptr(workspace), workspace.numel() * workspace.element_size(), a[-1])


_a_unfused_det_decode_noalloc = _a_fuse_det_decode


def _a_unfused_add_rmsnorm(x, r, w, h_out, out, workspace, eps: float = 1e-6, stream=None):
    _workspace("unfused_add_rmsnorm", workspace)
    a = _a_fuse_add_rmsnorm(x, r, w, h_out, out, eps, stream)
    _keep(stream, workspace)
    return a[:-1] + (_ptr(workspace), workspace.numel() * workspace.element_size(), a[-1])


def bind(name: str, *args, **kw):
    """Marshal the arguments of call `name` once; return a zero-argument callable
    that performs the C call (and raises NPError on failure) each time.

    The callable holds references to every tensor argument (and to the ctypes
    objects built from them): the marshalled pointers stay valid for as long as
    the callable exists, whatever happens to the caller's own names."""
    a = globals()["_a_" + name](*args, **kw)
    f = getattr(_lib, name)

    def call():
        rc = f(*a)
        if rc:
            _check(rc, name)
    call.args = a
    call.keep = (args, kw)
    return call


def fuse_chain(ops, inputs, out, stream=None):
    """out[i] = chain(inputs[0][i], ...); ops = [(kind, arg, const), ...]."""
    _check(_lib.fuse_chain(*_a_fuse_chain(ops, inputs, out, stream)), "fuse_chain")
    return out


def np_chain_cache_stats() -> dict:
    """Disk cache counters of specialised code objects: {"loads", "stores", "rejects"}."""
    v = [C.c_int64() for _ in range(3)]
    _lib.np_chain_cache_stats(*(C.byref(x) for x in v))
    return {"loads": v[0].value, "stores": v[1].value, "rejects": v[2].value}


def np_set_chain_table_min(n: int) -> int:
    """Element count from which a tabulated chain (one 16-bit input, 16-bit
    output) runs from its table; returns the previous value. n < 0 only
    queries; a huge n keeps every call on the per-element kernel."""
    return int(_lib.np_set_chain_table_min(n))


def fuse_chain_prepare(ops, n_inputs: int, in_dt: int, out_dt: int, n: int = 0):
    arr, k = _ops(ops)
    _check(_lib.fuse_chain_prepare(arr, k, n_inputs, in_dt, out_dt, n), "fuse_chain_prepare")


def fuse_det_decode(levels, strides, anchors, out, n_anchors: int = 3, n_ch: int = 85,
                    stream=None):
    """levels: [batch, n_anchors*n_ch, H, W] tensors; anchors: [[(w, h)] * n_anchors] per level;
    out: fp32 [batch, rows, n_ch]."""
    _check(_lib.fuse_det_decode(*_a_fuse_det_decode(levels, strides, anchors, out, n_anchors,
                                                    n_ch, stream)), "fuse_det_decode")
    return out


def fuse_add_rmsnorm(x, r, w, h_out, out, eps: float = 1e-6, stream=None):
    _check(_lib.fuse_add_rmsnorm(*_a_fuse_add_rmsnorm(x, r, w, h_out, out, eps, stream)),
           "fuse_add_rmsnorm")
    return h_out, out


def fuse_qkv_rope(qkv, q, k, v, n_heads: int, head_dim: int, positions=None,
                  base: float = 10000.0, q_scale: float | None = None, stream=None):
    _check(_lib.fuse_qkv_rope(*_a_fuse_qkv_rope(qkv, q, k, v, n_heads, head_dim, positions, base,
                                                q_scale, stream)), "fuse_qkv_rope")
    return q, k, v


def fuse_add_layernorm(x, r, gamma, beta, h_out, out, eps: float = 1e-5, stream=None):
    _check(_lib.fuse_add_layernorm(*_a_fuse_add_layernorm(x, r, gamma, beta, h_out, out, eps,
                                                          stream)), "fuse_add_layernorm")
    return h_out, out


def fuse_rmsnorm_linear(x, w_norm, Wt, bias, out, eps: float = 1e-6, scale: float = 1.0,
                        stream=None):
    """out = scale * (Linear(RMSNorm(x)) + bias) with the RMS factor applied to the
    accumulator: x [M, K], w_norm [K] or None, Wt [N, K], bias [N] or None, out [M, N]."""
    _check(_lib.fuse_rmsnorm_linear(*_a_fuse_rmsnorm_linear(x, w_norm, Wt, bias, out, eps, scale,
                                                            stream)), "fuse_rmsnorm_linear")
    return out


def np_fold_norm_weight(w_norm, Wt, Wt_folded, stream=None):
    """Wt_folded = round(w_norm * Wt) per element (the norm weight moved into the
    linear weight, once); Wt [N, K]."""
    fn = "np_fold_norm_weight"
    dt = _float_dtype(fn, Wt)
    _need(Wt.dim() == 2, fn, "Wt must be [N, K]")
    _need(w_norm is not None, fn, "w_norm is required")
    _dev(fn, "Wt", Wt, dt)
    _dev(fn, "w_norm", w_norm, dt, Wt.shape[1])
    _dev(fn, "Wt_folded", Wt_folded, dt, Wt.numel())
    _on_gpu(fn, w_norm, Wt, Wt_folded)
    _keep(stream, w_norm, Wt, Wt_folded)
    _check(_lib.np_fold_norm_weight(_ptr(w_norm), _ptr(Wt), _ptr(Wt_folded), Wt.shape[0],
                                    Wt.shape[1], dtype_code(Wt), _stream(stream)),
           "np_fold_norm_weight")
    return Wt_folded


def rmsnorm_linear_workspace_bytes(M: int, K: int) -> int:
    return M * K * 2


def unfused_rmsnorm_linear(x, w_norm, Wt, bias, out, workspace, eps: float = 1e-6,
                           scale: float = 1.0, stream=None):
    _check(_lib.unfused_rmsnorm_linear(*_a_unfused_rmsnorm_linear(x, w_norm, Wt, bias, out,
                                                                  workspace, eps, scale, stream)),
           "unfused_rmsnorm_linear")
    return out


def fuse_transpose021(x, out, shape=None, stream=None):
    """out[b, s, r, e] = x[b, r, s, e] for x of shape (B, R, S, E) (x.shape if
    4-D, else pass shape); any dtype, copied bit for bit."""
    _check(_lib.fuse_transpose021(*_a_fuse_transpose021(x, out, shape, stream)),
           "fuse_transpose021")
    return out


def naive_transpose021(x, out, shape=None, stream=None):
    _check(_lib.naive_transpose021(*_a_naive_transpose021(x, out, shape, stream)),
           "naive_transpose021")
    return out


def fuse_channel_shuffle(x, out, groups: int, layout="nchw", stream=None):
    _check(_lib.fuse_channel_shuffle(*_a_fuse_channel_shuffle(x, out, groups, layout, stream)),
           "fuse_channel_shuffle")
    return out


def naive_channel_shuffle(x, out, groups: int, layout="nchw", stream=None):
    _check(_lib.naive_channel_shuffle(*_a_naive_channel_shuffle(x, out, groups, layout, stream)),
           "naive_channel_shuffle")
    return out


TR_KERNELS = {1: "tile", 2: "small", 3: "items"}


def np_transpose_plan(in_ptr: int, out_ptr: int, shape, elem_bytes: int, naive: bool = False):
    """The kernel fuse_transpose021 / naive_transpose021 would launch for these
    addresses and sizes (host only): {"kernel", "item", "vec", "diag"} or None if
    empty."""
    B, R, S, E = shape
    rc = _lib.np_transpose_plan(C.c_void_p(in_ptr), C.c_void_p(out_ptr), B, R, S, E, elem_bytes,
                                int(naive))
    if rc < 0:
        _check(rc, "np_transpose_plan")
    if rc == 0:
        return None
    return {"kernel": TR_KERNELS[(rc >> 8) & 15], "item": rc & 255, "vec": bool(rc >> 12 & 1),
            "diag": bool(rc >> 13 & 1)}


# ------------------------------------------------------- unfused baselines

def unfused_chain(ops, inputs, out, stream=None):
    _check(_lib.unfused_chain(*_a_unfused_chain(ops, inputs, out, stream)), "unfused_chain")
    return out


def det_workspace_bytes(levels, n_anchors: int = 3, n_ch: int = 85) -> int:
    return 2 * levels[0].shape[0] * det_rows(levels, n_anchors) * n_ch * levels[0].element_size()


def unfused_det_decode(levels, strides, anchors, out, workspace, n_anchors: int = 3,
                       n_ch: int = 85, stream=None):
    _check(_lib.unfused_det_decode(*_a_unfused_det_decode(levels, strides, anchors, out,
                                                          workspace, n_anchors, n_ch, stream)),
           "unfused_det_decode")
    return out


def unfused_det_decode_noalloc(levels, strides, anchors, out, n_anchors: int = 3, n_ch: int = 85,
                               stream=None):
    """unfused_det_decode staged through the library's own 16 MiB device array
    (no workspace argument, no allocation)."""
    _check(_lib.unfused_det_decode_noalloc(*_a_unfused_det_decode_noalloc(
        levels, strides, anchors, out, n_anchors, n_ch, stream)), "unfused_det_decode_noalloc")
    return out


def rmsnorm_workspace_bytes(rows: int, cols: int, dtype, with_h: bool = True) -> int:
    es = _SIZE[dtype_code(dtype)]
    return (rows * cols + 2 * rows + (0 if with_h else rows * cols)) * es


def unfused_add_rmsnorm(x, r, w, h_out, out, workspace, eps: float = 1e-6, stream=None):
    _check(_lib.unfused_add_rmsnorm(*_a_unfused_add_rmsnorm(x, r, w, h_out, out, workspace, eps,
                                                            stream)), "unfused_add_rmsnorm")
    return h_out, out


def unfused_qkv_rope(qkv, q, k, v, n_heads: int, head_dim: int, positions=None,
                     base: float = 10000.0, q_scale: float | None = None, stream=None):
    _check(_lib.unfused_qkv_rope(*_a_unfused_qkv_rope(qkv, q, k, v, n_heads, head_dim, positions,
                                                      base, q_scale, stream)), "unfused_qkv_rope")
    return q, k, v


def layernorm_workspace_bytes(rows: int, cols: int, dtype, with_h: bool = True) -> int:
    es = _SIZE[dtype_code(dtype)]
    return (rows * cols + 3 * rows + (0 if with_h else rows * cols)) * es


def unfused_add_layernorm(x, r, gamma, beta, h_out, out, workspace, eps: float = 1e-5,
                          stream=None):
    _check(_lib.unfused_add_layernorm(*_a_unfused_add_layernorm(x, r, gamma, beta, h_out, out,
                                                                workspace, eps, stream)),
           "unfused_add_layernorm")
    return h_out, out
