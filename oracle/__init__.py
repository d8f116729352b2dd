"""CPU oracle for the fused-chain library -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the bench's ``cpu_baseline``
leg may import this package. It wraps ``liboracle.so`` (plain scalar C++ built
from ``oracle.cpp`` with the host compiler) with numpy-array marshalling; every
value it returns is computed by that C++ code. See ``oracle.h`` for the
definitions and the error-bound convention.

Functions whose parity is pinned only by invariants and special cases (no
worked example on the pages) say so in their docstrings.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
F32, F16, BF16 = 0, 1, 2
_NP = {F32: np.float32, F16: np.uint16, BF16: np.uint16}


def build(verbose: bool = False) -> str:
    """Compile liboracle.so with the host compiler (no GPU code involved)."""
    src = os.path.join(_HERE, "oracle.cpp")
    tmp = LIB_PATH + ".tmp"
    cmd = ["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-Wall", "-Wextra", "-o", tmp, src]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = C.CDLL(LIB_PATH)
        P = C.c_void_p
        i64 = C.c_int64
        L.oracle_f16_to_double.restype = C.c_double
        L.oracle_f16_to_double.argtypes = [C.c_uint16]
        L.oracle_double_to_f16.restype = C.c_uint16
        L.oracle_double_to_f16.argtypes = [C.c_double]
        L.oracle_bf16_to_double.restype = C.c_double
        L.oracle_bf16_to_double.argtypes = [C.c_uint16]
        L.oracle_double_to_bf16.restype = C.c_uint16
        L.oracle_double_to_bf16.argtypes = [C.c_double]
        L.oracle_double_to_f32.restype = C.c_float
        L.oracle_double_to_f32.argtypes = [C.c_double]
        L.oracle_round_array.restype = None
        L.oracle_round_array.argtypes = [P, i64, C.c_int, P]
        L.oracle_chain.argtypes = [P, P, P, C.c_int, P, C.c_int, C.c_int, P, C.c_int, i64,
                                   C.c_int, P, P]
        L.oracle_det_decode.argtypes = [P, C.c_int, P, P, P, P, C.c_int, C.c_int, C.c_int,
                                        C.c_int, P, C.c_int]
        L.oracle_add_rmsnorm.argtypes = [P, P, P, P, P, i64, i64, C.c_float, C.c_int, C.c_int, P]
        L.oracle_add_layernorm.argtypes = [P, P, P, P, P, P, i64, i64, C.c_float, C.c_int,
                                           C.c_int, P]
        L.oracle_qkv_rope.argtypes = [P, P, P, P, i64, C.c_int, C.c_int, P, C.c_float,
                                      C.c_float, C.c_int, C.c_int, P, P, P, P]
        L.oracle_rope_inv_freq.argtypes = [C.c_float, C.c_int, P]
        L.oracle_rmsnorm_linear.argtypes = [P, P, P, P, P, i64, i64, i64, C.c_float, C.c_float,
                                             C.c_int, C.c_int, P, P]
        L.oracle_channel_shuffle.argtypes = [P, P, i64, i64, i64, i64, i64, C.c_int, C.c_int]
        L.oracle_transpose021.argtypes = [P, P, i64, i64, i64, i64, C.c_int]
        for f in ("oracle_chain", "oracle_det_decode", "oracle_add_rmsnorm", "oracle_qkv_rope",
                  "oracle_rope_inv_freq", "oracle_add_layernorm", "oracle_channel_shuffle",
                  "oracle_transpose021", "oracle_rmsnorm_linear"):
            getattr(L, f).restype = C.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _dt_of(a: np.ndarray, dt: int | None) -> int:
    if dt is not None:
        return dt
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float16:
        return F16
    raise ValueError("uint16 arrays are ambiguous: pass dt=F16 or dt=BF16")


def _raw(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    return a.view(np.uint16) if a.dtype == np.float16 else a


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"{what}: oracle rejected the arguments (rc={rc})")


# --------------------------------------------------------------------------
# converters
# --------------------------------------------------------------------------

def round_array(x: np.ndarray, dt: int) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, _NP[dt])
    lib().oracle_round_array(_p(x), x.size, dt, _p(out))
    return out


def f16_to_double(bits: int) -> float:
    return lib().oracle_f16_to_double(bits)


def bf16_to_double(bits: int) -> float:
    return lib().oracle_bf16_to_double(bits)


_TABLES = {}


def decode(a: np.ndarray, dt: int) -> np.ndarray:
    """Values of an array of dt (float32 / fp16 bits / bf16 bits) as float64."""
    if dt == F32:
        return np.asarray(a, np.float64)
    if dt not in _TABLES:
        f = lib().oracle_f16_to_double if dt == F16 else lib().oracle_bf16_to_double
        _TABLES[dt] = np.array([f(i) for i in range(65536)], np.float64)
    flat = np.ascontiguousarray(a).view(np.uint16).ravel()
    return _TABLES[dt][flat].reshape(np.shape(a))


# --------------------------------------------------------------------------
# chains
# --------------------------------------------------------------------------

def chain(ops, inputs, out_dt: int, in_dt: int | None = None, eager: bool = False,
          want_bound: bool = False):
    """Evaluate an elementwise chain. ops: [(kind, arg, const)], inputs: arrays of n.

    Returns out (or (out, exact, bound) with want_bound).
    """
    kinds = np.array([o[0] for o in ops], np.int32)
    args = np.array([o[1] for o in ops], np.int32)
    consts = np.array([o[2] for o in ops], np.float32)
    ins = [_raw(a) for a in inputs]
    idt = _dt_of(np.asarray(inputs[0]), in_dt)
    n = ins[0].size
    ptrs = (C.c_void_p * len(ins))(*[a.ctypes.data for a in ins])
    out = np.empty(n, _NP[out_dt])
    exact = np.empty(n, np.float64) if want_bound else None
    bound = np.empty(n, np.float64) if want_bound else None
    rc = lib().oracle_chain(_p(kinds), _p(args), _p(consts), len(ops), C.cast(ptrs, C.c_void_p),
                            len(ins), idt, _p(out), out_dt, n, int(eager), _p(exact), _p(bound))
    _check(rc, "oracle_chain")
    if out_dt == F16:
        out = out.view(np.float16)
    return (out, exact, bound) if want_bound else out


def det_decode(levels, hw, strides, anchors, n_anchors: int = 3, n_ch: int = 85,
               in_dt: int | None = None, eager: bool = False) -> np.ndarray:
    """Detection-head decode; levels: arrays [batch, n_anchors*n_ch, H, W]."""
    ins = [_raw(a) for a in levels]
    idt = _dt_of(np.asarray(levels[0]), in_dt)
    batch = ins[0].shape[0]
    H = np.array([h for h, _ in hw], np.int32)
    W = np.array([w for _, w in hw], np.int32)
    st = np.array(strides, np.float32)
    an = np.ascontiguousarray(np.array(anchors, np.float32).reshape(-1))
    rows = int(sum(n_anchors * h * w for h, w in hw))
    out = np.empty((batch, rows, n_ch), np.float32)
    ptrs = (C.c_void_p * len(ins))(*[a.ctypes.data for a in ins])
    rc = lib().oracle_det_decode(C.cast(ptrs, C.c_void_p), len(ins), _p(H), _p(W), _p(st), _p(an),
                                 n_anchors, n_ch, batch, idt, _p(out), int(eager))
    _check(rc, "oracle_det_decode")
    return out


def add_rmsnorm(x, r, w, eps: float, dt: int, eager: bool = False, want_exact: bool = False):
    """Residual-add + RMSNorm over rows of x [rows, cols]; returns (h, out[, exact])."""
    x = _raw(x)
    rows, cols = x.shape
    rr = None if r is None else _raw(r)
    ww = None if w is None else _raw(w)
    h = np.empty((rows, cols), _NP[dt])
    out = np.empty((rows, cols), _NP[dt])
    exact = np.empty((rows, cols), np.float64) if want_exact else None
    rc = lib().oracle_add_rmsnorm(_p(x), _p(rr), _p(ww), _p(h), _p(out), rows, cols, eps, dt,
                                  int(eager), _p(exact))
    _check(rc, "oracle_add_rmsnorm")
    return (h, out, exact) if want_exact else (h, out)


def add_layernorm(x, r, gamma, beta, eps: float, dt: int, eager: bool = False,
                  want_exact: bool = False):
    """Residual-add + LayerNorm over rows of x [rows, cols]; returns (h, out[, exact])."""
    x = _raw(x)
    rows, cols = x.shape
    rr, gg, bb = (None if a is None else _raw(a) for a in (r, gamma, beta))
    h = np.empty((rows, cols), _NP[dt])
    out = np.empty((rows, cols), _NP[dt])
    exact = np.empty((rows, cols), np.float64) if want_exact else None
    rc = lib().oracle_add_layernorm(_p(x), _p(rr), _p(gg), _p(bb), _p(h), _p(out), rows, cols,
                                    eps, dt, int(eager), _p(exact))
    _check(rc, "oracle_add_layernorm")
    return (h, out, exact) if want_exact else (h, out)


def rope_inv_freq(base: float, head_dim: int) -> np.ndarray:
    inv = np.empty(head_dim // 2, np.float32)
    _check(lib().oracle_rope_inv_freq(base, head_dim, _p(inv)), "oracle_rope_inv_freq")
    return inv


def qkv_rope(qkv, n_heads: int, head_dim: int, base: float, q_scale: float, dt: int,
             positions=None, eager: bool = False, want_bound: bool = False):
    """QKV split + RoPE + Q scale. qkv: [T, 3*n_heads*head_dim]. Returns (q, k, v[, eq, ek, bq, bk])."""
    qkv = _raw(qkv)
    T = qkv.shape[0]
    shape = (n_heads, T, head_dim)
    q = np.empty(shape, _NP[dt])
    k = np.empty(shape, _NP[dt])
    v = np.empty(shape, _NP[dt])
    pos = None if positions is None else np.ascontiguousarray(positions, np.int32)
    extra = [np.empty(shape, np.float64) for _ in range(4)] if want_bound else [None] * 4
    rc = lib().oracle_qkv_rope(_p(qkv), _p(q), _p(k), _p(v), T, n_heads, head_dim, _p(pos),
                               base, q_scale, dt, int(eager), *[_p(e) for e in extra])
    _check(rc, "oracle_qkv_rope")
    return (q, k, v, *extra) if want_bound else (q, k, v)


def rmsnorm_linear(x, w_norm, Wt, bias, eps: float, scale: float, dt: int, eager: bool = False,
                   want_exact: bool = False):
    """RMSNorm + linear + scale (see oracle.h). x [M, K], Wt [N, K]; returns out
    [M, N] (and, with want_exact, the unrounded values and the per-output
    magnitude |scale| rstd sum|a W| of the dot product's terms)."""
    x = _raw(x)
    Wt = _raw(Wt)
    M, K = x.shape
    N = Wt.shape[0]
    if Wt.shape[1] != K:
        raise ValueError("Wt must be [N, K]")
    wn = None if w_norm is None else _raw(w_norm)
    b = None if bias is None else _raw(bias)
    out = np.empty((M, N), _NP[dt])
    ex = np.empty((M, N), np.float64) if want_exact else None
    cd = np.empty((M, N), np.float64) if want_exact else None
    _check(lib().oracle_rmsnorm_linear(_p(x), _p(wn), _p(Wt), _p(b), _p(out), M, N, K, eps,
                                       scale, dt, int(eager), _p(ex), _p(cd)), "rmsnorm_linear")
    return (out, ex, cd) if want_exact else out


# --------------------------------------------------------------------------
# layout: ChannelShuffle and the batched transpose behind it
# --------------------------------------------------------------------------

def _bytes_view(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a)


def channel_shuffle(x: np.ndarray, groups: int, layout: int = 0) -> np.ndarray:
    """ChannelShuffle of a 4-D array (NCHW for layout 0, NHWC for layout 1),
    bit for bit in x's dtype (see oracle.h)."""
    x = _bytes_view(x)
    if x.ndim != 4:
        raise ValueError("channel_shuffle: x must be 4-D")
    if layout == 0:
        N, Cc, H, W = x.shape
    else:
        N, H, W, Cc = x.shape
    out = np.empty_like(x)
    _check(lib().oracle_channel_shuffle(_p(x), _p(out), N, Cc, H, W, groups, layout,
                                        x.dtype.itemsize), "channel_shuffle")
    return out


def transpose021(x: np.ndarray) -> np.ndarray:
    """[B, R, S, E] -> [B, S, R, E], bit for bit (see oracle.h)."""
    x = _bytes_view(x)
    if x.ndim != 4:
        raise ValueError("transpose021: x must be 4-D [B, R, S, E]")
    B, R, S, E = x.shape
    out = np.empty((B, S, R, E), x.dtype)
    _check(lib().oracle_transpose021(_p(x), _p(out), B, R, S, E, x.dtype.itemsize),
           "transpose021")
    return out
