"""Seeded synthetic inputs for the fused-chain workloads.

This module only draws random numbers and lays them out in the shapes the
workloads use. It holds none of the chains' arithmetic: tests, the bench and
the smoke check take their inputs from here and hand the very same arrays to
both the CPU oracle and the GPU library.

Generator: numpy's Philox4x32-10 counter-based bit generator (Salmon et al.,
"Parallel random numbers: as easy as 1, 2, 3", SC 2011), keyed per 4 Mi-element
chunk from ``numpy.random.SeedSequence(seed).spawn``. Chunks are filled on a
small thread pool; the result does not depend on the number of threads.

Half-precision storage: fp16 values are produced by numpy's float32->float16
cast (round to nearest even); bf16 values are stored as ``uint16`` bit patterns
produced by round-to-nearest-even on the float32 draw (draws are finite, so no
NaN handling is needed).

The workload shapes follow the pages' examples:
- the DeepJIT write-up (hotelren.com/news/5350627), sections 3.3 and 4: fp32
  ``relu(a+b)*scale`` on 1,048,576 elements, and the detection-head tail of
  sigmoid / exp / mul / add / concat / cast (section 1.1);
- the TeleTron write-up (2kiu.com/news/5927820), sections 3.1 and 3.3:
  residual-add + RMSNorm and QKV split + RoPE + scale on activations with a
  hidden size in the thousands and sequences of tens of thousands of tokens;
- the NaiveRT write-up (zhaixingw.cn/coding/291.html): a layer of 29 separate
  GPU calls, here a seeded 29-op elementwise chain.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22
_THREADS = max(1, min(8, os.cpu_count() or 1))

# Op kinds shared by the chain description (same numbering the C ABI uses).
LOAD, ADD_IN, MUL_IN, ADD_C, MUL_C, SCALE, RELU, SIGMOID, EXP, TANH, CAST_F16, CAST_BF16 = range(12)
KIND_NAMES = ["load", "add_in", "mul_in", "add_c", "mul_c", "scale", "relu",
              "sigmoid", "exp", "tanh", "cast_f16", "cast_bf16"]


def _fill(n: int, seed: int, draw) -> np.ndarray:
    out = np.empty(n, np.float32)
    nch = (n + CHUNK - 1) // CHUNK
    keys = np.random.SeedSequence(seed).spawn(max(nch, 1))

    def one(i):
        g = np.random.Generator(np.random.Philox(keys[i]))
        lo = i * CHUNK
        hi = min(n, lo + CHUNK)
        draw(g, out[lo:hi])

    if nch <= 1:
        if n:
            one(0)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(one, range(nch)))
    return out


def normal_f32(n: int, seed: int, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """n float32 draws from N(mean, std^2)."""
    def draw(g, dst):
        g.standard_normal(dst.shape[0], dtype=np.float32, out=dst)
        if std != 1.0:
            dst *= np.float32(std)
        if mean != 0.0:
            dst += np.float32(mean)
    return _fill(n, seed, draw)


def uniform_f32(n: int, seed: int, lo: float, hi: float) -> np.ndarray:
    def draw(g, dst):
        g.random(dst.shape[0], dtype=np.float32, out=dst)
        dst *= np.float32(hi - lo)
        dst += np.float32(lo)
    return _fill(n, seed, draw)


def random_bytes(n: int, seed: int) -> np.ndarray:
    """n uniformly distributed bytes (uint8), Philox-keyed per chunk like the
    float draws (inputs of the bit-copying layout calls)."""
    out = np.empty(n, np.uint8)
    nch = (n + CHUNK - 1) // CHUNK
    keys = np.random.SeedSequence(seed).spawn(max(nch, 1))
    for i in range(nch):
        g = np.random.Generator(np.random.Philox(keys[i]))
        lo = i * CHUNK
        hi = min(n, lo + CHUNK)
        out[lo:hi] = np.frombuffer(g.bytes(hi - lo), np.uint8)
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def cast(x: np.ndarray, dtype: str) -> np.ndarray:
    """Store float32 draws as 'f32' (float32), 'f16' (float16) or 'bf16' (uint16 bits)."""
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        return to_bf16_bits(x)
    raise ValueError(dtype)


def normal(shape, seed: int, dtype: str, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    n = int(np.prod(shape)) if len(shape) else 1
    return cast(normal_f32(n, seed, mean, std), dtype).reshape(shape)


# --------------------------------------------------------------------------
# Workload recipes (seed = 1000 + workload number unless stated)
# --------------------------------------------------------------------------

def c1_inputs(n: int = 1 << 20, seed: int = 1001):
    """fp32 a, b ~ N(0,1) of n elements (relu(a+b)*0.5)."""
    return normal((n,), seed, "f32"), normal((n,), seed + 7919, "f32")


YOLO_LEVELS = ((80, 80, 8.0), (40, 40, 16.0), (20, 20, 32.0))
# Nine COCO anchor boxes (w, h) in pixels, smallest three at stride 8, as
# published in the YOLOv3 technical report (Redmon & Farhadi, 2018, sec. 2.3).
YOLO_ANCHORS = ((10, 13), (16, 30), (33, 23),
                (30, 61), (62, 45), (59, 119),
                (116, 90), (156, 198), (373, 326))


def c2_inputs(levels=YOLO_LEVELS, n_anchors: int = 3, n_ch: int = 85, batch: int = 1,
              seed: int = 1002, std: float = 2.0, dtype: str = "f16"):
    """Per-level NCHW logits [batch, n_anchors*n_ch, H, W] ~ N(0, std^2)."""
    out = []
    for li, (h, w, _s) in enumerate(levels):
        out.append(normal((batch, n_anchors * n_ch, h, w), seed + 101 * li, dtype, std=std))
    return out


def c3_inputs(rows: int = 16384, cols: int = 4096, seed: int = 1003, dtype: str = "bf16"):
    """x, r ~ N(0,1) [rows, cols]; w ~ N(1, 0.1) [cols]."""
    x = normal((rows, cols), seed, dtype)
    r = normal((rows, cols), seed + 7919, dtype)
    w = normal((cols,), seed + 15485863, dtype, mean=1.0, std=0.1)
    return x, r, w


def c4_inputs(tokens: int = 16384, heads: int = 24, head_dim: int = 128, seed: int = 1004,
              dtype: str = "bf16"):
    """Packed qkv [tokens, 3*heads*head_dim] ~ N(0,1)."""
    return normal((tokens, 3 * heads * head_dim), seed, dtype)


def c5_inputs(n: int, seed: int = 1005, dtype: str = "f16"):
    return normal((n,), seed, dtype)


def _ulp16(m: float) -> float:
    """Spacing of fp16 numbers at magnitude m (generator guard only)."""
    if m < 2.0 ** -14:
        return 2.0 ** -24
    return 2.0 ** (math.floor(math.log2(m)) - 10)


def c5_chain(n_ops: int = 29, seed: int = 29, min_ulps: float = 256.0):
    """Seeded mix of add/mul/sigmoid/exp/tanh/scale/cast ops, constants ~ U(-1,1).

    Returns a list of (kind, arg, const) beginning with LOAD(0). Kinds are drawn
    uniformly from the seven named kinds, constants uniformly from (-1, 1).
    A drawn op is rejected and redrawn when, on the interval [-4, 4] of inputs
    pushed through the ops drawn so far (every op is monotone), it would
    - let an exp argument exceed ln(32768), so an intermediate could leave the
      fp16 range (no chain produces inf or NaN), or
    - shrink the image interval below ``min_ulps`` fp16 spacings, so the output
      would no longer depend on the input (uniform draws otherwise collapse a
      29-op chain to a constant).
    """
    g = np.random.Generator(np.random.Philox(np.random.SeedSequence(seed)))
    kinds = [ADD_C, MUL_C, SIGMOID, EXP, TANH, SCALE, CAST_F16]
    ops = [(LOAD, 0, 0.0)]
    lo, hi = -4.0, 4.0
    limit = math.log(32768.0)
    sig = lambda t: 1.0 / (1.0 + math.exp(-t))
    while len(ops) < n_ops + 1:
        k = kinds[int(g.integers(0, len(kinds)))]
        c = float(np.float32(g.uniform(-1.0, 1.0)))
        if k == ADD_C:
            nlo, nhi = lo + c, hi + c
        elif k in (MUL_C, SCALE):
            nlo, nhi = sorted((lo * c, hi * c))
        elif k == SIGMOID:
            nlo, nhi = sig(lo), sig(hi)
        elif k == TANH:
            nlo, nhi = math.tanh(lo), math.tanh(hi)
        elif k == EXP:
            if hi > limit:
                continue
            nlo, nhi = math.exp(lo), math.exp(hi)
        else:
            nlo, nhi = lo, hi
        if nhi - nlo < min_ulps * _ulp16(max(abs(nlo), abs(nhi))):
            continue
        if k not in (ADD_C, MUL_C, SCALE):
            c = 0.0
        ops.append((k, 0, c))
        lo, hi = nlo, nhi
    return ops


C1_CHAIN = [(LOAD, 0, 0.0), (ADD_IN, 1, 0.0), (RELU, 0, 0.0), (MUL_C, 0, 0.5)]


def chain_arrays(ops):
    kinds = np.array([o[0] for o in ops], np.int32)
    args = np.array([o[1] for o in ops], np.int32)
    consts = np.array([o[2] for o in ops], np.float32)
    return kinds, args, consts


def chain_str(ops) -> str:
    parts = []
    for k, a, c in ops:
        name = KIND_NAMES[k]
        if k in (LOAD, ADD_IN, MUL_IN):
            parts.append(f"{name}({a})")
        elif k in (ADD_C, MUL_C, SCALE):
            parts.append(f"{name}({c:.6g})")
        else:
            parts.append(name)
    return " -> ".join(parts)


# --------------------------------------------------------------------------
# Layout workloads (the runtime page "CUDA算子与AI运行时", gtnt.cn/news/145880,
# section 2: ChannelShuffle of an [N, C, H, W] activation, and the strided
# transpose it reduces to). Channel counts and resolution follow ShuffleNet V2
# 1.0x (Ma et al., ECCV 2018), stage 2 at 224 x 224 input: 116 channels at
# 28 x 28, two groups.
# --------------------------------------------------------------------------

TRANSPOSE_2D = (1, 8192, 8192, 1)        # fp32 [8192, 8192] -> its transpose
SHUFFLE_NCHW = (1024, 116, 28, 28)       # fp16, groups 2
SHUFFLE_GROUPS = 2


def transpose_inputs(shape=TRANSPOSE_2D, seed: int = 1006, dtype: str = "f32"):
    return normal(shape, seed, dtype)


def shuffle_inputs(shape=SHUFFLE_NCHW, seed: int = 1007, dtype: str = "f16", layout: int = 0):
    """N(0, 1) activations of ShuffleNet-V2 stage-2 shape, NCHW (layout 0) or
    NHWC (layout 1)."""
    n, c, h, w = shape
    return normal((n, c, h, w) if layout == 0 else (n, h, w, c), seed, dtype)


# --------------------------------------------------------------------------
# RMSNorm + linear + scale (the TeleTron write-up, section 4.2): the norm of
# the residual-add workload (16384 tokens x hidden 4096) followed by a square
# 4096 -> 4096 projection, bf16 storage.
# --------------------------------------------------------------------------

RMS_LINEAR_SHAPE = (16384, 4096, 4096)  # M tokens, K hidden in, N out
RMS_LINEAR_SCALE = 0.5


def rmsnorm_linear_inputs(shape=RMS_LINEAR_SHAPE, seed: int = 1008, dtype: str = "bf16"):
    """x [M, K] ~ N(0, 1); w_norm [K] ~ N(1, 0.1^2); Wt [N, K] ~ N(0, 1/K)
    (unit-variance outputs); bias [N] ~ N(0, 0.1^2)."""
    M, K, N = shape
    x = normal((M, K), seed, dtype)
    w = normal((K,), seed + 1, dtype, mean=1.0, std=0.1)
    Wt = normal((N, K), seed + 2, dtype, std=K ** -0.5)
    b = normal((N,), seed + 3, dtype, std=0.1)
    return x, w, Wt, b
