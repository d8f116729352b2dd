#!/usr/bin/env python3
"""Fused vs N-launch unfused chains on one MI355X: achieved HBM GB/s and per-call us.

A step is one pass of the whole hot path over one batch of synthetic input:
  C1  fp32 relu(a+b)*0.5, 1,048,576 elements                     (fuse_chain)
  C2  YOLO decode, fp16 [1,255,80|40|20,..] -> fp32 [1,25200,85]  (fuse_det_decode)
  C3  bf16 residual add + RMSNorm [16384, 4096]                   (fuse_add_rmsnorm)
  C4  bf16 QKV split + RoPE + scale, 16384 tokens x 3x24x128     (fuse_qkv_rope)
  C5  seeded 29-op fp16 chain at 65,536 and 268,435,456 elements  (fuse_chain)
value = algorithmic bytes of the step (each input read once, each output written
once) / step time. Every fused call is also timed alone, next to its unfused
counterpart (one kernel per operator) and, for the small chain, next to the
NaiveRT write-up's launch-cost model L = (t_unfused - t_fused)/(K - 1).

Usage: python bench.py [--steps K] [--warmup W] [--no-cpu] [--quick]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
PROFILES = os.path.join(ROOT, "profiles")

# The NaiveRT write-up's two public timings (ms per decode round, 29 calls per
# layer fused into 1 kernel) and the figures it derives from them.
PAGES_COST_MODEL = {"t_unfused_ms": 12.3, "t_fused_ms": 3.4, "k": 29}


def cost_model(t_unfused: float, t_fused: float, k: int) -> dict:
    """K*L + T = t_unfused, L + T = t_fused  ->  L, T, launch share, reported cut."""
    L = (t_unfused - t_fused) / (k - 1)
    T = t_fused - L
    return {"L": L, "T": T, "launch_share": k * L / t_unfused, "cut": 1.0 - t_fused / t_unfused}


# ------------------------------------------------------------ byte models

def det_bytes(levels_hw, n_anchors=3, n_ch=85, in_size=2):
    e = sum(n_anchors * n_ch * h * w for h, w in levels_hw)  # input elements
    rows = sum(n_anchors * h * w for h, w in levels_hw)
    fused = e * in_size + rows * n_ch * 4
    per_ch = e / n_ch
    # permute, sigma(xy), sigma(obj+cls), exp(wh), x anchor, + grid, x stride: read + write
    unf = 2 * e * in_size + 2 * in_size * per_ch * (2 + (n_ch - 4) + 2 + 2 + 2 + 2)
    unf += 2 * e * in_size  # concat
    unf += e * in_size + rows * n_ch * 4  # cast to fp32
    return int(fused), int(unf)


def rms_bytes(rows, cols, es=2):
    s = rows * cols * es
    fused = 4 * s + cols * es
    unf = 3 * s + 2 * s + (s + rows * es) + 2 * rows * es + (2 * s + rows * es) + (2 * s + cols * es)
    return fused, unf


def ln_bytes(rows, cols, es=2):
    s = rows * cols * es
    fused = 4 * s + 2 * cols * es
    # add 3S; mean S; subtract 2S; square 2S; mean S; rsqrt; x rstd 2S; x gamma 2S; + beta 2S
    unf = 15 * s + 8 * rows * es + 2 * cols * es
    return fused, unf


def rope_bytes(T, H, D, es=2):
    q = T * H * D * es
    return 6 * q, 6 * q + 2 * q + 2 * q + 2 * q


SETTLE_S = 0.25  # seconds of untimed steps before the warm-up steps
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix-core peak of MI355X
VALU_PEAK = 256 * 64 * 2.4e9  # lane-instr/s: 256 CUs x 4 SIMD x 16 lanes x 2.4 GHz


def file_hash(*paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


_CHAIN_SRC = ["norm_pass_amd/csrc/chain.hip", "norm_pass_amd/csrc/device.h",
              "norm_pass_amd/csrc/fastmath.h", "norm_pass_amd/csrc/rtc.cpp"]
KERNEL_SOURCES = {
    "c1": _CHAIN_SRC,
    "c5_large": _CHAIN_SRC,
    "c5_large_pe": _CHAIN_SRC,  # the 2^28 chain evaluated per element (not its table)
    "c5_small": _CHAIN_SRC,
    "c2": ["norm_pass_amd/csrc/det_decode.hip", "norm_pass_amd/csrc/device.h"],
    "c3": ["norm_pass_amd/csrc/add_rmsnorm.hip", "norm_pass_amd/csrc/device.h"],
    "c4": ["norm_pass_amd/csrc/qkv_rope.hip", "norm_pass_amd/csrc/device.h"],
    "ln": ["norm_pass_amd/csrc/add_layernorm.hip", "norm_pass_amd/csrc/device.h"],
    "tr": ["norm_pass_amd/csrc/layout.hip", "norm_pass_amd/csrc/device.h"],
    "shuffle_nchw": ["norm_pass_amd/csrc/layout.hip", "norm_pass_amd/csrc/device.h"],
    "shuffle_nhwc": ["norm_pass_amd/csrc/layout.hip", "norm_pass_amd/csrc/device.h"],
    "rl": ["norm_pass_amd/csrc/rmsnorm_linear.hip", "norm_pass_amd/csrc/device.h"],
}


def _counter_row(name: str):
    """Row `| name | source hash | traffic bytes | ... | valu insts/element |` of
    the committed rocprofv3 counter summary, if the kernel sources still hash
    to what they were when the counters were taken."""
    path = os.path.join(PROFILES, "counters_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 3 and cells[0] == name and re.fullmatch(r"[0-9a-f]{16}", cells[1]):
            return cells if cells[1] == file_hash(*KERNEL_SOURCES[name]) else None
    return None


def measured_traffic(name: str):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated) or None."""
    row = _counter_row(name)
    return float(row[2]) if row else None


def measured_valu_per_element(name: str):
    """Dynamic VALU lane-instructions per element (SQ_INSTS_VALU) or None."""
    row = _counter_row(name)
    try:
        return float(row[-1]) if row else None
    except ValueError:
        return None


# ------------------------------------------------------------------ timing

def time_calls(torch, fn, reps: int, trials: int):
    """Median per-call seconds over `trials` trials of `reps` back-to-back calls,
    timed with HIP events on the current stream (the stream every call uses)."""
    res = []
    for _ in range(trials):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        e.synchronize()
        res.append(s.elapsed_time(e) / 1e3 / reps)
    res.sort()
    return res[len(res) // 2], res[max(0, len(res) // 10)], res[min(len(res) - 1, (9 * len(res)) // 10)]


def graph_time(torch, npa, spec, reps: int, trials: int):
    """Per-replay seconds of one call's launches captured in one HIP graph
    (bound inside the capture, so the launches go to the capturing stream)."""
    name, args = spec
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        npa.bind(name, *args)()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        npa.bind(name, *args)()
    med, _, _ = time_calls(torch, g.replay, reps, trials)
    torch.cuda.synchronize()
    return med


def pick_reps(torch, fn, target_s=0.003):
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    one = max(time.perf_counter() - t0, 2e-6)
    return int(min(2000, max(3, target_s / one)))


# ------------------------------------------------------------- workloads

def build_workloads(torch, npa, synth, quick: bool):
    dev = "cuda"
    W = {}
    import numpy as np

    def tdev(a, dt):
        a = np.ascontiguousarray(a)
        if dt == "f32":
            return torch.from_numpy(a).to(dev)
        if dt == "f16":
            return torch.from_numpy(a.view(np.float16)).to(dev)
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    # C1
    n1 = 1 << 20
    a, b = synth.c1_inputs(n1)
    ta, tb = tdev(a, "f32"), tdev(b, "f32")
    y1 = torch.empty(n1, device=dev)
    # warm-up specialisation of the chains (compiled once, off the timed path)
    t0 = time.perf_counter()
    npa.fuse_chain_prepare(synth.C1_CHAIN, 2, npa.NP_F32, npa.NP_F32, n1)
    compile_ms = {"c1": round((time.perf_counter() - t0) * 1e3, 1)}
    W["c1"] = dict(
        desc="fp32 relu(a+b)*0.5, 1,048,576 elements",
        fused=npa.bind("fuse_chain", synth.C1_CHAIN, [ta, tb], y1),
        unfused=npa.bind("unfused_chain", synth.C1_CHAIN, [ta, tb], y1),
        unfused_spec=("unfused_chain", (synth.C1_CHAIN, [ta, tb], y1)),
        bytes=12 * n1, unfused_bytes=28 * n1, launches=3, kernel="np_chain_spec_k4_n1048576")
    # C2
    lv = [tdev(x, "f16") for x in synth.c2_inputs()]
    hw = [(h, w) for h, w, _ in synth.YOLO_LEVELS]
    st = [s for _, _, s in synth.YOLO_LEVELS]
    an = np.array(synth.YOLO_ANCHORS, np.float32).reshape(3, 3, 2).tolist()
    out2 = torch.empty((1, 25200, 85), device=dev)
    ws2 = torch.empty(npa.det_workspace_bytes(lv), dtype=torch.uint8, device=dev)
    fb, ub = det_bytes(hw)
    W["c2"] = dict(
        desc="YOLO decode fp16 [1,255,80|40|20] -> fp32 [1,25200,85]",
        fused=npa.bind("fuse_det_decode", lv, st, an, out2),
        unfused=npa.bind("unfused_det_decode", lv, st, an, out2, ws2),
        unfused_spec=("unfused_det_decode", (lv, st, an, out2, ws2)),
        bytes=fb, unfused_bytes=ub, launches=23, kernel="det_decode_kernel")
    # C3
    rows = 2048 if quick else 16384
    x, r, w = synth.c3_inputs(rows=rows)
    tx, tr, tw = tdev(x, "bf16"), tdev(r, "bf16"), tdev(w, "bf16")
    del x, r
    h3 = torch.empty_like(tx)
    o3 = torch.empty_like(tx)
    ws3 = torch.empty(npa.rmsnorm_workspace_bytes(rows, 4096, torch.bfloat16), dtype=torch.uint8,
                      device=dev)
    fb, ub = rms_bytes(rows, 4096)
    # two more buffer sets: rotating through 3 x 512 MB defeats the 256 MB
    # Infinity Cache, so the "cold" figure is HBM-to-HBM
    sets3 = [(tx, tr, h3, o3)] + [tuple(torch.empty_like(tx) for _ in range(4)) for _ in range(2)]
    for st3 in sets3[1:]:
        st3[0].copy_(tx)
        st3[1].copy_(tr)
    cold3 = [npa.bind("fuse_add_rmsnorm", a_, b_, tw, c_, d_, 1e-6) for a_, b_, c_, d_ in sets3]
    W["c3"] = dict(cold=cold3,
        desc=f"bf16 residual add + RMSNorm [{rows}, 4096], eps 1e-6",
        fused=npa.bind("fuse_add_rmsnorm", tx, tr, tw, h3, o3, 1e-6),
        unfused=npa.bind("unfused_add_rmsnorm", tx, tr, tw, h3, o3, ws3, 1e-6),
        unfused_spec=("unfused_add_rmsnorm", (tx, tr, tw, h3, o3, ws3, 1e-6)),
        bytes=fb, unfused_bytes=ub, launches=6, kernel="rms_vec")
    # LayerNorm (the next row on the same machinery): same shape as C3, not in the step
    gam = tdev(synth.normal((4096,), 1013, "bf16", mean=1.0, std=0.1), "bf16")
    bet = tdev(synth.normal((4096,), 1014, "bf16", std=0.1), "bf16")
    hl = torch.empty_like(tx)
    ol = torch.empty_like(tx)
    wsl = torch.empty(npa.layernorm_workspace_bytes(rows, 4096, torch.bfloat16),
                      dtype=torch.uint8, device=dev)
    fb, ub = ln_bytes(rows, 4096)
    W["ln"] = dict(
        desc=f"bf16 residual add + LayerNorm [{rows}, 4096], eps 1e-5 (not in the step)",
        fused=npa.bind("fuse_add_layernorm", tx, tr, gam, bet, hl, ol, 1e-5),
        unfused=npa.bind("unfused_add_layernorm", tx, tr, gam, bet, hl, ol, wsl, 1e-5),
        unfused_spec=("unfused_add_layernorm", (tx, tr, gam, bet, hl, ol, wsl, 1e-5)),
        bytes=fb, unfused_bytes=ub, launches=9, kernel="ln_vec")
    # C4
    T = 2048 if quick else 16384
    qkv = tdev(synth.c4_inputs(tokens=T), "bf16")
    q4, k4, v4 = (torch.empty((24, T, 128), dtype=torch.bfloat16, device=dev) for _ in range(3))
    qs = float(np.float32(1.0 / math.sqrt(128.0)))
    fb, ub = rope_bytes(T, 24, 128)
    sets4 = [(qkv, q4, k4, v4)] + [tuple(torch.empty_like(t) for t in (qkv, q4, k4, v4))
                                   for _ in range(2)]
    for st4 in sets4[1:]:
        st4[0].copy_(qkv)
    cold4 = [npa.bind("fuse_qkv_rope", a_, b_, c_, d_, 24, 128, None, 10000.0, qs)
             for a_, b_, c_, d_ in sets4]
    W["c4"] = dict(cold=cold4,
        desc=f"bf16 QKV split + RoPE + scale, [{T}, 3x24x128] -> 3 x [24, {T}, 128]",
        fused=npa.bind("fuse_qkv_rope", qkv, q4, k4, v4, 24, 128, None, 10000.0, qs),
        unfused=npa.bind("unfused_qkv_rope", qkv, q4, k4, v4, 24, 128, None, 10000.0, qs),
        unfused_spec=("unfused_qkv_rope", (qkv, q4, k4, v4, 24, 128, None, 10000.0, qs)),
        bytes=fb, unfused_bytes=ub, launches=4, kernel="rope_tok")
    # C5
    ops = synth.c5_chain()
    t0 = time.perf_counter()
    npa.fuse_chain_prepare(ops, 1, npa.NP_F16, npa.NP_F16, 0)
    compile_ms["c5"] = round((time.perf_counter() - t0) * 1e3, 1)
    table_min = npa.np_set_chain_table_min(-1)
    for name, n in (("c5_small", 1 << 16), ("c5_large", (1 << 24) if quick else (1 << 28))):
        xin = tdev(synth.c5_inputs(n), "f16")
        yo = torch.empty_like(xin)
        fused = npa.bind("fuse_chain", ops, [xin], yo)

        def per_element(fused=fused):
            # the same call with the table threshold out of reach: the chain
            # evaluated per element by the specialised kernel
            old = npa.np_set_chain_table_min(1 << 62)
            fused()
            npa.np_set_chain_table_min(old)

        W[name] = dict(
            desc=f"seeded 29-op fp16 chain, {n:,} elements",
            fused=fused,
            unfused=npa.bind("unfused_chain", ops, [xin], yo),
            unfused_spec=("unfused_chain", (ops, [xin], yo)),
            bytes=4 * n, unfused_bytes=29 * 4 * n, launches=29,
            kernel="np_chain_spec_k30_n0_lut" if n >= table_min else "np_chain_scalar_k30_n0",
            path="table" if n >= table_min else "per element")
        if n >= table_min:
            W[name]["fused_per_element"] = per_element
    # Layout (the runtime page's strided transpose / ChannelShuffle; not in the
    # step): the LDS-staged kernels against the naive strided copy, and torch's
    # own permute().contiguous() for context. Three buffer sets each for the
    # cold figure.
    def layout(name, desc, x_np, dt, shape, fused_name, naive_name, extra_args, torch_fn,
               kernel):
        x = tdev(x_np, dt)
        sets = [(x, torch.empty_like(x))]
        for _ in range(2):
            y = torch.empty_like(x)
            y.copy_(x)
            sets.append((y, torch.empty_like(x)))
        xo = sets[0][1]
        nbytes = x.numel() * x.element_size()
        W[name] = dict(
            cold=[npa.bind(fused_name, a_, b_, *extra_args) for a_, b_ in sets],
            desc=desc,
            fused=npa.bind(fused_name, x, xo, *extra_args),
            unfused=npa.bind(naive_name, x, xo, *extra_args),
            unfused_spec=(naive_name, (x, xo) + tuple(extra_args)),
            torch=lambda: torch_fn(x), bytes=2 * nbytes, unfused_bytes=2 * nbytes,
            launches=1, kernel=kernel,
            plan=npa.np_transpose_plan(x.data_ptr(), xo.data_ptr(), shape, x.element_size()))

    B_, R_, S_, E_ = synth.TRANSPOSE_2D
    if quick:
        B_, R_, S_, E_ = 1, 2048, 2048, 1
    layout("tr", f"fp32 [{R_}, {S_}] transpose (not in the step; baseline: naive strided copy)",
           synth.transpose_inputs((B_, R_, S_, E_)), "f32", (B_, R_, S_, E_),
           "fuse_transpose021", "naive_transpose021", (),
           lambda t: t.transpose(1, 2).contiguous(), "tr_tile<4, true>")
    N_, C_, H_, Wd = synth.SHUFFLE_NCHW
    if quick:
        N_ = 64
    g = synth.SHUFFLE_GROUPS
    for lay, nm in ((0, "shuffle_nchw"), (1, "shuffle_nhwc")):
        xs = synth.shuffle_inputs((N_, C_, H_, Wd), layout=lay)
        if lay == 0:
            shp = (N_, g, C_ // g, H_ * Wd)
            tf = (lambda t, n=N_, c=C_, h=H_, wd=Wd:
                  t.view(n, g, c // g, h, wd).transpose(1, 2).contiguous())
        else:
            shp = (N_ * H_ * Wd, g, C_ // g, 1)
            tf = (lambda t, n=N_, c=C_, h=H_, wd=Wd:
                  t.view(n, h, wd, g, c // g).transpose(3, 4).contiguous())
        layout(nm, f"fp16 ChannelShuffle {nm[8:].upper()} [{N_}, {C_}, {H_}, {Wd}], groups {g} "
                   "(not in the step; baseline: naive strided copy)",
               xs, "f16", shp, "fuse_channel_shuffle", "naive_channel_shuffle", (g, lay), tf,
               "tr_items<16, true>" if lay == 0 else "tr_small<2, true>")
    # RMSNorm + linear + scale on the matrix cores (not in the step): fused
    # kernel vs RMSNorm -> GEMM + bias -> scale, and torch's bf16 linear
    # (the vendor GEMM) on the stored RMSNorm output, for context
    Mr, Kr, Nr = synth.RMS_LINEAR_SHAPE
    if quick:
        Mr = 2048
    xr, wr, Wr, br = (tdev(a_, "bf16") for a_ in synth.rmsnorm_linear_inputs((Mr, Kr, Nr)))
    orl = torch.empty((Mr, Nr), dtype=torch.bfloat16, device=dev)
    wsr = torch.empty(npa.rmsnorm_linear_workspace_bytes(Mr, Kr), dtype=torch.uint8, device=dev)
    yr = torch.empty((Mr, Kr), dtype=torch.bfloat16, device=dev)
    npa.fuse_add_rmsnorm(xr, None, wr, None, yr, 1e-6)
    sc = synth.RMS_LINEAR_SCALE
    # the norm weight folded into the (constant) linear weight once, outside
    # any timed region; the fused call then streams x and the weight straight
    # into LDS. The call with the norm weight kept separate is timed as well.
    Wf = torch.empty_like(Wr)
    npa.np_fold_norm_weight(wr, Wr, Wf)
    W["rl"] = dict(
        desc=f"bf16 RMSNorm + linear + scale, x [{Mr}, {Kr}] x Wt [{Nr}, {Kr}]^T, norm weight "
             "folded into Wt (not in the step)",
        fused=npa.bind("fuse_rmsnorm_linear", xr, None, Wf, br, orl, 1e-6, sc),
        fused_unfolded=npa.bind("fuse_rmsnorm_linear", xr, wr, Wr, br, orl, 1e-6, sc),
        unfused=npa.bind("unfused_rmsnorm_linear", xr, wr, Wr, br, orl, wsr, 1e-6, sc),
        unfused_spec=("unfused_rmsnorm_linear", (xr, wr, Wr, br, orl, wsr, 1e-6, sc)),
        torch=lambda: torch.nn.functional.linear(yr, Wr, br).mul_(sc),
        plan=None, bytes=2 * (Mr * Kr + Nr * Kr + Mr * Nr + Kr + Nr),
        unfused_bytes=2 * (3 * Mr * Kr + Nr * Kr + 3 * Mr * Nr + Kr + Nr),
        flops=2 * Mr * Nr * Kr, launches=3, kernel="rms_linear_dma4")
    W["_compile_ms"] = compile_ms
    return W


# ------------------------------------------------------------- CPU oracle

def disk_cache_timing(torch, npa, synth):
    """fuse_chain_prepare of the 29-op chain into an empty disk cache (a
    compile and a store), then again after np_shutdown has dropped every
    loaded module (a load from the cache): the restart case the DeepJIT
    write-up keeps compiled code on disk for (section 6.2). Both include the
    table fill. Runs last, since np_shutdown also unloads the workloads'
    prepared modules."""
    import shutil
    import tempfile
    ops = synth.c5_chain()
    d = tempfile.mkdtemp(prefix="np_chain_cache_")
    old = os.environ.get("NP_CACHE_DIR")
    os.environ["NP_CACHE_DIR"] = d
    try:
        times = []
        s0 = npa.np_chain_cache_stats()
        for _ in range(2):
            torch.cuda.synchronize()
            npa.np_shutdown()
            t0 = time.perf_counter()
            npa.fuse_chain_prepare(ops, 1, npa.NP_F16, npa.NP_F16, 0)
            times.append((time.perf_counter() - t0) * 1e3)
        s1 = npa.np_chain_cache_stats()
        torch.cuda.synchronize()
        npa.np_shutdown()
    finally:
        if old is None:
            os.environ.pop("NP_CACHE_DIR", None)
        else:
            os.environ["NP_CACHE_DIR"] = old
        shutil.rmtree(d, ignore_errors=True)
    return {"compile_ms": round(times[0], 1), "load_ms": round(times[1], 1),
            "loads": s1["loads"] - s0["loads"], "stores": s1["stores"] - s0["stores"],
            "rejects": s1["rejects"] - s0["rejects"]}


def cpu_baseline(synth, quick: bool):
    """The oracle, untuned, timed on the host on a bounded sample of every config;
    the step time is extrapolated from each config's measured oracle rate."""
    import numpy as np
    import oracle
    rates = {}
    samples = []

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    a, b = synth.c1_inputs()
    rates["c1"] = 12 * a.size / timed(lambda: oracle.chain(synth.C1_CHAIN, [a, b], 0))
    samples.append("c1 full")
    lv = synth.c2_inputs()
    hw = [(h, w) for h, w, _ in synth.YOLO_LEVELS]
    anc = np.array(synth.YOLO_ANCHORS, np.float32).reshape(3, 3, 2)
    rates["c2"] = det_bytes(hw)[0] / timed(
        lambda: oracle.det_decode(lv, hw, [8.0, 16.0, 32.0], anc, 3, 85, in_dt=1))
    samples.append("c2 full")
    rows = 256 if quick else 2048
    x, r, w = synth.c3_inputs(rows=rows)
    rates["c3"] = rms_bytes(rows, 4096)[0] / timed(lambda: oracle.add_rmsnorm(x, r, w, 1e-6, 2))
    samples.append(f"c3 {rows} of 16384 rows")
    toks = 256 if quick else 2048
    qkv = synth.c4_inputs(tokens=toks)
    rates["c4"] = rope_bytes(toks, 24, 128)[0] / timed(
        lambda: oracle.qkv_rope(qkv, 24, 128, 10000.0, 0.08838834764831845, 2))
    samples.append(f"c4 {toks} of 16384 tokens")
    ops = synth.c5_chain()
    xs = synth.c5_inputs(1 << 16)
    rates["c5_small"] = 4 * xs.size / timed(lambda: oracle.chain(ops, [xs], 1))
    samples.append("c5 65,536 full")
    nl = (1 << 20) if quick else (1 << 23)
    xl = synth.c5_inputs(nl, seed=77)
    rates["c5_large"] = 4 * nl / timed(lambda: oracle.chain(ops, [xl], 1))
    samples.append(f"c5 {nl:,} of 268,435,456 elements")
    # the next rows (not in the step): the same oracle, each on its own sample
    # (their GPU figures are reported beside these)
    gam = synth.normal((4096,), 1013, "bf16", mean=1.0, std=0.1)
    bet = synth.normal((4096,), 1014, "bf16", std=0.1)
    rates["ln"] = ln_bytes(rows, 4096)[0] / timed(
        lambda: oracle.add_layernorm(x, r, gam, bet, 1e-5, 2))
    samples.append(f"ln {rows} of 16384 rows")
    tr_rows = 256 if quick else 1024
    xt = synth.transpose_inputs((1, tr_rows, 8192, 1))
    rates["tr"] = 2 * xt.nbytes / timed(lambda: oracle.transpose021(xt))
    samples.append(f"tr {tr_rows} of 8192 rows")
    nb = 16 if quick else 128
    for name, layout in (("shuffle_nchw", 0), ("shuffle_nhwc", 1)):
        xs_ = synth.shuffle_inputs((nb,) + synth.SHUFFLE_NCHW[1:], layout=layout)
        rates[name] = 2 * xs_.nbytes / timed(
            lambda: oracle.channel_shuffle(xs_, synth.SHUFFLE_GROUPS, layout))
        samples.append(f"{name} batch {nb} of 1024")
    mr = 2 if quick else 8
    xr, wr, Wr, br = synth.rmsnorm_linear_inputs()
    M, K, N = synth.RMS_LINEAR_SHAPE
    rates["rl_flops"] = 2 * mr * K * N / timed(
        lambda: oracle.rmsnorm_linear(xr[:mr], wr, Wr, br, 1e-6, synth.RMS_LINEAR_SCALE, 2))
    samples.append(f"rl {mr} of {M} rows (flop/s)")
    return rates, "; ".join(samples)


# ------------------------------------------------------------------- main

def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--trials", type=int, default=11)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--quick", action="store_true", help="reduced sizes (smoke runs only)")
    ap.add_argument("--profile", action="store_true",
                    help="only a few launches of each kernel (for rocprofv3 runs)")
    ap.add_argument("--only", default="", help="profile mode: comma-separated workloads")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU: the fused chains shard without any exchange, so "
              "there is no multi-GPU path to run (use --gpus 1).", file=sys.stderr)
        return 2
    if os.environ.get("WORLD_SIZE", "1") not in ("", "1"):
        print("bench.py runs as a single process on one GPU.", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    sys.path.insert(0, ROOT)
    import synth
    import norm_pass_amd as npa

    t_setup = time.perf_counter()
    npa.np_init(0)
    props = torch.cuda.get_device_properties(0)
    W = build_workloads(torch, npa, synth, args.quick)
    compile_ms = W.pop("_compile_ms")
    torch.cuda.synchronize()
    log = lambda *a: print(*a, file=sys.stderr, flush=True)
    log(f"[bench] setup {time.perf_counter() - t_setup:.1f}s on {props.name} "
        f"({getattr(props, 'gcnArchName', '?')}, {props.multi_processor_count} CUs)")

    if args.profile:
        # a copy of known size for counter calibration, then each kernel a few times
        import numpy as _np  # noqa: F401
        n = 1 << 28
        src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            npa.unfused_chain([(synth.LOAD, 0, 0.0)], [src], dst)
        only = [x for x in args.only.split(",") if x]
        for name, w in W.items():
            if only and name not in only:
                continue
            for _ in range(20):  # warm clocks: rocprofv3 averages every dispatch
                w["fused"]()
            for _ in range(2):
                w["unfused"]()
        if "c5_large_pe" in only and "fused_per_element" in W["c5_large"]:
            for _ in range(20):  # the per-element kernel on the same data
                W["c5_large"]["fused_per_element"]()
        torch.cuda.synchronize()
        log("[bench] profile pass done")
        return 0

    order = ["c1", "c2", "c3", "c4", "c5_small", "c5_large"]
    step_fns = [W[k]["fused"] for k in order]
    step_bytes = sum(W[k]["bytes"] for k in order)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # clock settle (set-up, untimed): the GPU ramps its clocks over the first
    # tens of milliseconds of sustained load (the 2^28-element chain runs
    # ~500 us per launch at first, ~400 us once settled), so the step runs for
    # SETTLE_S seconds before the warm-up steps and the timed ones
    t_settle = time.perf_counter()
    settle_steps = 0
    while time.perf_counter() - t_settle < SETTLE_S:
        for f in step_fns:
            f()
        torch.cuda.synchronize()
        settle_steps += 1

    # warm-up steps, each call bracketed by events: the step's dominant kernel
    # (the config with the longest call) is the one the roofline times below
    warm = {k: [] for k in order}
    for _ in range(max(args.warmup, 1)):
        pairs = []
        for k, f in zip(order, step_fns):
            a, b = ev(), ev()
            a.record()
            f()
            b.record()
            pairs.append((k, a, b))
        torch.cuda.synchronize()
        for k, a, b in pairs:
            warm[k].append(a.elapsed_time(b))
    dom = max(order, key=lambda k: sum(warm[k]) / len(warm[k]))

    # the timed steps; the dominant kernel's launch inside each step is
    # bracketed by its own event pair on the same (current) stream, so its
    # per-launch duration is measured over the timed region itself
    dom_ev = [(ev(), ev()) for _ in range(args.steps)]
    s = ev()
    e = ev()
    t0 = time.perf_counter()
    s.record()
    for i in range(args.steps):
        for k, f in zip(order, step_fns):
            if k == dom:
                dom_ev[i][0].record()
                f()
                dom_ev[i][1].record()
            else:
                f()
    e.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_s = s.elapsed_time(e) / 1e3 / args.steps
    t_dom = sum(a.elapsed_time(b) for a, b in dom_ev) / args.steps / 1e3
    log(f"[bench] {args.steps} steps: {step_s * 1e6:.1f} us/step (wall {wall:.3f}s); "
        f"{dom} {t_dom * 1e6:.1f} us per launch in the step")

    per = {}
    extra = [k for k in W if k not in order]
    for k in order + extra:
        w = W[k]
        reps = pick_reps(torch, w["fused"])
        f_med, f_p10, f_p90 = time_calls(torch, w["fused"], reps, args.trials)
        reps_u = pick_reps(torch, w["unfused"])
        u_med, _, _ = time_calls(torch, w["unfused"], reps_u, max(5, args.trials // 2))
        # the same unfused launches captured once in a HIP graph and replayed:
        # launch cost removed, every intermediate HBM round trip kept
        g_med = graph_time(torch, npa, w["unfused_spec"], reps_u, max(5, args.trials // 2))
        gbps = w["bytes"] / f_med / 1e9
        cold = None
        if "cold" in w:
            calls = w["cold"]
            it = [0]

            def rot():
                calls[it[0] % len(calls)]()
                it[0] += 1
            c_med, _, _ = time_calls(torch, rot, max(3, reps), args.trials)
            cold = {"us_med": round(c_med * 1e6, 3), "GBps": round(w["bytes"] / c_med / 1e9, 1),
                    "pct_of_8TBps": round(100 * w["bytes"] / c_med / 1e9 / HBM_PEAK_GBPS, 1),
                    "buffer_sets": len(calls)}
        per[k] = {
            "desc": w["desc"], "us_med": round(f_med * 1e6, 3), "us_p10": round(f_p10 * 1e6, 3),
            "us_p90": round(f_p90 * 1e6, 3), "GBps": round(gbps, 1),
            "pct_of_8TBps": round(100 * gbps / HBM_PEAK_GBPS, 1), "bytes": w["bytes"],
            "unfused": {"launches": w["launches"], "us_med": round(u_med * 1e6, 3),
                        "GBps": round(w["unfused_bytes"] / u_med / 1e9, 1),
                        "bytes": w["unfused_bytes"],
                        "graph_us_med": round(g_med * 1e6, 3)},
            "speedup": round(u_med / f_med, 2),
        }
        if cold:
            per[k]["cold"] = cold
        if "torch" in w:
            t_med, _, _ = time_calls(torch, w["torch"], reps, max(5, args.trials // 2))
            per[k]["torch_us_med"] = round(t_med * 1e6, 3)
            if w.get("plan") is not None:
                per[k]["plan"] = w["plan"]
        if "path" in w:
            per[k]["path"] = w["path"]
        if "fused_per_element" in w:
            pe_med, _, _ = time_calls(torch, w["fused_per_element"], reps, max(5, args.trials // 2))
            per[k]["per_element_us_med"] = round(pe_med * 1e6, 3)
            per[k]["per_element_GBps"] = round(w["bytes"] / pe_med / 1e9, 1)
        if "fused_unfolded" in w:
            fu_med, _, _ = time_calls(torch, w["fused_unfolded"], reps, max(5, args.trials // 2))
            per[k]["fused_unfolded_us_med"] = round(fu_med * 1e6, 3)
            if "flops" in w:
                per[k]["fused_unfolded_TFLOPs"] = round(w["flops"] / fu_med / 1e12, 1)
        if "flops" in w:
            tf = w["flops"] / f_med / 1e12
            per[k]["TFLOPs"] = round(tf, 1)
            per[k]["mfma_frac"] = round(tf / MFMA_BF16_PEAK_TFLOPS, 4)
            per[k]["unfused"]["TFLOPs"] = round(w["flops"] / u_med / 1e12, 1)
            if "torch_us_med" in per[k]:
                per[k]["torch_TFLOPs"] = round(w["flops"] / (per[k]["torch_us_med"] * 1e-6) / 1e12, 1)
        log(f"[bench] {k}: fused {f_med * 1e6:.2f} us ({gbps:.0f} GB/s), "
            f"unfused {u_med * 1e6:.2f} us x{w['launches']} launches "
            f"(graph {g_med * 1e6:.2f} us)"
            + (f", cold {cold['us_med']:.2f} us ({cold['GBps']:.0f} GB/s)" if cold else ""))

    # achievable streaming ceiling: a plain 16-byte-per-lane copy of 1 GiB
    n_copy = 1 << 28
    csrc = torch.empty(n_copy, dtype=torch.float32, device="cuda").fill_(1.0)
    cdst = torch.empty_like(csrc)
    cp = npa.bind("unfused_chain", [(synth.LOAD, 0, 0.0)], [csrc], cdst)
    c_med, _, _ = time_calls(torch, cp, 10, 7)
    copy_gbps = 2 * 4 * n_copy / c_med / 1e9
    del csrc, cdst
    for k in order + extra:
        per[k]["frac_of_copy"] = round(per[k]["GBps"] / copy_gbps, 3)
    log(f"[bench] copy ceiling {copy_gbps:.0f} GB/s")

    # launch-cost model (NaiveRT write-up): the pages' own instance, then ours
    pages = cost_model(PAGES_COST_MODEL["t_unfused_ms"], PAGES_COST_MODEL["t_fused_ms"],
                       PAGES_COST_MODEL["k"])
    small = per["c5_small"]
    ours = cost_model(small["unfused"]["us_med"], small["us_med"], 29)
    reps = 50
    direct, _, _ = time_calls(torch, lambda: npa.np_empty_launches(29), reps, 5)
    ours["L_direct_us"] = round(direct * 1e6 / 29, 3)
    for key in ("L", "T"):
        ours[key] = round(ours[key], 3)

    # roofline of the dominant kernel of the step: HBM for the streaming
    # kernels; the 29-op chain is bound by VALU issue (its algorithmic slots
    # per element far exceed the ~20 that 8 TB/s leaves per fp16 element)
    d = per[dom]
    hbm_frac = d["bytes"] / t_dom / 1e9 / HBM_PEAK_GBPS
    if dom.startswith("c5") and W[dom].get("path") != "table":
        n_el = d["bytes"] // 4
        # executed VALU instructions per element from the committed rocprofv3
        # SQ_INSTS_VALU count; none (and no achieved figure) once the kernel
        # sources have changed since it was taken
        per_el = measured_valu_per_element(dom)
        achieved = per_el * n_el / t_dom / 1e12 if per_el is not None else None
        roof = {"kernel": dom, "launch_us": round(t_dom * 1e6, 2), "bound": "alu",
                "achieved": round(achieved, 2) if achieved is not None else None,
                "peak": round(VALU_PEAK / 1e12, 2), "unit": "T VALU lane-instr/s",
                "frac": round(achieved * 1e12 / VALU_PEAK, 4) if achieved is not None else None,
                "valu_per_element": round(per_el, 2) if per_el is not None else None,
                "valu_count_source": "rocprofv3 SQ_INSTS_VALU" if per_el is not None
                else "none for the current kernel sources",
                "hbm_frac": round(hbm_frac, 4), "traffic": measured_traffic(dom)}
    else:
        achieved = d["bytes"] / t_dom / 1e9
        roof = {"kernel": dom, "launch_us": round(t_dom * 1e6, 2), "bound": "hbm",
                "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(hbm_frac, 4),
                "traffic": measured_traffic(dom)}
    # every kernel's own roofline, for the record
    for k in order + extra:
        per[k]["hbm_frac"] = round(per[k]["bytes"] / (per[k]["us_med"] * 1e-6) / 1e9
                                   / HBM_PEAK_GBPS, 4)
    for k in ("c5_small", "c5_large"):
        n_el = per[k]["bytes"] // 4
        v = measured_valu_per_element(k if W[k].get("path") != "table" else "c5_large_pe")
        t_pe = (per[k]["us_med"] if W[k].get("path") != "table"
                else per[k].get("per_element_us_med"))
        per[k]["valu_frac"] = (round(v * n_el / (t_pe * 1e-6) / VALU_PEAK, 4)
                               if v is not None and t_pe else None)

    cpu = None
    if not args.no_cpu:
        t0 = time.perf_counter()
        rates, sample = cpu_baseline(synth, args.quick)
        est = sum(W[k]["bytes"] / rates[k] for k in order)
        cpu = {"value": round(step_bytes / est / 1e9, 4), "unit": "GB/s", "cores": 1,
               "kind": "oracle", "sample": sample,
               "per_config_GBps": {k: round(v / 1e9, 4) for k, v in rates.items()
                                   if k != "rl_flops"},
               "rl_GFLOPs": round(rates["rl_flops"] / 1e9, 4),
               "seconds": round(time.perf_counter() - t0, 1)}
        # beside each row's GPU figure: the oracle's rate on its sample
        for k in order + extra:
            if k in rates:
                per[k]["cpu_oracle_GBps"] = round(rates[k] / 1e9, 4)
                per[k]["gpu_over_cpu_oracle"] = round(per[k]["GBps"] * 1e9 / rates[k], 1)
        if "rl" in per:
            per["rl"]["cpu_oracle_GFLOPs"] = round(rates["rl_flops"] / 1e9, 4)
            per["rl"]["gpu_over_cpu_oracle"] = round(
                per["rl"]["TFLOPs"] * 1e12 / rates["rl_flops"], 1)
        log(f"[bench] cpu oracle {cpu['value']} GB/s ({cpu['seconds']} s)")

    disk = disk_cache_timing(torch, npa, synth)
    log(f"[bench] prepare of the 29-op chain: {disk['compile_ms']} ms compiling, "
        f"{disk['load_ms']} ms from the disk cache")

    value = step_bytes / step_s / 1e9
    out = {
        "metric": "achieved HBM GB/s (% of peak) + per-call us, fused vs N-launch unfused",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle_steps": settle_steps,
        "ms_per_step": round(step_s * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded Philox normals; see synth/)",
        "config": {"workload": "one fused pass over all five chains: C1 fp32 relu(a+b)*0.5 1M; "
                               "C2 YOLO decode fp16 3 levels; C3 bf16 add+RMSNorm 16384x4096; "
                               "C4 bf16 QKV split+RoPE+scale 16384x24x128; C5 29-op fp16 chain "
                               "65,536 and 268,435,456",
                   "pct_of_peak": round(100 * value / HBM_PEAK_GBPS, 1),
                   "step_bytes": step_bytes, "quick": args.quick},
        "roofline": roof,
        "cpu_baseline": cpu,
        "per_config": per,
        "cost_model": {"pages": {k: round(v, 4) for k, v in pages.items()}, "c5_small_us": ours},
        "rtc_compile_ms": compile_ms,
        "rtc_disk_cache_ms": disk,
        "copy_ceiling_GBps": round(copy_gbps, 1),
        "env": {"gpu": props.name, "arch": getattr(props, "gcnArchName", ""),
                "cus": props.multi_processor_count, "torch": torch.__version__},
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
