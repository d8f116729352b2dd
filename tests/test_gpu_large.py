"""Past 2^31 elements: the 64-bit index paths at sizes a 288 GB GPU holds with
room to spare (4-5 GB per tensor).

- the 29-op fp16 chain at 2^31 + 2^20 + 7 elements, through the table gather
  and through the per-element kernel of the same prepared module (their
  outputs must be the same bits), sampled against the oracle;
- add + RMSNorm and add + LayerNorm on [2^19 + 3, 4096] bf16 (2^31 + 12,288
  elements), sampled rows against the oracle;
- QKV split + RoPE + scale with 2^18 + 5 tokens (2.4 * 10^9 input elements),
  sampled tokens against the oracle at their positions.

A dispatch grid counts at most 2^32 work-items, so the library splits long
calls into several launches: the chain every 2^30 elements (the chain test
above crosses two such boundaries), the norms every 2^22 rows and QKV + RoPE
every 2^21 tokens. The boundary tests below run just past one such launch
and check the rows or tokens on both sides of it.

Inputs are drawn on the device (gpu_util.gpu_normal). Samples always include
both ends and the elements, rows or tokens around index 2^31 or the launch
boundary.
"""
import math

import numpy as np
import pytest
import torch

import synth
from gpu_util import empty, gpu_normal, need_gpu, to_host
from tolerance import check_half, half_values

pytestmark = pytest.mark.gpu
F16, BF16 = 1, 2
EDGE = 1 << 31


@pytest.fixture(scope="module")
def npa():
    need_gpu()
    import norm_pass_amd
    norm_pass_amd.np_init(0)
    return norm_pass_amd


@pytest.fixture(autouse=True)
def _free():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def sample(n: int, k: int, edge: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    parts = [rng.integers(0, n, k), np.arange(0, min(n, 64)), np.arange(max(0, n - 64), n),
             np.arange(max(0, edge - 64), min(n, edge + 64))]
    return np.unique(np.concatenate(parts))


def test_chain_past_2_31_elements(npa, orc):
    n = EDGE + (1 << 20) + 7
    ops = synth.c5_chain()
    x = gpu_normal((n,), "f16", seed=2031)
    out_tab, out_pe = empty((n,), "f16"), empty((n,), "f16")
    npa.fuse_chain_prepare(ops, 1, npa.NP_F16, npa.NP_F16, 0)
    old = npa.np_set_chain_table_min(-1)
    try:
        npa.np_set_chain_table_min(1 << 22)
        npa.fuse_chain(ops, [x], out_tab)
        npa.np_set_chain_table_min(1 << 62)
        npa.fuse_chain(ops, [x], out_pe)
        torch.cuda.synchronize()
    finally:
        npa.np_set_chain_table_min(old)
        torch.cuda.synchronize()
        npa.np_shutdown()
    assert torch.equal(out_tab.view(torch.int16), out_pe.view(torch.int16))
    idx = torch.from_numpy(sample(n, 1 << 18, EDGE, 1)).cuda()
    xs = to_host(x[idx]).view(np.float16)
    got = to_host(out_tab[idx])
    ref, exact, bound = orc.chain(ops, [xs], F16, want_bound=True)
    check_half(got, ref, "f16", half_values(got, "f16"), exact, bound,
               what=f"chain n = {n}, sampled")


@pytest.mark.parametrize("norm", ["rms", "layer"])
def test_norms_past_2_31_elements(npa, orc, norm):
    rows, cols = (1 << 19) + 3, 4096
    x = gpu_normal((rows, cols), "bf16", seed=2032)
    r = gpu_normal((rows, cols), "bf16", seed=2033)
    w = gpu_normal((cols,), "bf16", seed=2034, mean=1.0, std=0.1)
    b = gpu_normal((cols,), "bf16", seed=2035, std=0.1)
    h, out = empty((rows, cols), "bf16"), empty((rows, cols), "bf16")
    if norm == "rms":
        npa.fuse_add_rmsnorm(x, r, w, h, out, 1e-6)
    else:
        npa.fuse_add_layernorm(x, r, w, b, h, out, 1e-5)
    torch.cuda.synchronize()
    ri = torch.from_numpy(sample(rows, 256, EDGE // cols, 2)).cuda()
    xs, rs = to_host(x[ri]), to_host(r[ri])
    ws, bs = to_host(w), to_host(b)
    if norm == "rms":
        rh, ro = orc.add_rmsnorm(xs, rs, ws, 1e-6, BF16)
    else:
        rh, ro = orc.add_layernorm(xs, rs, ws, bs, 1e-5, BF16)
    assert np.array_equal(to_host(h[ri]).view(np.uint16), np.asarray(rh).view(np.uint16))
    check_half(to_host(out[ri]), ro, "bf16", max_ulp=2, what=f"{norm} [{rows}, {cols}], sampled rows")


def test_qkv_rope_past_2_31_elements(npa, orc):
    T, H, D = (1 << 18) + 5, 24, 128
    qs = float(np.float32(1 / math.sqrt(D)))
    qkv = gpu_normal((T, 3 * H * D), "bf16", seed=2036)
    q, k, v = (empty((H, T, D), "bf16") for _ in range(3))
    npa.fuse_qkv_rope(qkv, q, k, v, H, D, None, 10000.0, qs)
    torch.cuda.synchronize()
    ti = sample(T, 128, EDGE // (3 * H * D), 3)
    tt = torch.from_numpy(ti).cuda()
    rq, rk, rv, eq, ek, bq, bk = orc.qkv_rope(to_host(qkv[tt]), H, D, 10000.0, qs, BF16,
                                              positions=ti.astype(np.int32), want_bound=True)
    gq, gk, gv = (to_host(t[:, tt, :]) for t in (q, k, v))
    assert np.array_equal(gv.view(np.uint16), np.asarray(rv).view(np.uint16))
    check_half(gq, rq, "bf16", half_values(gq, "bf16"), eq, bq, what="Q, sampled tokens")
    check_half(gk, rk, "bf16", half_values(gk, "bf16"), ek, bk, what="K, sampled tokens")


ROW_CHUNK, TOK_CHUNK = 1 << 22, 1 << 21  # rows / tokens per launch in the library


@pytest.mark.parametrize("norm", ["rms", "layer"])
def test_norms_across_launch_boundary(npa, orc, norm):
    rows, cols = ROW_CHUNK + 5, 8
    x = gpu_normal((rows, cols), "bf16", seed=2041)
    r = gpu_normal((rows, cols), "bf16", seed=2042)
    w = gpu_normal((cols,), "bf16", seed=2043, mean=1.0, std=0.1)
    b = gpu_normal((cols,), "bf16", seed=2044, std=0.1)
    h, out = empty((rows, cols), "bf16"), empty((rows, cols), "bf16")
    if norm == "rms":
        npa.fuse_add_rmsnorm(x, r, w, h, out, 1e-6)
    else:
        npa.fuse_add_layernorm(x, r, w, b, h, out, 1e-5)
    torch.cuda.synchronize()
    ri = torch.from_numpy(sample(rows, 4096, ROW_CHUNK, 4)).cuda()
    xs, rs = to_host(x[ri]), to_host(r[ri])
    ws, bs = to_host(w), to_host(b)
    if norm == "rms":
        rh, ro = orc.add_rmsnorm(xs, rs, ws, 1e-6, BF16)
    else:
        rh, ro = orc.add_layernorm(xs, rs, ws, bs, 1e-5, BF16)
    assert np.array_equal(to_host(h[ri]).view(np.uint16), np.asarray(rh).view(np.uint16))
    check_half(to_host(out[ri]), ro, "bf16", max_ulp=2,
               what=f"{norm} [{rows}, {cols}] across the row launch boundary")


@pytest.mark.parametrize("D", [128, 64])  # token workgroups; (token, chunk) threads
def test_qkv_rope_across_launch_boundary(npa, orc, D):
    T, H = TOK_CHUNK + 3, 1
    qs = float(np.float32(1 / math.sqrt(D)))
    qkv = gpu_normal((T, 3 * H * D), "bf16", seed=2045 + D)
    pos_np = ((np.arange(T, dtype=np.int64) * 7) % 16384).astype(np.int32)
    pos = torch.from_numpy(pos_np).cuda()
    q, k, v = (empty((H, T, D), "bf16") for _ in range(3))
    npa.fuse_qkv_rope(qkv, q, k, v, H, D, pos, 10000.0, qs)
    torch.cuda.synchronize()
    ti = sample(T, 2048, TOK_CHUNK, 5)
    tt = torch.from_numpy(ti).cuda()
    rq, rk, rv, eq, ek, bq, bk = orc.qkv_rope(to_host(qkv[tt]), H, D, 10000.0, qs, BF16,
                                              positions=pos_np[ti],
                                              want_bound=True)
    gq, gk, gv = (to_host(t[:, tt, :]) for t in (q, k, v))
    assert np.array_equal(gv.view(np.uint16), np.asarray(rv).view(np.uint16))
    check_half(gq, rq, "bf16", half_values(gq, "bf16"), eq, bq, what="Q across the boundary")
    check_half(gk, rk, "bf16", half_values(gk, "bf16"), ek, bk, what="K across the boundary")
