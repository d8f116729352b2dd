"""GPU parity of fuse_rmsnorm_linear / unfused_rmsnorm_linear against the
oracle (TeleTron write-up, section 4.2: RMSNorm + linear + scale in one
kernel, the RMS factor applied to the linear layer's accumulation, the
weighted input x * w held in fp32).

Tolerance, from the arithmetic. The oracle's operand is x * w unrounded. The
matrix cores take dt operands, so the kernel rounds one operand to dt where a
norm weight is involved: x * w when the weight is passed, w * Wt when it was
folded into the linear weight (np_fold_norm_weight); without a norm weight
both operands are the inputs themselves and nothing is rounded. The kernel
then accumulates the K products in fp32 in its own order and applies rstd,
bias and scale in fp32. Per element, with t_k = scale * rstd * a_k * Wt_nk:
  - fp32 evaluation: at most 2^-24 (K + 16) * cond, cond = sum_k |t_k|;
  - operand rounding: sum_k d_k t_k with independent |d_k| <= u (u = 2^-8 for
    bf16, 2^-11 for fp16, the unit roundoff of dt). Hoeffding's inequality
    bounds it by 7 u l2, l2 = sqrt(sum_k t_k^2), except with probability
    2 exp(-24.5) < 1e-10 per element (the worst case u * cond is true but
    about twenty times looser at K = 4096 and would let a dropped bias pass);
  - the final rounding: one ulp of dt.
Every element must lie within the sum. Elements beyond 2 ulp of the oracle's
rounded value are counted and printed for each path; on the path that rounds
no operand at least 99.5 % of the elements must equal the oracle's rounded
value bit for bit.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import ORACLE_DT, empty, need_gpu, to_dev, to_host
from tolerance import bf16_bits_to_f32, ordinal16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def npa():
    need_gpu()
    import norm_pass_amd
    norm_pass_amd.np_init(0)
    return norm_pass_amd


def _vals(bits, dt):
    return bf16_bits_to_f32(bits).astype(np.float64) if dt == "bf16" else \
        bits.view(np.float16).astype(np.float64)


def _ulp(v, dt):
    mant = 7 if dt == "bf16" else 10
    emin = -126 if dt == "bf16" else -14
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** emin)))
    return 2.0 ** (e - mant)


def _inputs(M, K, N, seed, dt):
    x = synth.normal((M, K), seed, dt)
    w = synth.normal((K,), seed + 1, dt, mean=1.0, std=0.1)
    Wt = synth.normal((N, K), seed + 2, dt, std=K ** -0.5)
    b = synth.normal((N,), seed + 3, dt, std=0.1)
    return x, w, Wt, b


UNIT_ROUNDOFF = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}


def _l2(x, w, Wt, scale, dt):
    """|scale| rstd_m sqrt(sum_k (x_mk w_k Wt_nk)^2): the size of the terms for
    the operand-rounding part of the tolerance."""
    xv = _vals(x, dt)
    wv = np.ones(xv.shape[1]) if w is None else _vals(w, dt)
    Wv = _vals(Wt.reshape(-1), dt).reshape(Wt.shape)
    rstd = 1.0 / np.sqrt((xv * xv).mean(axis=1, keepdims=True) + float(np.float32(1e-6)))
    return abs(scale) * rstd * np.sqrt(((xv * wv) ** 2) @ (Wv ** 2).T)


def _check(got, exact, cond, K, dt, want_bits=None, l2=None, what="", min_equal=0.995):
    """l2 given: one operand was rounded to dt (the norm-weight paths)."""
    g = _vals(got, dt)
    err = np.abs(g - exact)
    lim = _ulp(exact, dt) + 2.0 ** -24 * (K + 16) * cond
    if l2 is not None:
        lim = lim + 7.0 * UNIT_ROUNDOFF[dt] * l2
    bad = err > lim
    assert not bad.any(), (int(bad.sum()), float((err - lim).max()))
    if want_bits is not None:
        d = np.abs(ordinal16(got) - ordinal16(want_bits))
        print(f"[{what}] {dt}: {int((d > 2).sum())} of {d.size} elements beyond 2 ulp "
              f"({(d > 2).mean():.4%}), {(d == 0).mean():.4%} bit-equal", flush=True)
        if l2 is None:
            assert (d == 0).mean() >= min_equal, float((d == 0).mean())


CASES = [  # M, N, K (K a multiple of 64: the four-wave kernels; otherwise the eight-wave ones)
    (256, 256, 512), (300, 260, 520), (1, 1, 8), (129, 130, 72), (64, 384, 1024), (517, 33, 136),
    (513, 257, 192), (1, 8, 64), (300, 250, 128),
]


@pytest.mark.parametrize("M,N,K", CASES)
@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("with_w,with_b,scale", [(True, True, 0.5), (False, False, 1.0),
                                                 (True, False, -2.0)])
def test_fused_matches_oracle(npa, orc, M, N, K, dt, with_w, with_b, scale):
    x, w, Wt, b = _inputs(M, K, N, 4000 + M + N + K, dt)
    w = w if with_w else None
    b = b if with_b else None
    want, exact, cond = orc.rmsnorm_linear(x, w, Wt, b, 1e-6, scale, ORACLE_DT[dt],
                                           want_exact=True)
    out = empty((M, N), dt)
    npa.fuse_rmsnorm_linear(to_dev(x, dt), None if w is None else to_dev(w, dt), to_dev(Wt, dt),
                            None if b is None else to_dev(b, dt), out, 1e-6, scale)
    torch.cuda.synchronize()
    _check(to_host(out), exact, cond, K, dt, want_bits=want,
           l2=_l2(x, w, Wt, scale, dt) if with_w else None, what=f"fused {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(256, 256, 512), (300, 260, 520)])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_unfused_matches_oracle_eager(npa, orc, M, N, K, dt):
    x, w, Wt, b = _inputs(M, K, N, 5000 + M, dt)
    want, exact, cond = orc.rmsnorm_linear(x, w, Wt, b, 1e-6, 0.5, ORACLE_DT[dt], eager=True,
                                           want_exact=True)
    out = empty((M, N), dt)
    ws = torch.empty(npa.rmsnorm_linear_workspace_bytes(M, K), dtype=torch.uint8, device="cuda")
    npa.unfused_rmsnorm_linear(to_dev(x, dt), to_dev(w, dt), to_dev(Wt, dt), to_dev(b, dt), out,
                               ws, 1e-6, 0.5)
    torch.cuda.synchronize()
    # the unfused GEMM's operand y = round(x rstd w) is computed with the fp32
    # rstd of the RMSNorm kernel: a y element may round the other way than the
    # oracle's (one ulp of y), which moves the sum by up to 2^-8 of one term
    g = _vals(to_host(out), dt)
    lim = 2 * _ulp(exact, dt) + 2.0 ** -24 * (K + 16) * cond + 2.0 ** -8 * cond / np.sqrt(K)
    assert (np.abs(g - exact) <= lim).all()
    assert (to_host(out) == want).mean() > 0.98


def test_full_size_sampled_rows(npa, orc):
    """The bench's workload (bf16, M 16384, K 4096, N 4096) in the bench's
    launch, sampled rows (all their 4096 outputs) against the oracle."""
    M, K, N = 16384, 4096, 4096
    x, w, Wt, b = synth.rmsnorm_linear_inputs()
    out = empty((M, N), "bf16")
    npa.fuse_rmsnorm_linear(to_dev(x, "bf16"), to_dev(w, "bf16"), to_dev(Wt, "bf16"),
                            to_dev(b, "bf16"), out, 1e-6, synth.RMS_LINEAR_SCALE)
    torch.cuda.synchronize()
    rng = np.random.default_rng(17)
    rows = np.unique(np.concatenate([[0, 127, 128, M - 1], rng.integers(0, M, 12)]))
    want, exact, cond = orc.rmsnorm_linear(x[rows], w, Wt, b, 1e-6, synth.RMS_LINEAR_SCALE,
                                           ORACLE_DT["bf16"], want_exact=True)
    got = to_host(out[torch.from_numpy(rows).cuda()])
    _check(got, exact, cond, K, "bf16", want_bits=want,
           l2=_l2(x[rows], w, Wt, synth.RMS_LINEAR_SCALE, "bf16"), what="weight passed, full size")


def _oracle_fold(orc, w, Wt, dt):
    """round_dt(w_k Wt_nk): the product of two dt values is exact in float64."""
    wv = _vals(w, dt)
    Wv = _vals(Wt.reshape(-1), dt).reshape(Wt.shape)
    return orc.round_array(Wv * wv[None, :], ORACLE_DT[dt])


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_fold_norm_weight_bit_exact(npa, orc, dt):
    N, K = 96, 200
    _, w, Wt, _ = _inputs(1, K, N, 6100, dt)
    out = empty((N, K), dt)
    npa.np_fold_norm_weight(to_dev(w, dt), to_dev(Wt, dt), out)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(out), _oracle_fold(orc, w, Wt, dt))


# the direct-to-LDS kernels: no norm weight and K a multiple of 32 (the
# four-wave kernel when K is a multiple of 64, the eight-wave one otherwise);
# ragged M and N, and N not a multiple of 8 (element-wise output stores)
# no norm weight: K % 64 == 0 -> the register-staged four-wave kernel (1, 2, 3,
# 8 and 64 K steps: its prologue stages steps 0..2, clamped past the end);
# K % 32 == 0 otherwise -> the eight-wave direct-to-LDS kernel
NO_W_CASES = [(300, 260, 512), (33, 1000, 96), (517, 40, 64), (256, 512, 4096), (1, 8, 32),
              (1, 8, 64), (513, 257, 192), (300, 250, 128), (70, 30, 96)]


@pytest.mark.parametrize("M,N,K", NO_W_CASES)
@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("with_b", [True, False])
def test_no_norm_weight_paths_match_oracle(npa, orc, M, N, K, dt, with_b):
    x, w, Wt, b = _inputs(M, K, N, 6200 + M + N + K, dt)
    b = b if with_b else None
    want, exact, cond = orc.rmsnorm_linear(x, None, Wt, b, 1e-6, 0.75, ORACLE_DT[dt],
                                           want_exact=True)
    out = empty((M, N), dt)
    npa.fuse_rmsnorm_linear(to_dev(x, dt), None, to_dev(Wt, dt),
                            None if b is None else to_dev(b, dt), out, 1e-6, 0.75)
    torch.cuda.synchronize()
    _check(to_host(out), exact, cond, K, dt, want_bits=want, what=f"no norm weight {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(300, 260, 512), (129, 130, 96)])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_folded_matches_oracle(npa, orc, M, N, K, dt):
    """The norm weight folded into Wt (np_fold_norm_weight), then the
    direct-to-LDS kernel, against the oracle given x, w and the unfolded Wt."""
    x, w, Wt, b = _inputs(M, K, N, 6300 + M + N + K, dt)
    want, exact, cond = orc.rmsnorm_linear(x, w, Wt, b, 1e-6, 0.5, ORACLE_DT[dt],
                                           want_exact=True)
    Wf = empty((N, K), dt)
    npa.np_fold_norm_weight(to_dev(w, dt), to_dev(Wt, dt), Wf)
    out = empty((M, N), dt)
    npa.fuse_rmsnorm_linear(to_dev(x, dt), None, Wf, to_dev(b, dt), out, 1e-6, 0.5)
    torch.cuda.synchronize()
    _check(to_host(out), exact, cond, K, dt, want_bits=want, l2=_l2(x, w, Wt, 0.5, dt),
           what=f"folded {M}x{N}x{K}")


def test_folded_full_size_sampled_rows(npa, orc):
    """The bench's folded launch: the norm weight folded into Wt once, then the
    direct-to-LDS kernel on the 16384 x 4096 x 4096 workload; sampled rows
    against the oracle given x, w and the unfolded Wt."""
    M, K, N = synth.RMS_LINEAR_SHAPE
    x, w, Wt, b = synth.rmsnorm_linear_inputs()
    Wf = empty((N, K), "bf16")
    npa.np_fold_norm_weight(to_dev(w, "bf16"), to_dev(Wt, "bf16"), Wf)
    out = empty((M, N), "bf16")
    npa.fuse_rmsnorm_linear(to_dev(x, "bf16"), None, Wf, to_dev(b, "bf16"), out, 1e-6,
                            synth.RMS_LINEAR_SCALE)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(Wf), _oracle_fold(orc, w, Wt, "bf16"))
    rng = np.random.default_rng(23)
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], rng.integers(0, M, 12)]))
    want, exact, cond = orc.rmsnorm_linear(x[rows], w, Wt, b, 1e-6, synth.RMS_LINEAR_SCALE,
                                           ORACLE_DT["bf16"], want_exact=True)
    got = to_host(out[torch.from_numpy(rows).cuda()])
    _check(got, exact, cond, K, "bf16", want_bits=want,
           l2=_l2(x[rows], w, Wt, synth.RMS_LINEAR_SCALE, "bf16"), what="folded, full size")


def test_empty_and_rejects(npa):
    x = torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda")
    Wt = torch.zeros(32, 64, dtype=torch.bfloat16, device="cuda")
    out = torch.zeros(0, 32, dtype=torch.bfloat16, device="cuda")
    npa.fuse_rmsnorm_linear(x, None, Wt, None, out)  # M = 0: nothing to do
    x = torch.zeros(4, 64, dtype=torch.float32, device="cuda")
    with pytest.raises(npa.NPError):
        npa.fuse_rmsnorm_linear(x, None, Wt.float(), None, torch.zeros(4, 32, device="cuda"))
    xb = torch.zeros(4, 60, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(npa.NPError):  # K % 8 != 0
        npa.fuse_rmsnorm_linear(xb, None, torch.zeros(32, 60, dtype=torch.bfloat16,
                                                      device="cuda"),
                                None, torch.zeros(4, 32, dtype=torch.bfloat16, device="cuda"))
    buf = torch.zeros(4 * 64 + 8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(npa.NPError):  # misaligned x
        npa.fuse_rmsnorm_linear(buf[1:1 + 256].view(4, 64), None, Wt, None,
                                torch.zeros(4, 32, dtype=torch.bfloat16, device="cuda"))


@pytest.mark.parametrize("with_w", [False, True])
def test_deterministic(npa, with_w):
    """Two runs on the same inputs give bit-identical outputs (fixed MFMA and
    row-sum order; no atomics)."""
    M, N, K = 513, 257, 192
    x, w, Wt, b = _inputs(M, K, N, 7100, "bf16")
    outs = []
    for _ in range(2):
        out = empty((M, N), "bf16")
        npa.fuse_rmsnorm_linear(to_dev(x, "bf16"), to_dev(w, "bf16") if with_w else None,
                                to_dev(Wt, "bf16"), to_dev(b, "bf16"), out, 1e-6, 0.5)
        torch.cuda.synchronize()
        outs.append(to_host(out))
    assert np.array_equal(outs[0], outs[1])
