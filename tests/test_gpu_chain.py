"""GPU parity of fuse_chain / unfused_chain against the oracle (relu(a+b)*0.5 and
the seeded 29-op fp16 chain; DeepJIT write-up sections 3.2-4.2, NaiveRT write-up).

fp32 relu(a+b)*0.5 must match bit for bit (one correctly rounded add, an exact
max and an exact halving). fp16 chains must be within 2 fp16 ulps of the
oracle, except ill-conditioned elements that lie within the oracle's fp32
evaluation bound (counted; < 1e-4 of the elements).
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import ORACLE_DT, empty, misaligned, need_gpu, to_dev, to_host
from tolerance import check_f32_counted, check_half, half_values

pytestmark = pytest.mark.gpu

F32, F16 = 0, 1


@pytest.fixture(scope="module")
def npa():
    need_gpu()
    import norm_pass_amd
    norm_pass_amd.np_init(0)
    return norm_pass_amd


def _c1(npa, orc, n, fn="fuse_chain", align=True):
    a, b = synth.c1_inputs(n, seed=17 + n)
    ta, tb = to_dev(a, "f32"), to_dev(b, "f32")
    if not align:
        ta, tb = misaligned(ta), misaligned(tb)
    out = empty((n,), "f32")
    getattr(npa, fn)(synth.C1_CHAIN, [ta, tb], out)
    torch.cuda.synchronize()
    ref = orc.chain(synth.C1_CHAIN, [a, b], F32, eager=(fn == "unfused_chain"))
    return to_host(out), ref


@pytest.mark.parametrize("n", [1, 3, 5, 4097, 65537, 1 << 20])
@pytest.mark.parametrize("fn", ["fuse_chain", "unfused_chain"])
def test_c1_bit_exact(npa, orc, n, fn):
    got, ref = _c1(npa, orc, n, fn)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_c1_misaligned_scalar_path(npa, orc):
    got, ref = _c1(npa, orc, 1001, align=False)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_c1_special_values(npa, orc):
    a = np.array([1.0, -3.0, 2.5, -0.0, 2.0 ** -149, 3e38, -1e-45, 7.0], np.float32)
    b = np.array([2.0, 1.0, -2.5, -0.0, 2.0 ** -149, 3e38, 0.0, np.inf], np.float32)
    out = empty((8,), "f32")
    npa.fuse_chain(synth.C1_CHAIN, [to_dev(a, "f32"), to_dev(b, "f32")], out)
    ref = orc.chain(synth.C1_CHAIN, [a, b], F32)
    got = to_host(out)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert not np.signbit(got).any()


def test_c1_specialised_bit_exact(npa, orc):
    n = 1 << 20
    npa.fuse_chain_prepare(synth.C1_CHAIN, 2, npa.NP_F32, npa.NP_F32, n)
    try:
        got, ref = _c1(npa, orc, n)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
        got, ref = _c1(npa, orc, 4099)  # no specialisation for this n: generic kernel
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    finally:
        torch.cuda.synchronize()
        npa.np_shutdown()


def test_c1_deterministic_and_in_bounds(npa):
    n = 65537
    a, b = synth.c1_inputs(n, seed=3)
    ta, tb = to_dev(a, "f32"), to_dev(b, "f32")
    canary = torch.full((n + 64,), 12345.0, device="cuda")
    out = canary[16:16 + n]
    npa.fuse_chain(synth.C1_CHAIN, [ta, tb], out)
    first = out.clone()
    npa.fuse_chain(synth.C1_CHAIN, [ta, tb], out)
    torch.cuda.synchronize()
    assert torch.equal(first, out)
    assert (canary[:16] == 12345.0).all() and (canary[16 + n:] == 12345.0).all()


def _c5(npa, orc, x, ops, fn="fuse_chain", dt="f16"):
    tx = to_dev(x, dt)
    out = empty(tx.shape, dt)
    getattr(npa, fn)(ops, [tx], out)
    torch.cuda.synchronize()
    got = to_host(out)
    ref, exact, bound = orc.chain(ops, [x], ORACLE_DT[dt], in_dt=ORACLE_DT[dt],
                                  eager=(fn == "unfused_chain"), want_bound=True)
    return check_half(got, ref, dt, half_values(got, dt), exact, bound,
                      what=f"{fn} n={x.size}")


@pytest.mark.parametrize("fn", ["fuse_chain", "unfused_chain"])
def test_c5_small_full(npa, orc, fn):
    x = synth.c5_inputs(65536)
    stats = _c5(npa, orc, x, synth.c5_chain(), fn)
    assert stats["n"] == 65536


@pytest.mark.parametrize("n", [1, 7, 9, 1000, 65543, (1 << 19) + 8 * 3 + 5])
def test_c5_ragged(npa, orc, n):
    _c5(npa, orc, synth.c5_inputs(n, seed=n), synth.c5_chain())


def test_c5_large_sampled(npa, orc):
    n = 1 << 28
    x = synth.c5_inputs(n)
    tx = to_dev(x, "f16")
    out = empty((n,), "f16")
    npa.fuse_chain(synth.c5_chain(), [tx], out)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    idx = np.unique(np.concatenate([rng.integers(0, n, 1 << 20), np.arange(n - 4096, n),
                                    np.arange(4096)]))
    got = to_host(out[torch.from_numpy(idx).cuda()])
    ref, exact, bound = orc.chain(synth.c5_chain(), [x[idx]], F16, want_bound=True)
    check_half(got, ref, "f16", half_values(got, "f16"), exact, bound, what="c5 2^28 sampled")


KINDS = [(synth.EXP, 0.0), (synth.SIGMOID, 0.0), (synth.TANH, 0.0), (synth.ADD_C, 0.883171),
         (synth.MUL_C, -0.563752), (synth.SCALE, 0.483334), (synth.CAST_F16, 0.0),
         (synth.CAST_BF16, 0.0), (synth.RELU, 0.0)]


@pytest.mark.parametrize("kind,c", KINDS)
def test_one_op_exhaustive_fp16(npa, orc, kind, c):
    """Every finite fp16 input through a one-op chain (the small chain size is 2^16)."""
    bits = np.arange(65536, dtype=np.uint16)
    x = bits.view(np.float16)
    x = x[np.isfinite(x)]
    if kind == synth.EXP:
        x = x[x.astype(np.float64) < 11.0]  # exp beyond fp16 range is not a valid chain
    ops = [(synth.LOAD, 0, 0.0), (kind, 0, float(np.float32(c)))]
    _c5(npa, orc, x, ops)
    _c5(npa, orc, x, ops, "unfused_chain")


@pytest.mark.parametrize("seed", range(6))
def test_random_short_chains(npa, orc, seed):
    """Random chains over 1-3 inputs, all op kinds, fp16 / bf16 / fp32 storage."""
    rng = np.random.default_rng(seed)
    dt = ["f16", "bf16", "f32"][seed % 3]
    n_in = 1 + seed % 3
    n = int(rng.integers(1, 5000))
    xs = [synth.cast(synth.normal_f32(n, 100 + seed * 7 + j), dt) for j in range(n_in)]
    ops = [(synth.LOAD, 0, 0.0)]
    for _ in range(int(rng.integers(1, 12))):
        k = int(rng.choice([synth.ADD_IN, synth.MUL_IN, synth.ADD_C, synth.MUL_C, synth.SCALE,
                            synth.RELU, synth.SIGMOID, synth.TANH, synth.CAST_F16,
                            synth.CAST_BF16]))
        ops.append((k, int(rng.integers(0, n_in)), float(np.float32(rng.uniform(-1, 1)))))
    ops.append((synth.SIGMOID, 0, 0.0))
    tins = [to_dev(a, dt) for a in xs]
    out = empty((n,), dt)
    npa.fuse_chain(ops, tins, out)
    torch.cuda.synchronize()
    got = to_host(out)
    od = ORACLE_DT[dt]
    ref, exact, bound = orc.chain(ops, xs, od, in_dt=od, want_bound=True)
    if dt == "f32":
        stats = check_f32_counted(got, ref, exact, bound, what=f"seed {seed}")
        print(f"seed {seed} fp32: {stats}", flush=True)
    else:
        check_half(got, ref, dt, half_values(got, dt), exact, bound, what=f"seed {seed}")


def test_c5_specialised(npa, orc):
    """Runtime-specialised kernels: one element per thread (small n) and 16-byte groups."""
    ops = synth.c5_chain()
    npa.fuse_chain_prepare(ops, 1, npa.NP_F16, npa.NP_F16, 0)
    try:
        _c5(npa, orc, synth.c5_inputs(65536), ops)
        _c5(npa, orc, synth.c5_inputs(1031, seed=9), ops)
        _c5(npa, orc, synth.c5_inputs((1 << 20) + 5, seed=10), ops)
    finally:
        torch.cuda.synchronize()
        npa.np_shutdown()


@pytest.mark.parametrize("seed", range(1, 9))
def test_specialised_folds(npa, orc, seed):
    """fp16-output specialisation folds constant runs, multiply-add pairs and
    affine maps around exp into fewer instructions; every folded chain must
    still match the oracle (the unfolded definition) to the fp16 bar."""
    ops = synth.c5_chain(n_ops=12, seed=seed)
    src = npa.np_chain_source(ops, 1, npa.NP_F16, npa.NP_F16, 0)
    body = src[src.index("float chain("):src.index("return v;")]
    assert body.count("\n  v = ") < len(ops)  # something was folded
    npa.fuse_chain_prepare(ops, 1, npa.NP_F16, npa.NP_F16, 0)
    try:
        _c5(npa, orc, synth.c5_inputs(65536, seed=seed), ops)
        _c5(npa, orc, synth.c5_inputs((1 << 20) + 3, seed=seed + 50), ops)
    finally:
        torch.cuda.synchronize()
        npa.np_shutdown()


@pytest.mark.parametrize("seed", [29, 200, 201, 202, 203, 204, 205])
def test_specialised_every_fp16_input(npa, orc, seed):
    """Every fp16 input that is not NaN (both zeros, subnormals, the largest
    finite values, both infinities) through a specialised 29-op chain: the
    tanh forms chosen from the argument ranges and the folded exps must hold
    over the whole input domain, not only over the workload's N(0, 1) draws."""
    ops = synth.c5_chain(n_ops=29, seed=seed)
    x = np.arange(1 << 16, dtype=np.uint16).view(np.float16)
    x = x[~np.isnan(x)]
    npa.fuse_chain_prepare(ops, 1, npa.NP_F16, npa.NP_F16, 0)
    try:
        _c5(npa, orc, x, ops)
    finally:
        torch.cuda.synchronize()
        npa.np_shutdown()


RARE_FORMS = [
    # tanh of an argument >= 1 (exp then + 1): the exponential form, no branch
    ([(synth.LOAD, 0, 0.0), (synth.EXP, 0, 0.0), (synth.ADD_C, 0, 1.0), (synth.TANH, 0, 0.0)],
     "np_fast_tanh_exp_pos(", True),
    # tanh of an argument <= -0.7 (-exp - 0.7): the negative exponential form
    ([(synth.LOAD, 0, 0.0), (synth.EXP, 0, 0.0), (synth.MUL_C, 0, -1.0), (synth.ADD_C, 0, -0.7),
      (synth.TANH, 0, 0.0)], "np_fast_tanh_exp_neg(", True),
    # an exp whose following factor is zero keeps the plain scaled form
    ([(synth.LOAD, 0, 0.0), (synth.EXP, 0, 0.0), (synth.MUL_C, 0, 0.0), (synth.ADD_C, 0, 0.5),
      (synth.TANH, 0, 0.0)], "np_fast_exp_affine(", False),
]


@pytest.mark.parametrize("case", range(len(RARE_FORMS)))
def test_specialised_rare_forms(npa, orc, case):
    """Forms the seeded chains seldom produce: each hand-made chain must
    generate the named form and match the oracle (every non-NaN fp16 input
    where the chain's output is finite for all of them, N(0, 1) draws
    otherwise)."""
    ops, form, every_input = RARE_FORMS[case]
    src = npa.np_chain_source(ops, 1, npa.NP_F16, npa.NP_F16, 0)
    assert form in src[src.index("float chain("):src.index("return v;")]
    if every_input:
        x = np.arange(1 << 16, dtype=np.uint16).view(np.float16)
        x = x[~np.isnan(x)]
    else:
        x = synth.c5_inputs(65536 + 7, seed=77)
    npa.fuse_chain_prepare(ops, 1, npa.NP_F16, npa.NP_F16, 0)
    try:
        _c5(npa, orc, x, ops)
    finally:
        torch.cuda.synchronize()
        npa.np_shutdown()


@pytest.mark.parametrize("in_dt,out_dt", [("f16", "f16"), ("bf16", "bf16"), ("f16", "bf16"),
                                          ("bf16", "f16")])
def test_table_path_equals_per_element_path(npa, in_dt, out_dt):
    """A specialised chain over one 16-bit input with a 16-bit output runs from
    its table once n reaches the threshold: every input bit pattern (NaNs
    included) must give the same output bits as the per-element kernel."""
    DT = {"f16": npa.NP_F16, "bf16": npa.NP_BF16}
    ops = synth.c5_chain()
    n = (1 << 22) + 13  # the table path, with a ragged tail
    pats = np.tile(np.arange(1 << 16, dtype=np.uint16), n // (1 << 16) + 1)[:n]
    x = torch.from_numpy(pats.view(np.int16)).cuda()
    x = x.view(torch.float16 if in_dt == "f16" else torch.bfloat16)
    npa.fuse_chain_prepare(ops, 1, DT[in_dt], DT[out_dt], 0)
    old = npa.np_set_chain_table_min(-1)
    try:
        outs = []
        for thr in (1 << 22, 1 << 62):  # table, then per element
            npa.np_set_chain_table_min(thr)
            out = empty((n,), out_dt)
            npa.fuse_chain(ops, [x], out)
            torch.cuda.synchronize()
            outs.append(to_host(out).view(np.uint16))
    finally:
        npa.np_set_chain_table_min(old)
        torch.cuda.synchronize()
        npa.np_shutdown()
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("n", [1 << 22, (1 << 22) + 1, (1 << 22) + 7 * 512 * 256 * 8 + 3,
                               (1 << 22) + 8 * (2048 * 37 + 1000) + 5])
def test_table_path_edges_and_in_place(npa, n):
    """The table path (blocks of 2048 16-byte vectors dealt round-robin to one
    workgroup per CU) at the threshold itself (one whole block per workgroup
    on 256 CUs), with a one-element tail, with block counts that leave some
    workgroups one block more than others, with 1000 vectors after the last
    whole block and five elements after the last vector, and in place (out is
    the input): the same bits as the per-element kernel out of place."""
    ops = synth.c5_chain()
    x = synth.c5_inputs(n, seed=n % 1000)
    npa.fuse_chain_prepare(ops, 1, npa.NP_F16, npa.NP_F16, 0)
    old = npa.np_set_chain_table_min(-1)
    try:
        npa.np_set_chain_table_min(1 << 62)
        ref = empty((n,), "f16")
        npa.fuse_chain(ops, [to_dev(x, "f16")], ref)
        npa.np_set_chain_table_min(1 << 22)
        inplace = to_dev(x, "f16")
        npa.fuse_chain(ops, [inplace], inplace)
        torch.cuda.synchronize()
    finally:
        npa.np_set_chain_table_min(old)
        torch.cuda.synchronize()
        npa.np_shutdown()
    assert np.array_equal(to_host(inplace), to_host(ref))


def test_c5_large_sampled_specialised(npa, orc):
    """The bench's launch: the prepared (folded) kernel on 2^28 elements,
    sampled outputs against the oracle."""
    n = 1 << 28
    ops = synth.c5_chain()
    x = synth.c5_inputs(n)
    tx = to_dev(x, "f16")
    out = empty((n,), "f16")
    npa.fuse_chain_prepare(ops, 1, npa.NP_F16, npa.NP_F16, 0)
    try:
        npa.fuse_chain(ops, [tx], out)
        torch.cuda.synchronize()
    finally:
        npa.np_shutdown()
    rng = np.random.default_rng(1)
    idx = np.unique(np.concatenate([rng.integers(0, n, 1 << 20), np.arange(n - 4096, n),
                                    np.arange(4096)]))
    got = to_host(out[torch.from_numpy(idx).cuda()])
    ref, exact, bound = orc.chain(ops, [x[idx]], F16, want_bound=True)
    check_half(got, ref, "f16", half_values(got, "f16"), exact, bound,
               what="c5 2^28 sampled, specialised")


def test_empty_launches(npa):
    npa.np_empty_launches(29)
    torch.cuda.synchronize()
