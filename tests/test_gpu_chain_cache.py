"""The disk cache of specialised code objects on the GPU (DeepJIT write-up,
section 6.2: a restarted process loads the compiled code from disk instead of
compiling).

With NP_CACHE_DIR set, the first fuse_chain_prepare compiles and stores the
code object; after np_shutdown (which drops every loaded module, as a restart
would) the next prepare of the same chain loads it from disk, and the chain's
outputs are the same bits. A file that does not hold this chain's code -- a
different key text, a truncated file, or a well-formed entry whose code object
the runtime cannot load -- is rejected, the chain is compiled again and the
file rewritten, with the same outputs. Both the per-element kernel and the
table gather of the prepared module are exercised.
"""
import os
import struct

import numpy as np
import pytest
import torch

import synth
from gpu_util import empty, need_gpu, to_dev, to_host

pytestmark = pytest.mark.gpu

F16 = 1
SIZES = (1 << 20, (1 << 22) + 5)  # per-element vector kernel; table gather


@pytest.fixture(scope="module")
def npa():
    need_gpu()
    import norm_pass_amd
    norm_pass_amd.np_init(0)
    return norm_pass_amd


@pytest.fixture
def cache_env(tmp_path, monkeypatch):
    monkeypatch.delenv("NP_DISABLE_RTC", raising=False)
    monkeypatch.setenv("NP_CACHE_DIR", str(tmp_path / "cache"))
    return tmp_path / "cache"


def run_prepared(npa, ops):
    """Prepare (compile or load), run at both sizes, drop the modules."""
    npa.fuse_chain_prepare(ops, 1, F16, F16, 0)
    outs = []
    try:
        for n in SIZES:
            x = to_dev(synth.c5_inputs(n, seed=n % 997), "f16")
            out = empty((n,), "f16")
            npa.fuse_chain(ops, [x], out)
            torch.cuda.synchronize()
            outs.append(to_host(out))
    finally:
        torch.cuda.synchronize()
        npa.np_shutdown()
    return outs


def only_file(d):
    names = [n for n in os.listdir(d) if n.endswith(".npco")]
    assert len(names) == 1, names
    return d / names[0]


def delta(a, b):
    return {k: b[k] - a[k] for k in a}


def test_restart_loads_from_disk(npa, cache_env):
    ops = synth.c5_chain()
    s0 = npa.np_chain_cache_stats()
    first = run_prepared(npa, ops)
    s1 = npa.np_chain_cache_stats()
    assert delta(s0, s1) == {"loads": 0, "stores": 1, "rejects": 0}
    again = run_prepared(npa, ops)
    assert delta(s1, npa.np_chain_cache_stats()) == {"loads": 1, "stores": 0, "rejects": 0}
    for a, b in zip(first, again):
        assert np.array_equal(a, b)


def _rewrite(path, key_edit=None, truncate=False, code=None):
    raw = open(path, "rb").read()
    klen = struct.unpack("<Q", raw[8:16])[0]
    key = raw[16:16 + klen]
    body = raw[24 + klen:]
    if key_edit is not None:
        key = key_edit(key)
    if code is not None:
        body = code
    new = raw[:8] + struct.pack("<Q", len(key)) + key + struct.pack("<Q", len(body)) + body
    if truncate:
        new = new[:len(new) // 2]
    open(path, "wb").write(new)


@pytest.mark.parametrize("damage", ["other key", "truncated", "unloadable code"])
def test_unusable_file_is_recompiled(npa, cache_env, damage):
    ops = synth.c5_chain(n_ops=12, seed=302)
    ref = run_prepared(npa, ops)
    path = only_file(cache_env)
    good = open(path, "rb").read()
    if damage == "other key":  # same length, one byte of the source changed
        _rewrite(path, key_edit=lambda k: k[:-2] + (b"#" if k[-2:-1] != b"#" else b"$") + k[-1:])
    elif damage == "truncated":
        _rewrite(path, truncate=True)
    else:  # a well-formed entry whose code object is plain text, not an ELF image
        _rewrite(path, code=b"not a code object " * 64)
    s0 = npa.np_chain_cache_stats()
    got = run_prepared(npa, ops)
    assert delta(s0, npa.np_chain_cache_stats()) == {"loads": 0, "stores": 1, "rejects": 1}
    assert open(path, "rb").read() == good  # rewritten with the freshly compiled object
    for a, b in zip(ref, got):
        assert np.array_equal(a, b)
