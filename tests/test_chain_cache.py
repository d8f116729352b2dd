"""The disk cache of specialised code objects, host side (no GPU needed).

DeepJIT write-up, section 6.2: the compiled output is kept on disk so that a
restarted process skips compilation. np_chain_compile compiles without a GPU
and, when NP_CACHE_DIR is set, stores the code object there; these tests
check that nothing is written without NP_CACHE_DIR, the file format (magic,
the key text ending in the generated source, the code object), that a file's
name depends on the chain alone, and that concurrent writers leave whole files
and no temporaries. Loading from the cache is checked on the GPU
(tests/test_gpu_chain_cache.py).
"""
import os
import struct
import threading

import pytest

import synth

F16 = 1


@pytest.fixture(scope="module")
def npa():
    import norm_pass_amd
    return norm_pass_amd


@pytest.fixture
def cache_env(tmp_path, monkeypatch):
    d = tmp_path / "a" / "b"
    monkeypatch.setenv("NP_CACHE_DIR", str(d))
    return d


def files(d):
    return sorted(os.listdir(d)) if os.path.isdir(d) else []


def read_entry(path):
    raw = open(path, "rb").read()
    assert raw[:8] == b"NPCHAIN1"
    klen = struct.unpack("<Q", raw[8:16])[0]
    key = raw[16:16 + klen].decode()
    clen = struct.unpack("<Q", raw[16 + klen:24 + klen])[0]
    code = raw[24 + klen:]
    assert len(code) == clen
    return key, code


def test_nothing_written_without_cache_dir(npa, tmp_path, monkeypatch):
    monkeypatch.delenv("NP_CACHE_DIR", raising=False)
    monkeypatch.chdir(tmp_path)
    before = npa.np_chain_cache_stats()
    npa.np_chain_compile(synth.C1_CHAIN, 2, npa.NP_F32, npa.NP_F32, 0)
    assert npa.np_chain_cache_stats() == before
    assert files(tmp_path) == []


def test_compile_stores_one_whole_file(npa, cache_env):
    ops = synth.c5_chain()
    before = npa.np_chain_cache_stats()
    ms, nbytes = npa.np_chain_compile(ops, 1, F16, F16, 0)
    after = npa.np_chain_cache_stats()
    assert after["stores"] == before["stores"] + 1 and after["loads"] == before["loads"]
    names = files(cache_env)
    assert len(names) == 1 and names[0].endswith(".npco") and len(names[0]) == 16 + 5
    key, code = read_entry(cache_env / names[0])
    assert key.startswith("hiprtc ") and "--offload-arch=gfx950" in key.splitlines()[0]
    assert key.endswith(npa.np_chain_source(ops, 1, F16, F16, 0))
    assert len(code) == nbytes > 0
    assert code[:4] == b"\x7fELF" or code.startswith(b"__CLANG_OFFLOAD_BUNDLE__")


def test_file_name_follows_the_chain(npa, cache_env):
    ops = synth.c5_chain()
    npa.np_chain_compile(ops, 1, F16, F16, 0)
    first = files(cache_env)
    npa.np_chain_compile(ops, 1, F16, F16, 0)  # same chain: the same file, rewritten
    assert files(cache_env) == first
    npa.np_chain_compile(ops, 1, F16, F16, 65536)  # the size is written into the source
    npa.np_chain_compile(synth.C1_CHAIN, 2, npa.NP_F32, npa.NP_F32, 0)
    assert len(files(cache_env)) == 3


def test_concurrent_writers_leave_whole_files(npa, cache_env):
    ops = synth.c5_chain(n_ops=12, seed=301)
    errs = []

    def work():
        try:
            npa.np_chain_compile(ops, 1, F16, F16, 0)
        except Exception as e:  # noqa: BLE001 - reported below
            errs.append(e)
    ts = [threading.Thread(target=work) for _ in range(4)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errs
    names = files(cache_env)
    assert len(names) == 1 and not any(".tmp." in n for n in names)
    key, code = read_entry(cache_env / names[0])
    assert key.endswith(npa.np_chain_source(ops, 1, F16, F16, 0)) and len(code) > 0
