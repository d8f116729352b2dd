"""Build libnorm_pass_amd.so in-tree with hipcc for gfx950.

Each source compiles to an object in norm_pass_amd/_build/ (in parallel),
then hipcc links the shared library. Every call compiles every source."""
from __future__ import annotations

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libnorm_pass_amd.so")
OBJ_DIR = os.path.join(PKG, "_build")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")) +
                  glob.glob(os.path.join(PKG, "csrc", "*.cpp")))


def compile_command(src: str, obj: str) -> list[str]:
    return ["/opt/rocm/bin/hipcc", *FLAGS, "-I", os.path.join(ROOT, "include"),
            "-I", os.path.join(PKG, "csrc"), "-c", src, "-o", obj]


def link_command(objs: list[str], out: str) -> list[str]:
    return ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *objs,
            "-lhiprtc", "-o", out]


def write_generated() -> None:
    """csrc/gen_fastmath.inc: fastmath.h as a C++ raw string literal, so that
    runtime-specialised kernels contain exactly the library's device functions."""
    src = open(os.path.join(PKG, "csrc", "fastmath.h")).read()
    assert ")NPFM\"" not in src
    text = 'R"NPFM(' + src + ')NPFM"\n'
    path = os.path.join(PKG, "csrc", "gen_fastmath.inc")
    if not os.path.exists(path) or open(path).read() != text:
        with open(path, "w") as f:
            f.write(text)


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


def build(verbose: bool = False, jobs: int | None = None) -> str:
    write_generated()
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(OBJ_DIR, os.path.basename(s) + ".o") for s in srcs]
    jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as pool:
        list(pool.map(lambda so: _run(compile_command(*so), verbose), zip(srcs, objs)))
    tmp = LIB + ".tmp"
    _run(link_command(objs, tmp), verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
