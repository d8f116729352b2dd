"""Build libnorm_pass_amd.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libnorm_pass_amd.so")


def hipcc_command(out: str) -> list[str]:
    srcs = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")) +
                  glob.glob(os.path.join(PKG, "csrc", "*.cpp")))
    return ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
            "-shared", "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
            *srcs, "-lhiprtc", "-o", out]


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


def build(verbose: bool = False) -> str:
    write_generated()
    tmp = LIB + ".tmp"
    cmd = hipcc_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
