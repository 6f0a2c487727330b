"""Build libcg.so (host compiler + C ABI + gfx950 kernels) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libcg.so")
ARCH = os.environ.get("CG_OFFLOAD_ARCH", "gfx950")
SOURCES = ["compiler.cpp", "capi.cpp", "contract.cpp", "pda.hip", "sample.hip"]
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "--offload-arch=" + ARCH,
         # keep hipcc from emitting packed fp32 instructions
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc():
    for p in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if p and os.path.exists(p):
            return p
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(bdir, src + ".o")
        cmd = [cc] + FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=3) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    build_floor(cc, bdir)
    return OUT


def build_floor(cc: str, bdir: str) -> str:
    """libcg_floor.so: the bench's read-only reference kernel (read_floor.hip),
    a library of its own that libcg does not link."""
    out = os.path.join(HERE, "libcg_floor.so")
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [cc] + FLAGS + ["-shared", "-Wl,--no-undefined", "-x", "hip", os.path.join(CSRC, "read_floor.hip"),
                          "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on read_floor.hip:\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
