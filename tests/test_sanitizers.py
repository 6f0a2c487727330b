"""CPU: the library's host paths (spec compiler, table walker, contract
transform, evaluators) and the oracle's recognizer built with
AddressSanitizer and UBSan (host code only: hipcc takes each -fsanitize=
after -Xarch_host), then driven by tests/sanitize_run.py in a child process
with the sanitizer runtime preloaded: page examples, the recursive-JSON pins,
tiny languages, random walks on small vocabularies and mutated specs.  Any
sanitizer report ends the child with an error (halt_on_error).
"""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "logit_masking_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
RUNTIME = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG) and RUNTIME),
                                reason="needs ROCm's clang and its sanitizer runtime")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, (cmd, r.stderr[-3000:])


def test_host_paths_under_sanitizers(tmp_path):
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-shared-libsan"]
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + san
    srcs = ["compiler.cpp", "capi.cpp", "contract.cpp", "pda.hip", "sample.hip"]
    objs = [str(tmp_path / (s + ".o")) for s in srcs]
    with ThreadPoolExecutor(max_workers=5) as ex:
        list(ex.map(_run, [[HIPCC] + flags + ["-x", "hip", "-c", os.path.join(CSRC, s), "-o", o]
                           for s, o in zip(srcs, objs)]))
    # host link with clang++ (each object carries its own device code)
    lib = str(tmp_path / "libcg_san.so")
    _run([CLANGXX, "-shared", "-fPIC", "-shared-libsan", "-fsanitize=address,undefined", "-o", lib] + objs +
         ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    rec = str(tmp_path / "recognizer_san.so")
    _run([CLANG, "-std=gnu11", "-O1", "-g", "-fsanitize=address,undefined", "-shared-libsan",
          "-fno-omit-frame-pointer", "-shared", "-fPIC", "-o", rec, os.path.join(ROOT, "oracle", "recognizer.c"),
          "-lpthread"])
    env = dict(os.environ, LD_PRELOAD=RUNTIME[-1], ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitize_run.py"), lib, rec],
                       capture_output=True, text=True, env=env, timeout=900)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-6000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-6000:]
    assert "sanitized runs ok" in r.stdout
