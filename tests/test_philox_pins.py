"""Philox4x32-10 of the oracle against PyTorch's independent Philox4_32
engine (its C++ header as installed, compiled here at test time)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from logit_masking_amd import workloads as W
from oracle import oracle as O

PROBE = r"""
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
#include <cstdlib>
int main(int argc, char** argv) {
  for (int a = 1; a + 2 < argc; a += 3) {
    unsigned long long seed = strtoull(argv[a], 0, 0), off = strtoull(argv[a + 1], 0, 0),
                       sub = strtoull(argv[a + 2], 0, 0);
    at::Philox4_32 e(seed, sub, off);   // key = seed, counter = (off lo, off hi, sub lo, sub hi)
    for (int i = 0; i < 4; i++) printf("%u\n", e());
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def torch_probe(tmp_path_factory):
    import torch
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    if not shutil.which("g++") or not os.path.exists(os.path.join(inc, "ATen/core/PhiloxRNGEngine.h")):
        pytest.skip("torch Philox header or g++ missing")
    d = tmp_path_factory.mktemp("philox")
    src = d / "probe.cpp"
    src.write_text(PROBE)
    exe = d / "probe"
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-I" + inc, str(src), "-o", str(exe)])
    return str(exe)


def test_against_torch_engine(torch_probe):
    rng = W.SplitMix(99)
    cases = []
    for _ in range(200):
        seed, j, step, lvl = rng.next(), rng.next() & 0xFFFFFFFF, rng.next() & 0xFFFFFFFF, rng.below(2)
        cases.append((seed, j, step, lvl))
    args = []
    for seed, j, step, lvl in cases:
        args += [str(seed), str(j | (step << 32)), str(lvl)]
    out = subprocess.check_output([torch_probe] + args).split()
    got = np.array([int(x) for x in out], dtype=np.uint64).reshape(-1, 4)
    for k, (seed, j, step, lvl) in enumerate(cases):
        mine = O.philox4x32_10(np.array([[j, step, lvl, 0]], dtype=np.uint64), (seed & 0xFFFFFFFF, seed >> 32))[0]
        assert [int(x) for x in mine] == [int(x) for x in got[k]]


def test_stream_layout():
    # element i of (seed, step, lvl) is word i & 3 of block (i >> 2, step, lvl, 0)
    seed = 0x0123456789ABCDEF
    ids = np.arange(12)
    w = O.philox_words(seed, 7, 1, ids)
    for i in ids:
        blk = O.philox4x32_10(np.array([[i >> 2, 7, 1, 0]], dtype=np.uint64), (seed & 0xFFFFFFFF, seed >> 32))[0]
        assert w[i] == blk[i & 3]


def test_uniform_words():
    w = O.philox_words(5, 3, 0, np.arange(200000))
    u = (w.astype(np.float64) + 0.5) / 2 ** 32
    assert abs(u.mean() - 0.5) < 0.005
    counts = np.bincount((u * 16).astype(int), minlength=16)
    e = len(u) / 16
    assert ((counts - e) ** 2 / e).sum() < 60
