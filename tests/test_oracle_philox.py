"""Pins of the oracle's uniform stream (Philox4x32-10 and the 24-bit uniform).

The pages fix no random-number convention; the oracle uses Philox4x32-10
(Salmon et al., SC'11) with key = seed and counter = (k, request, round_lo,
round_hi).  Pinned against (a) the published known-answer blocks and (b) an
independent implementation: ATen's header-only Philox engine, whose
(seed, subsequence, offset) constructor sets exactly that counter layout.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
from scipy import stats

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def test_known_answer_blocks():
    n = 0
    for line in open(GOLD):
        if line.startswith("#") or not line.strip():
            continue
        w = [int(t, 16) for t in line.split()]
        ctr, key, want = w[0:4], w[4:6], w[6:10]
        got = oracle.philox(np.array(ctr, np.uint32), np.array(key, np.uint32))
        assert [int(x) for x in got] == want
        n += 1
    assert n == 3


_ATEN_PROBE = r"""
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
int main() {
  unsigned long long seed, round; unsigned req, k;
  while (std::scanf("%llu %llu %u %u", &seed, &round, &req, &k) == 4) {
    at::philox_engine e(seed, round, ((unsigned long long)req << 32) | k);
    unsigned a = e(), b = e(), c = e(), d = e();
    std::printf("%u %u %u %u\n", a, b, c, d);
  }
  return 0;
}
"""


def test_matches_aten_philox_engine():
    torch_ext = pytest.importorskip("torch.utils.cpp_extension")
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    inc = []
    for p in torch_ext.include_paths():
        inc += ["-I", p]
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "probe.cpp")
        exe = os.path.join(d, "probe")
        open(src, "w").write(_ATEN_PROBE)
        subprocess.run(["g++", "-std=c++17", "-O1", *inc, src, "-o", exe], check=True)
        rng = np.random.default_rng(7)
        cases = [(1, 0, 0, 1), (2**64 - 1, 2**64 - 1, 2**31 - 1, 2**31 - 1), (0, 0, 0, 0)]
        for _ in range(2000):
            cases.append((int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2)),
                          int(rng.integers(0, 2**40)), int(rng.integers(0, 2**31)),
                          int(rng.integers(0, 64))))
        inp = "\n".join("%d %d %d %d" % c for c in cases) + "\n"
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        lines = out.strip().split("\n")
        assert len(lines) == len(cases)
        for c, line in zip(cases, lines):
            want = [int(t) for t in line.split()]
            got = [int(t) for t in oracle.draw(c[0], c[1], c[2], c[3])]
            assert got == want, c


def test_u24_range_and_resolution():
    assert oracle.u24(0) == 0.0
    assert oracle.u24(0xFFFFFFFF) == 1.0 - 2.0 ** -24
    assert oracle.u24(0x000000FF) == 0.0           # low 8 bits dropped
    assert oracle.u24(0x00000100) == 2.0 ** -24


def test_uniformity_chi_square():
    # 2^16 draws of word 0 over k = 1..4 requests, binned into 64 cells
    us = []
    for req in range(4096):
        for k in range(1, 5):
            w = oracle.draw(1, 0, req, k)
            us.extend(oracle.u24(int(x)) for x in w)
    counts = np.histogram(us, bins=64, range=(0.0, 1.0))[0]
    p = stats.chisquare(counts).pvalue
    assert p > 1e-4
