"""Pins for the oracle's Philox4x32-10 against the independent header-only
engine that ships in torch's C++ headers (compiled here as a test helper), and
for the statistics of its 16-bit draws."""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle

HELPER_SRC = r"""
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
#include <cstdlib>
// prints the four 32-bit outputs of counter (off_lo, off_hi, sub_lo, sub_hi), key = seed
int main(int argc, char** argv) {
  for (int i = 1; i + 2 < argc; i += 3) {
    unsigned long long seed = strtoull(argv[i], 0, 0), sub = strtoull(argv[i+1], 0, 0),
                       off = strtoull(argv[i+2], 0, 0);
    at::Philox4_32 e(seed, sub, off);
    unsigned a = e(), b = e(), c = e(), d = e();
    printf("%u %u %u %u\n", a, b, c, d);
  }
}
"""


@pytest.fixture(scope="module")
def torch_philox(tmp_path_factory):
    d = tmp_path_factory.mktemp("philox")
    src = d / "ph.cpp"
    src.write_text(HELPER_SRC)
    exe = d / "ph"
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    r = subprocess.run(["g++", "-std=c++17", "-O1", "-I", inc, str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("cannot compile torch's Philox header: " + r.stderr[-500:])

    def run(cases):
        args = []
        for seed, sub, off in cases:
            args += [str(seed), str(sub), str(off)]
        out = subprocess.run([str(exe)] + args, capture_output=True, text=True, check=True).stdout
        return [list(map(int, line.split())) for line in out.strip().splitlines()]
    return run


def test_philox_matches_torch_engine(torch_philox):
    g = np.random.default_rng(7)
    cases = [(0, 0, 0), (0, 1, 0), (0, 4, 0), (2**64 - 1, 2**32 - 1, 2**64 - 1), (123456789, 3, 17)]
    cases += [(int(g.integers(0, 2**63)), int(g.integers(0, 2**32)), int(g.integers(0, 2**63))) for _ in range(60)]
    ref = torch_philox(cases)
    for (seed, sub, off), r in zip(cases, ref):
        got = oracle.philox4x32_10([off & 0xFFFFFFFF, off >> 32, sub & 0xFFFFFFFF, sub >> 32],
                                   [seed & 0xFFFFFFFF, seed >> 32])
        assert got == r, (seed, sub, off)


def test_draw_u16_mapping(torch_philox):
    """Element i draws half (i & 1) of word (i >> 1) & 3 of counter i >> 3."""
    seed, stream = 0xDEADBEEF12345678, 3
    idx = [0, 1, 2, 3, 4, 5, 6, 7, 8, 15, 16, 2**35 + 5]
    ref = torch_philox([(seed, stream, i >> 3) for i in idx])
    for i, words in zip(idx, ref):
        want = (words[(i >> 1) & 3] >> (16 * (i & 1))) & 0xFFFF
        assert oracle.draw_u16(seed, stream, i) == want


def test_draw_u16_statistics():
    n = 1 << 16
    u = np.array([oracle.draw_u16(0, 1, i) for i in range(n)], dtype=np.float64)
    # uniform on [0, 65535]: mean 32767.5, sd 18918.6 -> 5 sigma of the mean
    assert abs(u.mean() - 32767.5) < 5 * 18918.6 / np.sqrt(n)
    bits = ((u.astype(np.int64)[:, None] >> np.arange(16)) & 1).mean(axis=0)
    assert np.all(np.abs(bits - 0.5) < 5 * 0.5 / np.sqrt(n))
    # streams are distinct sequences
    v = np.array([oracle.draw_u16(0, 2, i) for i in range(256)])
    assert not np.array_equal(u[:256], v)
