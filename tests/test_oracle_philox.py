"""Pins for the oracle's Philox4x32-10 (Salmon et al., SC'11).

The absolute pin is rocRAND's independent header-only implementation of the
same generator, compiled for the host with g++ at test time; the statistical
pins check the derived uniforms and child indices."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import philox

ROCRAND_HDR = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"

_PROG = r"""
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
#include <cstdlib>
// For each line "k0 k1 c0 c1 c2 c3" print the 4 output words of ten rounds.
int main() {
  unsigned long long k0, k1, c0, c1, c2, c3;
  while (std::scanf("%llu %llu %llu %llu %llu %llu", &k0, &k1, &c0, &c1, &c2, &c3) == 6) {
    unsigned long long seed = k0 | (k1 << 32);
    unsigned long long sub = c2 | (c3 << 32);
    unsigned long long x = c0 | (c1 << 32);
    rocrand_device::philox4x32_10_engine e(seed, sub, 0);
    while (x > 0) {  // advance by 4*x words in steps that do not overflow
      unsigned long long step = x < (1ull << 60) ? x : (1ull << 60);
      e.discard(4ull * step);
      x -= step;
    }
    unsigned a = e(), b = e(), c = e(), d = e();
    std::printf("%u %u %u %u\n", a, b, c, d);
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def rocrand_prog(tmp_path_factory):
    if not os.path.exists(ROCRAND_HDR) or shutil.which("g++") is None:
        pytest.skip("rocRAND header or g++ not available")
    d = tmp_path_factory.mktemp("rr")
    src = d / "rr.cpp"
    src.write_text(_PROG)
    exe = d / "rr"
    subprocess.run(["g++", "-O1", "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", str(src),
                    "-o", str(exe)], check=True, capture_output=True)
    return str(exe)


def test_against_rocrand(rocrand_prog):
    rng = np.random.default_rng(123)
    cases = [(0, 0, 0, 0, 0, 0), (0xFFFFFFFF,) * 6, (1, 2, 3, 4, 5, 6)]
    for _ in range(300):
        cases.append(tuple(int(x) for x in rng.integers(0, 2**32, size=6, dtype=np.uint64)))
    # the counters the verifier uses: (64*slot + round, request, offset_lo, offset_hi)
    for slot in (0, 1, 64):
        for rnd in (0, 1, 63):
            cases.append((2002, 0, 64 * slot + rnd, 7, 0, 0))
    inp = "\n".join(" ".join(str(v) for v in c) for c in cases) + "\n"
    res = subprocess.run([rocrand_prog], input=inp, capture_output=True, text=True, check=True)
    lines = res.stdout.strip().split("\n")
    assert len(lines) == len(cases)
    for c, line in zip(cases, lines):
        want = tuple(int(x) for x in line.split())
        got = philox.philox4x32_10(c[2:], c[:2])
        assert got == want, (c, got, want)


def test_words_counter_layout():
    seed, offset = (5 << 32) | 9, (3 << 32) | 11
    w = philox.words(seed, offset, request=4, node_slot=2, rnd=5)
    assert w == philox.philox4x32_10((64 * 2 + 5, 4, 11, 3), (9, 5))


def test_uniform_range_and_chi2():
    n = 40000
    us = np.array([philox.unit_open0(philox.philox4x32_10((i, 1, 2, 3), (17, 0))[1]) for i in range(n)])
    assert us.min() > 0.0 and us.max() <= 1.0
    # exact 24-bit grid
    assert np.all((us * 2**24) == np.round(us * 2**24))
    counts, _ = np.histogram(us, bins=64, range=(0.0, 1.0))
    chi2 = ((counts - n / 64) ** 2 / (n / 64)).sum()
    assert chi2 < 120.0          # 63 dof; p ~ 3e-5


def test_pick_index_uniform():
    for m in (1, 2, 3, 5, 8, 64):
        idx = [philox.pick_index(philox.philox4x32_10((i, 0, 0, 0), (3, 4))[0], m) for i in range(6000)]
        assert min(idx) >= 0 and max(idx) < m
        counts = np.bincount(idx, minlength=m)
        exp = 6000 / m
        assert ((counts - exp) ** 2 / exp).sum() < 3 * m + 30


def test_unit_extremes():
    assert philox.unit_open0(0) == 2.0 ** -24
    assert philox.unit_open0(0xFFFFFFFF) == 1.0
    assert philox.pick_index(0xFFFFFFFF, 7) == 6
    assert philox.pick_index(0, 7) == 0
