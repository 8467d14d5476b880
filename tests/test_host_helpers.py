"""Host-side helpers of the HIP library, checked on the CPU."""
from __future__ import annotations

import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "grouped_convolution_amd", "csrc")

FASTDIV_TEST = r"""
#include <cstdio>
#include <cstdint>
#include <random>
#include "fastdiv.h"
using namespace gconv;
int main() {
    std::mt19937_64 rng(7);
    long bad = 0, n_checked = 0;
    // every divisor up to 4096 against edge and random numerators,
    // plus random divisors up to 2^31 - 1
    auto check = [&](uint32_t d, uint32_t n) {
        FastDiv f = make_fastdiv(d);
        if (fastdiv(n, f) != n / d) { if (bad < 10) printf("d=%u n=%u\n", d, n); ++bad; }
        ++n_checked;
    };
    for (uint32_t d = 1; d <= 4096; ++d) {
        for (uint32_t n = 0; n < 3 * d + 5; ++n) check(d, n);
        for (int k = 0; k < 200; ++k) check(d, (uint32_t)(rng() % 0x80000000u));
        check(d, 0x7fffffffu); check(d, 0x7ffffffeu);
    }
    for (int k = 0; k < 200000; ++k) {
        uint32_t d = 1 + (uint32_t)(rng() % 0x7fffffffu);
        check(d, (uint32_t)(rng() % 0x80000000u));
        check(d, d); check(d, d - 1); check(d, 0x7fffffffu);
    }
    printf("%ld checked, %ld bad\n", n_checked, bad);
    return bad != 0;
}
"""


def test_fastdiv_matches_integer_division(tmp_path):
    src = tmp_path / "fd.cpp"
    src.write_text(FASTDIV_TEST)
    exe = tmp_path / "fd"
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
