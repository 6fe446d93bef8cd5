"""Host test of the multiply-shift division that splits a launch's workgroup
index (gdr_fastdiv.h): with the constants make_fastdiv computes, the formula
the kernels apply, q = (mulhi(x, mul) + x) >> shift, equals x / d for
non-negative x below 2^31.  A small C++ program (g++, the header only)
checks every divisor up to 1,024, powers of two and their neighbours, and
seeded random divisors below 2^31: all x below 2^16, every x within one of a
multiple of d (all multiples for d >= 2,048, a seeded sample below), and the
last 2^16 values below 2^31."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_loop_amd", "csrc")

CHECKER = r"""
#include "gdr_fastdiv.h"
#include <cstdint>
#include <cstdio>
#include <vector>

static uint64_t calls = 0;
static bool check(uint32_t d, gdr::FastDiv f, uint32_t x) {
    ++calls;
    const uint64_t hi = (static_cast<uint64_t>(x) * f.mul) >> 32;
    const uint64_t sum = hi + x;
    if (sum >> 32) { std::printf("overflow d=%u x=%u\n", d, x); return false; }
    const uint32_t q = static_cast<uint32_t>(sum) >> f.shift;
    if (q != x / d) { std::printf("d=%u x=%u got %u want %u\n", d, x, q, x / d); return false; }
    return true;
}

int main() {
    const uint32_t kTop = 0x80000000u;  // x < 2^31
    std::vector<uint32_t> ds;
    for (uint32_t d = 1; d <= 1024; ++d) ds.push_back(d);
    for (int k = 11; k <= 30; ++k) {
        ds.push_back((1u << k) - 1); ds.push_back(1u << k); ds.push_back((1u << k) + 1);
    }
    ds.push_back(kTop - 1);
    uint64_t s = 0x9E3779B97F4A7C15ull;  // splitmix64, fixed seed
    for (int i = 0; i < 200; ++i) {
        s += 0x9E3779B97F4A7C15ull;
        uint64_t z = s;
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        z ^= z >> 31;
        ds.push_back(static_cast<uint32_t>(z % (kTop - 1)) + 1);
    }
    for (uint32_t d : ds) {
        const gdr::FastDiv f = gdr::make_fastdiv(d);
        for (uint32_t x = 0; x < (1u << 16); ++x)
            if (!check(d, f, x)) return 1;
        for (uint32_t x = kTop - (1u << 16); x < kTop; ++x)
            if (!check(d, f, x)) return 1;
        const uint64_t mults = (kTop - 1) / d;
        const uint64_t step = mults > (1u << 16) ? mults / (1u << 16) : 1;
        for (uint64_t k = 1; k <= mults; k += step) {
            const uint64_t m = k * d;
            for (uint64_t x = m - 1; x <= m + 1 && x < kTop; ++x)
                if (!check(d, f, static_cast<uint32_t>(x))) return 1;
        }
    }
    std::printf("ok %zu divisors, %llu checks\n", ds.size(), static_cast<unsigned long long>(calls));
    return 0;
}
"""


def test_fastdiv_exact(tmp_path):
    src = tmp_path / "fastdiv_check.cpp"
    exe = tmp_path / "fastdiv_check"
    src.write_text(CHECKER)
    build = subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", "-I", CSRC, str(src), "-o", str(exe)],
                           capture_output=True, text=True)
    if build.returncode != 0:
        pytest.fail(f"g++ failed:\n{build.stderr}")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.startswith("ok "), run.stdout
