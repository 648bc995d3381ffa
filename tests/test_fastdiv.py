"""The launch-invariant division helper of the kernels (csrc/fastdiv.h, the unsigned
multiply-shift division of Granlund & Montgomery) against the C compiler's own integer
division, over its domain (numerators in [0, 2^31), divisors in [1, 2^31]): every divisor 1..4096 on the numerators where rounding could go wrong (multiples
of the divisor and their neighbours, 0, 2^31 - 1), large and power-of-two divisors, and a
seeded random sample over the whole range [0, 2^31). Compiled with the host C++ compiler."""
import os
import subprocess

from tests import conftest

SRC = r'''
#include <cstdio>
#include <cstdint>
#include <random>
#include "fastdiv.h"
using namespace mol;
static long bad = 0, checked = 0;
static void check(uint32_t n, uint32_t d) {
  if (n > 0x7fffffffu) return;
  const FastDiv f = make_fastdiv(d);
  const int q = fdiv((int)n, f), r = fmod((int)n, f);
  ++checked;
  if (q != (int)(n / d) || r != (int)(n % d)) {
    if (bad++ < 10) std::printf("n=%u d=%u got %d %d\n", n, d, q, r);
  }
}
int main() {
  for (uint32_t d = 1; d <= 4096; ++d) {
    for (uint32_t k = 0; k < 4096; k += (k < 64 ? 1 : 61)) {
      const uint64_t base = (uint64_t)k * d;
      for (int e = -1; e <= 1; ++e) check((uint32_t)(base + e), d);
    }
    check(0, d);
    check(0x7fffffffu, d);
    check(0x7fffffffu - (0x7fffffffu % d), d);
  }
  const uint32_t big[] = {8191, 8192, 8193, 65535, 65536, 1u << 20, (1u << 20) + 1, 12345679,
                          (1u << 30) - 1, 1u << 30, (1u << 30) + 1, 0x7fffffffu, 0x80000000u};
  for (uint32_t d : big) {
    for (uint32_t n : {0u, 1u, d - 1, d, d + 1, 2 * d - 1, 2 * d, 0x7fffffffu}) check(n, d);
  }
  std::mt19937_64 g(12345);
  for (int i = 0; i < 4000000; ++i) {
    const uint32_t n = (uint32_t)(g() & 0x7fffffffu);
    const int sh = 1 + (int)(g() % 31);
    uint32_t d = (uint32_t)(g() >> 32) >> sh;  // up to 2^31 - 1
    if (d == 0) d = 1;
    check(n, d);
  }
  std::printf("checked %ld bad %ld\n", checked, bad);
  return bad != 0;
}
'''


def test_fastdiv_matches_integer_division(tmp_path):
    csrc = os.path.join(conftest.ROOT, "virtual_expert_routed_amd", "csrc")
    src = tmp_path / "fd.cpp"
    src.write_text(SRC)
    exe = tmp_path / "fd"
    subprocess.run(["g++", "-std=c++17", "-O2", "-I", csrc, "-o", str(exe), str(src)],
                   check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "bad 0" in r.stdout
