"""Host-side logic of the native library, checked on the CPU.

The projection epilogue divides flat row and column indices by the token
count and head width with a multiply-high (csrc/fastdiv.hpp, after
Granlund and Montgomery, PLDI 1994).  Here that header is compiled with the
host C++ compiler and compared against plain integer division over every
divisor up to 4096 and sampled larger ones, at random numerators, at the
multiples of the divisor and their neighbours, and at the ends of the
supported range [0, 2^31).
"""
import os
import shutil
import subprocess
import tempfile

import pytest

CSRC = os.path.join(os.path.dirname(__file__), "..", "transformer_head_self_amd", "csrc")

CHECK = r"""
#include "fastdiv.hpp"
#include <cstdio>
#include <cstdint>
#include <initializer_list>
int main() {
  uint64_t state = 88172645463325252ull, bad = 0, n_checked = 0;
  auto next = [&]() { state ^= state << 13; state ^= state >> 7; state ^= state << 17; return state; };
  auto check = [&](uint32_t n, uint32_t d, const mha::FastDiv& f) {
    ++n_checked;
    if (mha::fastdiv(n, f) != n / d) { if (bad < 5) printf("n=%u d=%u\n", n, d); ++bad; }
  };
  for (uint32_t d = 1; d < 200000; d += (d < 4096 ? 1 : 97)) {
    const mha::FastDiv f = mha::make_fastdiv(d);
    for (int k = 0; k < 64; ++k) check((uint32_t)(next() & 0x7fffffffu), d, f);
    for (int k = 0; k < 64; ++k) {
      const uint32_t q = (uint32_t)(next() % (0x7fffffffu / d));
      check(q * d, d, f);
      check(q * d + d - 1, d, f);
    }
    for (uint32_t n : {0u, 1u, d - 1, d, d + 1, 0x7fffffffu - 1, 0x7fffffffu}) check(n, d, f);
  }
  for (uint32_t d : {0x7fffffffu, 0x40000000u, 0x40000001u, 65535u, 65537u, 12345679u}) {
    const mha::FastDiv f = mha::make_fastdiv(d);
    for (uint32_t n : {0u, d - 1, d, 0x7fffffffu}) check(n, d, f);
  }
  printf("checked %llu mismatches %llu\n", (unsigned long long)n_checked, (unsigned long long)bad);
  return bad != 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs a host C++ compiler")
def test_fastdiv_matches_integer_division():
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "check.cpp")
        exe = os.path.join(d, "check")
        with open(src, "w") as f:
            f.write(CHECK)
        subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC, src, "-o", exe], check=True)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stdout + r.stderr
        assert "mismatches 0" in r.stdout
