"""Host check of the multiply-high division the attention kernel uses to map a
visible token to its page (page = token / page_size, run-time page size).

device.h's div_magic is compiled with g++ into a small program that applies
(mulhi(m, n) + n) >> l, exactly as the kernel does, and compares with n / d:
every divisor 1..4096 on dense and edge numerators, and large divisors on
the edges of the range (n < 2^31)."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROG = r"""
#include <cstdint>
#include <cstdio>
#include <initializer_list>
#include "device.h"
static int check(uint32_t d, uint32_t n) {
  uint32_t m; int32_t l;
  psw::div_magic(d, &m, &l);
  const uint32_t hi = static_cast<uint32_t>((uint64_t{m} * n) >> 32);
  const uint32_t q = (hi + n) >> l;
  if (q != n / d) { std::printf("d=%u n=%u got %u\n", d, n, q); return 1; }
  return 0;
}
int main() {
  int bad = 0;
  for (uint32_t d = 1; d <= 4096 && !bad; ++d) {
    for (uint32_t n = 0; n < 70000; ++n) bad |= check(d, n);
    for (uint32_t k = 1; k < 2048; ++k) {
      const uint64_t base = uint64_t{d} * (k * 1021u % 500000u + 1);
      for (int e = -1; e <= 1; ++e) {
        const uint64_t n = base + e;
        if (n < (uint64_t{1} << 31)) bad |= check(d, static_cast<uint32_t>(n));
      }
    }
    bad |= check(d, 0x7fffffffu);
  }
  const uint32_t big[] = {65535u, 65536u, 65537u, 999999u, 1u << 20, (1u << 30) + 7u,
                          0x7fffffffu};
  for (uint32_t d : big)
    for (uint32_t n : {0u, 1u, d - 1, d, d + 1, 2 * d - 1, 0x7ffffffeu, 0x7fffffffu})
      if (n < (1u << 31)) bad |= check(d, n);
  std::printf(bad ? "FAIL\n" : "OK\n");
  return bad;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_div_magic_exact():
    with tempfile.TemporaryDirectory() as td:
        src = os.path.join(td, "t.cpp")
        exe = os.path.join(td, "t")
        with open(src, "w") as f:
            f.write(PROG)
        inc = os.path.join(ROOT, "paged_sliding_window_append_amd", "csrc")
        r = subprocess.run(["g++", "-O2", "-std=c++17", "-I", inc,
                            "-I", os.path.join(ROOT, "include"), src, "-o", exe],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0 and r.stdout.strip() == "OK", r.stdout
