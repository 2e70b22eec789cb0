"""The kernels' division by launch-time constants (csrc/fastdiv.h: multiply
high, add, shift) against exact integer division, on the host: the header
is compiled by the host C++ compiler with its device qualifiers defined
away, and checked exhaustively for small operands and at the 31-bit edge."""

import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "split_kv_paged_page_amd", "csrc", "fastdiv.h")

SRC = r"""
#include <stdio.h>
#include <stdint.h>
#define __host__
#define __device__
#include "%s"
using namespace splitkv;
static uint64_t lcg = 12345;
static uint32_t rnd31() { lcg = lcg * 6364136223846793005ull + 1442695040888963407ull; return (uint32_t)(lcg >> 33); }
int main() {
  long bad = 0, checked = 0;
  for (uint32_t d = 1; d <= 4200; ++d) {
    const FastDiv f = make_fastdiv(d);
    for (uint32_t n = 0; n < 70000; n += (d < 300 ? 1 : 7)) { bad += fdiv(n, f) != n / d; ++checked; }
    for (int k = 0; k < 2000; ++k) { const uint32_t n = rnd31(); bad += fdiv(n, f) != n / d; ++checked; }
    for (uint32_t n = 0x7fffffffu - 5000; n <= 0x7fffffffu - 1; ++n) { bad += fdiv(n, f) != n / d; ++checked; }
  }
  for (int k = 0; k < 200000; ++k) {
    const uint32_t d = rnd31() | 1u, n = rnd31();
    const FastDiv f = make_fastdiv(d);
    bad += fdiv(n, f) != n / d; ++checked;
  }
  printf("%%ld %%ld\n", bad, checked);
  return 0;
}
"""


def test_fastdiv_matches_integer_division(tmp_path):
    src = tmp_path / "fd.cpp"
    src.write_text(SRC % HDR)
    exe = tmp_path / "fd"
    subprocess.run(["g++", "-O2", "-std=c++17", str(src), "-o", str(exe)], check=True)
    bad, checked = map(int, subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split())
    assert checked > 10_000_000 and bad == 0
