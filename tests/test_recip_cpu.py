"""The launch-constant quotients of the attention and merge kernels:
floor(n / d) = quot32(n, recip32(d)) for every n with n * d <= 2^32.  A small
host program built with hipcc against the kernels' header checks every
divisor up to 4096 at the dividends where an error would show first (around
each multiple of d, and up to the bound), against integer division."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"

PROGRAM = r"""
#include <cstdio>
#include <cstdint>
#include "ring_kernels.h"
using ringkv::quot32;
using ringkv::recip32;
static uint64_t bad = 0, checked = 0;
static void check(uint64_t n, uint32_t d) {
  if (n * d > (uint64_t(1) << 32) || n > 0xFFFFFFFFull) return;
  ++checked;
  if (quot32((uint32_t)n, recip32(d)) != n / d) {
    if (bad < 5) printf("mismatch n=%llu d=%u\n", (unsigned long long)n, d);
    ++bad;
  }
}
int main() {
  for (uint32_t d = 1; d <= 4096; ++d) {
    const uint64_t top = (uint64_t(1) << 32) / d;      // largest n allowed
    for (uint64_t n = 0; n < 4 * d + 4; ++n) check(n, d);
    for (uint64_t k = 1; k <= 64; ++k) {               // around multiples of d
      const uint64_t m = top / k / d * d;
      for (int e = -2; e <= 2; ++e) check(m + e, d);
    }
    for (int e = -(int)d - 2; e <= 0; ++e) check(top + e, d);
  }
  printf("checked %llu bad %llu\n", (unsigned long long)checked, (unsigned long long)bad);
  return bad != 0;
}
"""


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_quotients_by_reciprocal(tmp_path):
    src = tmp_path / "quot.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "quot"
    inc = [f"-I{os.path.join(ROOT, 'draft_model_kv_amd', 'csrc')}", f"-I{os.path.join(ROOT, 'include')}"]
    subprocess.run([HIPCC, "-O2", "-std=c++17", *inc, "-o", str(exe), str(src)],
                   check=True, capture_output=True, timeout=300)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "bad 0" in r.stdout
