"""The work-item decomposition divides by launch constants with a multiply-high
and shift (Granlund and Montgomery, "Division by Invariant Integers using
Multiplication", PLDI 1994). The host computes the multiplier and shift
(``make_fast_div`` in csrc/decode_launch.h); the kernels evaluate
umulhi(n, mul) >> shr, or n itself when shr < 0. This compiles the host
function and checks that evaluation against exact division: every divisor up
to 4096 against every numerator below 2^14 plus edge numerators, and random
divisors and numerators up to 2^31."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_attention_14_amd", "csrc")

PROGRAM = r"""
#include <cstdio>
#include <cstdint>
#include <random>
#include "decode_launch.h"

static uint32_t quot(uint32_t n, const pdk::FastDiv& f) {
  if (f.shr < 0) return n;
  return static_cast<uint32_t>((static_cast<uint64_t>(n) * f.mul) >> 32) >> f.shr;
}

static int check(uint32_t n, uint32_t d, const pdk::FastDiv& f) {
  if (quot(n, f) != n / d) {
    std::printf("mismatch n=%u d=%u got=%u want=%u\n", n, d, quot(n, f), n / d);
    return 1;
  }
  return 0;
}

int main() {
  long checked = 0;
  const uint32_t top = 0x7fffffffu;
  for (uint32_t d = 1; d <= 4096; ++d) {
    const pdk::FastDiv f = pdk::make_fast_div(d);
    for (uint32_t n = 0; n < (1u << 14); ++n, ++checked)
      if (check(n, d, f)) return 1;
    const uint32_t edges[] = {top, top - 1, top - d, top / d * d, top / d * d - 1, d - 1, d, d + 1,
                              2 * d - 1, 2 * d};
    for (uint32_t n : edges) {
      if (n > top) continue;
      ++checked;
      if (check(n, d, f)) return 1;
    }
  }
  std::mt19937_64 rng(20261203);
  for (int i = 0; i < 2000000; ++i, ++checked) {
    const uint32_t d = 1 + static_cast<uint32_t>(rng() % top);
    const uint32_t n = static_cast<uint32_t>(rng() % (static_cast<uint64_t>(top) + 1));
    if (check(n, d, pdk::make_fast_div(d))) return 1;
    if (check(n / d * d, d, pdk::make_fast_div(d))) return 1;
  }
  std::printf("ok %ld\n", checked);
  return 0;
}
"""


def test_fast_div_matches_exact_division(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no C++ compiler")
    src = tmp_path / "fast_div.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "fast_div"
    subprocess.run([cxx, "-O2", "-std=c++17", "-D__HIP_PLATFORM_AMD__", f"-I{CSRC}",
                    "-I/opt/rocm/include", str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok ")
