"""The launch-time division (attention_softmax_amd/csrc/fastdiv.hpp), compiled
for the host with g++, against the '/' operator on edge and random operands."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER_DIR = os.path.join(ROOT, "attention_softmax_amd", "csrc")

CHECK = r"""
#include <cstdio>
#include <cstdint>
#include <random>
#include "fastdiv.hpp"
int main() {
  std::mt19937_64 rng(12345);
  const uint32_t edges_d[] = {1u, 2u, 3u, 5u, 7u, 31u, 32u, 33u, 1000u, 1024u, 4096u, 4097u,
                              65535u, 65536u, 65537u, 1u << 20, (1u << 31) - 1, 1u << 31,
                              (1u << 31) + 1, 0xfffffffeu, 0xffffffffu};
  long checked = 0;
  auto check = [&](uint32_t n, uint32_t d, const sms::FastDiv& f) {
    const uint32_t got = sms::fast_div(n, f);
    if (got != n / d) { std::printf("FAIL n=%u d=%u got=%u want=%u\n", n, d, got, n / d); return false; }
    ++checked;
    return true;
  };
  for (uint32_t d : edges_d) {
    const sms::FastDiv f = sms::make_fastdiv(d);
    const uint64_t ns[] = {0, 1, d - 1ull, d, d + 1ull, 2ull * d - 1, 2ull * d, 0x7fffffffull,
                           0x80000000ull, 0xfffffffeull, 0xffffffffull};
    for (uint64_t n : ns) if (n <= 0xffffffffull && !check((uint32_t)n, d, f)) return 1;
    for (int i = 0; i < 20000; ++i) if (!check((uint32_t)rng(), d, f)) return 1;
    // multiples and their neighbours
    for (int i = 0; i < 2000; ++i) {
      const uint64_t k = rng() % (0xffffffffull / d + 1);
      for (int64_t dn = -1; dn <= 1; ++dn) {
        const int64_t n = (int64_t)(k * d) + dn;
        if (n >= 0 && n <= 0xffffffffll && !check((uint32_t)n, d, f)) return 1;
      }
    }
  }
  for (int i = 0; i < 3000; ++i) {
    uint32_t d = (uint32_t)rng() >> (rng() % 32);
    if (!d) d = 1;
    const sms::FastDiv f = sms::make_fastdiv(d);
    for (int j = 0; j < 300; ++j) if (!check((uint32_t)rng() >> (rng() % 32), d, f)) return 1;
  }
  std::printf("ok %ld\n", checked);
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_fast_division_matches_operator(tmp_path):
    src = tmp_path / "check.cpp"
    exe = tmp_path / "check"
    src.write_text(CHECK)
    subprocess.run(["g++", "-O2", "-std=c++17", f"-I{HEADER_DIR}", str(src), "-o", str(exe)],
                   check=True, capture_output=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.startswith("ok"), out.stdout + out.stderr
