"""Host check of FastDiv (csrc/device_common.h), the multiply-shift division
the GEMM epilogues and the rotary helper use for run-time divisors (tokens per
stream, per frame, grid width, head widths).

The struct's own source is compiled with the host compiler (device qualifiers
stubbed, the 32-bit high multiply written out) and compared with exact integer
division over divisor and dividend ranges that include every boundary the
method depends on: powers of two and their neighbours, the Wan-layer sizes,
and dividends up to 2^31 - 1."""
import pathlib
import shutil
import subprocess

import pytest

SRC = pathlib.Path(__file__).resolve().parents[1] / "mla_latent_kv_vmla_amd" / "csrc" / "device_common.h"

PROG = r"""
#include <cstdint>
#include <cstdio>
#include <random>
#define __device__
static inline uint32_t __umulhi(uint32_t a, uint32_t b) { return (uint32_t)(((uint64_t)a * b) >> 32); }
%s
int main() {
  std::mt19937 rng(7);
  uint32_t ds[4200];
  int nd = 0;
  for (uint32_t d = 1; d <= 2100; ++d) ds[nd++] = d;
  for (int k = 1; k < 31; ++k) { ds[nd++] = 1u << k; ds[nd++] = (1u << k) + 1; ds[nd++] = (1u << k) - 1; }
  const uint32_t wan[] = {1560, 4680, 52, 30, 224, 128, 96, 192, 480, 18720, 56160};
  for (uint32_t d : wan) ds[nd++] = d;
  while (nd < 4200) ds[nd++] = 1 + rng() %% 0x7fffffffu;
  long bad = 0, checked = 0;
  for (int i = 0; i < nd; ++i) {
    const FastDiv f(ds[i]);
    const uint32_t d = ds[i];
    uint32_t xs[16] = {0, 1, d - 1, d, d + 1, 2 * d - 1, 2 * d, 0x7fffffffu, 0x7ffffffeu};
    for (int j = 9; j < 16; ++j) xs[j] = rng() & 0x7fffffffu;
    for (uint32_t x : xs) {
      if (x > 0x7fffffffu) continue;
      ++checked;
      if (f.div(x) != x / d || f.mod(x) != x %% d) ++bad;
    }
    for (uint32_t x = 0; x < 70000; x += 1 + (d & 7)) {
      ++checked;
      if (f.div(x) != x / d || f.mod(x) != x %% d) ++bad;
    }
  }
  std::printf("%%ld %%ld\n", checked, bad);
  return 0;
}
"""


def test_fastdiv_matches_integer_division(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    s = SRC.read_text()
    a = s.index("struct FastDiv {")
    e = s.index("\n};", a) + 3
    (tmp_path / "fd.cpp").write_text(PROG % s[a:e])
    subprocess.run([gxx, "-std=c++17", "-O2", str(tmp_path / "fd.cpp"), "-o", str(tmp_path / "fd")], check=True)
    checked, bad = map(int, subprocess.run([str(tmp_path / "fd")], check=True, capture_output=True,
                                           text=True).stdout.split())
    assert checked > 1_000_000 and bad == 0
