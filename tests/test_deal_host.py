"""The dealt decode's mapping of workgroups to units, checked on the host.

`dealt_unit` and `deal_blocks` (csrc/pa_launch.h) are plain host/device
functions; compiled here with g++ they must map the workgroups of a dealt
launch onto units 0..T-1 exactly once each (the rest getting units >= T, which
exit), and give each even-numbered XCD (workgroup id % 8) 7 of every 52 units
and each odd one 6.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SRC = r"""
#include "pa_launch.h"
#include <cstdio>
#include <vector>
int main() {
  const long Ts[] = {1, 7, 8, 51, 52, 53, 104, 10920, 20480, 100001};
  for (long T : Ts) {
    const long g = pa::deal_blocks(T);
    if (g % pa::kXcds != 0) { printf("grid %ld not whole rounds\n", g); return 1; }
    std::vector<int> seen(T, 0);
    long per_xcd[pa::kXcds] = {0};
    for (long b = 0; b < g; ++b) {
      const int t = pa::dealt_unit((int)b);
      if (t < 0) { printf("negative unit\n"); return 1; }
      if (t < T) { seen[t]++; per_xcd[b % pa::kXcds]++; }
    }
    for (long t = 0; t < T; ++t)
      if (seen[t] != 1) { printf("T=%ld unit %ld taken %d times\n", T, t, seen[t]); return 1; }
    if (T % pa::kDealPeriod == 0)
      for (int x = 0; x < pa::kXcds; ++x)
        if (per_xcd[x] != (T / pa::kDealPeriod) * ((x & 1) ? 6 : 7)) {
          printf("T=%ld xcd %d got %ld\n", T, x, per_xcd[x]); return 1;
        }
  }
  printf("ok\n");
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP headers")
def test_dealt_units_cover_each_unit_once(tmp_path):
    src = tmp_path / "deal.cpp"
    src.write_text(SRC)
    exe = tmp_path / "deal"
    subprocess.run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    f"-I{ROOT}/include", f"-I{ROOT}/paged_kv_cache_453_amd/csrc", str(src), "-o",
                    str(exe)], check=True, capture_output=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout
