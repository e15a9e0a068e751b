"""Host check of the launch tile order (planner.hpp ``xcd_balance``).

A small C++ driver compiled with g++ runs the library's own header on random
launches (runs of equal K, like the tile lists of a grouped launch) and checks
what the device remap relies on: the result is a permutation; the range of XCD
x is [x*q + min(x, r), +q + (x < r)) and is ordered longest first; every run of
equal K is split over the XCDs with counts that differ by at most one.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "matrix_optimizer_step_owner_amd", "csrc")
GXX = shutil.which("g++")

DRIVER = r"""
#include <cstdio>
#include <map>
#include <random>
#include "planner.hpp"

int main() {
  std::mt19937 rng(1);
  for (int trial = 0; trial < 5000; ++trial) {
    const int n_xcd = trial % 5 == 0 ? 4 : 8;
    const int ncls = 1 + static_cast<int>(rng() % 5);
    std::vector<int> t;
    std::vector<int64_t> c;
    int id = 0;
    for (int k = 0; k < ncls; ++k) {
      const int n = static_cast<int>(rng() % (trial % 3 == 0 ? 40 : 700));
      for (int i = 0; i < n; ++i) { t.push_back(id++); c.push_back(100 - k); }
    }
    const int64_t T = static_cast<int64_t>(t.size());
    std::vector<int> out(T, -1);
    mfsdp::xcd_balance(t, c, n_xcd, out.data());
    std::vector<int> seen(T, 0);
    for (int v : out) {
      if (v < 0 || v >= T) { std::printf("bad entry\n"); return 1; }
      ++seen[v];
    }
    for (int64_t i = 0; i < T; ++i)
      if (seen[i] != 1) { std::printf("not a permutation\n"); return 1; }
    const int64_t q = T / n_xcd, r = T % n_xcd;
    std::vector<std::map<int64_t, int>> cnt(n_xcd);
    int64_t end = 0;
    for (int x = 0; x < n_xcd; ++x) {
      const int64_t s0 = x * q + (x < r ? x : r), len = q + (x < r ? 1 : 0);
      if (s0 != end) { std::printf("ranges not contiguous\n"); return 1; }
      end = s0 + len;
      for (int64_t i = s0; i < s0 + len; ++i) {
        if (i > s0 && c[out[i]] > c[out[i - 1]]) { std::printf("not longest first\n"); return 1; }
        ++cnt[x][c[out[i]]];
      }
    }
    if (end != T) { std::printf("ranges do not cover the launch\n"); return 1; }
    for (int k = 0; k < ncls; ++k) {
      int lo = 1 << 30, hi = 0;
      for (int x = 0; x < n_xcd; ++x) {
        const auto it = cnt[x].find(100 - k);
        const int v = it == cnt[x].end() ? 0 : it->second;
        lo = v < lo ? v : lo;
        hi = v > hi ? v : hi;
      }
      if (hi - lo > 1) { std::printf("run of equal K unbalanced\n"); return 1; }
    }
  }
  std::printf("ok\n");
  return 0;
}
"""


@pytest.mark.skipif(GXX is None, reason="g++ not available")
def test_xcd_balance_properties(tmp_path):
    src = tmp_path / "drv.cpp"
    src.write_text(DRIVER)
    exe = tmp_path / "drv"
    res = subprocess.run([GXX, "-O2", "-std=c++17", "-I", CSRC, "-o", str(exe), str(src)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
