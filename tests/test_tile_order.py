"""The matrix-core launches' tile order (csrc/tile_order.hpp) compiled on the host
with g++: every workgroup-to-tile mapping is a bijection onto the tile grid, a
launch of fewer workgroups covers exactly the first logical ids, the fixed chained
walk (a fixed number of workgroups, each taking every (nwg/8)-th id of its XCD's
run) computes every tile exactly once, and so do the per-XCD queues with stealing
(queue_next), under random interleavings of the workgroups' takes and with
workgroups that keep taking after every run is empty."""
import os
import shutil
import subprocess

import pytest

from tests.conftest import ROOT

HDR = os.path.join(ROOT, "lm_head_selected_amd", "csrc")

DRIVER = r"""
#include <cstdio>
#include <cstdlib>
#include <vector>
#include "tile_order.hpp"
int main(int argc, char** argv) {
  const int tm_ = atoi(argv[1]), tn_ = atoi(argv[2]), g = atoi(argv[3]), nwg = atoi(argv[4]);
  std::vector<int> seen(tm_ * tn_, 0), logical(nwg, 0);
  for (int b = 0; b < nwg; ++b) {
    const int l = gh::xcd_logical(b, nwg);
    if (l < 0 || l >= nwg) { printf("logical out of range\n"); return 1; }
    logical[l]++;
    int m, n;
    gh::tile_coords(b, nwg, tm_, tn_, g, m, n);
    if (m < 0 || m >= tm_ || n < 0 || n >= tn_) { printf("tile out of range\n"); return 1; }
    seen[m * tn_ + n]++;
  }
  for (int l = 0; l < nwg; ++l) if (logical[l] != 1) { printf("logical not a bijection\n"); return 1; }
  // the tail (ids nwg .. total-1) mapped directly completes the grid exactly once
  for (int l = nwg; l < tm_ * tn_; ++l) {
    int m, n;
    gh::logical_coords(l, tm_, tn_, g, m, n);
    seen[m * tn_ + n]++;
  }
  for (int i = 0; i < tm_ * tn_; ++i) if (seen[i] != 1) { printf("tile %d seen %d\n", i, seen[i]); return 1; }
  // each XCD's run is the set of ids xcd_logical gives that XCD's workgroups
  const int total = tm_ * tn_;
  for (int x = 0; x < 8; ++x) {
    int start, len;
    gh::xcd_run(x, total, start, len);
    int count = 0;
    for (int b = x; b < total; b += 8) {
      const int l = gh::xcd_logical(b, total);
      if (l < start || l >= start + len) { printf("run mismatch\n"); return 1; }
      ++count;
    }
    if (count != len) { printf("run length mismatch\n"); return 1; }
  }
  // the chained walk with 8, 256 and ceil8(total) workgroups
  const int chains[3] = {8, 256, (total + 7) / 8 * 8};
  for (int c = 0; c < 3; ++c) {
    const int g8 = chains[c], per = g8 >> 3;
    std::vector<int> hit(total, 0);
    for (int b = 0; b < g8; ++b) {
      int start, len;
      gh::xcd_run(b & 7, total, start, len);
      for (int id = b >> 3; id < len; id += per) {
        int m, n;
        gh::logical_coords(start + id, tm_, tn_, g, m, n);
        if (m < 0 || m >= tm_ || n < 0 || n >= tn_) { printf("chain out of range\n"); return 1; }
        hit[m * tn_ + n]++;
      }
    }
    for (int i = 0; i < total; ++i) if (hit[i] != 1) { printf("chain tile %d hit %d\n", i, hit[i]); return 1; }
  }
  // the queues: workgroups on random XCDs take ids in a random order (every XCD's
  // own run first, then the others'), each until it gets -1; every id is handed
  // out once, and an XCD steals only once its own run is empty
  for (int trial = 0; trial < 4; ++trial) {
    unsigned rng = 12345u + 977u * (unsigned)trial + (unsigned)total;
    auto rnd = [&rng]() { rng = rng * 1664525u + 1013904223u; return rng >> 8; };
    int counter[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    std::vector<int> hit(total, 0);
    const int wgs = 8 * (1 + (int)(rnd() % 40));
    std::vector<int> done(wgs, 0);
    int live = wgs;
    while (live > 0) {
      const int b = (int)(rnd() % wgs);
      if (done[b]) continue;
      const int xcd = b & 7;
      int own_start, own_len;
      gh::xcd_run(xcd, total, own_start, own_len);
      const bool own_left = counter[xcd] < own_len;
      auto take = [&counter](int x) { return counter[x]++; };
      const int id = gh::queue_next(take, xcd, total);
      if (id < 0) { done[b] = 1; --live; continue; }
      if (id >= total) { printf("queue id out of range\n"); return 1; }
      const bool own = id >= own_start && id < own_start + own_len;
      if (own_left != own) { printf("stole while the own run had ids\n"); return 1; }
      hit[id]++;
    }
    for (int i = 0; i < total; ++i) if (hit[i] != 1) { printf("queue id %d hit %d\n", i, hit[i]); return 1; }
  }
  printf("ok\n");
  return 0;
}
"""


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("tile_order")
    src = d / "driver.cpp"
    src.write_text(DRIVER)
    exe = d / "driver"
    subprocess.run([gxx, "-std=c++17", "-O1", "-DGH_HOST_DEVICE=", f"-I{HDR}", str(src), "-o",
                    str(exe)], check=True)
    return str(exe)


@pytest.mark.parametrize("tm,tn,g,frac", [
    (594, 32, 8, 1.0), (594, 64, 4, 1.0), (32, 16, 4, 1.0), (16, 594, 4, 1.0),
    (16, 594, 4, 9472 / 9504), (16, 20, 4, 1.0), (1, 2, 8, 1.0), (7, 3, 4, 1.0),
    (13, 11, 8, 0.5), (594, 32, 8, 0.9)])
def test_tile_order_is_a_bijection(driver, tm, tn, g, frac):
    nwg = max(1, int(round(tm * tn * frac)))
    out = subprocess.run([driver, str(tm), str(tn), str(g), str(nwg)], capture_output=True,
                         text=True)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout
