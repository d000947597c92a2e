"""Host-side checks of the causal launch order (fa_params.h: head_rank_order,
head_group), compiled with hipcc as host code and run on the CPU.

Every workgroup of a launch must compute a distinct (head, tile) and every
(head, tile) must be computed: the order is a permutation whatever group
size the launcher picks. The GPU visit-map tests check the same through the
kernels; this test covers many grid shapes cheaply.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_io_aware_69_amd", "csrc")

PROGRAM = r"""
#include <cstdio>
#include <vector>
#include "fa_params.h"

static int fails = 0;
#define CHECK(c, ...) do { if (!(c)) { if (fails++ < 20) { std::printf(__VA_ARGS__); std::printf("\n"); } } } while (0)

int main() {
  // head_rank_order: a bijection for every G dividing the head count; G = 1
  // is head-by-head order; each run of G * ntile indices holds G heads, ranks
  // non-decreasing along the run.
  for (int BH : {1, 2, 3, 8, 12, 16, 24, 64, 128}) {
    for (int ntile : {1, 2, 5, 16, 32, 33, 128}) {
      for (int G = 1; G <= BH; ++G) {
        if (BH % G) continue;
        std::vector<int> seen(BH * ntile, 0);
        int prev_rank = -1;
        for (int lid = 0; lid < BH * ntile; ++lid) {
          int bh = -1, rank = -1;
          fa::head_rank_order(lid, ntile, G, bh, rank);
          CHECK(bh >= 0 && bh < BH && rank >= 0 && rank < ntile, "range BH=%d ntile=%d G=%d lid=%d", BH, ntile, G, lid);
          if (bh < 0 || bh >= BH || rank < 0 || rank >= ntile) continue;
          seen[bh * ntile + rank]++;
          CHECK(bh / G == lid / (G * ntile), "group BH=%d ntile=%d G=%d lid=%d", BH, ntile, G, lid);
          if (lid % (G * ntile) == 0) prev_rank = -1;
          CHECK(rank >= prev_rank, "rank order BH=%d ntile=%d G=%d lid=%d", BH, ntile, G, lid);
          prev_rank = rank;
          if (G == 1) CHECK(bh == lid / ntile && rank == lid % ntile, "head order lid=%d", lid);
        }
        for (int i = 0; i < BH * ntile; ++i) CHECK(seen[i] == 1, "coverage BH=%d ntile=%d G=%d i=%d n=%d", BH, ntile, G, i, seen[i]);
      }
    }
  }
  // head_group: 1 unless 8 divides BH; otherwise the smallest divisor of
  // BH / 8 with G * ntile >= cover * slots, or BH / 8 when none reaches it,
  // capped at the largest divisor of BH / 8 not above `cap`. Checked for the
  // default (cover 2, cap kMaxHeadGroup) and the dense causal dK/dV setting
  // (cover 8, cap 8).
  for (int mode = 0; mode < 2; ++mode) {
    const int cover = mode ? 8 : 2, capv = mode ? 8 : fa::kMaxHeadGroup;
    for (int BH : {1, 4, 8, 12, 16, 32, 64, 128, 256}) {
      for (int ntile : {1, 16, 32, 64, 128, 512}) {
        for (int wgs : {1, 2, 3, 4}) {
          const int cus = 32, slots = wgs * cus;
          const int G = mode ? fa::head_group(wgs, cus, BH, ntile, cover, capv) : fa::head_group(wgs, cus, BH, ntile);
          if (BH % 8) { CHECK(G == 1, "not /8 BH=%d G=%d", BH, G); continue; }
          const int hx = BH / 8;
          CHECK(G >= 1 && hx % G == 0, "divisor BH=%d ntile=%d wgs=%d G=%d", BH, ntile, wgs, G);
          int cap = 1;  // largest divisor of hx not above the cap
          for (int g = 1; g <= capv && g <= hx; ++g)
            if (hx % g == 0) cap = g;
          CHECK(G <= cap, "cap BH=%d ntile=%d wgs=%d G=%d mode=%d", BH, ntile, wgs, G, mode);
          CHECK(G == hx || G == cap || G * ntile >= cover * slots, "cover BH=%d ntile=%d wgs=%d G=%d mode=%d", BH, ntile,
                wgs, G, mode);
          for (int g = 1; g < G; ++g)
            CHECK(hx % g != 0 || g * ntile < cover * slots, "minimal BH=%d ntile=%d wgs=%d G=%d g=%d mode=%d", BH, ntile,
                  wgs, G, g, mode);
        }
      }
    }
  }
  if (fails) { std::printf("FAILED %d\n", fails); return 1; }
  std::printf("OK\n");
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"), reason="hipcc not found")
def test_launch_order_is_a_permutation(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    src = tmp_path / "order.hip"
    exe = tmp_path / "order"
    src.write_text(PROGRAM)
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", CSRC, str(src), "-o", str(exe)],
                   check=True, capture_output=True, text=True, timeout=300)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and out.stdout.strip().endswith("OK"), out.stdout + out.stderr
