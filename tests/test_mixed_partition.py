"""The weighted partitions of a mixed history (CPU test).

A partition decode over a mixed history (a bf16 sink and recent window around a low-bit
middle) cuts each sequence's joint block list over weighted positions, a bf16 block counting
kMixedBf16Weight.  The kernel (its partition's blocks), the host planner and the merge (the
partition count) all use mixed_positions and mixed_blocks_before from the internal header.
This test compiles a host program against that header and checks, by brute force over
random part sizes and partition lengths, that mixed_blocks_before(x) counts the blocks whose
first weighted position is below x, that the partitions cover every block exactly once, in
order, and that none holds more than tpc blocks (the kernel's block-id table has tpc
entries).
"""
import os
import shutil
import subprocess
import tempfile

import pytest

from mla_latent_kv_02_amd import build as libbuild

PROGRAM = r"""
#include <cstdio>
#include <cstdlib>
#include <vector>
#include "mla_internal.hpp"
int main() {
  const int W = mla::kMixedBf16Weight;
  unsigned s = 12345u;
  auto rnd = [&](int n) { s = s * 1103515245u + 12345u; return (int)((s >> 8) % (unsigned)n); };
  for (int it = 0; it < 20000; ++it) {
    const int nS = rnd(6), nM = rnd(80), nR = rnd(14), tpc = 1 + rnd(48);
    std::vector<int> start;
    for (int i = 0; i < nS; ++i) start.push_back(W * i);
    for (int j = 0; j < nM; ++j) start.push_back(W * nS + j);
    for (int k = 0; k < nR; ++k) start.push_back(W * nS + nM + W * k);
    const int P = mla::mixed_positions(nS, nM, nR);
    if (P != W * (nS + nR) + nM) { printf("positions %d %d %d\n", nS, nM, nR); return 1; }
    for (int x = -3; x <= P + 2 * tpc; ++x) {
      int cnt = 0;
      for (int v : start) cnt += v < x;
      if (mla::mixed_blocks_before(x, nS, nM, nR) != cnt) { printf("before %d %d %d %d\n", x, nS, nM, nR); return 1; }
    }
    const int nch = P > 0 ? (P + tpc - 1) / tpc : 1;
    int next = 0;
    for (int c = 0; c < nch; ++c) {
      const int a = mla::mixed_blocks_before(c * tpc, nS, nM, nR), b = mla::mixed_blocks_before((c + 1) * tpc, nS, nM, nR);
      if (a != next || b < a || b - a > tpc) { printf("partition %d of %d %d %d tpc %d\n", c, nS, nM, nR, tpc); return 1; }
      next = b;
    }
    if (next != nS + nM + nR) { printf("cover %d %d %d\n", nS, nM, nR); return 1; }
  }
  printf("ok\n");
  return 0;
}
"""


def test_weighted_partitions_cover_every_block_once():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "part.cpp")
        exe = os.path.join(d, "part")
        open(src, "w").write(PROGRAM)
        r = subprocess.run([hipcc, "-O2", "-std=c++17", "-I", libbuild.CSRC, src, "-o", exe],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout + out.stderr
