"""The weight-streaming kernels' vocabulary split (CPU: a host build of
csrc/korder.hpp). split_plan (the launchers' choice of grid, blocks per wave
and groups) and split_cols (each wave's own column blocks, computed in the
kernels) are run here, in the library's own code, over vocabularies from 1 to
2^20 columns, the row lengths of the workloads and others, every launcher's
(waves, blocks per wave) and several compute-unit counts, and checked for:

- every 16-column block owned by exactly one wave;
- no wave owning more than the plan's blocks per wave (the kernels'
  accumulator count);
- a work-group's waves owning consecutive blocks;
- every column of a work-group under the K start its group has
  (korder_start), so that one hidden stream serves the work-group;
- no more work-groups than slots unless the blocks-per-wave cap forced it.
"""
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
CSRC = ROOT / "lm_head_logits_amd" / "csrc"

_PROG = r"""
#include "korder.hpp"
#include <cstdio>
#include <vector>
using namespace lmhead;
static int fail(const char *what, long V, long H, int w, int nbm, long slots, long a, long b) {
  std::printf("FAIL %s V=%ld H=%ld waves=%d nb_max=%d slots=%ld (%ld, %ld)\n", what, V, H, w, nbm,
              slots, a, b);
  return 1;
}
int main() {
  const long Vs[] = {1, 15, 16, 17, 4096, 10240, 10241, 10257, 16032, 20480, 20483, 30001, 32000,
                     50000, 65536, 100000, 128256, 151936, 152064, 200000, 262144, 1000000, 1048576};
  const long Hs[] = {32, 256, 512, 768, 896, 2048, 2304, 4096, 8192};
  const int tiers[][2] = {{4, 1}, {8, 1}, {16, 3}, {16, 4}, {16, 2}, {8, 6}, {8, 5}};
  const long slotss[] = {256, 304, 80, 1};
  long plans = 0, blocks = 0;
  for (long V : Vs)
    for (long H : Hs)
      for (auto &t : tiers)
        for (long slots : slotss) {
          const int waves = t[0], nbm = t[1];
          const long ncb = (V + 15) / 16;
          const VSplit sp = split_plan(ncb, H, waves, nbm, slots);
          if (sp.nvs < 1 || sp.nb < 1 || sp.nb > nbm || sp.gblocks < 1 || sp.kwg < 1)
            return fail("plan fields", V, H, waves, nbm, slots, sp.nvs, sp.nb);
          if (sp.nvs > slots && sp.nb < nbm) return fail("grid beyond slots", V, H, waves, nbm, slots, sp.nvs, sp.nb);
          std::vector<int> own(ncb, 0);
          for (long wg = 0; wg < sp.nvs; ++wg) {
            long prev_end = -1, ks = -1;
            for (int w = 0; w < waves; ++w) {
              const WaveCols c = split_cols(wg, sp.nvs, w, waves, ncb, sp.gblocks, sp.kwg, H);
              if (c.cb1 < c.cb0 || c.cb1 - c.cb0 > sp.nb) return fail("blocks per wave", V, H, waves, nbm, slots, c.cb0, c.cb1);
              if (prev_end >= 0 && c.cb0 != prev_end) return fail("not consecutive", V, H, waves, nbm, slots, prev_end, c.cb0);
              prev_end = c.cb1;
              if (ks >= 0 && c.kstart != ks) return fail("two starts in one work-group", V, H, waves, nbm, slots, ks, c.kstart);
              ks = c.kstart;
              for (long b = c.cb0; b < c.cb1; ++b) {
                if (b < 0 || b >= ncb) return fail("block out of range", V, H, waves, nbm, slots, b, ncb);
                ++own[b];
                const long last = b * 16 + 15 < V - 1 ? b * 16 + 15 : V - 1;
                if (korder_start(b * 16, H) != c.kstart || korder_start(last, H) != c.kstart)
                  return fail("column under another start", V, H, waves, nbm, slots, b, c.kstart);
              }
            }
          }
          for (long b = 0; b < ncb; ++b)
            if (own[b] != 1) return fail("block not owned once", V, H, waves, nbm, slots, b, own[b]);
          ++plans;
          blocks += ncb;
        }
  std::printf("OK %ld plans %ld blocks\n", plans, blocks);
  return 0;
}
"""


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and Path(c).exists():
            return c
    return None


def test_split_covers_every_block_once_within_one_start(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    src = tmp_path / "split.hip"
    src.write_text(_PROG)
    exe = tmp_path / "split"
    r = subprocess.run([hipcc, "--cuda-host-only", "-O2", "-std=c++17", "-I", str(CSRC), str(src),
                        "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0 and out.stdout.startswith("OK"), out.stdout[-2000:]
