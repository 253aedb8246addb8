// korder.hpp -- where each column's K reduction starts, and the split of the
// vocabulary over the weight-streaming kernels' waves that keeps a
// work-group's columns on one starting point (internal, host and device).
//
// Every kernel builds output column v with the K-step chain of kstep.hpp
// begun at K element korder_start(v, H) and wrapped around the row end:
// columns come in groups of KORDER_COLS, and group i starts
// (5 i mod (H / 256)) * 256 elements into the row (rows whose length is not
// a multiple of 256 all start at 0). The start depends on the column and H
// only -- not on the row count, the kernel or the launch -- so a row's logits
// stay bit-identical across calls.
//
// What the staggered start buys is the spread of the weight stream over HBM.
// A weight-streaming grid walks K in near lockstep, so with one common start
// the ~4000 weight rows in flight are all read at the same offset within
// their rows (rows of 4 or 8 KB), and on some allocations those addresses
// use only part of the memory channels. Measured on MI355X: the decode head
// (H = 4096, V = 128256) ran at 5.9 TB/s on one allocation and 4.3-4.6 TB/s
// on others; the H = 2048, V = 151936 head at M = 32 took 148 µs with one
// start and 120 µs with the starts staggered by group.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmhead {

// Columns per group: a multiple of every kernel's column tile (16-column
// blocks; 128-, 160- and 256-column tiles), so no tile spans two groups.
constexpr int64_t KORDER_COLS = 10240;
constexpr int64_t KORDER_BLOCKS = KORDER_COLS / 16;
// The start's granularity: a multiple of every kernel's K stage (64, 128 and
// 256 elements).
constexpr int64_t KORDER_STEP = 256;

__host__ __device__ constexpr int64_t korder_start(int64_t col, int64_t H) {
  return H % KORDER_STEP != 0 ? 0 : ((col / KORDER_COLS) * 5 % (H / KORDER_STEP)) * KORDER_STEP;
}

// Whether the columns of a [V, H] head have more than one start.
__host__ __device__ constexpr bool korder_staggered(int64_t H, int64_t V) {
  return H % KORDER_STEP == 0 && H / KORDER_STEP > 1 && V > KORDER_COLS;
}

// Split of `ncb` vocabulary column blocks (16 weight rows each) of a head of
// row length H over the waves of a weight-streaming kernel with `waves` waves
// per work-group: `nvs` work-groups along V, each wave owning at most `nb`
// consecutive blocks. The weight stream's bandwidth grows with the number of
// CUs streaming, so the grid is about `slots` work-groups (one per CU; fewer
// when V is small). When the head's K orders have several starts the blocks
// are split group by group -- `kwg` work-groups per full group of `gblocks`
// blocks, about in proportion to its blocks, the rest to the last -- so that
// a work-group's columns share one start; otherwise one group of all blocks.
// Within a group every wave owns floor or ceil of the mean (the kernels
// derive their own range with split_cols below). Past nb_max blocks per wave
// the grid grows instead. Host code.
struct VSplit {
  int64_t nvs;
  int nb;
  int64_t gblocks, kwg;
};
inline VSplit split_plan(int64_t ncb, int64_t H, int waves, int nb_max, int64_t slots) {
  // work-groups that give `blocks` blocks at most nb per wave
  auto need = [&](int64_t blocks, int64_t nb) { return (blocks + nb * waves - 1) / (nb * waves); };
  if (!korder_staggered(H, ncb * 16) || ncb <= KORDER_BLOCKS) {
    int64_t nvs = need(ncb, 1);  // at least one block per wave
    if (nvs > slots) nvs = slots;
    int64_t nb = (ncb + nvs * waves - 1) / (nvs * waves);
    if (nb > nb_max) {
      nb = nb_max;
      nvs = need(ncb, nb);
    }
    return VSplit{nvs, (int)nb, ncb > 0 ? ncb : 1, nvs};
  }
  // groups of KORDER_BLOCKS blocks, the last one of lb
  const int64_t gb = KORDER_BLOCKS, ng = (ncb + gb - 1) / gb, lb = ncb - (ng - 1) * gb;
  auto clamp = [](int64_t v, int64_t lo, int64_t hi) { return v < lo ? lo : (v > hi ? hi : v); };
  int64_t kf = clamp(slots * gb / ncb, 1, need(gb, 1));
  int64_t kl = clamp((kf * lb + gb - 1) / gb, 1, need(lb, 1));
  if ((ng - 1) * kf + kl > slots && kl > 1) --kl;  // never two work-groups on one CU
  const int64_t nbf = (gb + kf * waves - 1) / (kf * waves), nbl = (lb + kl * waves - 1) / (kl * waves);
  int64_t nb = nbf > nbl ? nbf : nbl;
  if (nb > nb_max) {
    nb = nb_max;
    kf = need(gb, nb);
    kl = need(lb, nb);
  }
  return VSplit{(ng - 1) * kf + kl, (int)nb, gb, kf};
}

// Split of ncb column blocks over a weight-streaming grid of nwg work-groups
// of nw waves: the blocks come in groups of gblocks (KORDER_BLOCKS when the
// starts are staggered, else all of them); each full group has kwg
// work-groups, the last group the rest, and a group's blocks are spread
// evenly over its waves (floor or ceil of the mean each). Returns wave w's
// blocks [cb0, cb1) of work-group wg, and the first K element of the
// work-group's columns.
struct WaveCols {
  int64_t cb0, cb1, kstart;
};
__host__ __device__ inline WaveCols split_cols(int64_t wg, int64_t nwg, int64_t w, int64_t nw,
                                               int64_t ncb, int64_t gblocks, int64_t kwg,
                                               int64_t H) {
  const int64_t ng = (ncb + gblocks - 1) / gblocks;
  const int64_t grp = wg / kwg < ng - 1 ? wg / kwg : ng - 1;
  const int64_t wi = wg - grp * kwg;
  const int64_t gwg = grp < ng - 1 ? kwg : nwg - (ng - 1) * kwg;
  const int64_t gb0 = grp * gblocks;
  const int64_t gn = ncb - gb0 < gblocks ? ncb - gb0 : gblocks;
  const int64_t t = gwg * nw, x = wi * nw + w;
  return WaveCols{gb0 + x * gn / t, gb0 + (x + 1) * gn / t, korder_start(gb0 * 16, H)};
}

}  // namespace lmhead
