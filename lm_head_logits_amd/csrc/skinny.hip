// skinny.hip -- the weight-streaming split-V kernel for decode-sized M (<= 64).
//
// At decode sizes the projection is one stream of the whole bf16 weight from
// HBM (the sglang digest's motivation section: the fp32 head's cost was weight
// traffic, which the bf16 x bf16 -> fp32 path cuts to one read of the bf16
// weight). Each wave owns NB column blocks of 16 vocabulary rows and walks the
// full H for them. Its weight goes to LDS by direct-to-LDS buffer loads of
// 8 rows x 128 contiguous bytes per instruction into a ring of NSL stage
// slots per wave; a slot holds one block's 16 rows x 64 K-elements (two
// K-steps, 2 KB) and is refilled with the block-stage NSL places ahead as
// soon as the wave has read it, so the bytes in flight per wave do not depend
// on NB. The MFMA B operand comes from the slot by ds_read_b128. The hidden
// rows (<= 64) are staged through LDS in 64-element K chunks, double-buffered,
// one LDS-only barrier per chunk, so the waves of a work-group read them from
// L2 once. The K-step chain is the one of kstep.hpp, so the results equal the
// tiled GEMM's bit for bit.
//
// Measured on MI355X: the order in which the GPU as a whole walks the weight
// decides the bandwidth. Waves that drift apart in K reach ~4.8 TB/s; the
// waves of a work-group held in lockstep by the per-chunk barrier (~512
// consecutive weight rows at the same K) reach ~5.8 TB/s. Reading each weight
// row 128 contiguous bytes per load instruction (8 rows per instruction)
// streams rows of 4 KB (H = 2048) much faster than 64 bytes per row and
// instruction (16 rows, the MFMA operand layout read straight into
// registers), which capped the H = 2048 head at about 4.4 TB/s.
//
// The waves' lockstep also means that the ~4000 weight rows read at any one
// time are read at one offset within their rows, which on some allocations
// uses only part of HBM's channels (the same decode head measured at 5.9 or
// at 4.3-4.6 TB/s). The K orders of korder.hpp start 10240-column groups at
// different offsets, so the grid's reads spread over eight or sixteen
// offsets.
//
// Launch: one work-group per CU, the vocabulary's column blocks split group
// by group over the work-groups (about in proportion to the group's blocks:
// a work-group's columns share one K order) and evenly over a group's waves
// (each owns floor or ceil of the mean, NB = the largest).
// The stream's bandwidth follows the number of CUs streaming, and a CU that
// holds two work-groups while others hold one finishes last (at V = 151936:
// 297 work-groups of 32 blocks took 1.4x as long as 238 of 40). With few
// blocks per CU (a small vocabulary, or one GPU's share of a
// vocabulary-sharded head) the work-group has 4 or 8 waves of one block and
// an 8-slot ring, or 16 waves with 4 slots: sixteen waves with two slots
// left most waves idle and too few bytes in flight (V = 16032: 28 against
// 52 µs per call; V = 32000: 52 against 57 µs).
// Grid (1-D): vocabulary slices times 64-row blocks of M (one for M <= 64;
// the forced-path test drives more).
#include "kstep.hpp"
#include "launch.hpp"
#include "ring.hpp"

namespace lmhead {

namespace {

constexpr int SK_KC = 64;            // K elements per stage and per hidden chunk (two K-steps)
constexpr int SK_CPR = SK_KC / 8;    // 16-byte pieces per hidden row per chunk
constexpr int SK_WSLOT = 128;        // 16-byte LDS slots of one wave's block-stage (16 rows x 128 B)

// Column blocks per wave at most: with 16 waves per CU a wave has 128 VGPRs,
// which hold 4 NB R accumulators and the 8 R registers of the two K-steps'
// hidden operands without spilling up to NB = 4 (R <= 3) or NB = 3 (R = 4).
template <int R>
constexpr int sk_nb_max() { return R >= 4 ? 3 : 4; }

// LDS slot of 16-byte piece `ch` of hidden row `row` (xor swizzle: the 16
// rows one K-step reads land in different banks).
__device__ __forceinline__ int hslot(int row, int ch) { return row * SK_CPR + (ch ^ (row & 7)); }

// LDS slot of 16-byte piece `p` (of 8) of row `row` of a block-stage: rows of
// 128 bytes, pieces xor-swizzled by row pair so the 16 rows one MFMA operand
// read touches fall in distinct banks.
__device__ __forceinline__ int wslot(int row, int p) { return row * 8 + (p ^ ((row >> 1) & 7)); }

// NW waves per work-group, NB column blocks per wave, NSL stage slots per
// wave (NSL - 1 block-stages in flight while one is read).
template <int R, int NB, bool F16, typename OutT, int NW, int NSL>
__global__ __launch_bounds__(64 * NW, NW >= 8 ? 1 : 2) void skinny_kernel(
    const uint16_t *__restrict__ hidden, int64_t M, int64_t H, const uint16_t *__restrict__ W,
    int64_t V, float alpha, const float *__restrict__ bias, OutT *__restrict__ out,
    RowPart *__restrict__ part, int64_t gblocks, int64_t kwg) {
  constexpr int THREADS = 64 * NW;
  constexpr int ROWS = 16 * R;
  constexpr int HPC = ROWS * SK_CPR;                 // hidden pieces per chunk
  constexpr int HL = (HPC + THREADS - 1) / THREADS;  // ... per thread
  using S = Schedule<NB, NSL, HL, 2>;
  constexpr int NHR = S::NHR;
  constexpr int PERIOD = S::PERIOD;
  static_assert(NSL >= 2 && NSL <= 8, "a ring of 2 to 8 slots");
  constexpr int WLDS = NW * SK_WSLOT;  // 16-byte slots of one ring slot, all waves
  __shared__ u32x4 hs[2][HPC];
  // Separately declared slots, so the compiler tells the slot being loaded
  // from the ones being read (and waits for the right loads).
  __shared__ u32x4 Wl0[WLDS], Wl1[WLDS], Wl2[NSL > 2 ? WLDS : 1], Wl3[NSL > 3 ? WLDS : 1],
      Wl4[NSL > 4 ? WLDS : 1], Wl5[NSL > 5 ? WLDS : 1], Wl6[NSL > 6 ? WLDS : 1],
      Wl7[NSL > 7 ? WLDS : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: resources stay scalar
  const int li = lane & 15;
  const int lg = lane >> 4;
  const int64_t nmb = (M + 63) / 64;
  const int64_t m0 = ((int64_t)blockIdx.x % nmb) * 64;
  // This wave's column blocks [cb0, cb1): the ncb blocks split over the
  // grid's waves along V, group by group (korder.hpp), at most NB each (the
  // host sized NB so); kstart: the K element where the chains of the
  // work-group's columns start.
  const int64_t ncb = (V + 15) / 16;
  const WaveCols wc = split_cols((int64_t)blockIdx.x / nmb, (int64_t)gridDim.x / nmb, wave, NW, ncb,
                                 gblocks, kwg, H);
  const int64_t cb0 = wc.cb0, cb1 = wc.cb1;
  const bool active = cb1 > cb0;  // wave-uniform
  const int nbw = (int)(cb1 - cb0);  // blocks this wave owns (<= NB)
  const int64_t cend = cb1 * 16 < V ? cb1 * 16 : V;  // end of this wave's columns

  // Weight: one buffer resource per wave over its rows [16 cb0, cend)
  // (blocks j >= cb1 - cb0 read as zero); block j at j*16*H elements.
  const rsrc_t wr = make_rsrc(W + (active ? cb0 * 16 : 0) * H,
                              active ? (uint32_t)((cend - cb0 * 16) * H * 2) : 0u);
  const uint32_t wjstride = (uint32_t)(16 * H * 2);
  // Direct-load plan: load h of a block-stage fills rows 8h..8h+7 of the
  // wave's 2 KB; lane l writes slot l % 8 of row l / 8, which must hold
  // piece (l % 8) ^ swizzle(row): the swizzle of row 8h + l/16... is
  // (4h + l/16) & 7, so the lane offset depends on h only.
  uint32_t lvoff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int piece = (lane % 8) ^ ((4 * h + lane / 16) & 7);
    lvoff[h] = (uint32_t)(((lane / 8) * H + 8 * piece) * 2);
  }

  // Hidden: one resource over the work-group's <= 64 rows (rows past M read
  // as zero); this thread stages pieces (row, 16-byte piece) of each chunk.
  const int64_t hrows = M - m0 < 64 ? M - m0 : 64;
  const rsrc_t hr = make_rsrc(hidden + m0 * H, (uint32_t)(hrows * H * 2));
  uint32_t hvoff[HL];
  int hsl[HL], hch[HL];
#pragma unroll
  for (int i = 0; i < HL; ++i) {
    // threads past the chunk's last piece re-stage the last piece (same bytes, same slot)
    const int idx = i * THREADS + tid < HPC ? i * THREADS + tid : HPC - 1;
    const int row = idx / SK_CPR, ch = idx % SK_CPR;
    hvoff[i] = (uint32_t)((row * H + 8 * ch) * 2);
    hsl[i] = hslot(row, ch);
    hch[i] = ch;
  }

  const int64_t nk = H / KSTEP;
  const int64_t hpieces = H / 8;
  const int64_t nchunks = (nk + 1) / 2;  // the last may hold one K-step (H % 64 == 32)
  const int64_t nunits = nchunks * NB;
  const bool odd_tail = (nk & 1) != 0;
  // chunk c of the order -> chunk of the row (a start other than 0 only when
  // H % 256 == 0, so then there is no half chunk)
  const int64_t krot = wc.kstart / SK_KC;
  auto rowchunk = [&](int64_t c) { return c + krot < nchunks ? c + krot : c + krot - nchunks; };

  u32x4 hring[NHR][HL];
  auto load_hidden = [&](u32x4 (&dst)[HL], int64_t c) {
    const int64_t pc = c < nchunks ? rowchunk(c) : c;
    const uint32_t soff = c < nchunks ? (uint32_t)(pc * SK_KC * 2) : OFF_NONE;
#pragma unroll
    for (int i = 0; i < HL; ++i) {
      // a piece past the row end (H % 64 == 32) reads zero through an
      // out-of-range offset
      const uint32_t v = (pc * SK_CPR + hch[i] < hpieces) ? hvoff[i] : OFF_NONE;
      dst[i] = load16(hr, v, soff);
    }
  };
  auto store_hidden = [&](const u32x4 (&src)[HL], int buf) {
#pragma unroll
    for (int i = 0; i < HL; ++i) hs[buf][hsl[i]] = src[i];
  };

  // slot J of the ring (compile-time J)
  auto wbuf = [&](auto jc) -> u32x4 * {
    constexpr int J = decltype(jc)::value;
    if constexpr (J == 0) return Wl0;
    else if constexpr (J == 1) return Wl1;
    else if constexpr (J == 2) return Wl2;
    else if constexpr (J == 3) return Wl3;
    else if constexpr (J == 4) return Wl4;
    else if constexpr (J == 5) return Wl5;
    else if constexpr (J == 6) return Wl6;
    else return Wl7;
  };
  // Unit u into slot wl: two direct loads (rows 0-7 and 8-15 of the block),
  // or two loads of nothing (an out-of-range offset: no memory traffic, LDS
  // slot unused) past the last unit, which keep the load counts of the
  // schedule exact.
  auto issue_unit = [&](int64_t u, u32x4 *wl, int j) {
    const uint32_t soff = u < nunits ? (uint32_t)(rowchunk(u / NB) * 128 + j * wjstride) : OFF_NONE;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      dma16_lds(wr, &wl[wave * SK_WSLOT + 64 * h], lvoff[h],
                u < nunits ? soff + (uint32_t)(h * 8 * H * 2) : OFF_NONE);
  };

  f32x4 acc[NB][R];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[j][r] = zero4();
  u32x4 a0[R], a1[R];  // the current chunk's hidden operands (K-steps 0 and 1)

  // Unit P of the period starting at unit ub (ub a multiple of PERIOD).
  auto unit = [&](auto pc, int64_t ub) {
    constexpr int P = decltype(pc)::value;
    constexpr int J = P % NB;              // block
    constexpr int BUF = (P / NB) & 1;      // LDS hidden buffer of this chunk
    const int64_t u = ub + P;
    const int64_t c = u / NB;
    u32x4 *wl = wbuf(std::integral_constant<int, P % NSL>{});
    wait_vm<S::wait_unit(P)>();
    if constexpr (J == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        a0[r] = hs[BUF][hslot(16 * r + li, lg)];
        a1[r] = hs[BUF][hslot(16 * r + li, 4 + lg)];
      }
    }
    // A wave may own fewer blocks than NB: the slot of a block it does not
    // own holds zeros (its loads are still issued, to keep the schedule's
    // counts); its K-steps are skipped (wave-uniform). At M = 64, H = 2048,
    // V = 151936 (up to 3 blocks a wave, most waves 2) this took the call from
    // 116 to 104 µs.
    if (J < nbw) {
      const u32x4 b0 = wl[wave * SK_WSLOT + wslot(li, lg)];
#pragma unroll
      for (int r = 0; r < R; ++r) acc[J][r] = kstep<F16>(acc[J][r], a0[r], b0);
      if (!(odd_tail && c == nchunks - 1)) {  // wave-uniform
        const u32x4 b1 = wl[wave * SK_WSLOT + wslot(li, 4 + lg)];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[J][r] = kstep<F16>(acc[J][r], a1[r], b1);
      }
    }
    // Refill the slot with unit u + NSL. A direct load writes LDS on its own
    // path, not behind the wave's earlier ds_reads: wait until they have
    // returned (lgkmcnt(0)) before overwriting the slot.
    wait_lds();
    issue_unit(u + NSL, wl, (P + NSL) % NB);
    if constexpr ((P + NSL) % NB == 0) {
      // the hidden loads after the unit's direct loads, as the wait counts
      // assume: issued before them, they would make the count that retires
      // the second direct load one too large
      sched_fence();
      load_hidden(hring[((P + NSL) / NB) % NHR], (u + NSL) / NB);
    }
    if constexpr (J == NB - 1) {
      // end of chunk c: hidden chunk c + 1 to LDS, then the barrier that
      // hands both hidden buffers over
      wait_vm<S::wait_hidden(P)>();
      store_hidden(hring[(P / NB + 1) % NHR], BUF ^ 1);
      lds_barrier();
    }
  };

  // prologue: units 0 .. NSL - 1 and their chunks' hidden loads in flight,
  // hidden chunk 0 in LDS
  static_for<NSL>([&](auto wc) {
    constexpr int W_ = decltype(wc)::value;
    issue_unit(W_, wbuf(wc), W_ % NB);
    if constexpr (W_ % NB == 0) {
      sched_fence();
      load_hidden(hring[(W_ / NB) % NHR], W_ / NB);
    }
    sched_fence();
  });
  wait_vm<S::wait_hidden(-1)>();
  store_hidden(hring[0], 0);
  lds_barrier();

  int64_t ub = 0;
  for (; ub + PERIOD <= nunits; ub += PERIOD) static_for<PERIOD>([&](auto pc) { unit(pc, ub); });
  static_for<PERIOD>([&](auto pc) {
    if (ub + decltype(pc)::value < nunits) unit(pc, ub);  // wave- and work-group-uniform
  });

  if (!active) return;
  const int64_t rows = M - m0 < 16 * R ? M - m0 : 16 * R;
  auto at = [&](int i, int j) -> f32x4 & { return acc[j][i]; };
  if (out != nullptr)
    store_blocks<R, NB, LOAD_DEFAULT>(at, out, m0, rows, cb0 * 16, cend, V, alpha, bias);
  if (part != nullptr) {
    // the wave's ring slot 0 stages the reduction: every direct load that
    // could still write it (the ring's loads of nothing past the end
    // included) has landed first
    wait_vm<0>();
    float *stg = reinterpret_cast<float *>(&Wl0[wave * SK_WSLOT]);
    static_assert(SK_WSLOT * 4 >= RED_STG_FLOATS, "reduction staging fits a ring slot");
    reduce_blocks<R, NB>(at, part, stg, m0, rows, cb0 * 16, cend, V, alpha, bias);
  }
}

template <int R, int NB, bool F16, typename OutT, int NW, int NSL>
hipError_t launch_nb(const GemmArgs &a, const VSplit &sp, hipStream_t stream) {
  dim3 grid((unsigned)(sp.nvs * ((a.M + 63) / 64)));
  return launch_kernel(skinny_kernel<R, NB, F16, OutT, NW, NSL>, grid, dim3(64 * NW), stream,
                       a.hidden, a.M, a.H, a.W, a.V, a.alpha, a.bias, static_cast<OutT *>(a.out),
                       static_cast<RowPart *>(a.part), sp.gblocks, sp.kwg);
}

// The variant with NB = the split's blocks per wave (NB <= NBM), sixteen
// waves with four slots each (128 KB of LDS).
template <int R, int NBM, bool F16, typename OutT>
hipError_t launch_split(const GemmArgs &a, const VSplit &sp, hipStream_t stream) {
  if constexpr (NBM > 1) {
    if (sp.nb < NBM) return launch_split<R, NBM - 1, F16, OutT>(a, sp, stream);
  }
  return launch_nb<R, NBM, F16, OutT, 16, 4>(a, sp, stream);
}

template <int R, bool F16, typename OutT>
hipError_t launch_r(const GemmArgs &a, hipStream_t stream) {
  const int64_t ncb = (a.V + 15) / 16, cus = device_cus();
  // few column blocks per CU: one block per wave, fewer waves, a deeper ring
  // (at most 128 KB of stage slots per work-group)
  if (ncb <= 4 * cus) return launch_nb<R, 1, F16, OutT, 4, 8>(a, vsplit(ncb, a.H, 4, 1), stream);
  if (ncb <= 8 * cus) return launch_nb<R, 1, F16, OutT, 8, 8>(a, vsplit(ncb, a.H, 8, 1), stream);
  constexpr int NBM = sk_nb_max<R>();
  return launch_split<R, NBM, F16, OutT>(a, vsplit(ncb, a.H, 16, NBM), stream);
}

template <bool F16, typename OutT>
hipError_t launch_t(const GemmArgs &a, hipStream_t stream) {
  // Row blocks per 64-row chunk: only as many as the rows present need.
  const int64_t rows = a.M < 64 ? a.M : 64;
  switch ((rows + 15) / 16) {
    case 1: return launch_r<1, F16, OutT>(a, stream);
    case 2: return launch_r<2, F16, OutT>(a, stream);
    case 3: return launch_r<3, F16, OutT>(a, stream);
    default: return launch_r<4, F16, OutT>(a, stream);
  }
}

}  // namespace

hipError_t launch_skinny(const GemmArgs &a, hipStream_t stream) {
  if (a.in_f16)
    return a.out_type == OUT_F32 ? launch_t<true, float>(a, stream)
                                 : launch_t<true, _Float16>(a, stream);
  return a.out_type == OUT_F32 ? launch_t<false, float>(a, stream)
                               : launch_t<false, uint16_t>(a, stream);
}

}  // namespace lmhead
