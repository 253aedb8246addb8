// skinny.hip -- the weight-streaming split-V kernel for decode-sized M (<= 64).
//
// At decode sizes the projection is one stream of the whole bf16 weight from
// HBM (the sglang digest's motivation section: the fp32 head's cost was weight
// traffic, which the bf16 x bf16 -> fp32 path cuts to one read of the bf16
// weight). Each wave owns NB column blocks of 16 vocabulary rows and walks the
// full H for them, its weight loads running ahead of their use: by
// direct-to-LDS loads of 8 rows x 128 bytes into a ring of stage buffers of
// two K-steps each, when the work-group's blocks fit in LDS (NB <= 2); else
// by register loads of 16 bytes per lane and K-step straight into the MFMA B
// operand, P K-steps ahead. The hidden rows (<= 64) are staged through LDS in
// KC-element K chunks, double-buffered, so the waves of a work-group read
// them from L2 once. The K-step chain is the one of kstep.hpp, so the results
// equal the tiled GEMM's bit for bit.
//
// Measured on MI355X (HBM read of the 1.05 GB decode weight): the order in
// which the GPU as a whole walks the weight decides the bandwidth. Waves that
// drift apart in K reach ~4.8 TB/s; the waves of a work-group held in
// lockstep by the per-chunk LDS barrier (~512 consecutive weight rows at the
// same K) reach ~5.8 TB/s. The barrier is an LDS-only barrier so prefetched
// weight loads stay in flight across it. Sixteen waves of two column blocks
// with 64-element chunks and a two-step prefetch beat eight waves of four
// blocks with 128-element chunks by 2-4% (decode, M = 1..64).
//
// Launch: one work-group per CU, the vocabulary's column blocks split evenly
// over all waves (each owns floor or ceil of the mean, NB = the ceiling).
// Measured: the stream's bandwidth follows the number of CUs streaming, and a
// CU that holds two work-groups while others hold one finishes last (at
// V = 151936: 297 work-groups of 32 blocks took 1.4x as long as 238 of 40).
// With few blocks per CU (a small vocabulary, or one GPU's share of a
// vocabulary-sharded head) the work-group has 4 or 8 waves of one block and
// an 8-stage ring, or 16 waves with 4 stages: sixteen waves with two stages
// left most waves idle and too few bytes in flight (V = 16032: 28 against
// 52 µs per call; V = 32000: 52 against 57 µs).
// Grid (1-D): vocabulary slices times 64-row blocks of M (one for M <= 64;
// the forced-path test drives more).
#include <type_traits>

#include "kstep.hpp"
#include "launch.hpp"

namespace lmhead {

namespace {

#ifndef LMHEAD_SK_WAVES
#define LMHEAD_SK_WAVES 16
#endif
#ifndef LMHEAD_SK_KC
#define LMHEAD_SK_KC 64
#endif
constexpr int SK_WAVES = LMHEAD_SK_WAVES;
constexpr int SK_KC = LMHEAD_SK_KC;     // K elements per LDS chunk of hidden (one barrier each)
constexpr int SK_SPC = SK_KC / KSTEP;   // K-steps per chunk
constexpr int SK_CPR = SK_KC / 8;       // 16-byte pieces per hidden row per chunk
#ifndef LMHEAD_SK_P
#define LMHEAD_SK_P 2
#endif
#ifndef LMHEAD_SK_POLICY
#define LMHEAD_SK_POLICY LOAD_DEFAULT
#endif
constexpr int SK_P = LMHEAD_SK_P;       // weight prefetch depth, in K-steps (divides SK_SPC)
// Column blocks per wave at most: with 16 waves per CU a wave has 128 VGPRs,
// which hold 4 * NB * R accumulators and 4 * P * NB weight registers without
// spilling up to NB = 4 (R <= 3) or NB = 3 (R = 4).
template <int R>
constexpr int sk_nb_max() { return R >= 4 ? 3 : 4; }
// Cache policy of the weight stream. Measured on MI355X: the non-temporal
// hint makes this access pattern about 1.5x slower, so the default policy.
constexpr int SK_POLICY = LMHEAD_SK_POLICY;

// LDS slot of 16-byte piece `ch` of hidden row `row` (xor swizzle: the 16
// rows one K-step reads land in different banks).
__device__ __forceinline__ int hslot(int row, int ch) {
  return row * SK_CPR + (ch ^ (row & (SK_CPR < 16 ? SK_CPR - 1 : 15)));
}

// LDS slot of 16-byte piece `p` (of 8) of row `row` of a weight block staged
// by direct loads: rows of 128 bytes, pieces xor-swizzled by row pair so the
// 16 rows one MFMA operand read touches fall in distinct banks.
__device__ __forceinline__ int wslot(int row, int p) { return row * 8 + (p ^ ((row >> 1) & 7)); }

typedef __attribute__((address_space(3))) void sk_lds_void;

// Calls f(std::integral_constant<int, 0>{}) ... f(integral_constant<N - 1>)
// in order: loops whose index must be a compile-time constant.
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

// DMA: the weight goes to LDS by direct-to-LDS buffer loads of 8 rows x 128
// bytes (two K-steps of 8 rows) per instruction, two stages per wave in
// flight, and reaches the MFMA through ds_read. Otherwise each lane loads its
// own 16 bytes of a 16-row x 64-byte K-step into registers. The direct loads
// read each weight row 128 contiguous bytes at a time (measured 2-4% faster
// at the decode shape) but need 4 KB of LDS per column block, so they are
// used while the work-group's blocks fit (NB <= 2).
//
// NW waves per work-group and, with direct loads, NS stage buffers per wave
// (NS - 1 stages in flight while one is read). Sixteen waves with two stages
// serve vocabularies of more than 8 column blocks per CU; below that most of
// sixteen waves would own no block and the few that do would keep too few
// bytes in flight, so four waves with eight stages (up to 4 blocks per CU) or
// eight waves with four stages (up to 8) keep about 64 KB per CU in flight.
template <int R, int NB, bool DMA, bool F16, typename OutT, int NW = SK_WAVES, int NS = 2>
__global__ __launch_bounds__(64 * NW, NW >= 8 ? 1 : 2) void skinny_kernel(
    const uint16_t *__restrict__ hidden, int64_t M, int64_t H, const uint16_t *__restrict__ W,
    int64_t V, float alpha, const float *__restrict__ bias, OutT *__restrict__ out,
    RowPart *__restrict__ part) {
  constexpr int THREADS = 64 * NW;
  constexpr int ROWS = 16 * R;
  constexpr int HPC = ROWS * SK_CPR;                           // hidden pieces per chunk
  constexpr int HL = (HPC + THREADS - 1) / THREADS;            // ... per thread
  static_assert(!DMA || SK_KC == 64, "a direct-load stage is one 64-element hidden chunk");
  static_assert(NS == 2 || NS == 4 || NS == 8, "stage ring of 2, 4 or 8");
  static_assert(DMA || NS == 2, "the register path keeps its own prefetch ring");
  constexpr int WLDS = DMA ? NW * NB * 128 : 1;                // 16-byte slots per stage buffer
  __shared__ u32x4 hs[2][ROWS * SK_CPR];
  // Separately declared stage buffers, so the compiler tells the stage being
  // loaded from the ones being read (and waits for the right loads).
  __shared__ u32x4 Wl0[WLDS], Wl1[WLDS], Wl2[NS > 2 ? WLDS : 1], Wl3[NS > 2 ? WLDS : 1],
      Wl4[NS > 4 ? WLDS : 1], Wl5[NS > 4 ? WLDS : 1], Wl6[NS > 4 ? WLDS : 1],
      Wl7[NS > 4 ? WLDS : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: resources stay scalar
  const int li = lane & 15;
  const int lg = lane >> 4;
  const int64_t nmb = (M + 63) / 64;
  const int64_t m0 = ((int64_t)blockIdx.x % nmb) * 64;
  // This wave's column blocks [cb0, cb1): the ncb blocks split evenly over
  // all waves of the grid along V, at most NB each (the host sized NB so).
  const int64_t ncb = (V + 15) / 16;
  const int64_t tw = (int64_t)(gridDim.x / nmb) * NW;
  const int64_t g = ((int64_t)blockIdx.x / nmb) * NW + wave;
  const int64_t cb0 = g * ncb / tw, cb1 = (g + 1) * ncb / tw;
  const bool active = cb1 > cb0;  // wave-uniform
  const int64_t cend = cb1 * 16 < V ? cb1 * 16 : V;  // end of this wave's columns

  // Weight: one buffer resource per wave over its rows [16 cb0, cend)
  // (blocks j >= cb1 - cb0 read as zero); lane offset li*H + 8*lg elements,
  // column block j at j*16*H elements (a scalar offset), K-step s at 32*s.
  const rsrc_t wr = make_rsrc(W + (active ? cb0 * 16 : 0) * H,
                              active ? (uint32_t)((cend - cb0 * 16) * H * 2) : 0u);
  const uint32_t wvoff = (uint32_t)((li * H + 8 * lg) * 2);
  const uint32_t wjstride = (uint32_t)(16 * H * 2);

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
  const int64_t nchunks = (nk + SK_SPC - 1) / SK_SPC;

  auto load_hidden_into = [&](u32x4 (&dst)[HL], int64_t c) {
    const uint32_t soff = (uint32_t)(c * SK_KC * 2);
#pragma unroll
    for (int i = 0; i < HL; ++i) {
      // a piece past the row end (H % 256 != 0) gets an offset past the
      // resource (2^31 + soff cannot wrap), which reads zero without a branch
      const uint32_t v = (c * SK_CPR + hch[i] < hpieces) ? hvoff[i] : 0x80000000u;
      dst[i] = load16(hr, v, soff);
    }
  };
  auto store_hidden_from = [&](const u32x4 (&src)[HL], int buf) {
#pragma unroll
    for (int i = 0; i < HL; ++i) hs[buf][hsl[i]] = src[i];
  };
  u32x4 hreg[HL];
  auto load_hidden = [&](int64_t c) { load_hidden_into(hreg, c); };
  auto store_hidden = [&](int buf) { store_hidden_from(hreg, buf); };

  f32x4 acc[NB][R];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[j][r] = zero4();

  // The wave's logits and / or row-reduction partials (acc is indexed
  // [column block][row block]).
  auto epilogue_all = [&](f32x4 (&a)[NB][R]) {
    const int64_t rows = M - m0 < 16 * R ? M - m0 : 16 * R;
    auto at = [&](int i, int j) -> f32x4 & { return a[j][i]; };
    if (out != nullptr) store_blocks<R, NB>(at, out, m0, rows, cb0 * 16, cend, V, alpha, bias);
    if (part != nullptr) reduce_blocks<R, NB>(at, part, m0, rows, cb0 * 16, cend, V, alpha, bias);
  };

  u32x4 wb[SK_P][NB];
  auto load_w = [&](int slot, int64_t step) {
    const uint32_t soff = (uint32_t)(step * KSTEP * 2);
#pragma unroll
    for (int j = 0; j < NB; ++j) wb[slot][j] = load16<SK_POLICY>(wr, wvoff, soff + j * wjstride);
  };

  // One K-step of the chain on LDS buffer `buf`, slot `slot` of the weight
  // ring; then the ring slot is refilled P steps ahead (clamped to the last
  // step: the refetch of an already-read piece costs a cache hit, not a branch).
  auto kstep_all = [&](int buf, int s, int slot, int64_t step) {
    u32x4 a[R];
#pragma unroll
    for (int r = 0; r < R; ++r) a[r] = hs[buf][hslot(16 * r + li, 4 * s + lg)];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[j][r] = kstep<F16>(acc[j][r], a[r], wb[slot][j]);
    const int64_t next = step + SK_P < nk ? step + SK_P : nk - 1;
    load_w(slot, next);
  };

  if constexpr (DMA) {
    // Direct-load plan (as the tiled kernel's): load h of block j fills rows
    // 8h..8h+7 of the block's 2 KB; lane l writes slot l % 8 of row l / 8,
    // which must hold piece (l % 8) ^ swizzle(row): the swizzle of row
    // 8h + l/8 is (4h + l/16) & 7, so the lane offset depends on h only.
    uint32_t lvoff[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int piece = (lane % 8) ^ ((4 * h + lane / 16) & 7);
      lvoff[h] = (uint32_t)(((lane / 8) * H + 8 * piece) * 2);
    }
    const int64_t nst = (nk + 1) / 2;  // stages of two K-steps (the last may hold one)
    // stage buffer J of the ring (compile-time J)
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
    auto dma_stage = [&](int64_t st, u32x4 *wl) {
      const uint32_t soff = (uint32_t)(st * 128);
      // The buffer was just read by this wave's ds_reads, and a direct load
      // writes LDS on its own path, not behind them: wait until they have
      // returned (lgkmcnt(0)) before overwriting the buffer.
      __builtin_amdgcn_s_waitcnt(0xC07F);
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              wr, (sk_lds_void *)&wl[(wave * NB + j) * 128 + 64 * h], 16, lvoff[h],
              soff + j * wjstride + (uint32_t)(h * 8 * H * 2), 0, 0);
    };
    // Hidden chunks come through a ring of NS register sets, loaded NS chunks
    // ahead like the weight stages: a chunk's hidden loads are issued right
    // after the same chunk's weight loads, so the in-order wait for them
    // (before they are stored to LDS, one chunk ahead of use) never waits for
    // a weight stage earlier than that stage is needed.
    u32x4 hring[NS][HL];
    // Before the first read of a stage buffer: wait for its direct loads.
    // Issued after them: that chunk's hidden loads (HL), then NS - 1 chunks
    // of weight (2 NB) and hidden (HL) loads. The compiler's own wait
    // placement once let a read of the second block slip ahead of its load
    // (single-chunk path, NB = 2), so the wait is explicit, fenced.
    constexpr int VM_AFTER = (NS - 1) * 2 * NB + NS * HL;
    static_assert(VM_AFTER < 64, "vmcnt field");
    constexpr int VM_WAIT = (VM_AFTER & 15) | ((VM_AFTER >> 4) << 14) | 0x70 | 0xF00;
    auto wait_stage = [&]() {
      sched_fence();
      __builtin_amdgcn_s_waitcnt(VM_WAIT);
      sched_fence();
    };
    auto kstep_dma = [&](int buf, int s, const u32x4 *wl) {
      if (s == 0) wait_stage();
      u32x4 a[R], b[NB];
#pragma unroll
      for (int r = 0; r < R; ++r) a[r] = hs[buf][hslot(16 * r + li, 4 * s + lg)];
#pragma unroll
      for (int j = 0; j < NB; ++j) b[j] = wl[(wave * NB + j) * 128 + wslot(li, 4 * s + lg)];
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[j][r] = kstep<F16>(acc[j][r], a[r], b[j]);
    };
    // One 64-element chunk c (= one stage, in ring slot J = c % NS): its two
    // K-steps, then stage c + NS into the buffer just read and hidden chunk
    // c + NS into the register set just freed, with the hand-over of hidden
    // chunk c + 1 to LDS in between.
    auto chunk = [&](auto jc, int64_t c) {
      constexpr int J = decltype(jc)::value;
      constexpr int BUF = J & 1;  // == c & 1 (NS is even)
      u32x4 *wl = wbuf(jc);
      kstep_dma(BUF, 0, wl);
      kstep_dma(BUF, 1, wl);
      dma_stage(c + NS < nst ? c + NS : nst - 1, wl);
      sched_fence();
      store_hidden_from(hring[(J + 1) % NS], BUF ^ 1);
      lds_barrier();
      load_hidden_into(hring[J], c + NS < nchunks ? c + NS : nchunks - 1);
    };
    // prologue: the first NS stages and hidden chunks in flight (stage and
    // chunk j interleaved, as in the loop), hidden chunk 0 in LDS
    static_for<NS>([&](auto jc) {
      constexpr int J = decltype(jc)::value;
      dma_stage(J < nst ? J : nst - 1, wbuf(jc));
      load_hidden_into(hring[J], J < nchunks ? J : nchunks - 1);
    });
    store_hidden_from(hring[0], 0);
    lds_barrier();
    const int64_t nfull = nk / 2;
    int64_t c = 0;
    for (; c + NS <= nfull; c += NS) static_for<NS>([&](auto jc) { chunk(jc, c + decltype(jc)::value); });
    static_for<NS>([&](auto jc) {
      if (c + decltype(jc)::value < nfull) chunk(jc, c + decltype(jc)::value);
    });
    // H % 64 == 32: the last stage holds one K-step
    if (nfull < nst)
      static_for<NS>([&](auto jc) {
        if (nfull % NS == decltype(jc)::value) kstep_dma((int)(nfull & 1), 0, wbuf(jc));
      });
    if (!active) return;
    epilogue_all(acc);
    return;
  }

  // prologue: hidden chunk 0 in LDS, the first P weight K-steps in flight,
  // hidden chunk 1 in flight. Waves past the vocabulary end run the same
  // code on zero-filled loads (their resource is empty) and store nothing.
  load_hidden(0);
#pragma unroll
  for (int p = 0; p < SK_P; ++p) load_w(p, p < nk ? p : nk - 1);
  store_hidden(0);  // waits for hidden chunk 0 only: loads complete in issue order
  load_hidden(nchunks > 1 ? 1 : 0);
  lds_barrier();

  // Full chunks: straight-line code with no branches around the loads, so
  // the waits before each MFMA count exactly the loads still in flight.
  const int64_t nfull = nk / SK_SPC;
  for (int64_t c = 0; c < nfull; ++c) {
    const int buf = (int)(c & 1);
#pragma unroll
    for (int s = 0; s < SK_SPC; ++s) kstep_all(buf, s, s % SK_P, c * SK_SPC + s);
    sched_fence();
    store_hidden(buf ^ 1);
    lds_barrier();
    load_hidden(c + 2 < nchunks ? c + 2 : nchunks - 1);
  }
  // Partial last chunk (H % 256 != 0).
  if (nfull < nchunks) {
    const int buf = (int)(nfull & 1);
#pragma unroll
    for (int s = 0; s < SK_SPC; ++s)
      if (nfull * SK_SPC + s < nk) kstep_all(buf, s, s % SK_P, nfull * SK_SPC + s);
  }

  if (!active) return;
  epilogue_all(acc);
}

template <int R, int NB, bool F16, typename OutT, int NW = SK_WAVES, int NS = 2>
hipError_t launch_nb(const GemmArgs &a, int64_t nvs, hipStream_t stream) {
  dim3 grid((unsigned)(nvs * ((a.M + 63) / 64)));
  constexpr bool DMA = NB <= 2;
  return launch_kernel(skinny_kernel<R, NB, DMA, F16, OutT, NW, NS>, grid, dim3(64 * NW), stream,
                       a.hidden, a.M, a.H, a.W, a.V, a.alpha, a.bias, static_cast<OutT *>(a.out),
                       static_cast<RowPart *>(a.part));
}

// The variant with NB = the split's blocks per wave (NB <= NBM).
template <int R, int NBM, bool F16, typename OutT>
hipError_t launch_split(const GemmArgs &a, const VSplit &sp, hipStream_t stream) {
  if constexpr (NBM > 1) {
    if (sp.nb < NBM) return launch_split<R, NBM - 1, F16, OutT>(a, sp, stream);
  }
  return launch_nb<R, NBM, F16, OutT>(a, sp.nvs, stream);
}

template <int R, bool F16, typename OutT>
hipError_t launch_r(const GemmArgs &a, hipStream_t stream) {
  const int64_t ncb = (a.V + 15) / 16, cus = device_cus();
  // few column blocks per CU: one block per wave, fewer waves, a deeper ring
  // (at most 128 KB of stage buffers per work-group)
  if (ncb <= 4 * cus) return launch_nb<R, 1, F16, OutT, 4, 8>(a, vsplit(ncb, 4, 1).nvs, stream);
  if (ncb <= 8 * cus) return launch_nb<R, 1, F16, OutT, 8, 8>(a, vsplit(ncb, 8, 1).nvs, stream);
  if (ncb <= 16 * cus) return launch_nb<R, 1, F16, OutT, 16, 4>(a, vsplit(ncb, 16, 1).nvs, stream);
  constexpr int NBM = sk_nb_max<R>();
  return launch_split<R, NBM, F16, OutT>(a, vsplit(ncb, SK_WAVES, NBM), stream);
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
