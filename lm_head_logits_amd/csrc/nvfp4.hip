// nvfp4.hip -- the W4A16 NVFP4 head: 4-bit E2M1 weights with one E4M3 scale
// per 16 consecutive weights of a row, bf16 activations, bf16 logits.
//
// The metrale "lm_head_nvfp4_rows.rs" source page (module documentation)
// describes the head: weights stay NVFP4, activations stay 16-bit (casting
// them to E4M3 would fall below the declared precision), rows go through in
// calls of at most 64, and a row's logits do not depend on the row count.
//
// Here a call of up to 64 rows runs the weight-streaming kernels below, in
// which each lane decodes the 8 codes it feeds to one MFMA B operand --
// e2m1 * e4m3 is exact in bf16 (at most 6 significant bits, exponent inside
// bf16's range) -- and the K-step chain of kstep.hpp runs unchanged. A call
// of more rows runs the tiled kernel (tiled.hip), which decodes each weight
// element once per 128-row tile into LDS and runs the same chain. Either way
// the logits equal lmhead_logits on the dequantised weight with
// alpha = fl32(g * alpha), bit for bit, so a row's bits do not depend on M.
#include "kstep.hpp"
#include "launch.hpp"
#include "nvfp4_decode.hpp"
#include "ring.hpp"

namespace lmhead {

namespace {

constexpr int NV_WAVES = 4;
constexpr int NV_NB = 4;  // 16-column blocks per wave

// OCP E2M1 nibble -> fp32: sign bit 3; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
__device__ __forceinline__ float e2m1_f32(uint32_t nib) {
  const uint32_t mag = nib & 7u;
  const uint32_t e = mag >> 1, m = mag & 1u;
  uint32_t bits = mag == 0u ? 0u : (mag == 1u ? 0x3F000000u : (((126u + e) << 23) | (m << 22)));
  bits |= (nib & 8u) << 28;
  return __builtin_bit_cast(float, bits);
}

// OCP E4M3 byte -> fp32: bias 7, subnormals below exponent field 1, the one NaN
// pattern S.1111.111, no infinities.
__device__ __forceinline__ float e4m3_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float mag;
  if (e == 0u)
    mag = (float)m * 0x1p-9f;
  else if (e == 15u && m == 7u)
    mag = __builtin_nanf("");
  else
    mag = __builtin_bit_cast(float, ((e + 120u) << 23) | (m << 20));
  return (b & 0x80u) ? -mag : mag;
}

// Eight codes (one 32-bit word, element 2i in the low nibble of byte i) times
// their block scale -> the eight bf16 values of one B-operand slot group.
// The products are exact in fp32 and in bf16, so taking the upper half of the
// fp32 pattern is the exact bf16 value.
__device__ __forceinline__ u32x4 dequant8(uint32_t codes, float scale) {
  u32x4 r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float lo = e2m1_f32((codes >> (8 * p)) & 15u) * scale;
    const float hi = e2m1_f32((codes >> (8 * p + 4)) & 15u) * scale;
    r[p] = (__builtin_bit_cast(uint32_t, lo) >> 16) | (__builtin_bit_cast(uint32_t, hi) & 0xFFFF0000u);
  }
  return r;
}

template <int R>
__global__ __launch_bounds__(256) void nvfp4_generic_kernel(const uint16_t *__restrict__ hidden, int64_t M,
                                                    int64_t H, const uint8_t *__restrict__ codes,
                                                    const uint8_t *__restrict__ scales, int64_t V,
                                                    float scale, const float *__restrict__ bias,
                                                    uint16_t *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int li = lane & 15;
  const int lg = lane >> 4;
  const int64_t nmb = (M + 63) / 64;
  const int64_t m0 = ((int64_t)blockIdx.x % nmb) * 64;
  const int64_t col0 = (((int64_t)blockIdx.x / nmb) * NV_WAVES + wave) * (NV_NB * 16);
  if (col0 >= V) return;

  const uint32_t *cp[NV_NB];
  const uint8_t *sp[NV_NB];
  bool bv[NV_NB];
#pragma unroll
  for (int j = 0; j < NV_NB; ++j) {
    int64_t col = col0 + 16 * j + li;
    bv[j] = col < V;
    const int64_t c = bv[j] ? col : 0;
    // lane group lg feeds k0 + 8*lg .. k0 + 8*lg + 7: bytes 4*lg .. 4*lg + 3 of
    // the step's 16 code bytes, and scale (k0 + 8*lg) / 16 = k0/16 + lg/2.
    cp[j] = reinterpret_cast<const uint32_t *>(codes + c * (H / 2)) + lg;
    sp[j] = scales + c * (H / 16) + (lg >> 1);
  }
  const u32x4 *ap[R];
  bool av[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int64_t row = m0 + 16 * r + li;
    av[r] = row < M;
    ap[r] = reinterpret_cast<const u32x4 *>(hidden + (av[r] ? row : 0) * H + 8 * lg);
  }

  f32x4 acc[NV_NB][R];
#pragma unroll
  for (int j = 0; j < NV_NB; ++j)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[j][r] = zero4();

  const u32x4 z = {0u, 0u, 0u, 0u};
  const int64_t nk = H / KSTEP;
  // the wave's 64 columns lie in one group of korder.hpp: their chains start
  // at K-step krot of the row
  const int64_t krot = korder_start(col0, H) / KSTEP;
  for (int64_t s0 = 0; s0 < nk; ++s0) {
    const int64_t s = s0 + krot < nk ? s0 + krot : s0 + krot - nk;  // K-step of the row
    u32x4 b[NV_NB], a[R];
#pragma unroll
    for (int j = 0; j < NV_NB; ++j) {
      if (bv[j]) {
        const uint32_t cw = cp[j][s * 4];
        const float sc = e4m3_f32(sp[j][s * 2]);
        b[j] = dequant8(cw, sc);
      } else {
        b[j] = z;
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) a[r] = av[r] ? ap[r][s * 4] : z;
#pragma unroll
    for (int j = 0; j < NV_NB; ++j)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[j][r] = kstep(acc[j][r], a[r], b[j]);
  }

#pragma unroll
  for (int j = 0; j < NV_NB; ++j) {
    const int64_t col = col0 + 16 * j + li;
    if (col >= V) continue;
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = m0 + 16 * r + 4 * lg + q;
        if (row < M) out[row * V + col] = bf16_rne(epilogue(acc[j][r][q], scale, bias, col));
      }
    }
  }
}

template <int R>
hipError_t launch_generic_r(const Nvfp4Args &a, hipStream_t stream) {
  dim3 grid((unsigned)(((a.V + NV_WAVES * NV_NB * 16 - 1) / (NV_WAVES * NV_NB * 16)) *
                       ((a.M + 63) / 64)));
  dim3 block(64 * NV_WAVES);
  return launch_kernel(nvfp4_generic_kernel<R>, grid, block, stream, a.hidden, a.M, a.H, a.codes,
                       a.scales, a.V, a.scale, a.bias, a.out);
}

// ---------------------------------------------------------------------------
// Streaming kernels for H % 128 == 0 (the common case): the decode-sized
// NVFP4 head at HBM speed.
// ---------------------------------------------------------------------------
constexpr int NR_KC = 256;          // K per chunk
constexpr int NR_CPR = NR_KC / 8;   // 16-byte hidden pieces per row per chunk
constexpr int NR_CB = NR_KC / 2;    // code bytes per weight row per chunk
constexpr int NR_SB = NR_KC / 16;   // scale bytes per weight row per chunk

__device__ __forceinline__ int nr_hslot(int row, int ch) { return row * NR_CPR + (ch ^ (row & 15)); }

// LDS slot of 16-byte piece p (K-step p of the chunk) of row `row` of a code
// unit: rows of 128 bytes, pieces xor-swizzled by row pair so the 16 rows one
// operand read touches fall in distinct banks.
__device__ __forceinline__ int nr_cslot(int row, int p) { return row * 8 + (p ^ ((row >> 1) & 7)); }

// 4 x 4 transpose of 32-bit words across the four 16-lane rows of a wave:
// on entry row g holds words D[g][0..3] in x0..x3; on exit x_t in row g
// holds D[t][g].
__device__ __forceinline__ void transpose4(uint32_t &x0, uint32_t &x1, uint32_t &x2, uint32_t &x3) {
  auto a = __builtin_amdgcn_permlane32_swap(x0, x2, false, false);
  auto b = __builtin_amdgcn_permlane32_swap(x1, x3, false, false);
  auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  x0 = c[0];
  x1 = c[1];
  x2 = d[0];
  x3 = d[1];
}

// Ring kernel, one or two row blocks (M <= 32). K is walked in chunks of 256
// elements: per weight row 128 code bytes and 16 scale bytes. Each wave owns
// NB column blocks of 16 rows; a block's chunk is one "unit", whose codes
// come to LDS by two direct-to-LDS loads of 8 rows x 128 contiguous bytes
// into a ring of NSL slots per wave. Units are read and refilled one at a
// time, as in the bf16 weight-streaming kernel, so NSL - 1 units stay in
// flight. A lane's ds_read_b128 takes the 16 code bytes of one K-step of its
// row; a 4 x 4 transpose of 32-bit words across the four 16-lane groups (two
// v_permlane32_swap, two v_permlane16_swap) hands each lane the 8 codes of
// its MFMA slots for four K-steps. Dequantisation stays in registers:
// v_cvt_scalef32_pk_f32_fp4 (scale 1.0) turns two codes into two fp32 values,
// a multiply by the E4M3 block scale (v_cvt_f32_fp8) gives the exact weight,
// whose upper 16 bits are its bf16 pattern. Hidden rows come through LDS in
// the same 256-element chunks, double-buffered, one LDS barrier per chunk.
//
// Block scales are 16 bytes per row and chunk. Loaded per chunk (16 rows x
// 16 bytes per instruction) the same 128-byte scale lines are read eight
// times, a chunk apart, with the code stream passing through L2 in between:
// measured without the K-steps, that stream took 78 µs instead of 37 µs
// (M = 1, H = 2048, V = 151936). So a block's scales are loaded for a group of
// eight chunks at once, 16 rows x 64 contiguous bytes per instruction (two
// instructions): lane (i, k) holds row i's scales of chunk 4h + k of the
// group, and at each chunk a ds_bpermute hands every lane of row i the
// 16 bytes of that chunk. The next group's scales are loaded at the group's
// last chunk, into the registers just read.
//
// The kernel is bound by its waves' instruction streams, not by the weight
// stream. Timing-only copies (M = 1, H = 2048, V = 151936, one MI355X): with
// every code load hitting L2 it ran as fast as with the codes from HBM
// (42.6 against 42.8 µs); without the dequantisation (about 2 VALU
// instructions per weight) in 31 µs; without that and the direct loads in
// 22 µs, and that skeleton fell to 9-12 µs when either its MFMAs or its lane
// transposes were removed: transposes interleaved with MFMAs stall. Reading
// the codes with eight 4-byte LDS reads instead of transposing them was
// slower. A wave may own fewer blocks than NB; its K-steps for the others
// are skipped (6-8% at this shape).
//
// Issue order: at the read of unit v (and in the prologue for v < 0) a
// "batch": unit v + NSL's two direct loads; the hidden loads of chunk
// (v + NSL) / NB when unit v + NSL starts a chunk; and, when v lies in the
// last chunk of a scale group, the next group's two scale loads of v's
// block. The prologue issues the batches of v = -NSL .. -1 with the first
// group's scale loads where a steady-state batch would carry scale loads, so
// every batch size is a function of the position only and each wait is a
// compile-time count of the loads issued after the ones it needs
// (NvSchedule, ring.hpp).
template <int R, int NB, int NW, int NSL>
__global__ __launch_bounds__(64 * NW, 1) void nvfp4_ring_kernel(
    const uint16_t *__restrict__ hidden, int64_t M, int64_t H, const uint8_t *__restrict__ codes,
    const uint8_t *__restrict__ scales, int64_t V, float scale, const float *__restrict__ bias,
    uint16_t *__restrict__ out, int64_t gblocks, int64_t kwg) {
  constexpr int THREADS = 64 * NW;
  constexpr int ROWS = 16 * R;
  constexpr int HPC = ROWS * NR_CPR;                 // hidden pieces per chunk
  constexpr int HL = (HPC + THREADS - 1) / THREADS;  // ... per thread
  using S = NvSchedule<NB, NSL, HL>;
  constexpr int NHR = S::NHR;
  constexpr int PERIOD = S::PERIOD;
  constexpr int GROUP = S::GROUP;
  static_assert(NSL > NB && NSL <= 8, "a ring of more slots than blocks, at most 8");
  constexpr int CW = NW * 128;  // 16-byte slots of one ring slot's codes, all waves
  __shared__ u32x4 hs[2][HPC];
  __shared__ u32x4 C0[CW], C1[CW], C2[NSL > 2 ? CW : 1], C3[NSL > 3 ? CW : 1],
      C4[NSL > 4 ? CW : 1], C5[NSL > 5 ? CW : 1], C6[NSL > 6 ? CW : 1], C7[NSL > 7 ? CW : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15;
  const int lg = lane >> 4;
  const int64_t nmb = (M + 63) / 64;
  const int64_t m0 = ((int64_t)blockIdx.x % nmb) * 64;
  const int64_t ncb = (V + 15) / 16;
  const WaveCols wc = split_cols((int64_t)blockIdx.x / nmb, (int64_t)gridDim.x / nmb, wave, NW, ncb,
                                 gblocks, kwg, H);
  const int64_t cb0 = wc.cb0, cb1 = wc.cb1;
  const bool active = cb1 > cb0;
  const int nbw = (int)(cb1 - cb0);  // blocks this wave owns (<= NB)
  const int64_t cend = cb1 * 16 < V ? cb1 * 16 : V;

  const int64_t HC = H / 2, HS = H / 16;
  const int64_t wrows = active ? cend - cb0 * 16 : 0;
  const rsrc_t cr = make_rsrc(codes + (active ? cb0 * 16 : 0) * HC, (uint32_t)(wrows * HC));
  const rsrc_t sr = make_rsrc(scales + (active ? cb0 * 16 : 0) * HS, (uint32_t)(wrows * HS));
  const uint32_t cjs = (uint32_t)(16 * HC), sjs = (uint32_t)(16 * HS);
  uint32_t cvoff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int piece = (lane % 8) ^ ((4 * h + lane / 16) & 7);
    cvoff[h] = (uint32_t)((lane / 8 + 8 * h) * HC + 16 * piece);
  }

  const int64_t nc = (H + NR_KC - 1) / NR_KC;
  const int64_t nunits = nc * NB;
  const bool half_tail = (H % NR_KC) != 0;
  // chunk c of the order -> chunk of the row (a start other than 0 only when
  // H % 256 == 0: then no chunk is half)
  const int64_t krot = wc.kstart / NR_KC;
  auto rowchunk = [&](int64_t c) { return c + krot < nc ? c + krot : c + krot - nc; };

  auto cslot = [&](auto jc) -> u32x4 * {
    constexpr int J = decltype(jc)::value;
    if constexpr (J == 0) return C0;
    else if constexpr (J == 1) return C1;
    else if constexpr (J == 2) return C2;
    else if constexpr (J == 3) return C3;
    else if constexpr (J == 4) return C4;
    else if constexpr (J == 5) return C5;
    else if constexpr (J == 6) return C6;
    else return C7;
  };
  // Unit u (block j) into ring slot jc: two direct loads, or two loads of
  // nothing past the last unit (the schedule's counts stay exact).
  auto issue_unit = [&](int64_t u, auto jc, int j) {
    const bool ok = u < nunits;
    const int64_t pc = ok ? rowchunk(u / NB) : 0;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      dma16_lds(cr, &cslot(jc)[wave * 128 + 64 * h], cvoff[h],
                ok ? (uint32_t)(j * cjs + pc * NR_CB) : OFF_NONE);
  };

  // Scales of block j, group q: load h (chunks 4h .. 4h + 3 of the group) gives
  // lane (i, k) row i's 16 bytes of chunk 8q + 4h + k; past the last chunk,
  // an out-of-range offset (zeros).
  u32x4 sc[NB][2];
  auto load_scales = [&](int j, int64_t q) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t c = GROUP * q + 4 * h + lg;
      sc[j][h] = load16(sr, c < nc ? (uint32_t)(li * HS + rowchunk(c) * NR_SB) : OFF_NONE,
                        (uint32_t)(j * sjs));
    }
  };

  const int64_t hrows = M - m0 < 64 ? M - m0 : 64;
  const rsrc_t hr = make_rsrc(hidden + m0 * H, (uint32_t)(hrows * H * 2));
  const int64_t hpieces = H / 8;
  uint32_t hvoff[HL];
  int hsl[HL], hch[HL];
#pragma unroll
  for (int i = 0; i < HL; ++i) {
    const int idx = i * THREADS + tid < HPC ? i * THREADS + tid : HPC - 1;
    const int row = idx / NR_CPR, ch = idx % NR_CPR;
    hvoff[i] = (uint32_t)((row * H + 8 * ch) * 2);
    hsl[i] = nr_hslot(row, ch);
    hch[i] = ch;
  }
  u32x4 hring[NHR][HL];
  auto load_hidden = [&](u32x4 (&dst)[HL], int64_t c) {
    const int64_t pc = c < nc ? rowchunk(c) : c;
    const uint32_t soff = c < nc ? (uint32_t)(pc * NR_KC * 2) : OFF_NONE;
#pragma unroll
    for (int i = 0; i < HL; ++i)
      dst[i] = load16(hr, (pc * NR_CPR + hch[i] < hpieces) ? hvoff[i] : OFF_NONE, soff);
  };
  auto store_hidden = [&](const u32x4 (&src)[HL], int buf) {
#pragma unroll
    for (int i = 0; i < HL; ++i) hs[buf][hsl[i]] = src[i];
  };

  f32x4 acc[NB][R];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[j][r] = zero4();

  // A unit's codes and scale bytes in registers, copied from its slot (which
  // is then refilled at once).
  struct Regs {
    uint32_t x[8];   // codes of K-step t for this lane's slot group
    uint32_t sw[4];  // scale bytes, pre-shifted for this lane's group
  };

  // Reads unit ub + Q's slot into registers and issues its batch.
  auto read_slot = [&](auto qc, int64_t ub, Regs &rg) {
    constexpr int Q = decltype(qc)::value;  // position of the schedule
    constexpr int J = Q % NB;
    constexpr int SLOT = Q % NSL;
    constexpr int C8 = (Q / NB) % GROUP;
    const int64_t w = ub + Q;
    wait_vm<S::wait_first(Q)>();
    const u32x4 *cs = cslot(std::integral_constant<int, SLOT>{}) + wave * 128;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const u32x4 v = cs[nr_cslot(li, 4 * q + lg)];
      rg.x[4 * q + 0] = v[0];
      rg.x[4 * q + 1] = v[1];
      rg.x[4 * q + 2] = v[2];
      rg.x[4 * q + 3] = v[3];
    }
    // this chunk's scale bytes of row li, from lane li + 16 (C8 % 4)
    const int src = 4 * (li + 16 * (C8 % 4));
#pragma unroll
    for (int d = 0; d < 4; ++d)
      rg.sw[d] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)sc[J][C8 / 4][d]) >> (8 * (lg >> 1));
    // the batch: refill the slot once its reads have returned, the next
    // chunk's hidden loads, the next scale group
    wait_lds();
    issue_unit(w + NSL, std::integral_constant<int, SLOT>{}, (Q + NSL) % NB);
    // the batch in this order (direct loads, hidden, scales), as the wait
    // counts assume: a load issued above a direct load would make the count
    // that retires that direct load one too large
    if constexpr ((Q + NSL) % NB == 0) {
      sched_fence();
      load_hidden(hring[((Q + NSL) / NB) % NHR], (w + NSL) / NB);
    }
    if constexpr (C8 == GROUP - 1) {
      sched_fence();
      load_scales(J, w / NB / GROUP + 1);
    }
    transpose4(rg.x[0], rg.x[1], rg.x[2], rg.x[3]);
    transpose4(rg.x[4], rg.x[5], rg.x[6], rg.x[7]);
  };

  // Unit P of the period starting at unit ub (a multiple of PERIOD): its
  // slot read and batch, then its K-steps.
  auto unit = [&](auto pc, int64_t ub) {
    constexpr int P = decltype(pc)::value;
    constexpr int J = P % NB;
    constexpr int BUF = (P / NB) & 1;
    const int64_t u = ub + P;
    const int64_t c = u / NB;
    Regs rg;
    read_slot(pc, ub, rg);
    const bool half = half_tail && c == nc - 1;  // wave-uniform
    auto kstep_t = [&](auto tc) {
      constexpr int T = decltype(tc)::value;
      u32x4 a[R];
#pragma unroll
      for (int r = 0; r < R; ++r)
        a[r] = hs[BUF][nr_hslot(16 * r + li, 4 * T + lg)];
      const float s = __builtin_amdgcn_cvt_f32_fp8(rg.sw[T / 2], 2 * (T % 2));
      const u32x4 b = dequant8_fast(rg.x[T], s);
#pragma unroll
      for (int r = 0; r < R; ++r) acc[J][r] = kstep(acc[J][r], a[r], b);
    };
    // a wave may own fewer blocks than NB: the slot of a block it does not
    // own holds zeros (its loads are still issued, to keep the schedule's
    // counts), and its K-steps are skipped (a wave-uniform branch)
    if (J < nbw) {
      static_for<4>([&](auto tc) { kstep_t(tc); });
      if (!half) static_for<4>([&](auto tc) { kstep_t(std::integral_constant<int, 4 + decltype(tc)::value>{}); });
    }
    if constexpr (J == NB - 1) {
      wait_vm<S::wait_hidden(P)>();
      store_hidden(hring[(P / NB + 1) % NHR], BUF ^ 1);
      lds_barrier();
    }
  };

  // prologue: the batches of v = -NSL .. -1 (the first scale group where a
  // steady-state batch carries scale loads), hidden chunk 0 to LDS
  static_for<NSL>([&](auto wc) {
    constexpr int W_ = decltype(wc)::value;
    constexpr int VB = W_ - NSL;  // the batch this is
    issue_unit(W_, wc, W_ % NB);
    if constexpr (W_ % NB == 0) {
      sched_fence();
      load_hidden(hring[(W_ / NB) % NHR], W_ / NB);
    }
    if constexpr (S::scl(VB) != 0) {
      sched_fence();
      load_scales(S::md(VB, NB), 0);
    }
    sched_fence();
  });
  wait_vm<S::wait_hidden(-1)>();
  store_hidden(hring[0], 0);
  lds_barrier();

  int64_t ub = 0;
  for (; ub + PERIOD <= nunits; ub += PERIOD) static_for<PERIOD>([&](auto pc) { unit(pc, ub); });
  static_for<PERIOD>([&](auto pc) {
    if (ub + decltype(pc)::value < nunits) unit(pc, ub);
  });

  if (!active) return;
  store_blocks<R, NB>([&](int i, int j) -> f32x4 & { return acc[j][i]; }, out, m0,
                      M - m0 < 16 * R ? M - m0 : 16 * R, cb0 * 16, cend, V, scale, bias);
}

template <int R, int NB, int NW, int NSL>
hipError_t launch_ring_nb(const Nvfp4Args &a, const VSplit &sp, hipStream_t stream) {
  dim3 grid((unsigned)(sp.nvs * ((a.M + 63) / 64)));
  return launch_kernel(nvfp4_ring_kernel<R, NB, NW, NSL>, grid, dim3(64 * NW), stream,
                       a.hidden, a.M, a.H, a.codes, a.scales, a.V, a.scale, a.bias, a.out,
                       sp.gblocks, sp.kwg);
}

template <int R, int NBM, int NW, int NSL>
hipError_t launch_ring_split(const Nvfp4Args &a, const VSplit &sp, hipStream_t stream) {
  if constexpr (NBM > 1) {
    if (sp.nb < NBM) return launch_ring_split<R, NBM - 1, NW, NSL>(a, sp, stream);
  }
  return launch_ring_nb<R, NBM, NW, NSL>(a, sp, stream);
}

// ---------------------------------------------------------------------------
// Three or four row blocks (M = 33 .. 64): the MFMA work per unit is four
// times larger, and the ring's hidden chunks (48-64 KB) and registers do not
// fit beside four slots per wave; this kernel streams the codes straight
// into registers instead.
//
constexpr int NS_WAVES = 8;
constexpr int NS_THREADS = 64 * NS_WAVES;
constexpr int NS_KC = 128;          // K per quad == K per LDS chunk of hidden
constexpr int NS_CPR = NS_KC / 8;   // 16-byte hidden pieces per row per chunk
constexpr int NS_P = 2;             // quads of weight loads in flight ahead of use
constexpr int NS_NB_MAX = 6;        // column blocks per wave

constexpr int NS_SEGQ = 16;                 // quads per LDS segment of block scales
constexpr int NS_SROW = NS_SEGQ + 1;        // 8-byte LDS words per weight row (1 word pad: banks)

__device__ __forceinline__ int ns_hslot(int row, int ch) { return row * NS_CPR + (ch ^ (row & 15)); }

template <int R, int NB>
__global__ __launch_bounds__(NS_THREADS, 1) void nvfp4_quad_kernel(
    const uint16_t *__restrict__ hidden, int64_t M, int64_t H, const uint8_t *__restrict__ codes,
    const uint8_t *__restrict__ scales, int64_t V, float scale, const float *__restrict__ bias,
    uint16_t *__restrict__ out, int64_t gblocks, int64_t kwg) {
  constexpr int ROWS = 16 * R;
  constexpr int HPC = ROWS * NS_CPR;
  constexpr int HL = (HPC + NS_THREADS - 1) / NS_THREADS;
  // Weight prefetch depth in quads: with three or four row blocks a quad has
  // enough MFMA work to cover the load latency with one quad in flight, and
  // the registers go to the accumulators.
  constexpr int P = R >= 3 ? 1 : NS_P;
  constexpr int WROWS = NS_WAVES * NB * 16;              // weight rows of the work-group
  constexpr int SPIECES = WROWS * NS_SEGQ;               // 8-byte scale pieces per segment
  constexpr int SL = (SPIECES + NS_THREADS - 1) / NS_THREADS;
  __shared__ u32x4 hs[2][HPC];
  __shared__ u32x2 ss[WROWS * NS_SROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15;
  const int lg = lane >> 4;
  const int64_t nmb = (M + 63) / 64;
  const int64_t m0 = ((int64_t)blockIdx.x % nmb) * 64;
  // Column blocks [cb0, cb1) of this wave: the ncb blocks split over the
  // grid's waves along V group by group (at most NB each), as in the bf16
  // kernel; [wg_cb0, wg_cb1) those of the work-group.
  const int64_t ncb = (V + 15) / 16;
  const int64_t wg = (int64_t)blockIdx.x / nmb, nwg = (int64_t)gridDim.x / nmb;
  const WaveCols wc = split_cols(wg, nwg, wave, NS_WAVES, ncb, gblocks, kwg, H);
  const int64_t cb0 = wc.cb0, cb1 = wc.cb1;
  const int64_t wg_cb0 = split_cols(wg, nwg, 0, NS_WAVES, ncb, gblocks, kwg, H).cb0;
  const int64_t wg_cb1 = split_cols(wg, nwg, NS_WAVES, NS_WAVES, ncb, gblocks, kwg, H).cb0;
  const bool active = cb1 > cb0;
  const int64_t cend = cb1 * 16 < V ? cb1 * 16 : V;

  const int64_t HC = H / 2, HS = H / 16;  // code and scale bytes per weight row
  const int64_t base_row = active ? cb0 * 16 : 0;
  const rsrc_t cr = make_rsrc(codes + base_row * HC, active ? (uint32_t)((cend - cb0 * 16) * HC) : 0u);
  const uint32_t cvoff = (uint32_t)(li * HC + 16 * lg);
  const uint32_t cjs = (uint32_t)(16 * HC);
  // scale byte of K-step t of a quad for this lane group: 2t + lg/2
  const uint32_t ssel = (lg >> 1) ? 0x07050301u : 0x06040200u;

  // Block scales: the work-group's weight rows (at most WROWS) are contiguous
  // in memory; each segment of NS_SEGQ quads (8 scale bytes per row per quad)
  // is loaded cooperatively into LDS, so the scale stream is read once, in
  // order.
  const int64_t wg_row0 = wg_cb0 * 16;
  const int64_t wg_rows = (wg_cb1 * 16 < V ? wg_cb1 * 16 : V) - wg_row0;
  const rsrc_t sr = make_rsrc(scales + wg_row0 * HS, (uint32_t)(wg_rows * HS));
  const int64_t nq = H / NS_KC;
  // quad q of the order -> quad of the row
  const int64_t krot = wc.kstart / NS_KC;
  auto rowquad = [&](int64_t q) { return q + krot < nq ? q + krot : q + krot - nq; };
  // Scale piece i of this thread in segment `seg`: its load offset (pieces past
  // the segment or the tile get an out-of-range offset and read zero) and its
  // LDS word.
  auto scale_off = [&](int i, int64_t seg) -> uint32_t {
    const int64_t seg_quads = nq - seg * NS_SEGQ < NS_SEGQ ? nq - seg * NS_SEGQ : NS_SEGQ;
    const int p = i * NS_THREADS + tid;
    const int row = p / NS_SEGQ, e = p % NS_SEGQ;
    return (i < SL && p < SPIECES && e < seg_quads)
               ? (uint32_t)(row * HS + rowquad(seg * NS_SEGQ + e) * 8) : 0x80000000u;
  };
  auto scale_store = [&](int i, u32x2 v) {
    const int p = i * NS_THREADS + tid;
    if (i < SL && p < SPIECES) ss[(p / NS_SEGQ) * NS_SROW + p % NS_SEGQ] = v;
  };
  // Copies scale segment `seg` into LDS four pieces per thread at a time (few
  // registers: it also runs inside the quad loop when H > 2048).
  auto copy_scales = [&](int64_t seg) {
#pragma unroll 1
    for (int i0 = 0; i0 < SL; i0 += 4) {
      u32x2 sreg[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        sreg[u] = __builtin_amdgcn_raw_buffer_load_b64(sr, scale_off(i0 + u, seg), 0, 0);
#pragma unroll
      for (int u = 0; u < 4; ++u) scale_store(i0 + u, sreg[u]);
    }
  };
  // LDS row of this lane's weight row in column block j
  const int srow0 = (int)((cb0 - wg_cb0) * 16 + li) * NS_SROW;

  const int64_t hrows = M - m0 < 64 ? M - m0 : 64;
  const rsrc_t hr = make_rsrc(hidden + m0 * H, (uint32_t)(hrows * H * 2));
  uint32_t hvoff[HL];
  int hsl[HL];
#pragma unroll
  for (int i = 0; i < HL; ++i) {
    const int idx = i * NS_THREADS + tid < HPC ? i * NS_THREADS + tid : HPC - 1;
    const int row = idx / NS_CPR, ch = idx % NS_CPR;
    hvoff[i] = (uint32_t)((row * H + 8 * ch) * 2);
    hsl[i] = ns_hslot(row, ch);
  }
  u32x4 hreg[HL];
  auto load_hidden = [&](int64_t q) {
#pragma unroll
    for (int i = 0; i < HL; ++i) hreg[i] = load16(hr, hvoff[i], (uint32_t)(rowquad(q) * NS_KC * 2));
  };
  auto store_hidden = [&](int buf) {
#pragma unroll
    for (int i = 0; i < HL; ++i) hs[buf][hsl[i]] = hreg[i];
  };

  u32x4 cq[P][NB];
  auto load_q = [&](int slot, int64_t q) {
#pragma unroll
    // default policy: a quad reads 64 bytes of each 128-byte line of codes,
    // the next quad the other half, from the cache
    for (int j = 0; j < NB; ++j) cq[slot][j] = load16(cr, cvoff, (uint32_t)(rowquad(q) * 64 + j * cjs));
  };

  f32x4 acc[NB][R];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[j][r] = zero4();

  // One quad: transpose codes, pick scales, then four K-steps of the chain.
  auto do_quad = [&](int slot, int64_t q) {
    const int buf = (int)(q & 1);
    if (q > 0 && q % NS_SEGQ == 0) {  // next scale segment (only when H > 2048)
      lds_barrier();
      copy_scales(q / NS_SEGQ);
      lds_barrier();
    }
    uint32_t x[NB][4], sdw[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      x[j][0] = cq[slot][j][0];
      x[j][1] = cq[slot][j][1];
      x[j][2] = cq[slot][j][2];
      x[j][3] = cq[slot][j][3];
      transpose4(x[j][0], x[j][1], x[j][2], x[j][3]);
      const u32x2 sv = ss[srow0 + j * 16 * NS_SROW + (int)(q % NS_SEGQ)];
      sdw[j] = __builtin_amdgcn_perm(sv[1], sv[0], ssel);
    }
    load_q(slot, q + P < nq ? q + P : nq - 1);
    auto kstep_t = [&](auto tc) {
      constexpr int t = decltype(tc)::value;
      u32x4 a[R];
#pragma unroll
      for (int r = 0; r < R; ++r) a[r] = hs[buf][ns_hslot(16 * r + li, 4 * t + lg)];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const u32x4 b = dequant8_fast(x[j][t], __builtin_amdgcn_cvt_f32_fp8(sdw[j], t));
#pragma unroll
        for (int r = 0; r < R; ++r) acc[j][r] = kstep(acc[j][r], a[r], b);
      }
    };
    kstep_t(std::integral_constant<int, 0>{});
    kstep_t(std::integral_constant<int, 1>{});
    kstep_t(std::integral_constant<int, 2>{});
    kstep_t(std::integral_constant<int, 3>{});
    sched_fence();
    store_hidden(buf ^ 1);
    lds_barrier();
    load_hidden(q + 2 < nq ? q + 2 : nq - 1);
  };

  // Prologue: segment 0's scales into LDS, hidden chunk 0 into LDS, the first
  // P code quads and hidden chunk 1 in flight.
  copy_scales(0);
  load_hidden(0);
#pragma unroll
  for (int p = 0; p < P; ++p) load_q(p, p < nq ? p : nq - 1);
  store_hidden(0);
  load_hidden(nq > 1 ? 1 : 0);
  lds_barrier();

  // ring slot of quad q is q % P: unroll P quads per iteration so every slot
  // index is a compile-time constant
  int64_t q = 0;
  for (; q + P <= nq; q += P) {
#pragma unroll
    for (int p = 0; p < P; ++p) do_quad(p, q + p);
  }
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (q + p < nq) do_quad(p, q + p);

  if (!active) return;
  store_blocks<R, NB>([&](int i, int j) -> f32x4 & { return acc[j][i]; }, out, m0,
                      M - m0 < 16 * R ? M - m0 : 16 * R, cb0 * 16, cend, V, scale, bias);
}

template <int R, int NB>
hipError_t launch_quad_nb(const Nvfp4Args &a, const VSplit &sp, hipStream_t stream) {
  dim3 grid((unsigned)(sp.nvs * ((a.M + 63) / 64)));
  return launch_kernel(nvfp4_quad_kernel<R, NB>, grid, dim3(NS_THREADS), stream, a.hidden, a.M,
                       a.H, a.codes, a.scales, a.V, a.scale, a.bias, a.out, sp.gblocks, sp.kwg);
}

// The variant with NB = the split's blocks per wave (NB <= NBM).
template <int R, int NBM>
hipError_t launch_quad_split(const Nvfp4Args &a, const VSplit &sp, hipStream_t stream) {
  if constexpr (NBM > 1) {
    if (sp.nb < NBM) return launch_quad_split<R, NBM - 1>(a, sp, stream);
  }
  return launch_quad_nb<R, NBM>(a, sp, stream);
}

// One or two row blocks: the ring kernel, sixteen waves of up to three blocks
// (16 or 32 KB of hidden chunks, 4 slots of 2 KB per wave); three or four:
// the register-streaming kernel, eight waves of up to six blocks.
template <int R>
hipError_t launch_stream_r(const Nvfp4Args &a, hipStream_t stream) {
  const int64_t ncb = (a.V + 15) / 16;
  if constexpr (R <= 2)
    return launch_ring_split<R, 3, 16, 4>(a, vsplit(ncb, a.H, 16, 3), stream);
  else
    return launch_quad_split<R, NS_NB_MAX>(a, vsplit(ncb, a.H, NS_WAVES, NS_NB_MAX), stream);
}

}  // namespace

hipError_t launch_nvfp4(const Nvfp4Args &a, hipStream_t stream) {
  // More than one 64-row block: the tiled kernel decodes each weight element
  // once per 256-row tile instead of once per 64-row block.
  if (a.M > 64) return launch_tiled_nvfp4(a, stream);
  const int64_t rows = a.M < 64 ? a.M : 64;
  const int rb = (int)((rows + 15) / 16);
  // the streaming kernels load 8 or 16 scale bytes per row at a time: rows of
  // 8k bytes on a 16-byte aligned base
  if (a.H % 128 == 0 && reinterpret_cast<uintptr_t>(a.scales) % 16 == 0) {
    switch (rb) {
      case 1: return launch_stream_r<1>(a, stream);
      case 2: return launch_stream_r<2>(a, stream);
      case 3: return launch_stream_r<3>(a, stream);
      default: return launch_stream_r<4>(a, stream);
    }
  }
  switch (rb) {  // any H % 32 == 0: per-K-step byte loads, same K-step chain
    case 1: return launch_generic_r<1>(a, stream);
    case 2: return launch_generic_r<2>(a, stream);
    case 3: return launch_generic_r<3>(a, stream);
    default: return launch_generic_r<4>(a, stream);
  }
}

}  // namespace lmhead
