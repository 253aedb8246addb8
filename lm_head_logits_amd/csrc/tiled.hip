// tiled.hip -- LDS-tiled MFMA GEMM for large M (verify and prefill).
//
// logits[M, V] = alpha * hidden[M, H] . W[V, H]^T (+ bias) with bf16 inputs,
// fp32 accumulation and fp32 or bf16 output: the fast path of the sglang
// digest (key source excerpt of _compute_lm_head: a bf16 x bf16 -> fp32 mm
// with no fp32 copy of either operand) with the alpha of vLLM PR 49120
// folded into the epilogue (section "muP is folded into the fp32 GEMM").
//
// Work-group tile 256 x 256 output elements with eight waves in a 4 x 2
// arrangement (64 x 128 per wave), or 128 x 128 / 128 x 160 with four waves
// of 64 x 64 / 64 x 80 when M <= 128. Each wave's 16 x 16 MFMA blocks keep
// their fp32 accumulators in registers for the whole K loop. K is staged
// through LDS 64 elements at a time, double-buffered: the loads of stage k+1
// are issued as direct-to-LDS buffer loads (buffer_load_dwordx4 ... lds, no
// registers) before the MFMAs of stage k run, and one barrier per stage
// (which also waits for those loads) hands the buffers over. Every output
// element is built by the K-step chain of kstep.hpp -- ascending K, one
// accumulator, the same operand map -- so a row's bits equal the
// weight-streaming kernel's and do not depend on M. After the K loop the
// stage buffers are idle; each wave stages its logits there one 16-row block
// at a time and writes them as whole rows with 16-byte stores
// (store_rows_lds), which measured 6% (fp32) and 13% (bf16 logits) faster at
// prefill than per-element stores of partial cache lines.
//
// LDS layout of a stage: [row][8 pieces of 16 bytes]; piece c of row r sits in
// slot c ^ ((r >> 1) & 7), so the 16 rows one MFMA operand read touches land
// on 16 distinct 4-bank groups (conflict-free ds_read_b128). The direct loads
// write 64 consecutive slots per instruction; the swizzle is applied on the
// global side by choosing which piece each lane fetches.
//
// Tile order: work-groups are dispatched to the eight XCDs round-robin, so
// block b is remapped to tile t such that consecutive tiles run on one XCD;
// tiles are numbered M-fastest, so the work-groups sharing a weight tile share
// that XCD's L2 and the weight is read from HBM about once.
#include "kstep.hpp"
#include "launch.hpp"
#include "nvfp4_decode.hpp"

namespace lmhead {

namespace {

constexpr int TL_TK = 64;                 // two K-steps per LDS stage
constexpr int TL_PPR = TL_TK / 8;         // 16-byte pieces per row per stage
constexpr int TL_XCDS = 8;

__device__ __forceinline__ int tl_slot(int row, int piece) {
  return row * TL_PPR + (piece ^ ((row >> 1) & 7));
}

typedef __attribute__((address_space(3))) void lds_void;

// One direct-to-LDS load: 64 lanes x 16 bytes into 1 KB of LDS at `dst`
// (wave-uniform), lane l landing at dst + 16 l; POLICY: the cache hint.
template <int POLICY = LOAD_DEFAULT>
__device__ __forceinline__ void dma16(rsrc_t r, void *dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)dst, 16, voff, soff, 0, POLICY);
}

// Arguments of one tiled launch. The B operand is either a 16-bit weight W
// (bf16, or fp16 with fp16 hidden) or an NVFP4 weight (codes, scales)
// decoded on its way into LDS.
struct TiledArgs {
  const uint16_t *hidden;  // [M, H] bf16 or fp16
  int64_t M, H;
  const uint16_t *W;       // [V, H] bf16 or fp16 (16-bit weight)
  const uint8_t *codes;    // [V, H/2] E2M1 pairs (NVFP4 weight)
  const uint8_t *scales;   // [V, H/16] E4M3 (NVFP4 weight)
  int64_t V;
  float alpha;             // epilogue scale (NVFP4: fl32(global_scale * alpha))
  const float *bias;       // [V] or nullptr
  void *out;               // [M, V], or nullptr
  void *part;              // row-reduction partials [M, ceil(V / 16)], or nullptr
};

// WM x WN waves; each owns a (TM / WM) x (TN / WN) sub-tile of at most 4 x 8
// MFMA blocks: <= 128 fp32 accumulators per lane, which the compiler keeps in
// ordinary VGPRs next to the operand fragments (two waves per SIMD).
//
// NV: the B stage is produced from NVFP4 codes instead of a direct load. Each
// thread owns half a stage row (32 elements: 16 code bytes, 2 scale bytes),
// loads it one stage ahead into registers, and at the stage's turn decodes it
// (exact bf16, nvfp4_decode.hpp) into the same swizzled LDS layout the direct
// loads fill. Every weight element is decoded once per tile, whatever M.
//
// RED: the epilogue also writes the row-reduction partials (args.part); a
// separate instantiation, so the plain kernel's register allocation does not
// carry the reduction's code.
//
// TAIL: the stages left after the two-stage loop, 1 or 2 (the parity of the
// stage count, fixed by the launch), or 0 to decide at run time. With the
// 256 x 256 tile a run-time choice makes the compiler hold two copies of the
// accumulators at the join and spill.
template <int TM, int TN, int WM, int WN, bool NV, bool F16, typename OutT, bool RED, int TAIL>
__global__ __launch_bounds__(64 * WM * WN, 1) void tiled_kernel(TiledArgs args) {
  const uint16_t *__restrict__ hidden = args.hidden;
  const int64_t M = args.M, H = args.H, V = args.V;
  const float alpha = args.alpha;
  const float *__restrict__ bias = args.bias;
  OutT *__restrict__ out = static_cast<OutT *>(args.out);
  constexpr int NW = WM * WN;
  constexpr int SM = TM / WM, SN = TN / WN;   // wave sub-tile
  constexpr int FM = SM / 16;                    // 16-row blocks per wave
  constexpr int FN = SN / 16;                    // 16-column blocks per wave
  constexpr int A_DMA = TM * TL_PPR / 64 / NW;     // direct loads per wave per stage (A)
  constexpr int B_DMA = TN * TL_PPR / 64 / NW;  // (B)
  static_assert(A_DMA * 64 * NW == TM * TL_PPR && B_DMA * 64 * NW == TN * TL_PPR, "tiling");
  // Two separately declared buffers per operand (not one array indexed by a
  // variable), so the compiler can tell the stage being loaded from the stage
  // being read and does not wait for the former before reading the latter.
  __shared__ u32x4 As0[TM * TL_PPR], As1[TM * TL_PPR];
  __shared__ u32x4 Bs0[TN * TL_PPR], Bs1[TN * TL_PPR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15;
  const int lg = lane >> 4;
  const int wm = wave / WN;
  const int wn = wave % WN;

  // XCD-aware tile index, M-tiles fastest.
  const int64_t nmt = (M + TM - 1) / TM;
  const int64_t ntiles = nmt * ((V + TN - 1) / TN);
  const int64_t b = blockIdx.x;
  const int64_t q = ntiles / TL_XCDS, r = ntiles % TL_XCDS;
  const int64_t xcd = b % TL_XCDS, pos = b / TL_XCDS;
  const int64_t t = xcd < r ? xcd * (q + 1) + pos : r * (q + 1) + (xcd - r) * q + pos;
  const int64_t m0 = (t % nmt) * TM;
  const int64_t n0 = (t / nmt) * TN;
  // The 128-row tiles serve calls of at most 128 rows (one tile of rows):
  // there the 16-bit weight is read once per call, in whole 128-byte lines,
  // and its direct loads carry the read-once (non-temporal) hint, as in the
  // weight-streaming kernels (M = 128, H = 2048: 125 against 130 µs). The
  // 256-row tiles keep the default: prefill's row tiles share each weight
  // tile through L2, and at M = 256 the hint measured 5% slower. A compile-
  // time choice: a run-time one put a branch in the stage loop, and the
  // prefill kernel ran 8% slower for it.
  constexpr bool B_STREAM = !NV && TM == 128;

  const int64_t arows = M - m0 < TM ? M - m0 : TM;
  const int64_t brows = V - n0 < TN ? V - n0 : TN;
  const rsrc_t ar = make_rsrc(hidden + m0 * H, (uint32_t)(arows * H * 2));
  const rsrc_t br = NV ? make_rsrc(args.codes + n0 * (H / 2), (uint32_t)(brows * (H / 2)))
                       : make_rsrc(args.W + n0 * H, (uint32_t)(brows * H * 2));
  const rsrc_t sr = make_rsrc(NV ? args.scales + n0 * (H / 16) : args.scales,
                              NV ? (uint32_t)(brows * (H / 16)) : 0u);

  // Direct-load plan: instruction u of this wave fills LDS bytes
  // [1 KB * (wave * N + u), ...): 8 rows x 8 slots; lane l -> slot l % 8 of
  // row 8 * (wave * N + u) + l / 8, holding piece (slot ^ swizzle(row)). The
  // swizzle of row 8g + l/8 is (4g + l/16) & 7, so the lane's part of the
  // offset depends only on the parity of g; the row part is a scalar offset.
  uint32_t lvoff[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int piece = (lane % 8) ^ ((4 * par + lane / 16) & 7);
    lvoff[par] = (uint32_t)(((lane / 8) * H + 8 * piece) * 2);
  }
  const uint32_t row8 = (uint32_t)(8 * H * 2);  // bytes of 8 rows

  // H % 32 == 0 but not necessarily % 64: the last stage may hold one K-step
  // (its second half is loaded but never read).
  const int64_t nsteps = H / KSTEP;  // >= 1
  const int64_t nstages = (nsteps + 1) / 2;
  // Stage kt of the tile's K order -> stage of the row: the chains of the
  // tile's columns start korder_start(n0, H) elements into the row (a start
  // other than 0 only when H % 256 == 0, so then every stage is whole).
  // Stages past the last stay past it.
  const int64_t krot = korder_start(n0, H) / TL_TK;
  auto rowstage = [&](int64_t kt) {
    return kt >= nstages ? kt : (kt + krot < nstages ? kt + krot : kt + krot - nstages);
  };

  // NVFP4 producer: unit u = tid + i * threads is half `u % 2` (32 elements)
  // of stage row u / 2; its codes and scales for one stage sit in registers.
  constexpr int NT = 64 * NW;
  constexpr int NU = NV ? TN * 2 / NT : 0;  // units per thread
  static_assert(!NV || NU * NT == TN * 2, "NVFP4 producer tiling");
  u32x4 cq[NU > 0 ? NU : 1];
  uint32_t sq[NU > 0 ? NU : 1];
  // Unit u's stage row and half. Rows 2k and 2k + 1 share their swizzle, so
  // with the two halves of a row on neighbouring lanes, lanes writing rows
  // 2k and 2k + 1 hit the same banks. Instead each group of 8 units takes
  // the even or odd rows of 8 (0, 2, 4, 6 or 1, 3, 5, 7), both halves: the
  // eight 16-byte pieces one decode store of the group writes then sit in
  // eight distinct slots.
  auto unit_row = [](int u) { return (u >> 4) * 8 + ((u >> 1) & 3) * 2 + ((u >> 3) & 1); };
  auto load_codes = [&](int64_t kt) {
    const int64_t pk = rowstage(kt);
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = tid + i * NT, row = unit_row(u), half = u & 1;
      // a half past the row's end (H % 64 == 32, or the stage after the
      // last) reads zero through an out-of-range offset
      const bool in = pk * TL_TK + 32 * half < H;
      const uint32_t co = in ? (uint32_t)(row * (H / 2) + pk * 32 + 16 * half) : OFF_NONE;
      const uint32_t so = in ? (uint32_t)(row * (H / 16) + pk * 4 + 2 * half) : OFF_NONE;
      // default policy: a stage reads 32 bytes of each 128-byte line of
      // codes, and the next stages read the rest of the line from the cache
      // (non-temporal loads here took the M = 256 call from 187 to 280 µs)
      cq[i] = load16(br, co, 0);
      sq[i] = __builtin_amdgcn_raw_buffer_load_b16(sr, so, 0, 0);
    }
  };
  auto decode_codes = [&](u32x4 *bs) {
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = tid + i * NT, row = unit_row(u), half = u & 1;
      // elements 0-15 of the half take scale byte 0, elements 16-31 byte 1
      const float s0 = __builtin_amdgcn_cvt_f32_fp8((int)sq[i], 0);
      const float s1 = __builtin_amdgcn_cvt_f32_fp8((int)sq[i], 1);
#pragma unroll
      for (int w = 0; w < 4; ++w)  // 8 elements per code word
        bs[tl_slot(row, 4 * half + w)] = dequant8_fast(cq[i][w], w < 2 ? s0 : s1);
    }
  };

  // Stage kt into (as, bs): A by direct loads; B by direct loads (bf16) or
  // decoded from the codes loaded one stage earlier, whose registers are then
  // refilled with stage kt+1's.
  auto issue_stage = [&](int64_t kt, u32x4 *as, u32x4 *bs) {
    const uint32_t soff = (uint32_t)(rowstage(kt) * TL_TK * 2);
    if constexpr (NV) decode_codes(bs);
#pragma unroll
    for (int u = 0; u < A_DMA; ++u) {
      const int g = wave * A_DMA + u;
      dma16(ar, &as[g * 64], lvoff[g & 1], soff + g * row8);
    }
    if constexpr (NV) {
      load_codes(kt + 1);
    } else {
#pragma unroll
      for (int u = 0; u < B_DMA; ++u) {
        const int g = wave * B_DMA + u;
        dma16<B_STREAM ? LOAD_STREAM : LOAD_DEFAULT>(br, &bs[g * 64], lvoff[g & 1], soff + g * row8);
      }
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = zero4();


  auto compute = [&](const u32x4 *as, const u32x4 *bs, int s) {
    u32x4 a[FM], bb[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) a[i] = as[tl_slot(wm * SM + 16 * i + li, 4 * s + lg)];
#pragma unroll
    for (int j = 0; j < FN; ++j) bb[j] = bs[tl_slot(wn * SN + 16 * j + li, 4 * s + lg)];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = kstep<F16>(acc[i][j], a[i], bb[j]);
  };

  // The barrier that hands a stage over waits for its direct loads. With NV
  // the next stage's code and scale loads are issued after them, so a full
  // vmcnt(0) would wait for those too; there the compiler's barrier, which
  // waits for the direct loads with vmcnt(number of later loads), is used
  // (checked on the generated code by the test suite).
  auto stage_barrier = [&]() {
    if constexpr (NV)
      __syncthreads();
    else
      dma_barrier();
  };

  // Stages alternate between the two buffers; the loop body covers two stages
  // and has no branches, the last one or two stages are peeled off.
  if constexpr (NV) load_codes(0);
  issue_stage(0, As0, Bs0);
  stage_barrier();  // waits for the direct loads and meets the other waves
  int64_t kt = 0;
  for (; kt + 2 < nstages; kt += 2) {
    issue_stage(kt + 1, As1, Bs1);
    sched_fence();  // keep the loads ahead of the MFMAs they overlap with
    compute(As0, Bs0, 0);
    compute(As0, Bs0, 1);
    stage_barrier();  // stage kt+1 landed; every wave is done with buffer 0
    issue_stage(kt + 2, As0, Bs0);
    sched_fence();
    compute(As1, Bs1, 0);
    compute(As1, Bs1, 1);
    stage_barrier();
  }
  // one or two stages left; the very last may hold a single K-step (H % 64 == 32)
  const bool last_full = (nsteps % 2) == 0;
  const bool two_left = TAIL == 0 ? kt + 1 < nstages : TAIL == 2;
  if (two_left) {
    issue_stage(kt + 1, As1, Bs1);
    sched_fence();
    compute(As0, Bs0, 0);
    compute(As0, Bs0, 1);
    stage_barrier();
    compute(As1, Bs1, 0);
    if (last_full) compute(As1, Bs1, 1);
  } else {
    compute(As0, Bs0, 0);
    if (last_full) compute(As0, Bs0, 1);
  }

  const int64_t rb = m0 + wm * SM;
  const int64_t rows = M - rb < SM ? M - rb : SM;
  const int64_t cb = n0 + wn * SN;
  auto at = [&](int i, int j) -> f32x4 & { return acc[i][j]; };
  // The stage buffers are free once every wave has read its last stage; each
  // wave then stages its epilogue in an LDS area of its own.
  constexpr int STG = stage_rows_floats<FN>();
  constexpr int PER_A = TM * TL_PPR * 16 / (4 * STG), PER_B = TN * TL_PPR * 16 / (4 * STG);
  static_assert(2 * PER_A + 2 * PER_B >= NW, "epilogue staging fits the stage buffers");
  static_assert(STG >= RED_STG_FLOATS, "the reduction's staging fits the logits' area");
  auto wave_stg = [&]() -> float * {
    int w = wave;
    if (w < PER_A) return reinterpret_cast<float *>(As0) + w * STG;
    if ((w -= PER_A) < PER_A) return reinterpret_cast<float *>(As1) + w * STG;
    if ((w -= PER_A) < PER_B) return reinterpret_cast<float *>(Bs0) + w * STG;
    return reinterpret_cast<float *>(Bs1) + (w - PER_B) * STG;
  };
  if (!RED || out != nullptr) {
    // Logits in whole rows; waves whose columns run past V, or rows not
    // 16-byte aligned (V % 8 != 0), store block by block.
    __syncthreads();
    if (V % 8 == 0 && cb + SN <= V)
      store_rows_lds<FM, FN>(at, out, wave_stg(), rb, rows, cb, V, alpha, bias);
    else
      store_blocks<FM, FN>(at, out, rb, rows, cb, V, V, alpha, bias);
  }
  if constexpr (RED) {
    if (out == nullptr) __syncthreads();
    reduce_blocks<FM, FN>(at, static_cast<RowPart *>(args.part), wave_stg(), rb, rows, cb, V, V,
                          alpha, bias);
  }
}

template <int TM, int TN, int WM, int WN, bool NV, bool F16, typename OutT, int TAIL>
hipError_t launch_tail(const TiledArgs &a, hipStream_t stream) {
  const int64_t tiles = ((a.M + TM - 1) / TM) * ((a.V + TN - 1) / TN);
  if constexpr (!NV) {
    if (a.part != nullptr)
      return launch_kernel(tiled_kernel<TM, TN, WM, WN, NV, F16, OutT, true, TAIL>,
                           dim3((unsigned)tiles), dim3(64 * WM * WN), stream, a);
  }
  return launch_kernel(tiled_kernel<TM, TN, WM, WN, NV, F16, OutT, false, TAIL>,
                       dim3((unsigned)tiles), dim3(64 * WM * WN), stream, a);
}

template <int TM, int TN, int WM, int WN, bool NV, bool F16, typename OutT>
hipError_t launch_tm(const TiledArgs &a, hipStream_t stream) {
  if constexpr (TM == 256) {
    const int64_t nstages = (a.H / KSTEP + 1) / 2;  // as in the kernel
    return nstages % 2 == 0 ? launch_tail<TM, TN, WM, WN, NV, F16, OutT, 2>(a, stream)
                            : launch_tail<TM, TN, WM, WN, NV, F16, OutT, 1>(a, stream);
  } else {
    return launch_tail<TM, TN, WM, WN, NV, F16, OutT, 0>(a, stream);
  }
}

template <bool F16, typename OutT>
hipError_t launch_t(const TiledArgs &a, hipStream_t stream) {
  if (a.M > 128) return launch_tm<256, 256, 4, 2, false, F16, OutT>(a, stream);
  // M <= 128: one 128-row tile covers M; four waves (2 x 2), two tiles
  // resident per CU. The tile width (128 or 160) is the one
  // with the smaller (rounds of resident tiles) x width, since a partial last
  // round costs a whole round: at V = 151936, 160 gives 950 tiles (2 rounds
  // of 512) against 1187 (3 rounds), measured 8-11% faster; at V = 128256,
  // 128 gives 1002 tiles (2 rounds).
  const int64_t slots = 2 * (int64_t)device_cus();
  auto cost = [&](int64_t tn) { return ((a.V + tn - 1) / tn + slots - 1) / slots * tn; };
  return cost(160) < cost(128) ? launch_tm<128, 160, 2, 2, false, F16, OutT>(a, stream)
                               : launch_tm<128, 128, 2, 2, false, F16, OutT>(a, stream);
}

}  // namespace

hipError_t launch_tiled(const GemmArgs &a, hipStream_t stream) {
  const TiledArgs t{a.hidden, a.M, a.H, a.W, nullptr, nullptr, a.V, a.alpha, a.bias, a.out, a.part};
  if (a.in_f16)
    return a.out_type == OUT_F32 ? launch_t<true, float>(t, stream)
                                 : launch_t<true, _Float16>(t, stream);
  return a.out_type == OUT_F32 ? launch_t<false, float>(t, stream)
                               : launch_t<false, uint16_t>(t, stream);
}

hipError_t launch_tiled_nvfp4(const Nvfp4Args &a, hipStream_t stream) {
  const TiledArgs t{a.hidden, a.M, a.H, nullptr, a.codes, a.scales, a.V, a.scale, a.bias, a.out,
                    nullptr};
  // More than 128 rows: 256 x 256 tiles of eight waves, which decode each
  // weight element once per 256 rows (M = 256: 190 against 213 µs for
  // 128 x 128 tiles, measured once the decode stores were free of bank
  // conflicts; before, the larger tile was 12% slower). Up to 128 rows:
  // 128 x 128 tiles of four waves, two resident per CU.
  if (a.M > 128) return launch_tm<256, 256, 4, 2, true, false, uint16_t>(t, stream);
  return launch_tm<128, 128, 2, 2, true, false, uint16_t>(t, stream);
}

}  // namespace lmhead
