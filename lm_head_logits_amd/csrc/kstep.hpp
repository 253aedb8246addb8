// kstep.hpp -- the one K-reduction order every kernel of the library runs.
//
// A row's logits must not depend on the row count of the call (metrale
// "lm_head_nvfp4_rows.rs" source page, module documentation: its row-tile head
// was chosen over a GEMV/GEMM switch whose summation order changes with the
// row count). Here every kernel -- the weight-streaming kernel for decode,
// the LDS-tiled GEMM for prefill and the NVFP4 kernel -- builds each output
// element with exactly this chain and nothing else:
//
//   acc = +0.0f
//   for k0 = s, s + 32, ..., H - 32, 0, 32, ..., s - 32   (s = korder_start(v, H)):
//       acc = MFMA_F32_16x16x32_BF16(acc, h[m, k0 .. k0+31], w[v, k0 .. k0+31])
//
// with one fixed placement of the 32 products inside the instruction (the
// operand map below). The start s depends on the column v and H only
// (korder.hpp: it staggers the weight stream over HBM). There is no split-K,
// no second accumulator and no cross-lane reduction of partial sums, so the
// bits of (m, v) depend only on hidden row m, weight row v and the index v:
// not on M, on the 16-row block or row slot the row lands in, or on which
// kernel ran.
//
// Operand map of one K-step (16 x 16 output block at rows r0.., cols c0..):
//   lane l = 16*g + i  (i = l % 16, g = l / 16)
//   A operand, slot s (0..7): hidden[r0 + i][k0 + 8*g + s]
//   B operand, slot s (0..7): W     [c0 + i][k0 + 8*g + s]
//   accumulator register j : output (r0 + 4*g + j, c0 + i)
// so each lane feeds 16 contiguous bytes of one hidden row and of one weight
// row per K-step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace lmhead {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int KSTEP = 32;  // K consumed by one MFMA

// One step of the chain: acc += A(16 x 32) * B(32 x 16), fp32 out; bf16
// inputs, or fp16 inputs (F16) through the fp16 MFMA of the same shape and
// operand map.
template <bool F16 = false>
__device__ __forceinline__ f32x4 kstep(f32x4 acc, u32x4 a, u32x4 b) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.0f, 0.0f, 0.0f, 0.0f}; }

// ---------------------------------------------------------------------------
// Buffer loads. A buffer resource bounds every access: offsets at or past
// `bytes` read as zero, which is how the kernels fill padding rows and the
// ragged vocabulary tail without branches. Offsets are 32-bit, so each
// resource is based at the start of the region one wave or work-group reads.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Word 3 of a gfx9-family raw (stride 0) buffer resource: 32-bit data format.
constexpr int RSRC_WORD3 = 0x00020000;
// Cache-policy bits of a load: nt marks a read-once stream.
constexpr int LOAD_DEFAULT = 0;
constexpr int LOAD_STREAM = 2;

// The base and size are wave-uniform by construction; readfirstlane makes the
// compiler see that too, so the resource lives in scalar registers (a resource
// it believes divergent turns every load into a loop over lanes).
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  void *ub = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                           RSRC_WORD3);
}

template <int POLICY = LOAD_DEFAULT>
__device__ __forceinline__ u32x4 load16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, POLICY);
}

template <int POLICY = LOAD_DEFAULT>
__device__ __forceinline__ uint32_t load4(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, POLICY);
}

// Work-group barrier that orders LDS only: waits for this wave's LDS
// operations, then meets the other waves. Unlike __syncthreads() it does not
// wait for outstanding global loads, so prefetched weight streams stay in
// flight across it. The memory clobber keeps the compiler from moving LDS
// accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Work-group barrier after which every wave's direct-to-LDS loads have
// landed: waits for all of this wave's vector memory loads (vmcnt) and LDS
// operations, then meets the other waves. A direct load's LDS write is
// counted by vmcnt, and __syncthreads() does not necessarily wait for it:
// this compiler emits vmcnt(0) before the barrier in some loop layouts and
// not in others (seen in the generated code).
__device__ __forceinline__ void dma_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Keeps the compiler from moving any instruction across this point. Used
// before a chunk's hidden rows are written to LDS: hoisting that write above
// the chunk's MFMAs would make it wait for every load issued since the hidden
// load (the whole weight prefetch), draining the stream once per chunk.
__device__ __forceinline__ void sched_fence() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// The epilogue (fp32): t = fl32(alpha * acc); with a bias t = fl32(t + b).
// Two separately rounded operations -- the same bits as the projection
// followed by an elementwise multiply and then an add (vLLM PR 49120, sections
// Purpose and "muP is folded into the fp32 GEMM"). __fmul_rn / __fadd_rn keep
// the compiler from contracting them into one fused multiply-add.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float epilogue(float acc, float alpha, const float *__restrict__ bias,
                                          int64_t col) {
  float t = __fmul_rn(alpha, acc);
  if (bias != nullptr) t = __fadd_rn(t, bias[col]);
  return t;
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// The epilogue with the bias value already loaded (has_bias false: no add).
__device__ __forceinline__ float epilogue_v(float acc, float alpha, bool has_bias, float b) {
  float t = __fmul_rn(alpha, acc);
  if (has_bias) t = __fadd_rn(t, b);
  return t;
}

// Logits are written with the streaming hint by default: they are not
// re-read by this kernel, and keeping them out of the caches spares the next
// call's weight stream (measured: the M = 128 tiled call 7% faster than with
// the default policy). The weight-streaming kernel, whose weight loads carry
// the read-once hint themselves, writes with the default policy (spec-decode
// draft M = 32: 104.5 against 106.5 µs).
constexpr int STORE_POLICY = LOAD_STREAM;

// One output element through a buffer resource: fp32, or bf16 / fp16
// rounded to nearest even (the fp16 conversion's default mode). Offsets past
// the resource are dropped by the hardware.
template <typename OutT, int POLICY = STORE_POLICY>
__device__ __forceinline__ void store_c(rsrc_t r, uint32_t voff, uint32_t soff, float t) {
  if constexpr (sizeof(OutT) == 4)
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, t), r, voff, soff, POLICY);
  else if constexpr (std::is_same_v<OutT, _Float16>)
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (_Float16)t), r, voff, soff,
                                          POLICY);
  else
    __builtin_amdgcn_raw_buffer_store_b16(bf16_rne(t), r, voff, soff, POLICY);
}

// An offset past any output resource (resources are < 1 GiB and scalar
// offsets < 1 GiB, so the sum cannot wrap into range): the store is dropped.
constexpr uint32_t OFF_NONE = 0x80000000u;

// Epilogue of one wave's output blocks, shared by every kernel.
//   acc(i, j)   accumulator of 16-row block i, 16-column block j
//   rows        output rows of the block (from the wave's first row), <= 16*FM
//   rbase       row of the wave's first output row; cbase: its first column
//   cend        end (exclusive) of the columns this wave owns, <= V
// Output element (rbase + 16 i + 4 lg + q, cbase + 16 j + li) of a row-major
// [M, V] matrix. Rows past `rows` are dropped by the resource bound, columns
// >= cend by an out-of-range offset; the bias is read once per column.
template <int FM, int FN, int POLICY = STORE_POLICY, typename OutT, typename Acc>
__device__ __forceinline__ void store_blocks(Acc &&acc, OutT *out, int64_t rbase, int64_t rows,
                                             int64_t cbase, int64_t cend, int64_t V,
                                             float alpha, const float *__restrict__ bias) {
  const int lane = threadIdx.x & 63;
  const int li = lane & 15, lg = lane >> 4;
  // Based at the wave's first element; its size runs to the end of the last
  // row the wave owns, so no store of a valid (row, column) is dropped. A wave
  // with no valid row or no column gets an empty resource (a negative size
  // would wrap to a huge one and let the out-of-range column offset below
  // land inside it).
  const bool any = rows > 0 && cbase < cend;
  const rsrc_t r = make_rsrc(any ? out + rbase * V + cbase : out,
                             any ? (uint32_t)(((rows - 1) * V + (cend - cbase)) * sizeof(OutT)) : 0u);
  const uint32_t lvoff = (uint32_t)((4 * lg * V + li) * sizeof(OutT));
  const bool has_bias = bias != nullptr;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int64_t col = cbase + 16 * j + li;
    const bool ok = col < cend;
    const float b = (has_bias && ok) ? bias[col] : 0.0f;
    const uint32_t voff = ok ? lvoff + (uint32_t)(16 * j * sizeof(OutT)) : OFF_NONE;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        store_c<OutT, POLICY>(r, voff, (uint32_t)((16 * i + q) * V * sizeof(OutT)),
                              epilogue_v(acc(i, j)[q], alpha, has_bias, b));
  }
}

// Bits of the 16-bit output types (round to nearest even).
template <typename OutT>
__device__ __forceinline__ uint16_t out_bits16(float t);
template <>
__device__ __forceinline__ uint16_t out_bits16<uint16_t>(float t) { return bf16_rne(t); }
template <>
__device__ __forceinline__ uint16_t out_bits16<_Float16>(float t) {
  return __builtin_bit_cast(uint16_t, (_Float16)t);
}

// Floats of LDS one wave needs for store_rows_lds with FN column blocks.
template <int FN>
constexpr int stage_rows_floats() { return 16 * (16 * FN + 4); }

// The epilogue of one wave's output through LDS, for whole rows in 16-byte
// stores. Block-row i (16 rows x 16 FN columns) goes to the wave-private LDS
// area `stg` row by row (row stride 16 FN + 4 floats: the four 4-row groups
// of a block write distinct banks), is read back along its rows and written
// with 16-byte buffer stores, so the bytes of a row leave as full cache lines
// instead of one 64-byte (fp32) or 32-byte (16-bit) piece per store and row.
// The values are those store_blocks writes. Requires: columns
// [cbase, cbase + 16 FN) all inside the output (the caller checks), V % 8 == 0
// (16-byte aligned rows), `stg` 16-byte aligned with
// stage_rows_floats<FN>() floats. Rows from `rows` on are dropped.
template <int FM, int FN, typename OutT, typename Acc>
__device__ __forceinline__ void store_rows_lds(Acc &&acc, OutT *out, float *stg, int64_t rbase,
                                               int64_t rows, int64_t cbase, int64_t V,
                                               float alpha, const float *__restrict__ bias) {
  constexpr int SN = 16 * FN, STR = SN + 4;
  constexpr bool F32 = sizeof(OutT) == 4;
  constexpr int EPS = F32 ? 4 : 8;        // elements per 16-byte store
  constexpr int SPR = SN / EPS;           // stores per row
  constexpr int NITEM = 16 * SPR;         // stores per block-row
  static_assert(SN % EPS == 0, "whole 16-byte stores per row");
  const int lane = threadIdx.x & 63;
  const int li = lane & 15, lg = lane >> 4;
  const rsrc_t r = make_rsrc(rows > 0 ? out + rbase * V + cbase : out,
                             rows > 0 ? (uint32_t)(((rows - 1) * V + SN) * sizeof(OutT)) : 0u);
  const bool has_bias = bias != nullptr;
  float b[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) b[j] = has_bias ? bias[cbase + 16 * j + li] : 0.0f;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        stg[(4 * lg + q) * STR + 16 * j + li] = epilogue_v(acc(i, j)[q], alpha, has_bias, b[j]);
    __builtin_amdgcn_wave_barrier();  // other lanes' values: LDS keeps a wave's order
#pragma unroll
    for (int k = 0; k < (NITEM + 63) / 64; ++k) {
      const int u = 64 * k + lane;
      const bool ok = u < NITEM;
      const int row = ok ? u / SPR : 0, c = u % SPR;
      const uint32_t voff = ok ? (uint32_t)(((16 * i + row) * V + EPS * c) * sizeof(OutT)) : OFF_NONE;
      const f32x4 *src = reinterpret_cast<const f32x4 *>(stg + row * STR + EPS * c);
      u32x4 v;
      if constexpr (F32) {
        v = __builtin_bit_cast(u32x4, src[0]);
      } else {
        const f32x4 lo = src[0], hi = src[1];
        v = u32x4{(uint32_t)out_bits16<OutT>(lo[0]) | ((uint32_t)out_bits16<OutT>(lo[1]) << 16),
                  (uint32_t)out_bits16<OutT>(lo[2]) | ((uint32_t)out_bits16<OutT>(lo[3]) << 16),
                  (uint32_t)out_bits16<OutT>(hi[0]) | ((uint32_t)out_bits16<OutT>(hi[1]) << 16),
                  (uint32_t)out_bits16<OutT>(hi[2]) | ((uint32_t)out_bits16<OutT>(hi[3]) << 16)};
      }
      __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, 0, STORE_POLICY);
    }
    __builtin_amdgcn_wave_barrier();  // reads of this block-row before the next one's writes
  }
}

// ---------------------------------------------------------------------------
// Row-reduction epilogue: instead of (or besides) the logits, per-row
// partials over each 16-column block -- the block's largest logit t_max, the
// lowest column holding it, and the sum of exp(t - t_max) over the block's
// columns -- for the softmax quantities of a row (its maximum, argmax with
// the lowest index winning ties, and log-sum-exp) without a second pass over
// [M, V] logits. The logit t is the epilogue value above, so the partials
// reduce exactly the fp32 logits the plain call writes.
//
// Logits of -inf (masked entries) are allowed: a block of only -inf keeps
// its lowest column and sums 0, and contributes nothing to a row that has a
// finite logit. +inf and NaN logits are outside the contract.
//
// A block's partial depends only on the block's 16 logits and their column
// positions: the maximum and its column are exact, and the sum has one fixed
// order. Each row's 16 logits pass through a wave-private LDS area so that
// four lanes hold four consecutive columns each: a lane sums its four terms
// in column order, then the four lanes meet in a butterfly (pairs, then
// quads), in which both partners of every step add the same two values (the
// same bits). So the partials, and the combined row results, are the same
// whichever kernel ran and however many rows the call had. (When the
// maximum is a zero present with both signs, the sign of the zero stored is
// the hardware maximum's.)
//
// Record of row m, block cb at part[m * ncb + cb] (ncb = ceil(V / 16)).
// ---------------------------------------------------------------------------
// Written and read as a struct: with this compiler, __builtin_bit_cast of a
// vector element (v.y of a u32x4) compiled to a read of element 0.
struct alignas(16) RowPart {
  float m;    // the block's largest logit
  float s;    // sum over the block's columns of exp(logit - m)
  int32_t i;  // lowest column holding m
  int32_t pad;
};

// (value, column) maximum with the lowest column winning ties; the same
// answer for either argument order.
__device__ __forceinline__ void max_lowest(float &m, int &mi, float om, int oi) {
  if (om > m || (om == m && oi < mi)) {
    m = om;
    mi = oi;
  }
}

// Butterfly steps over the four lanes of a quad (lanes 4 r .. 4 r + 3):
// partner lane l ^ 1, then l ^ 2.
constexpr int DPP_QUAD_SWAP1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int DPP_QUAD_SWAP2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;  // lane i <-> 7 - i within 8
constexpr int DPP_ROW_MIRROR = 0x140;       // lane i <-> 15 - i within 16

template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, dpp<CTRL>(__builtin_bit_cast(int, v)));
}

// e^x as 2^(x log2 e) (the hardware exp2 of a rounded product).
__device__ __forceinline__ float exp_fast(float x) { return __expf(x); }

// Floats of LDS one wave needs for reduce_blocks (16 rows of 16 logits,
// row stride 20: the writes of one register, rows 4 g + q at lanes 16 g + i,
// land in distinct banks, and each row's four 16-byte pieces stay aligned).
constexpr int RED_STRIDE = 20;
constexpr int RED_STG_FLOATS = 16 * RED_STRIDE;

// The row partials of a wave's FM x FN blocks (rows rbase.., columns cbase..,
// columns from cend on absent). `stg`: RED_STG_FLOATS floats of LDS of this
// wave's own, 16-byte aligned, free for the duration.
template <int FM, int FN, typename Acc>
__device__ __forceinline__ void reduce_blocks(Acc &&acc, RowPart *__restrict__ part, float *stg,
                                              int64_t rbase, int64_t rows, int64_t cbase,
                                              int64_t cend, int64_t V, float alpha,
                                              const float *__restrict__ bias) {
  const int lane = threadIdx.x & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int rr = lane >> 2, t = lane & 3;  // reading side: row rr, columns 4 t .. 4 t + 3
  const int64_t ncb = (V + 15) / 16;
  const bool has_bias = bias != nullptr;
  constexpr float NEG_INF = -__builtin_inff();
  // every block's bias first: its loads in flight together, not one
  // round trip per block
  float bj[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int64_t col = cbase + 16 * j + li;
    bj[j] = (has_bias && col < cend) ? bias[col] : 0.0f;
  }
  // columns fit 32 bits (V <= 2^20 by the shape contract); this lane's record
  // slot for block 0 of its row
  const int cw = (int)cbase + 4 * t;  // the reading lane's first column in block 0
  RowPart *prow = part + (rbase + rr) * ncb + (cbase >> 4);
  const int nok = (int)(cend - cbase);  // columns present from cbase on
  // the body once with and once without the bias add (a uniform choice)
  auto run = [&](auto hb) {
    constexpr bool HB = decltype(hb)::value;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if (16 * j >= nok) break;  // wave-uniform: this and later blocks have no column
      const bool ok = 16 * j + li < nok;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        // the block's logits, row-major (absent columns -inf)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float tv = epilogue_v(acc(i, j)[q], alpha, HB, bj[j]);
          stg[(4 * lg + q) * RED_STRIDE + li] = ok ? tv : NEG_INF;
        }
        __builtin_amdgcn_wave_barrier();  // other lanes' values: LDS keeps a wave's order
        const f32x4 v = *reinterpret_cast<const f32x4 *>(stg + rr * RED_STRIDE + 4 * t);
        __builtin_amdgcn_wave_barrier();  // this read before the next block's writes
        float m = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
        m = fmaxf(m, dpp<DPP_QUAD_SWAP1>(m));
        m = fmaxf(m, dpp<DPP_QUAD_SWAP2>(m));
        // lowest column holding m: the absent columns (-inf) come after every
        // present one, and a block has a present column, so one of those wins
        int mi = 0x7FFFFFFF;
#pragma unroll
        for (int k = 3; k >= 0; --k)
          if (v[k] == m) mi = cw + 16 * j + k;
        mi = min(mi, dpp<DPP_QUAD_SWAP1>(mi));
        mi = min(mi, dpp<DPP_QUAD_SWAP2>(mi));
        // a block whose logits are all -inf (a masked vocabulary range) has
        // m = -inf and sums nothing: its terms are taken against 0 instead
        // (exp(-inf - 0) = 0), never exp(-inf + inf)
        const float mz = m == NEG_INF ? 0.0f : m;
        float e = exp_fast(__fsub_rn(v[0], mz));
#pragma unroll
        for (int k = 1; k < 4; ++k) e = __fadd_rn(e, exp_fast(__fsub_rn(v[k], mz)));
        e = __fadd_rn(e, dpp<DPP_QUAD_SWAP1>(e));
        e = __fadd_rn(e, dpp<DPP_QUAD_SWAP2>(e));
        if (t == 0 && 16 * i + rr < rows) prow[16 * i * ncb + j] = RowPart{m, e, mi, 0};
      }
    }
  };
  if (has_bias)
    run(std::true_type{});
  else
    run(std::false_type{});
}

}  // namespace lmhead
