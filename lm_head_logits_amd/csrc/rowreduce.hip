// rowreduce.hip -- folds the per-block row partials of the GEMM epilogue into
// each row's softmax quantities: the largest logit, its column (the lowest
// one among equal maxima) and s = sum over columns of exp(logit - max), so
// that log-sum-exp = max + log(s).
//
// These are the quantities the pages need after the projection: the target
// and draft heads' acceptance distributions (vLLM PR 49120, section Purpose)
// and greedy selection that is stable under ties, the lowest index first
// (tokenspeed PR 720: its summary on target-equivalent greedy MTP and routing
// ties, and the stable descending sort in its review thread). A vocabulary
// shard's triple is also all a multi-GPU head would exchange per row.
//
// Order: work-group = one row, RC_THREADS threads; thread t folds blocks t,
// t + RC_THREADS, t + 2 RC_THREADS, ... in ascending order (their loads are
// issued RC_BATCH at a time, ahead of the folds), then the 64 lanes of a wave
// meet in a butterfly (DPP steps within each 16-lane row, then xor 16 and
// 32) and the waves' results in a 16-lane DPP butterfly. Every fold is
// symmetric (both partners of a butterfly
// step compute the same bits), and the order depends only on V, so a row's
// result does not depend on M or on which GEMM kernel wrote the partials.
#include "kstep.hpp"
#include "launch.hpp"

namespace lmhead {

namespace {

constexpr int RC_THREADS = 1024;
constexpr int RC_WAVES = RC_THREADS / 64;
constexpr int RC_BATCH = 16;  // one round of loads for V <= 16 * RC_BATCH * RC_THREADS

struct RowAcc {
  float m;  // largest logit so far (-inf: nothing yet)
  float s;  // sum of exp(logit - m) so far
  int i;    // column of m
};

// (m, i) is the larger maximum, ties to the lower column; each sum is
// rescaled to the new maximum and the two are added. Symmetric in a and b.
// An empty side (s == 0: no column yet, or only -inf logits) contributes
// nothing and never reaches the exponential with an infinite difference; a
// side with s > 0 has a finite maximum, and r.m >= it, so its difference is
// finite or the exponential of -inf (0).
__device__ __forceinline__ RowAcc fold(RowAcc a, RowAcc b) {
  RowAcc r = a;
  max_lowest(r.m, r.i, b.m, b.i);
  const float ta = a.s == 0.0f ? 0.0f : __fmul_rn(a.s, exp_fast(__fsub_rn(a.m, r.m)));
  const float tb = b.s == 0.0f ? 0.0f : __fmul_rn(b.s, exp_fast(__fsub_rn(b.m, r.m)));
  r.s = __fadd_rn(ta, tb);
  return r;
}

__device__ __forceinline__ RowAcc shfl_xor(RowAcc a, int d) {
  return RowAcc{__shfl_xor(a.m, d), __shfl_xor(a.s, d), __shfl_xor(a.i, d)};
}

// The partner's RowAcc within a 16-lane row by DPP (no LDS round trip).
template <int CTRL>
__device__ __forceinline__ RowAcc dpp_acc(RowAcc a) {
  return RowAcc{dpp<CTRL>(a.m), dpp<CTRL>(a.s), dpp<CTRL>(a.i)};
}

// Butterfly over the 16 lanes of each row: partner lane l ^ 1, l ^ 2 (quad
// permutations), then the mirror inside 8 lanes and inside 16 lanes -- the
// same pairs of groups an xor butterfly 4, 8 meets, so every lane ends with
// the row's fold and both partners of each step fold the same two values.
__device__ __forceinline__ RowAcc row16_fold(RowAcc a) {
  a = fold(a, dpp_acc<DPP_QUAD_SWAP1>(a));
  a = fold(a, dpp_acc<DPP_QUAD_SWAP2>(a));
  a = fold(a, dpp_acc<DPP_ROW_HALF_MIRROR>(a));
  return fold(a, dpp_acc<DPP_ROW_MIRROR>(a));
}

constexpr RowAcc EMPTY{-__builtin_inff(), 0.0f, 0x7FFFFFFF};

__global__ __launch_bounds__(RC_THREADS) void row_combine_kernel(
    const RowPart *__restrict__ part, int64_t ncb, float *__restrict__ row_max,
    int32_t *__restrict__ row_argmax, float *__restrict__ row_sumexp) {
  const int64_t row = blockIdx.x;
  const RowPart *p = part + row * ncb;
  RowAcc a = EMPTY;
  for (int64_t c0 = threadIdx.x; c0 < ncb; c0 += (int64_t)RC_BATCH * RC_THREADS) {
    RowPart v[RC_BATCH];
#pragma unroll
    for (int k = 0; k < RC_BATCH; ++k) {
      const int64_t cb = c0 + (int64_t)k * RC_THREADS;
      v[k] = cb < ncb ? p[cb] : RowPart{-__builtin_inff(), 0.0f, 0x7FFFFFFF, 0};
    }
#pragma unroll
    for (int k = 0; k < RC_BATCH; ++k) a = fold(a, RowAcc{v[k].m, v[k].s, v[k].i});
  }
  a = row16_fold(a);
  a = fold(a, shfl_xor(a, 16));
  a = fold(a, shfl_xor(a, 32));
  __shared__ RowAcc w[RC_WAVES];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) w[wave] = a;
  __syncthreads();
  if (wave == 0) {
    a = lane < RC_WAVES ? w[lane] : EMPTY;
    static_assert(RC_WAVES == 16, "the waves' results meet within one 16-lane row");
    a = row16_fold(a);
    if (lane == 0) {
      row_max[row] = a.m;
      row_argmax[row] = a.i;
      row_sumexp[row] = a.s;
    }
  }
}

}  // namespace

hipError_t launch_row_combine(const void *part, int64_t M, int64_t V, float *row_max,
                              int32_t *row_argmax, float *row_sumexp, hipStream_t stream) {
  return launch_kernel(row_combine_kernel, dim3((unsigned)M), dim3(RC_THREADS), stream,
                       static_cast<const RowPart *>(part), (V + 15) / 16, row_max, row_argmax,
                       row_sumexp);
}

}  // namespace lmhead
