// tiled.hip -- LDS-tiled MFMA GEMM for large M (verify and prefill).
//
// logits[M, V] = alpha * hidden[M, H] . W[V, H]^T (+ bias) with bf16 inputs,
// fp32 accumulation and fp32 or bf16 output, the fast path of the sglang
// digest (key source excerpt of _compute_lm_head: a bf16 x bf16 -> fp32 mm
// with no fp32 copies of either operand) and the fused alpha of vLLM PR 49120
// (section "muP is folded into the fp32 GEMM").
//
// Work-group tile BM x BN, K staged through LDS BK at a time; four waves in a
// 2 x 2 arrangement, each owning a (BM/2) x (BN/2) sub-tile of 16 x 16 MFMA
// blocks. Every output element is built by the K-step chain of kstep.hpp --
// ascending K, one accumulator, the same operand map -- so a row's bits equal
// the skinny kernel's and do not depend on M.
//
// LDS layout: [row][16-byte chunk] with the chunk index xor-ed by (row & 7),
// so the 16 rows a K-step reads spread over the banks.
#include "kstep.hpp"
#include "launch.hpp"

namespace lmhead {

namespace {

constexpr int TL_BM = 128;
constexpr int TL_BN = 128;
constexpr int TL_BK = 64;                 // two K-steps per LDS stage
constexpr int TL_CH = TL_BK / 8;          // 16-byte chunks per row per stage
constexpr int TL_THREADS = 256;
constexpr int TL_WM = TL_BM / 2;          // rows per wave
constexpr int TL_WN = TL_BN / 2;          // columns per wave
constexpr int TL_FM = TL_WM / 16;         // 16-row blocks per wave
constexpr int TL_FN = TL_WN / 16;         // 16-column blocks per wave
constexpr int TL_LOADS_A = TL_BM * TL_CH / TL_THREADS;
constexpr int TL_LOADS_B = TL_BN * TL_CH / TL_THREADS;

__device__ __forceinline__ int swz(int row, int chunk) { return row * TL_CH + (chunk ^ (row & 7)); }

template <typename OutT>
__global__ __launch_bounds__(TL_THREADS) void tiled_kernel(const uint16_t *__restrict__ hidden,
                                                           int64_t M, int64_t H,
                                                           const uint16_t *__restrict__ W,
                                                           int64_t V, float alpha,
                                                           const float *__restrict__ bias,
                                                           OutT *__restrict__ out) {
  __shared__ u32x4 As[TL_BM * TL_CH];
  __shared__ u32x4 Bs[TL_BN * TL_CH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 15;
  const int lg = lane >> 4;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  // 1-D grid: the M tiles of one weight tile are neighbours in launch order.
  const int64_t nmt = (M + TL_BM - 1) / TL_BM;
  const int64_t m0 = ((int64_t)blockIdx.x % nmt) * TL_BM;
  const int64_t n0 = ((int64_t)blockIdx.x / nmt) * TL_BN;

  // Global -> register staging: each thread moves TL_LOADS_{A,B} 16-byte chunks.
  const u32x4 *ga[TL_LOADS_A];
  bool va[TL_LOADS_A];
  int la[TL_LOADS_A], ca[TL_LOADS_A];
#pragma unroll
  for (int p = 0; p < TL_LOADS_A; ++p) {
    int idx = p * TL_THREADS + tid;
    int row = idx / TL_CH, ch = idx % TL_CH;
    int64_t grow = m0 + row;
    va[p] = grow < M;
    ga[p] = reinterpret_cast<const u32x4 *>(hidden + (va[p] ? grow : 0) * H) + ch;
    la[p] = swz(row, ch);
    ca[p] = ch;
  }
  const u32x4 *gb[TL_LOADS_B];
  bool vb[TL_LOADS_B];
  int lb[TL_LOADS_B], cb[TL_LOADS_B];
#pragma unroll
  for (int p = 0; p < TL_LOADS_B; ++p) {
    int idx = p * TL_THREADS + tid;
    int row = idx / TL_CH, ch = idx % TL_CH;
    int64_t gcol = n0 + row;
    vb[p] = gcol < V;
    gb[p] = reinterpret_cast<const u32x4 *>(W + (vb[p] ? gcol : 0) * H) + ch;
    lb[p] = swz(row, ch);
    cb[p] = ch;
  }

  const u32x4 z = {0u, 0u, 0u, 0u};
  u32x4 ra[TL_LOADS_A], rb[TL_LOADS_B];
  // A stage covers k in [kt*BK, kt*BK + BK); its second half lies past the
  // row end when H / 32 is odd, and those chunks are never read from memory.
  const int64_t hch = H / 8;  // 16-byte chunks per row
  auto load_stage = [&](int64_t kt) {
    const int64_t off = kt * TL_CH;  // in 16-byte chunks
#pragma unroll
    for (int p = 0; p < TL_LOADS_A; ++p) ra[p] = (va[p] && off + ca[p] < hch) ? ga[p][off] : z;
#pragma unroll
    for (int p = 0; p < TL_LOADS_B; ++p) rb[p] = (vb[p] && off + cb[p] < hch) ? gb[p][off] : z;
  };
  auto store_stage = [&]() {
#pragma unroll
    for (int p = 0; p < TL_LOADS_A; ++p) As[la[p]] = ra[p];
#pragma unroll
    for (int p = 0; p < TL_LOADS_B; ++p) Bs[lb[p]] = rb[p];
  };

  f32x4 acc[TL_FM][TL_FN];
#pragma unroll
  for (int i = 0; i < TL_FM; ++i)
#pragma unroll
    for (int j = 0; j < TL_FN; ++j) acc[i][j] = zero4();

  // H % 32 == 0 but not necessarily % 64: the last stage may hold one K-step.
  const int64_t nsteps = H / KSTEP;
  const int64_t nstages = (nsteps + 1) / 2;

  load_stage(0);
  store_stage();
  __syncthreads();
  for (int64_t kt = 0; kt < nstages; ++kt) {
    if (kt + 1 < nstages) load_stage(kt + 1);
    const int ks_here = (kt * 2 + 1 < nsteps) ? 2 : 1;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s < ks_here) {
        u32x4 a[TL_FM], b[TL_FN];
#pragma unroll
        for (int i = 0; i < TL_FM; ++i) a[i] = As[swz(wm * TL_WM + 16 * i + li, 4 * s + lg)];
#pragma unroll
        for (int j = 0; j < TL_FN; ++j) b[j] = Bs[swz(wn * TL_WN + 16 * j + li, 4 * s + lg)];
#pragma unroll
        for (int i = 0; i < TL_FM; ++i)
#pragma unroll
          for (int j = 0; j < TL_FN; ++j) acc[i][j] = kstep(acc[i][j], a[i], b[j]);
      }
    }
    __syncthreads();
    if (kt + 1 < nstages) {
      store_stage();
      __syncthreads();
    }
  }

#pragma unroll
  for (int j = 0; j < TL_FN; ++j) {
    const int64_t col = n0 + wn * TL_WN + 16 * j + li;
    if (col >= V) continue;
#pragma unroll
    for (int i = 0; i < TL_FM; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = m0 + wm * TL_WM + 16 * i + 4 * lg + q;
        if (row < M) store_out<OutT>(out, row * V + col, epilogue(acc[i][j][q], alpha, bias, col));
      }
    }
  }
}

}  // namespace

hipError_t launch_tiled(const Bf16Args &a, hipStream_t stream) {
  dim3 grid((unsigned)(((a.V + TL_BN - 1) / TL_BN) * ((a.M + TL_BM - 1) / TL_BM)));
  dim3 block(TL_THREADS);
  if (a.out_bf16)
    hipLaunchKernelGGL((tiled_kernel<uint16_t>), grid, block, 0, stream, a.hidden, a.M, a.H, a.W,
                       a.V, a.alpha, a.bias, static_cast<uint16_t *>(a.out));
  else
    hipLaunchKernelGGL((tiled_kernel<float>), grid, block, 0, stream, a.hidden, a.M, a.H, a.W, a.V,
                       a.alpha, a.bias, static_cast<float *>(a.out));
  return hipGetLastError();
}

}  // namespace lmhead
