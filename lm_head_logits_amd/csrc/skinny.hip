// skinny.hip -- the weight-streaming split-V kernel for decode-sized M (<= 64).
//
// At decode sizes the projection is a stream of the whole bf16 weight from
// HBM (the sglang digest's motivation section: the fp32 head's cost was the
// weight traffic, which the bf16 x bf16 -> fp32 path cuts to one read of the
// bf16 weight). Each wave owns NB column blocks of 16 vocabulary rows and
// walks the full H for them, loading 16 contiguous bytes per lane per weight
// row straight into the MFMA B operand; the hidden rows (<= 64, L2-resident)
// feed the A operand the same way. The K-step chain is the one of kstep.hpp,
// so the results equal the tiled GEMM's bit for bit.
//
// Grid (1-D): vocabulary slices of 4 waves * NB * 16 columns times 64-row
// blocks of M (one block for M <= 64; the forced-path test drives more).
#include "kstep.hpp"
#include "launch.hpp"

namespace lmhead {

namespace {

constexpr int SK_WAVES = 4;
constexpr int SK_NB = 4;  // 16-column blocks per wave

template <int R, typename OutT>
__global__ __launch_bounds__(256) void skinny_kernel(const uint16_t *__restrict__ hidden, int64_t M,
                                                     int64_t H, const uint16_t *__restrict__ W,
                                                     int64_t V, float alpha,
                                                     const float *__restrict__ bias,
                                                     OutT *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int li = lane & 15;
  const int lg = lane >> 4;
  // 1-D grid: the 64-row blocks of one vocabulary slice are neighbours.
  const int64_t nmb = (M + 63) / 64;
  const int64_t m0 = ((int64_t)blockIdx.x % nmb) * 64;
  const int64_t col0 = (((int64_t)blockIdx.x / nmb) * SK_WAVES + wave) * (SK_NB * 16);
  if (col0 >= V) return;  // no barriers in this kernel: a wave may leave early

  const u32x4 *bp[SK_NB];
  bool bv[SK_NB];
#pragma unroll
  for (int j = 0; j < SK_NB; ++j) {
    int64_t col = col0 + 16 * j + li;
    bv[j] = col < V;
    bp[j] = reinterpret_cast<const u32x4 *>(W + (bv[j] ? col : 0) * H + 8 * lg);
  }
  const u32x4 *ap[R];
  bool av[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int64_t row = m0 + 16 * r + li;
    av[r] = row < M;
    ap[r] = reinterpret_cast<const u32x4 *>(hidden + (av[r] ? row : 0) * H + 8 * lg);
  }

  f32x4 acc[SK_NB][R];
#pragma unroll
  for (int j = 0; j < SK_NB; ++j)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[j][r] = zero4();

  const u32x4 z = {0u, 0u, 0u, 0u};
  const int64_t nk = H / KSTEP;
#pragma unroll 4
  for (int64_t s = 0; s < nk; ++s) {
    u32x4 b[SK_NB], a[R];
#pragma unroll
    for (int j = 0; j < SK_NB; ++j) b[j] = bv[j] ? bp[j][s * 4] : z;
#pragma unroll
    for (int r = 0; r < R; ++r) a[r] = av[r] ? ap[r][s * 4] : z;
#pragma unroll
    for (int j = 0; j < SK_NB; ++j)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[j][r] = kstep(acc[j][r], a[r], b[j]);
  }

#pragma unroll
  for (int j = 0; j < SK_NB; ++j) {
    const int64_t col = col0 + 16 * j + li;
    if (col >= V) continue;
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = m0 + 16 * r + 4 * lg + q;
        if (row < M) store_out<OutT>(out, row * V + col, epilogue(acc[j][r][q], alpha, bias, col));
      }
    }
  }
}

template <int R>
hipError_t launch_r(const Bf16Args &a, hipStream_t stream) {
  dim3 grid((unsigned)(((a.V + SK_WAVES * SK_NB * 16 - 1) / (SK_WAVES * SK_NB * 16)) *
                       ((a.M + 63) / 64)));
  dim3 block(64 * SK_WAVES);
  if (a.out_bf16)
    hipLaunchKernelGGL((skinny_kernel<R, uint16_t>), grid, block, 0, stream, a.hidden, a.M, a.H,
                       a.W, a.V, a.alpha, a.bias, static_cast<uint16_t *>(a.out));
  else
    hipLaunchKernelGGL((skinny_kernel<R, float>), grid, block, 0, stream, a.hidden, a.M, a.H, a.W,
                       a.V, a.alpha, a.bias, static_cast<float *>(a.out));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_skinny(const Bf16Args &a, hipStream_t stream) {
  // Row blocks per 64-row chunk: only as many as the rows present need.
  const int64_t rows = a.M < 64 ? a.M : 64;
  switch ((rows + 15) / 16) {
    case 1: return launch_r<1>(a, stream);
    case 2: return launch_r<2>(a, stream);
    case 3: return launch_r<3>(a, stream);
    default: return launch_r<4>(a, stream);
  }
}

}  // namespace lmhead
