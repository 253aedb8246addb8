// quant_nvfp4.hip -- BF16 -> NVFP4 quantisation of a head, the step before
// the NVFP4 projection.
//
// Two passes over the weight, as the metrale page
// "layers/mtp_head/new_bf16_moe.rs" runs quantize_to_nvfp4 with an absmax
// kernel and then an NVFP4 kernel (new_nvfp4_draft_moe): the tensor's
// absolute maximum fixes the per-tensor scale, and each block of 16
// consecutive elements of a row is then scaled and rounded. The pages give no
// arithmetic; the two-level recipe here, every step a binary32 operation
// (division correctly rounded), is
//
//   amax = max |w|;  g = amax / (6 * 448), or 1 when that is 0
//   per block:   s = bmax / (6 g)  ->  E4M3, nearest even, at most 448
//                d = e4m3(s) * g
//   per element: code = sign bit of w | E2M1(|w| / d), nearest even, at
//                most 6 (magnitude 0 when d == 0)
//
// so the largest block scale lands on E4M3's largest value and a block's
// largest element on E2M1's. Output layout as the NVFP4 projection reads it:
// codes [V, H/2] (element 2i in the low nibble of byte i), scales [V, H/16].
//
// Both kernels stream: the absmax pass reads the weight once (2 bytes per
// element), the quantiser reads it again and writes 9/16 byte per element.
// Measured at V = 151936, H = 2048 (622 MB of bf16): absmax pass 104 us
// (6.0 TB/s), quantiser 162 us (797 MB, 4.9 TB/s).
#include "kstep.hpp"
#include "launch.hpp"

namespace lmhead {

namespace {

constexpr int QA_BLOCKS = 1024;  // work-groups of the absmax pass = its partial maxima
constexpr int Q_THREADS = 256;
constexpr int QB_BLOCKS = 2048;  // work-groups of the quantiser (grid-stride)

// Largest |x| of the 8 bf16 values in one 16-byte vector, as the bf16
// magnitude bits: for finite values the magnitude order is the integer order.
__device__ __forceinline__ uint32_t absmax8(u32x4 v) {
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    m = max(m, v[k] & 0x7FFFu);
    m = max(m, (v[k] >> 16) & 0x7FFFu);
  }
  return m;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) v = max(v, (uint32_t)__shfl_xor((int)v, d));
  return v;
}

// Pass 1: each work-group's maximum of |w| (bf16 magnitude bits) over a
// grid-stride share of the n8 16-byte vectors.
__global__ __launch_bounds__(Q_THREADS) void absmax_kernel(const u32x4 *__restrict__ w, int64_t n8,
                                                           uint32_t *__restrict__ partial) {
  constexpr int U = 4;  // vectors in flight per thread
  const int64_t stride = (int64_t)gridDim.x * Q_THREADS;
  uint32_t m = 0;
  for (int64_t i0 = (int64_t)blockIdx.x * Q_THREADS + threadIdx.x; i0 < n8; i0 += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + u * stride;
      v[u] = i < n8 ? __builtin_nontemporal_load(&w[i]) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) m = max(m, absmax8(v[u]));
  }
  m = wave_max(m);
  __shared__ uint32_t wm[Q_THREADS / 64];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = wm[0];
#pragma unroll
    for (int k = 1; k < Q_THREADS / 64; ++k) r = max(r, wm[k]);
    partial[blockIdx.x] = r;
  }
}

// binary32 -> OCP E4M3 byte for s >= 0: nearest even, saturating at 448.
// Below 448 the hardware conversion (v_cvt_pk_fp8_f32) rounds to nearest
// even; checked on this part against the rounding written from the format
// (binade [2^e, 2^(e+1)), e >= -6, 4 significant bits) for every
// non-negative finite binary32. From 464 up it does not saturate, hence the
// explicit bound.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float s) {
  if (!(s < 448.0f)) return 0x7Eu;
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(s, 0.0f, 0, false) & 0xFFu;
}

// Two E2M1 codes (x0 in the low nibble, x1 in the high one) into byte `sel`
// of `word`: sign bit of x | magnitude rounded to nearest, ties to the even
// code (the one whose mantissa bit is 0), saturating at 6. The hardware
// conversion with scale 1 (v_cvt_scalef32_pk_fp4_f32) was checked on this
// part to give exactly that -- the threshold rounding below for the
// magnitude, the sign bit of the input (-0 included) -- for every finite
// binary32, and to leave the other bytes of `word` unchanged.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pair(uint32_t word, float x0, float x1) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, x0, x1, 1.0f, SEL);
}

// The same rounding written out: the number of midpoints between
// neighbouring E2M1 values (0, .5, 1, 1.5, 2, 3, 4, 6) that x passes, the
// midpoints below an even code counting when reached (>=), the others only
// when passed (>).
__device__ __forceinline__ uint32_t e2m1_code(float x) {
  return (uint32_t)(x > 0.25f) + (uint32_t)(x >= 0.75f) + (uint32_t)(x > 1.25f) +
         (uint32_t)(x >= 1.75f) + (uint32_t)(x > 2.5f) + (uint32_t)(x >= 3.5f) +
         (uint32_t)(x > 5.0f);
}

// Pass 2: the per-tensor scale from the partial maxima, then the blocks. Two
// neighbouring lanes share a 16-element block: each loads its 16 contiguous
// bytes (8 elements; a wave's loads cover 1 KB without gaps), the pair
// exchanges its maxima, and each lane writes its 4 bytes of codes; the even
// lane writes the block's scale byte.
//
// Codes: fl(w / d) rounded to E2M1 with w's sign. With a normal d whose
// hardware reciprocal r (within 1 ulp) is normal, q = fl(w r) is within
// 2^-22 (relative) of w / d and fl(w / d) within 2^-24, with w's sign. Every
// midpoint the rounding compares against has a 3-bit significand, so when
// |q| lies within 2^-20 of such a value the low 21 bits of its significand
// are near 0 or near 2^21 (flagged below with a margin of 32). Otherwise
// w / d, fl(w / d) and q lie strictly on the same side of every midpoint,
// and q rounds to the same code. Flagged elements (rare) take the division
// itself; so do the blocks whose d is outside the normal range.
__global__ __launch_bounds__(Q_THREADS) void quant_kernel(const u32x4 *__restrict__ w,
                                                          int64_t n8,
                                                          const uint32_t *__restrict__ partial,
                                                          uint32_t *__restrict__ codes,
                                                          uint8_t *__restrict__ scales,
                                                          float *__restrict__ g_out) {
  uint32_t m = 0;
  for (int k = threadIdx.x; k < QA_BLOCKS; k += Q_THREADS) m = max(m, partial[k]);
  m = wave_max(m);
  __shared__ uint32_t wm[Q_THREADS / 64];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  m = wm[0];
#pragma unroll
  for (int k = 1; k < Q_THREADS / 64; ++k) m = max(m, wm[k]);
  const float amax = __uint_as_float(m << 16);
  float g = __fdiv_rn(amax, 2688.0f);  // 6 * 448
  if (g == 0.0f) g = 1.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0) *g_out = g;
  const float g6 = __fmul_rn(6.0f, g);

  // unit u = half of block u / 2; n8 is even and the stride a multiple of 64,
  // so both halves of a block are always in neighbouring lanes of one wave,
  // and both lanes run the same iterations. Each thread takes QU units per
  // iteration, their loads issued together: the stream needs several loads
  // in flight per lane to reach the HBM rate.
  constexpr int QU = 4;
  const int64_t stride = (int64_t)gridDim.x * Q_THREADS;
  for (int64_t u0 = (int64_t)blockIdx.x * Q_THREADS + threadIdx.x; u0 < n8; u0 += QU * stride) {
    u32x4 v[QU];
#pragma unroll
    for (int j = 0; j < QU; ++j) {
      const int64_t u = u0 + j * stride;
      v[j] = u < n8 ? __builtin_nontemporal_load(&w[u]) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < QU; ++j) {
      const int64_t u = u0 + j * stride;
      const uint32_t hm = absmax8(v[j]);
      const uint32_t bm = max(hm, (uint32_t)__shfl_xor((int)hm, 1));
      if (u >= n8) break;  // the same for both lanes of a block
      const uint32_t sb = e4m3_rne_sat(__fdiv_rn(__uint_as_float(bm << 16), g6));
      const float d = __fmul_rn(__builtin_amdgcn_cvt_f32_fp8((int)sb, 0), g);
      // the 8 elements (element 2i + 1 in the upper half of word i)
      float e[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e[2 * i] = __uint_as_float(v[j][i] << 16);
        e[2 * i + 1] = __uint_as_float(v[j][i] & 0xFFFF0000u);
      }
      uint32_t word;
      if (d >= 0x1p-120f && d <= 0x1p120f) {
        const float r = __builtin_amdgcn_rcpf(d);
        float q[8];
        // near: the low 21 significand bits of max(|q|, 0.1) within 32 of 0
        // or of 2^21 ((bits + 32) << 11 drops the bits above them). 0.1 is
        // no 3-bit value and rounds to code 0, as every smaller |q| does.
        uint32_t lowmin = 0xFFFFFFFFu;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          q[k] = __fmul_rn(e[k], r);
          const uint32_t qb = __float_as_uint(fmaxf(fabsf(q[k]), 0.1f));
          lowmin = min(lowmin, (qb << 11) + (32u << 11));
        }
        if (lowmin < (64u << 11)) {  // rare: some quotient is near a rounding boundary
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const uint32_t qb = __float_as_uint(fmaxf(fabsf(q[k]), 0.1f));
            if ((qb << 11) + (32u << 11) < (64u << 11)) q[k] = __fdiv_rn(e[k], d);
          }
        }
        word = e2m1_pair<0>(0u, q[0], q[1]);
        word = e2m1_pair<1>(word, q[2], q[3]);
        word = e2m1_pair<2>(word, q[4], q[5]);
        word = e2m1_pair<3>(word, q[6], q[7]);
      } else {
        // d == 0: the sign bits alone; d outside the normal range: the
        // division itself, rounded by the threshold form
        word = 0u;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint32_t mag = d == 0.0f ? 0u : e2m1_code(__fdiv_rn(fabsf(e[k]), d));
          word |= (mag | (__float_as_uint(e[k]) >> 31 << 3)) << (4 * k);
        }
      }
      codes[u] = word;
      if ((u & 1) == 0) scales[u >> 1] = (uint8_t)sb;
    }
  }
}

}  // namespace

size_t quantize_nvfp4_workspace_bytes() { return QA_BLOCKS * sizeof(uint32_t); }

hipError_t launch_quantize_nvfp4(const uint16_t *W, int64_t V, int64_t H, uint8_t *codes,
                                 uint8_t *scales, float *g, void *workspace, hipStream_t stream) {
  const int64_t n = V * H;  // H % 32 == 0: whole 16-byte vectors and 16-element blocks
  uint32_t *partial = static_cast<uint32_t *>(workspace);
  hipError_t e = launch_kernel(absmax_kernel, dim3(QA_BLOCKS), dim3(Q_THREADS), stream,
                               reinterpret_cast<const u32x4 *>(W), n / 8, partial);
  if (e != hipSuccess) return e;
  return launch_kernel(quant_kernel, dim3(QB_BLOCKS), dim3(Q_THREADS), stream,
                       reinterpret_cast<const u32x4 *>(W), n / 8,
                       static_cast<const uint32_t *>(partial), reinterpret_cast<uint32_t *>(codes),
                       scales, g);
}

}  // namespace lmhead
