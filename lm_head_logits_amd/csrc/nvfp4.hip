// nvfp4.hip -- the W4A16 NVFP4 head: 4-bit E2M1 weights with one E4M3 scale
// per 16 consecutive weights of a row, bf16 activations, bf16 logits.
//
// The metrale "lm_head_nvfp4_rows.rs" source page (module documentation)
// describes the head: weights stay NVFP4, activations stay 16-bit (casting
// them to E4M3 would fall below the declared precision), rows go through in
// calls of at most 64, and a row's logits do not depend on the row count.
//
// Here one launch covers every 64-row block of the call (the blocks of one
// vocabulary slice are neighbours in launch order, so a weight slice is read
// from HBM once and re-read from cache by the other blocks). Each lane decodes
// the 8 codes it feeds to one MFMA B operand -- e2m1 * e4m3 is exact in bf16
// (at most 6 significant bits, exponent inside bf16's range) -- and the
// K-step chain of kstep.hpp runs unchanged. So this kernel's logits equal
// lmhead_logits on the dequantised weight with alpha = fl32(g * alpha), bit
// for bit.
#include "kstep.hpp"
#include "launch.hpp"

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
__global__ __launch_bounds__(256) void nvfp4_kernel(const uint16_t *__restrict__ hidden, int64_t M,
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
#pragma unroll 2
  for (int64_t s = 0; s < nk; ++s) {
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
hipError_t launch_r(const Nvfp4Args &a, hipStream_t stream) {
  dim3 grid((unsigned)(((a.V + NV_WAVES * NV_NB * 16 - 1) / (NV_WAVES * NV_NB * 16)) *
                       ((a.M + 63) / 64)));
  dim3 block(64 * NV_WAVES);
  hipLaunchKernelGGL((nvfp4_kernel<R>), grid, block, 0, stream, a.hidden, a.M, a.H, a.codes,
                     a.scales, a.V, a.scale, a.bias, a.out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_nvfp4(const Nvfp4Args &a, hipStream_t stream) {
  const int64_t rows = a.M < 64 ? a.M : 64;
  switch ((rows + 15) / 16) {
    case 1: return launch_r<1>(a, stream);
    case 2: return launch_r<2>(a, stream);
    case 3: return launch_r<3>(a, stream);
    default: return launch_r<4>(a, stream);
  }
}

}  // namespace lmhead
