// nvfp4_decode.hpp -- NVFP4 weight decoding on gfx950 (internal).
//
// An NVFP4 weight is an OCP E2M1 code times the OCP E4M3 scale of its block
// of 16 consecutive elements of a weight row (metrale "lm_head_nvfp4_rows.rs"
// source page, module documentation). The product has at most 2 + 4 = 6
// significant bits and an exponent inside bf16's range, so it is exact in
// fp32 and in bf16: the upper 16 bits of the fp32 product are its bf16 value.
#pragma once

#include "kstep.hpp"

namespace lmhead {

// Two codes of byte P of `codes` (element 2P in the low nibble, 2P + 1 in the
// high nibble) times the block scale s, as a pair of bf16 (element 2P in the
// low half). v_cvt_scalef32_pk_f32_fp4 with scale 1.0 is the exact E2M1 value.
template <int P>
__device__ __forceinline__ uint32_t dequant_pair(uint32_t codes, float s) {
  const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, P);
  const uint32_t lo = __builtin_bit_cast(uint32_t, v[0] * s);
  const uint32_t hi = __builtin_bit_cast(uint32_t, v[1] * s);
  return __builtin_amdgcn_perm(hi, lo, 0x07060302u);  // upper halves: (lo.bf16, hi.bf16)
}

// Eight codes (one 32-bit word, element 2p in the low nibble of byte p) times
// their block scale -> eight bf16 weights in element order.
__device__ __forceinline__ u32x4 dequant8_fast(uint32_t codes, float s) {
  return u32x4{dequant_pair<0>(codes, s), dequant_pair<1>(codes, s), dequant_pair<2>(codes, s),
               dequant_pair<3>(codes, s)};
}

}  // namespace lmhead
