// launch.hpp -- host-side launchers of the library's kernels (internal).
// Shapes and alignment are validated by the C ABI before any of these runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lmhead.h"
#include "korder.hpp"

namespace lmhead {

// Element type of the logits.
enum OutType { OUT_F32 = 0, OUT_BF16 = 1, OUT_F16 = 2 };

struct GemmArgs {
  const uint16_t *hidden;  // [M, H] bf16, or fp16 when in_f16
  int64_t M, H;
  const uint16_t *W;       // [V, H] of the same type as hidden
  int64_t V;
  float alpha;
  const float *bias;       // [V] or nullptr
  int in_f16;              // 0: bf16 inputs, 1: fp16 inputs
  OutType out_type;        // OUT_F32, or the input type
  void *out;               // [M, V], or nullptr (no logits written)
  void *part;              // row-reduction partials, 16 B x [M, ceil(V / 16)], or nullptr
};

struct Nvfp4Args {
  const uint16_t *hidden;  // [M, H] bf16
  int64_t M, H;
  const uint8_t *codes;    // [V, H/2] packed E2M1
  const uint8_t *scales;   // [V, H/16] E4M3
  int64_t V;
  float scale;             // fl32(global_scale * alpha)
  const float *bias;       // [V] or nullptr
  uint16_t *out;           // [M, V] bf16
};

// Launches `kernel` on `stream` and returns the launch's own status (not an
// error some earlier, unrelated HIP call left behind). The argument types are
// taken from the kernel's parameter list.
template <typename T>
struct arg_of {
  using type = T;
};
template <typename... P>
hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream,
                         typename arg_of<P>::type... args) {
  void *ptrs[] = {static_cast<void *>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, ptrs, 0, stream);
}

// Compute units of the current device (queried once per device).
int device_cus();

// The vocabulary split of a weight-streaming launch (split_plan in
// korder.hpp) for `per_cu` work-groups per compute unit of the current device.
VSplit vsplit(int64_t ncb, int64_t H, int waves, int nb_max, int per_cu = 1);

// Folds the partials of each row into its (max, argmax, sum of exp(x - max)).
hipError_t launch_row_combine(const void *part, int64_t M, int64_t V, float *row_max,
                              int32_t *row_argmax, float *row_sumexp, hipStream_t stream);

// BF16 -> NVFP4 quantisation of a [V, H] head (two kernels); the workspace
// holds the absmax pass's partial maxima.
size_t quantize_nvfp4_workspace_bytes();
hipError_t launch_quantize_nvfp4(const uint16_t *W, int64_t V, int64_t H, uint8_t *codes,
                                 uint8_t *scales, float *g, void *workspace, hipStream_t stream);

// lmhead_logits_rowreduce in two parts, shared with the entry point that
// takes no workspace: the host checks of everything but the workspace
// (LMHEAD_OK also when M == 0), and the launches with a workspace of at
// least 16 M ceil(V / 16) bytes, 16-byte aligned.
lmhead_status rowreduce_check(const void *hidden, int64_t M, int64_t H, const void *W, int64_t V,
                              const float *bias, int in_dtype, int out_dtype, const void *out,
                              const float *row_max, const int32_t *row_argmax,
                              const float *row_sumexp, int path);
lmhead_status rowreduce_run(const void *hidden, int64_t M, int64_t H, const void *W, int64_t V,
                            float alpha, const float *bias, int in_dtype, int out_dtype, void *out,
                            float *row_max, int32_t *row_argmax, float *row_sumexp,
                            void *workspace, void *stream, int path);

hipError_t launch_skinny(const GemmArgs &a, hipStream_t stream);
hipError_t launch_tiled(const GemmArgs &a, hipStream_t stream);
hipError_t launch_nvfp4(const Nvfp4Args &a, hipStream_t stream);
hipError_t launch_tiled_nvfp4(const Nvfp4Args &a, hipStream_t stream);

}  // namespace lmhead
