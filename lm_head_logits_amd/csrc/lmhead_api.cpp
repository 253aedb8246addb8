// lmhead_api.cpp -- the C ABI: argument checks, path choice, launch.
//
// Every check is host-side integer work done before anything is enqueued; a
// call that fails one launches nothing (metrale "lm_head_nvfp4_rows.rs"
// page: its row-tile head returns false and launches nothing when it does not
// apply; vLLM PR 49120, section Purpose: cases the fused op does not cover
// fall back). The shape predicates never touch the device.
#include "../../include/lmhead.h"

#include <hip/hip_runtime.h>

#include <atomic>

#include "launch.hpp"

namespace {

constexpr int64_t MAX_MV = (int64_t)1 << 42;  // M * V bound: keeps every grid < 2^31 blocks

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Contract shared by both entry points; returns LMHEAD_OK when the shape is in.
lmhead_status check_shape(int64_t M, int64_t H, int64_t V) {
  if (M < 0 || H <= 0 || V <= 0) return LMHEAD_ERR_INVALID;
  if (M > LMHEAD_MAX_M || H > LMHEAD_MAX_H || V > LMHEAD_MAX_V) return LMHEAD_ERR_INVALID;
  if (M > 0 && M > MAX_MV / V) return LMHEAD_ERR_INVALID;
  if (H % 32 != 0) return LMHEAD_NOT_HANDLED;  // one K-step consumes 32 elements
  return LMHEAD_OK;
}

int auto_path(int64_t M) { return M <= 64 ? LMHEAD_PATH_SKINNY : LMHEAD_PATH_TILED; }

bool known_dtype(int d) { return d == LMHEAD_F32 || d == LMHEAD_BF16 || d == LMHEAD_F16; }

// Host checks shared by the 16-bit entry points, in the order: shape, dtype
// and path values, dtype pair; LMHEAD_OK when the call may proceed.
lmhead_status check_call(int64_t M, int64_t H, int64_t V, int in_dtype, int out_dtype, int path) {
  lmhead_status st = check_shape(M, H, V);
  if (st != LMHEAD_OK) return st;
  if (!known_dtype(in_dtype) || !known_dtype(out_dtype)) return LMHEAD_ERR_INVALID;
  if (path != LMHEAD_PATH_AUTO && path != LMHEAD_PATH_SKINNY && path != LMHEAD_PATH_TILED)
    return LMHEAD_ERR_INVALID;
  // 16-bit inputs of one type; logits fp32 or of the input type
  if (in_dtype == LMHEAD_F32 || (out_dtype != LMHEAD_F32 && out_dtype != in_dtype))
    return LMHEAD_NOT_HANDLED;
  return LMHEAD_OK;
}

// Launches the GEMM with its epilogue writing the logits (out) and / or the
// row-reduction partials (part); arguments already checked.
hipError_t run_gemm(const void *hidden, int64_t M, int64_t H, const void *W, int64_t V,
                    float alpha, const float *bias, lmhead_dtype in_dtype, lmhead_dtype out_dtype,
                    void *out, void *part, hipStream_t s, int path) {
  lmhead::GemmArgs a;
  a.hidden = static_cast<const uint16_t *>(hidden);
  a.M = M;
  a.H = H;
  a.W = static_cast<const uint16_t *>(W);
  a.V = V;
  a.alpha = alpha;
  a.bias = bias;
  a.in_f16 = in_dtype == LMHEAD_F16 ? 1 : 0;
  a.out_type = out_dtype == LMHEAD_F32    ? lmhead::OUT_F32
               : out_dtype == LMHEAD_BF16 ? lmhead::OUT_BF16
                                          : lmhead::OUT_F16;
  a.out = out;
  a.part = part;
  const int p = path == LMHEAD_PATH_AUTO ? auto_path(M) : path;
  return p == LMHEAD_PATH_SKINNY ? lmhead::launch_skinny(a, s) : lmhead::launch_tiled(a, s);
}

int64_t part_bytes(int64_t M, int64_t V) { return 16 * M * ((V + 15) / 16); }

}  // namespace

namespace lmhead {

int device_cus() {
  constexpr int CACHED = 64;
  static std::atomic<int> cache[CACHED];  // zero: not queried yet
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < CACHED && (cus = cache[dev].load(std::memory_order_relaxed)) > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;  // the MI355X count; only the balance of the split depends on it
  if (dev >= 0 && dev < CACHED) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

VSplit vsplit(int64_t ncb, int64_t H, int waves, int nb_max, int per_cu) {
  return split_plan(ncb, H, waves, nb_max, (int64_t)device_cus() * per_cu);
}

lmhead_status rowreduce_check(const void *hidden, int64_t M, int64_t H, const void *W, int64_t V,
                              const float *bias, int in_dtype, int out_dtype, const void *out,
                              const float *row_max, const int32_t *row_argmax,
                              const float *row_sumexp, int path) {
  lmhead_status st = check_call(M, H, V, in_dtype, out_dtype, path);
  if (st != LMHEAD_OK || M == 0) return st;
  if (hidden == nullptr || W == nullptr || row_max == nullptr || row_argmax == nullptr ||
      row_sumexp == nullptr)
    return LMHEAD_ERR_INVALID;
  if (!aligned(hidden, 16) || !aligned(W, 16) || (out != nullptr && !aligned(out, 16)) ||
      !aligned(row_max, 4) || !aligned(row_argmax, 4) || !aligned(row_sumexp, 4) ||
      (bias != nullptr && !aligned(bias, 4)))
    return LMHEAD_ERR_ALIGN;
  return LMHEAD_OK;
}

lmhead_status rowreduce_run(const void *hidden, int64_t M, int64_t H, const void *W, int64_t V,
                            float alpha, const float *bias, int in_dtype, int out_dtype, void *out,
                            float *row_max, int32_t *row_argmax, float *row_sumexp,
                            void *workspace, void *stream, int path) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = run_gemm(hidden, M, H, W, V, alpha, bias, static_cast<lmhead_dtype>(in_dtype),
                          static_cast<lmhead_dtype>(out_dtype), out, workspace, s, path);
  if (e == hipSuccess) e = launch_row_combine(workspace, M, V, row_max, row_argmax, row_sumexp, s);
  return e == hipSuccess ? LMHEAD_OK : LMHEAD_ERR_DEVICE;
}

}  // namespace lmhead

extern "C" {

int lmhead_shape_ok(int64_t M, int64_t H, int64_t V, int nvfp4) {
  (void)nvfp4;  // both entry points share one shape contract
  return check_shape(M, H, V) == LMHEAD_OK ? 1 : 0;
}

int lmhead_path_for(int64_t M, int64_t H, int64_t V, int nvfp4) {
  if (!lmhead_shape_ok(M, H, V, nvfp4)) return LMHEAD_PATH_NONE;
  return nvfp4 ? LMHEAD_PATH_NVFP4 : auto_path(M);
}

const char *lmhead_status_string(int status) {
  switch (status) {
    case LMHEAD_OK: return "ok";
    case LMHEAD_NOT_HANDLED: return "not handled: shape or dtype outside the kernels' contract (caller falls back)";
    case LMHEAD_ERR_INVALID: return "invalid argument";
    case LMHEAD_ERR_ALIGN: return "misaligned pointer";
    case LMHEAD_ERR_DEVICE: return "HIP launch error";
    default: return "unknown status";
  }
}

const char *lmhead_version(void) { return "0.1.0"; }

lmhead_status lmhead_logits_ex(const void *hidden, int64_t M, int64_t H, const void *W, int64_t V,
                               float alpha, const float *bias, lmhead_dtype in_dtype,
                               lmhead_dtype out_dtype, void *out, void *stream, int path) {
  lmhead_status st = check_call(M, H, V, in_dtype, out_dtype, path);
  if (st != LMHEAD_OK) return st;
  if (M == 0) return LMHEAD_OK;  // nothing to do, nothing launched
  if (hidden == nullptr || W == nullptr || out == nullptr) return LMHEAD_ERR_INVALID;
  if (!aligned(hidden, 16) || !aligned(W, 16) || !aligned(out, 16) ||
      (bias != nullptr && !aligned(bias, 4)))
    return LMHEAD_ERR_ALIGN;
  hipError_t e = run_gemm(hidden, M, H, W, V, alpha, bias, in_dtype, out_dtype, out, nullptr,
                          static_cast<hipStream_t>(stream), path);
  return e == hipSuccess ? LMHEAD_OK : LMHEAD_ERR_DEVICE;
}

size_t lmhead_rowreduce_workspace_bytes(int64_t M, int64_t V) {
  if (check_shape(M, 32, V) == LMHEAD_ERR_INVALID) return 0;
  return (size_t)part_bytes(M, V);
}

lmhead_status lmhead_logits_rowreduce(const void *hidden, int64_t M, int64_t H, const void *W,
                                      int64_t V, float alpha, const float *bias,
                                      lmhead_dtype in_dtype, lmhead_dtype out_dtype, void *out,
                                      float *row_max, int32_t *row_argmax, float *row_sumexp,
                                      void *workspace, size_t workspace_bytes, void *stream,
                                      int path) {
  lmhead_status st = lmhead::rowreduce_check(hidden, M, H, W, V, bias, in_dtype, out_dtype, out,
                                             row_max, row_argmax, row_sumexp, path);
  if (st != LMHEAD_OK || M == 0) return st;
  if (workspace == nullptr || workspace_bytes < (size_t)part_bytes(M, V)) return LMHEAD_ERR_INVALID;
  if (!aligned(workspace, 16)) return LMHEAD_ERR_ALIGN;
  return lmhead::rowreduce_run(hidden, M, H, W, V, alpha, bias, in_dtype, out_dtype, out, row_max,
                               row_argmax, row_sumexp, workspace, stream, path);
}

lmhead_status lmhead_logits_path(const void *hidden, int64_t M, int64_t H, const void *W,
                                 int64_t V, float alpha, const float *bias,
                                 lmhead_dtype out_dtype, void *out, void *stream, int path) {
  // the bf16 entry points take fp32 or bf16 logits only
  if (out_dtype != LMHEAD_F32 && out_dtype != LMHEAD_BF16) {
    const lmhead_status st = check_shape(M, H, V);
    return st != LMHEAD_OK ? st : LMHEAD_ERR_INVALID;
  }
  return lmhead_logits_ex(hidden, M, H, W, V, alpha, bias, LMHEAD_BF16, out_dtype, out, stream,
                          path);
}

lmhead_status lmhead_logits(const void *hidden, int64_t M, int64_t H, const void *W, int64_t V,
                            float alpha, const float *bias, lmhead_dtype out_dtype, void *out,
                            void *stream) {
  return lmhead_logits_path(hidden, M, H, W, V, alpha, bias, out_dtype, out, stream,
                            LMHEAD_PATH_AUTO);
}

size_t lmhead_quantize_nvfp4_workspace_bytes(void) { return lmhead::quantize_nvfp4_workspace_bytes(); }

lmhead_status lmhead_quantize_nvfp4(const void *W, int64_t V, int64_t H, uint8_t *w_e2m1,
                                    uint8_t *w_scale, float *global_scale, void *workspace,
                                    size_t workspace_bytes, void *stream) {
  lmhead_status st = check_shape(1, H, V);
  if (st != LMHEAD_OK) return st;
  if (W == nullptr || w_e2m1 == nullptr || w_scale == nullptr || global_scale == nullptr ||
      workspace == nullptr)
    return LMHEAD_ERR_INVALID;
  if (workspace_bytes < lmhead::quantize_nvfp4_workspace_bytes()) return LMHEAD_ERR_INVALID;
  if (!aligned(W, 16) || !aligned(w_e2m1, 4) || !aligned(global_scale, 4) ||
      !aligned(workspace, 4))
    return LMHEAD_ERR_ALIGN;
  hipError_t e = lmhead::launch_quantize_nvfp4(static_cast<const uint16_t *>(W), V, H, w_e2m1,
                                               w_scale, global_scale, workspace,
                                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LMHEAD_OK : LMHEAD_ERR_DEVICE;
}

lmhead_status lmhead_logits_nvfp4(const void *hidden, int64_t M, int64_t H,
                                  const uint8_t *w_e2m1, const uint8_t *w_scale,
                                  float global_scale, int64_t V, float alpha, const float *bias,
                                  void *out, void *stream) {
  lmhead_status st = check_shape(M, H, V);
  if (st != LMHEAD_OK) return st;
  if (M == 0) return LMHEAD_OK;
  if (hidden == nullptr || w_e2m1 == nullptr || w_scale == nullptr || out == nullptr)
    return LMHEAD_ERR_INVALID;
  if (!aligned(hidden, 16) || !aligned(w_e2m1, 16) || !aligned(w_scale, 2) || !aligned(out, 16) ||
      (bias != nullptr && !aligned(bias, 4)))
    return LMHEAD_ERR_ALIGN;

  lmhead::Nvfp4Args a;
  a.hidden = static_cast<const uint16_t *>(hidden);
  a.M = M;
  a.H = H;
  a.codes = w_e2m1;
  a.scales = w_scale;
  a.V = V;
  a.scale = global_scale * alpha;  // one binary32 multiply, rounded once
  a.bias = bias;
  a.out = static_cast<uint16_t *>(out);
  hipError_t e = lmhead::launch_nvfp4(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LMHEAD_OK : LMHEAD_ERR_DEVICE;
}

}  // extern "C"
