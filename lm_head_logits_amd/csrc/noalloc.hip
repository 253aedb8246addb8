// noalloc.hip -- lmhead_logits_rowreduce for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, hosts
// that forbid allocation): the same kernels, with the per-(row, 16-column
// block) partials in a buffer the library holds instead of a caller-provided
// workspace.
//
// The buffer is a file-scope device array of a fixed size. Each GPU the
// library runs on holds its own copy until the process ends, at its own
// device address, which is looked up once per device (with that device
// current) and used from then on; the array's name on the host is only a
// stand-in for the symbol and is never handed to a kernel. Every call on one
// GPU shares that GPU's array: calls that overlap in time on one GPU (on
// different streams, or from different host threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/lmhead.h"
#include "launch.hpp"

namespace {

static_assert(LMHEAD_NOALLOC_SCRATCH_BYTES % 256 == 0, "whole 256-byte pieces");

// The partials of one call: 16 bytes per row and 16-column block. Every
// record of a call is written by its GEMM before the combine kernel reads it,
// so nothing has to start at zero.
__device__ __align__(256) unsigned char scratch[LMHEAD_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mutex;
void *scratch_ptr[MAX_DEVICES];  // device address of `scratch` per device, once looked up

// The device address of the current device's copy of `scratch`, or nullptr
// when it cannot be had (no device, a device index past the table, or the
// lookup failed).
void *device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

}  // namespace

extern "C" lmhead_status lmhead_logits_rowreduce_noalloc(
    const void *hidden, int64_t M, int64_t H, const void *W, int64_t V, float alpha,
    const float *bias, lmhead_dtype in_dtype, lmhead_dtype out_dtype, void *out, float *row_max,
    int32_t *row_argmax, float *row_sumexp, void *stream, int path) {
  lmhead_status st = lmhead::rowreduce_check(hidden, M, H, W, V, bias, in_dtype, out_dtype, out,
                                             row_max, row_argmax, row_sumexp, path);
  if (st != LMHEAD_OK || M == 0) return st;
  // host-only size check, before any device call
  if (lmhead_rowreduce_workspace_bytes(M, V) > (size_t)LMHEAD_NOALLOC_SCRATCH_BYTES)
    return LMHEAD_ERR_INVALID;
  void *ws = device_scratch();
  if (ws == nullptr) return LMHEAD_ERR_DEVICE;
  return lmhead::rowreduce_run(hidden, M, H, W, V, alpha, bias, in_dtype, out_dtype, out, row_max,
                               row_argmax, row_sumexp, ws, stream, path);
}
