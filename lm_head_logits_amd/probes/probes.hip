// probes.hip -- measurement probes: the HBM read rate and the bf16 MFMA rate
// this part sustains, as context for the projection's fractions of the
// published peaks. Not part of the projection: built into a library of its
// own (liblmhead_probes.so), which only the benchmark and its tests load.
#include "../csrc/kstep.hpp"
#include "../csrc/launch.hpp"
#include "lmhead_probes.h"

namespace lmhead {

namespace {

// Compute units of the current device (256 on MI355X if the query fails:
// only the probes' grid size depends on it).
int probe_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return 256;
  return cus;
}

constexpr int PR_THREADS = 256;
constexpr int PR_U = 8;                      // 4 KB steps in flight per work-group
constexpr int PR_STEP = PR_THREADS * 16;     // bytes per step

// Streams `bytes` (a multiple of 16) once: work-group w reads its own
// contiguous segment [w * seg, (w + 1) * seg), 4 KB per step across its 256
// lanes, PR_U steps in flight, xor-folded (the pattern that reached the
// highest read rate among those measured on this part), with the read-once
// (non-temporal) hint the weight streams of the projection carry. The fold is stored
// only when `flag` is set (the caller passes 0), which keeps the loads live.
__global__ __launch_bounds__(PR_THREADS) void hbm_read_kernel(const uint8_t *__restrict__ buf,
                                                              uint64_t bytes, uint64_t seg,
                                                              int flag,
                                                              uint32_t *__restrict__ sink) {
  uint64_t lo = (uint64_t)blockIdx.x * seg, hi = lo + seg;
  if (lo > bytes) lo = bytes;
  if (hi > bytes) hi = bytes;
  const rsrc_t r = make_rsrc(buf + lo, (uint32_t)(hi - lo));  // reads past hi return zero
  const uint32_t lane = (uint32_t)threadIdx.x * 16;
  uint32_t x = 0;
  for (uint64_t o = 0; o < seg; o += (uint64_t)PR_STEP * PR_U) {
    u32x4 v[PR_U];
#pragma unroll
    for (int u = 0; u < PR_U; ++u)
      v[u] = load16<LOAD_STREAM>(r, lane, (uint32_t)(o + (uint64_t)u * PR_STEP));
#pragma unroll
    for (int u = 0; u < PR_U; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (flag) sink[(uint64_t)blockIdx.x * PR_THREADS + threadIdx.x] = x;
}

// Each wave runs `iters` rounds of 16 independent 16x16x32 bf16 MFMAs on
// register operands: bf16 values near +-1 with varied mantissas (the operand
// bits toggle as real data do; all-zero operands run faster on this part).
__global__ __launch_bounds__(PR_THREADS) void mfma_kernel(int64_t iters, int flag,
                                                          float *__restrict__ sink) {
  const uint32_t lane = threadIdx.x & 63;
  uint32_t s = 0x9E3779B9u * (lane + 1) ^ (0x85EBCA6Bu * (blockIdx.x + 1));
  auto next = [&]() {
    s ^= s << 13;
    s ^= s >> 17;
    s ^= s << 5;
    return s;
  };
  auto bf16_pair = [&]() {
    const uint32_t r = next();
    const uint32_t lo = 0x3F80u | (r & 0x807Fu), hi = 0x3F80u | ((r >> 16) & 0x807Fu);
    return lo | (hi << 16);
  };
  u32x4 a = {bf16_pair(), bf16_pair(), bf16_pair(), bf16_pair()};
  u32x4 b = {bf16_pair(), bf16_pair(), bf16_pair(), bf16_pair()};
  f32x4 acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = zero4();
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = kstep<false>(acc[i], a, b);
    a[0] ^= 0x00010001u;  // a new operand each round, magnitudes unchanged
  }
  float t = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) t += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  if (flag) sink[(uint64_t)blockIdx.x * PR_THREADS + threadIdx.x] = t;
}

}  // namespace

}  // namespace lmhead

extern "C" {

int64_t lmhead_probe_grid(void) { return 4 * (int64_t)lmhead::probe_cus(); }

lmhead_status lmhead_probe_hbm_read(const void *buf, size_t bytes, int flag, uint32_t *sink,
                                    void *stream) {
  if (buf == nullptr || sink == nullptr || bytes % 16 != 0 ||
      reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return LMHEAD_ERR_INVALID;
  if (bytes == 0) return LMHEAD_OK;
  const uint64_t grid = (uint64_t)lmhead_probe_grid();
  const uint64_t unit = (uint64_t)lmhead::PR_STEP * lmhead::PR_U;
  const uint64_t seg = ((bytes + grid - 1) / grid + unit - 1) / unit * unit;
  if (seg > 0xFFFFFFFFull - unit) return LMHEAD_ERR_INVALID;  // 32-bit offsets within a segment
  const hipError_t e = lmhead::launch_kernel(
      lmhead::hbm_read_kernel, dim3((unsigned)grid), dim3(lmhead::PR_THREADS),
      static_cast<hipStream_t>(stream), static_cast<const uint8_t *>(buf), (uint64_t)bytes, seg,
      flag, sink);
  return e == hipSuccess ? LMHEAD_OK : LMHEAD_ERR_DEVICE;
}

lmhead_status lmhead_probe_mfma_bf16(int64_t iters, int flag, float *sink, void *stream,
                                     double *flops) {
  if (iters <= 0 || sink == nullptr) return LMHEAD_ERR_INVALID;
  // two work-groups of four waves per CU: two waves per SIMD
  const int64_t grid = 2 * (int64_t)lmhead::probe_cus();
  if (flops != nullptr) *flops = (double)grid * 4 * (double)iters * 16 * 16384.0;
  const hipError_t e = lmhead::launch_kernel(lmhead::mfma_kernel, dim3((unsigned)grid),
                                             dim3(lmhead::PR_THREADS),
                                             static_cast<hipStream_t>(stream), iters, flag, sink);
  return e == hipSuccess ? LMHEAD_OK : LMHEAD_ERR_DEVICE;
}

}  // extern "C"
