/*
 * lmhead.h -- C ABI of the MI355X (gfx950) LM-head logits library.
 *
 *   logits[m, v] = alpha * (hidden[m, :] . W[v, :]) + bias[v]
 *
 * bf16 inputs, fp32 accumulation, fp32 or bf16 output; an NVFP4 weight-only
 * (W4A16) variant with bf16 output. Every output row depends only on its own
 * hidden row, the weight, alpha, bias and the output type: never on how many
 * rows are in the call, where the row sits in it, or which entry point (bf16
 * weight at any M) produced it. Each logit is summed over K in one fixed
 * order, starting at a point that depends on H and on the column's index v
 * within the call (in groups of 10240 columns) and wrapping around; so a call
 * on a row sub-range W + v0*H of the vocabulary (one GPU's shard) gives the
 * full call's columns bit for bit when v0 is a multiple of
 * 10240 * (H / 256) / gcd(5, H / 256) (any v0 when H % 256 != 0 or
 * H == 256: every column then starts at 0), and agrees with them within the
 * fp32 accumulation tolerance otherwise.
 *
 * Where the operation is defined (page title, then section):
 *  - bf16 x bf16 products accumulated at fp32 with fp32 logits and no fp32
 *    copy of the weight: sglang PR 32370 digest "FP32 LM head skips the FP32
 *    cast" (motivation; implementation breakdown; key source excerpt of
 *    _compute_lm_head), and vLLM PR 49120 "Honor fp32 head_dtype in Inkling
 *    muP logits (target + MTP draft)", section Purpose.
 *  - alpha = 1/mup folded into the projection's epilogue, equal bit for bit
 *    to the projection followed by a separate multiply: vLLM PR 49120,
 *    sections Purpose and "muP is folded into the fp32 GEMM (not a bypass)".
 *  - the embedding bias added to the logits: sglang digest, _compute_lm_head
 *    excerpt (embedding_bias argument).
 *  - the NVFP4 head with 16-bit activations and bf16 logits, whose rows do
 *    not depend on the row count, run in calls of at most 64 rows: metrale
 *    "lm_head_nvfp4_rows.rs" source page, module documentation and the row
 *    loop of lm_head_nvfp4_rows_run.
 *  - "launch nothing and report that the fast path does not cover the case",
 *    leaving the caller to fall back: the same metrale page (the Ok(false)
 *    return of lm_head_nvfp4_rows_run) and vLLM PR 49120, section Purpose
 *    (fallback cases the fused op does not cover).
 *
 * Conventions shared by every entry point:
 *  - Every tensor pointer is a DEVICE pointer to memory the caller owns and
 *    keeps alive until the enqueued work has finished. The library never
 *    allocates, frees or synchronises; it only enqueues kernels on `stream`.
 *  - All tensors are dense and row-major: hidden [M, H], W [V, H] (the
 *    nn.Linear layout, used transposed), logits [M, V].
 *  - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *  - `out` must not overlap any input.
 *  - Work is checked on the host before anything is launched; on any non-OK
 *    status nothing was launched. Faults inside a kernel surface at the
 *    caller's next synchronisation, as for any HIP work.
 *  - The library keeps no state between calls apart from HIP's own
 *    once-per-process code-object load; calls from several threads are safe.
 */
#ifndef LMHEAD_H
#define LMHEAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LMHEAD_F32 = 0,   /* fp32, 4 bytes per element */
  LMHEAD_BF16 = 1,  /* bf16, 2 bytes per element (logits: rounded to nearest even) */
  LMHEAD_F16 = 2    /* IEEE fp16, 2 bytes per element (logits: rounded to nearest even) */
} lmhead_dtype;

typedef enum {
  LMHEAD_OK = 0,           /* work enqueued on `stream`, or M == 0 and nothing to do */
  LMHEAD_NOT_HANDLED = 1,  /* well-formed, outside the shape or dtype contract: nothing
                              launched, the caller falls back */
  LMHEAD_ERR_INVALID = -1, /* NULL pointer with M > 0, M < 0, H <= 0, V <= 0, unknown dtype
                              or path, sizes beyond the documented maxima */
  LMHEAD_ERR_ALIGN = -2,   /* a base pointer below its required alignment */
  LMHEAD_ERR_DEVICE = -3   /* HIP reported an error when the kernel was launched */
} lmhead_status;

typedef enum {
  LMHEAD_PATH_NONE = -1,   /* outside the contract: NOT_HANDLED */
  LMHEAD_PATH_AUTO = -2,   /* let the library choose (the normal use) */
  LMHEAD_PATH_SKINNY = 0,  /* weight-streaming split-V kernel, chosen for M <= 64 */
  LMHEAD_PATH_TILED = 1,   /* LDS-tiled MFMA GEMM, chosen for M > 64 */
  LMHEAD_PATH_NVFP4 = 2    /* NVFP4 W4A16 kernel */
} lmhead_path;

/* Shape contract (both entry points):
 *   M >= 0, H >= 32 and H % 32 == 0, V >= 1,
 *   M <= LMHEAD_MAX_M, H <= LMHEAD_MAX_H, V <= LMHEAD_MAX_V.
 * (The kernels address one work-group's block of output rows, and one wave's
 * slice of weight rows, with 32-bit byte offsets; the maxima keep every such
 * block below 1 GiB. V <= 2^20 covers every vocabulary in use.)
 * Alignment: hidden, W, w_e2m1 and out 16-byte aligned; bias 4-byte aligned;
 * w_scale 2-byte aligned. (torch allocations are 256-byte aligned; a row
 * sub-range W + v0*H stays 16-byte aligned because H % 32 == 0.) */
#define LMHEAD_MAX_M ((int64_t)1 << 24)
#define LMHEAD_MAX_H ((int64_t)1 << 16)
#define LMHEAD_MAX_V ((int64_t)1 << 20)

/* The projection with a bf16 weight.
 *   hidden    bf16 [M, H]                       (device, read)
 *   W         bf16 [V, H]                       (device, read)
 *   alpha     fp32 scale applied to the fp32 accumulator: t = fl32(alpha * acc)
 *   bias      fp32 [V] or NULL                  (device, read): t = fl32(t + bias[v]),
 *             a separate rounding, never fused with the multiply
 *   out_dtype LMHEAD_F32 or LMHEAD_BF16
 *   out       [M, V] of out_dtype               (device, written; every element)
 * Returns LMHEAD_OK, LMHEAD_NOT_HANDLED (H % 32 != 0) or an error. */
lmhead_status lmhead_logits(const void *hidden, int64_t M, int64_t H, const void *W, int64_t V,
                            float alpha, const float *bias, lmhead_dtype out_dtype, void *out,
                            void *stream);

/* As lmhead_logits, with the kernel chosen by the caller: LMHEAD_PATH_AUTO,
 * LMHEAD_PATH_SKINNY (any M; the chunked skinny kernel walks 64-row blocks)
 * or LMHEAD_PATH_TILED (any M). Both kernels run the same K-step chain, so
 * their results are bit-identical; this entry point exists to show that. */
lmhead_status lmhead_logits_path(const void *hidden, int64_t M, int64_t H, const void *W,
                                 int64_t V, float alpha, const float *bias,
                                 lmhead_dtype out_dtype, void *out, void *stream, int path);

/* The projection with 16-bit inputs of either kind: hidden and W both bf16,
 * or both IEEE fp16 (sglang PR 32370 digest, implementation breakdown and the
 * key source excerpt: the fp32-output fast path takes bf16 or fp16 inputs of
 * one dtype and falls back otherwise). fp16 inputs run the fp16 MFMA of the
 * same shape through the same K-step chain and epilogue, so everything said
 * of lmhead_logits holds with fp16 in place of bf16.
 *   in_dtype   LMHEAD_BF16 or LMHEAD_F16: the type of hidden and of W
 *   out_dtype  LMHEAD_F32, or in_dtype (logits rounded to nearest even)
 *   path       as in lmhead_logits_path
 * Returns LMHEAD_NOT_HANDLED for any other (in_dtype, out_dtype) pair, for
 * instance fp32 inputs (nothing launched; the caller falls back), else as
 * lmhead_logits. lmhead_logits(...) is lmhead_logits_ex(..., LMHEAD_BF16,
 * out_dtype, out, stream, LMHEAD_PATH_AUTO). */
lmhead_status lmhead_logits_ex(const void *hidden, int64_t M, int64_t H, const void *W, int64_t V,
                               float alpha, const float *bias, lmhead_dtype in_dtype,
                               lmhead_dtype out_dtype, void *out, void *stream, int path);

/* The projection with a row-reduction epilogue: for every row m, over the
 * fp32 logits t[m, v] the call computes (the epilogue values of
 * lmhead_logits_ex, before any rounding to a 16-bit out_dtype):
 *   row_max[m]    = max over v of t[m, v]
 *   row_argmax[m] = the lowest v with t[m, v] == row_max[m]
 *   row_sumexp[m] = sum over v of exp(t[m, v] - row_max[m])   (>= 1)
 * Logits of -inf (a masked vocabulary entry, through a -inf bias) are
 * allowed and contribute exp(-inf) = 0; a row whose logits are all -inf gets
 * row_max -inf, row_argmax its lowest column and row_sumexp 0. +inf and NaN
 * logits are outside the contract.
 * so that the row's log-sum-exp is row_max + log(row_sumexp) and
 * softmax(t)[m, v] = exp(t[m, v] - row_max[m]) / row_sumexp[m]. These feed
 * the target and draft heads' acceptance distributions (vLLM PR 49120,
 * section Purpose) and greedy selection whose ties keep the lowest index, as
 * a stable descending sort does (tokenspeed PR 720, summary and review
 * thread). They are computed inside the GEMM's epilogue, so the [M, V] logits
 * need not be written at all.
 *   hidden, W, alpha, bias, in_dtype, out_dtype, path   as in lmhead_logits_ex
 *   out         [M, V] of out_dtype, or NULL: the logits are then not written
 *   row_max     fp32 [M]                          (device, written)
 *   row_argmax  int32 [M]                         (device, written)
 *   row_sumexp  fp32 [M]                          (device, written)
 *   workspace   device memory of at least lmhead_rowreduce_workspace_bytes(M, V)
 *               bytes, 16-byte aligned; the call overwrites it (it holds one
 *               16-byte partial per row and 16-column block) and it must not be
 *               in use by other work until this call's work has finished
 * row_max and row_argmax are exact: the maximum and the lowest argmax of the
 * fp32 logits lmhead_logits_ex writes (a zero maximum present with both signs
 * may be returned as either zero). row_sumexp is accumulated at fp32 in a
 * fixed order that depends only on V, each exponential taken as
 * 2^(x log2 e). All three are the same, bit for bit, whatever the row count
 * of the call and the path.
 * Returns as lmhead_logits_ex; LMHEAD_ERR_INVALID also for a NULL row output
 * or workspace, or a workspace smaller than required (M > 0); LMHEAD_ERR_ALIGN
 * for a misaligned workspace or row output (4-byte). */
lmhead_status lmhead_logits_rowreduce(const void *hidden, int64_t M, int64_t H, const void *W,
                                      int64_t V, float alpha, const float *bias,
                                      lmhead_dtype in_dtype, lmhead_dtype out_dtype, void *out,
                                      float *row_max, int32_t *row_argmax, float *row_sumexp,
                                      void *workspace, size_t workspace_bytes, void *stream,
                                      int path);

/* Host-only: bytes of workspace lmhead_logits_rowreduce needs for (M, V):
 * 16 * M * ceil(V / 16); 0 when M or V is outside the shape contract. */
size_t lmhead_rowreduce_workspace_bytes(int64_t M, int64_t V);

/* Bytes of the partials buffer the library holds for
 * lmhead_logits_rowreduce_noalloc, per GPU it runs on (32 MiB). */
#define LMHEAD_NOALLOC_SCRATCH_BYTES ((int64_t)32 << 20)

/* lmhead_logits_rowreduce for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, hosts that forbid
 * allocation. It takes no workspace: the partials go to a buffer of
 * LMHEAD_NOALLOC_SCRATCH_BYTES that the library keeps in a file-scope device
 * array, one per GPU, held until the process ends. The call allocates and
 * frees nothing (no hipMalloc, no allocating library routine); the caller
 * still passes the inputs and outputs. Arguments, results and bits are those
 * of lmhead_logits_rowreduce with the same arguments.
 * Limit: lmhead_rowreduce_workspace_bytes(M, V) <= LMHEAD_NOALLOC_SCRATCH_BYTES
 * (16 M ceil(V / 16) bytes: M <= 220 rows at V = 151936), else
 * LMHEAD_ERR_INVALID with nothing launched.
 * Every call on one GPU shares that GPU's buffer: calls whose work overlaps in
 * time on one GPU (other streams, other host threads) race on it and must be
 * ordered by the caller. The buffer's device address is looked up on the
 * first call on each device (LMHEAD_ERR_DEVICE if that fails). */
lmhead_status lmhead_logits_rowreduce_noalloc(const void *hidden, int64_t M, int64_t H,
                                              const void *W, int64_t V, float alpha,
                                              const float *bias, lmhead_dtype in_dtype,
                                              lmhead_dtype out_dtype, void *out, float *row_max,
                                              int32_t *row_argmax, float *row_sumexp,
                                              void *stream, int path);

/* The NVFP4 W4A16 head (bf16 logits).
 *   hidden       bf16 [M, H]                    (device, read)
 *   w_e2m1       uint8 [V, H/2]: two OCP E2M1 codes per byte, element 2i in the
 *                low nibble and 2i+1 in the high nibble (device, read)
 *   w_scale      uint8 [V, H/16]: one OCP E4M3 scale per 16 consecutive
 *                elements of a weight row (device, read)
 *   global_scale fp32 per-tensor scale g
 *   alpha, bias  as in lmhead_logits; the epilogue multiplies the accumulator
 *                by s = fl32(global_scale * alpha), then adds the bias
 *   out          bf16 [M, V]                    (device, written)
 * The weight w[v, k] = e2m1 * e4m3 is exact in bf16 and runs through the same
 * K-step chain as lmhead_logits: lmhead_logits_nvfp4 equals lmhead_logits on
 * the dequantised weight with alpha' = s, bit for bit. */
lmhead_status lmhead_logits_nvfp4(const void *hidden, int64_t M, int64_t H,
                                  const uint8_t *w_e2m1, const uint8_t *w_scale,
                                  float global_scale, int64_t V, float alpha, const float *bias,
                                  void *out, void *stream);

/* BF16 -> NVFP4 quantisation of a head: the weight lmhead_logits_nvfp4 reads,
 * made from a bf16 weight in two passes -- the tensor's absolute maximum, then
 * block quantisation -- as the metrale page "layers/mtp_head/new_bf16_moe.rs"
 * requantises BF16 weights to NVFP4 at load with an absmax kernel and an NVFP4
 * kernel (quantize_to_nvfp4, new_nvfp4_draft_moe). Every step is a binary32
 * operation (division correctly rounded):
 *   g = amax / 2688 (6 * 448; 1 when that is 0), amax = max |W|
 *   per 16 consecutive elements of a row: s = bmax / (6 g) rounded to E4M3
 *     (nearest even, at most 448); d = e4m3(s) * g
 *   per element: code = sign bit of W | E2M1(|W| / d) (nearest even,
 *     at most 6; magnitude 0 when d == 0)
 *   W             bf16 [V, H], finite               (device, read)
 *   w_e2m1        uint8 [V, H/2], layout as in lmhead_logits_nvfp4 (device, written)
 *   w_scale       uint8 [V, H/16]                   (device, written)
 *   global_scale  one fp32, g                       (device, written)
 *   workspace     at least lmhead_quantize_nvfp4_workspace_bytes() bytes of
 *                 device memory, 4-byte aligned, overwritten by the call
 * Shape contract as for the projection with M = 1 (H % 32 != 0:
 * LMHEAD_NOT_HANDLED). Alignment: W 16, w_e2m1 4, global_scale 4 bytes.
 * The result is deterministic (maxima are exact, the per-element steps fixed). */
lmhead_status lmhead_quantize_nvfp4(const void *W, int64_t V, int64_t H, uint8_t *w_e2m1,
                                    uint8_t *w_scale, float *global_scale, void *workspace,
                                    size_t workspace_bytes, void *stream);

/* Host-only: bytes of workspace lmhead_quantize_nvfp4 needs (a constant). */
size_t lmhead_quantize_nvfp4_workspace_bytes(void);

/* Host-only shape predicate (no device access): 1 when (M, H, V) is inside the
 * shape contract of the bf16 (nvfp4 = 0) or NVFP4 (nvfp4 = 1) entry point,
 * else 0. Like the shape check the metrale page's install step runs before
 * enabling its row-tile head. */
int lmhead_shape_ok(int64_t M, int64_t H, int64_t V, int nvfp4);

/* Host-only: the lmhead_path the AUTO choice takes for this shape, or
 * LMHEAD_PATH_NONE when the shape is outside the contract. The tests use it
 * to assert which kernel a call takes, as the sglang PR 32370 digest's test
 * changes (test coverage of test_fp32_lm_head.py: the probe_mm interceptor
 * asserts which torch operation, input dtype and out_dtype a call used, and a
 * fallback case checks the explicit-fp32 path) check the path as well as the
 * values. */
int lmhead_path_for(int64_t M, int64_t H, int64_t V, int nvfp4);

/* Static, human-readable name of a status code. */
const char *lmhead_status_string(int status);

/* Library version string, "major.minor.patch". */
const char *lmhead_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LMHEAD_H */
