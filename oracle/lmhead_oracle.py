"""CPU oracle for the LM-head logits projection -- TEST INFRASTRUCTURE ONLY.

    logits[m, v] = alpha * (hidden[m, :] . W[v, :]) + bias[v]

This module is the slow, plain definition that the GPU library is checked
against. It is imported only by the test-suite, by the smoke check and by the
CPU-baseline leg of the benchmark; the library itself never calls it and
shares no code with it (its own bf16 / E2M1 / E4M3 decoders and roundings are
written here from the format definitions).

What the pages fix, and where (page title, then section):

* The projection accumulates bf16 inputs at fp32 precision and never builds an
  fp32 copy of the weight -- sglang PR 32370 digest ("FP32 LM head skips the
  FP32 cast"), sections on motivation and implementation breakdown; vLLM PR
  49120 ("Honor fp32 head_dtype in Inkling muP logits"), section Purpose.
* The muP divisor enters as alpha = 1/mup, and folding it into the GEMM gives
  the same bits as the projection followed by a separate elementwise multiply
  -- vLLM PR 49120, sections Purpose and "muP is folded into the fp32 GEMM".
  The oracle therefore applies alpha *after* rounding the dot product to fp32,
  as that separate multiply does.
* An embedding bias may be added to the logits -- sglang digest, key source
  excerpt of ``_compute_lm_head`` (the ``embedding_bias`` argument).
* The NVFP4 head is weight-only 4-bit with 16-bit activations, and a row's
  logits may not depend on how many rows are in the call -- metrale
  ``lm_head_nvfp4_rows.rs`` source page, module documentation.

Readings where the pages are silent (each listed in the design notes):

* fp32 output: r = fl32(S); r = fl32(r * alpha); with bias r = fl32(r + b),
  every step an IEEE binary32 round-to-nearest-even operation, S the dot
  product accumulated in binary64 (each bf16 x bf16 product is exact there).
* bf16 output: the binary64 value alpha*S (+ b) correctly rounded to bf16
  (round-to-odd into binary32, then nearest-even into bf16: S. Boldo and
  G. Melquiond, "Emulation of FMA and correctly rounded sums: proved
  algorithms using rounding to odd", IEEE Trans. Computers 57(4), 2008).
* fp16 inputs (the fast path admits fp16 or bf16 of one dtype -- sglang
  digest, implementation breakdown): decoded from the IEEE binary16
  definition; each fp16 x fp16 product is exact in binary64. fp32 output as
  above; fp16 output: alpha*S (+ b) correctly rounded to binary16, with
  gradual underflow and overflow to infinity.
* Row reduction (the fused epilogue of the library's row-reduction entry
  point): over a row's fp32 logits, the maximum, the lowest column holding it
  (ties keep the lowest index, as a stable descending sort does -- tokenspeed
  PR 720, summary and review thread) and sum exp(x - max) in binary64, the
  pieces of the softmax that drives acceptance (vLLM PR 49120, Purpose).
* BF16 -> NVFP4 quantisation (two passes, as the metrale mtp_head page's
  quantize_to_nvfp4 runs an absmax kernel and an NVFP4 kernel): the pages
  give no arithmetic; the reading is the two-level recipe g = amax / (6*448),
  block scale E4M3_RNE(bmax / (6 g)), codes E2M1_RNE(|w| / (scale * g)),
  every step a binary32 operation (the decisions are integers, so both sides
  take them in the same precision).
* NVFP4 layout: codes [V, H/2] row-major, element 2i in the low nibble of byte
  i and 2i+1 in the high nibble; one OCP E4M3 scale per 16 consecutive
  elements of a weight row, [V, H/16] row-major; one fp32 per-tensor scale g.
  w = e2m1(code) * e4m3(scale) (exact), and the output is g*alpha*S (+ b)
  correctly rounded to bf16.

Parity pins (tests marked "not gpu"): a hand-computed 2x3x4 example and a
hand-computed NVFP4 example (tests/golden), exact rational brute force with
``fractions.Fraction`` on tiny random cases, exact integer arithmetic checked
against numpy's int64 matmul, E4M3 decoding checked against torch's
float8_e4m3fn, bf16 decoding and rounding checked against torch.bfloat16, the
E2M1 magnitudes of the OCP MX specification, one-hot weights (a gather) and
zero hidden rows (bias only); for fp16, a hand-computed example (tests/golden),
binary16 decoding against numpy's float16 for every bit pattern, binary16
rounding against exact rational rounding, rational brute force and integer
inputs past bf16's range against numpy's int64 matmul; for the row reduction,
a hand example with ties (tests/golden), scipy's logsumexp on random rows,
exact shift and reversal invariants and closed forms (constant rows).
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# Number formats, written from their definitions.
# ----------------------------------------------------------------------------


def bf16_to_f64(bits) -> np.ndarray:
    """bfloat16 is the upper 16 bits of an IEEE binary32; widening is exact."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):          # NaN patterns widen to NaN
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f16_to_f64(bits) -> np.ndarray:
    """IEEE binary16: sign bit 15, exponent bits 14..10 (bias 15), fraction
    bits 9..0. Exponent field 0 is subnormal: value = f * 2^-24; field 31 is
    infinity (f = 0) or NaN. Widening to binary64 is exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = (b >> 15) & 1
    e = (b >> 10) & 31
    f = b & 1023
    mag = np.where(e == 0, np.ldexp(f.astype(np.float64), -24),
                   np.ldexp((1024 + f).astype(np.float64), e - 25))
    mag = np.where(e == 31, np.where(f == 0, np.inf, np.nan), mag)
    return np.where(sign == 1, -mag, mag).astype(np.float64)


def f64_to_f16_correct(x) -> np.ndarray:
    """binary64 -> binary16 bits, correctly rounded (nearest, ties to even),
    with gradual underflow and overflow to infinity. Finite inputs only.

    |x| lies in the binade [2^q, 2^(q+1)); binary16 keeps 11 significant bits
    there, so its spacing is 2^(max(q, -14) - 10) (the subnormals share the
    spacing of the lowest binade). x / spacing is exact (a power-of-two
    scaling), rint rounds it to nearest even, and a result of 2^16 or more
    (beyond the largest finite value 65504 after rounding) is infinity."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    sign = np.where(np.signbit(x), 0x8000, 0).astype(np.int64)
    _, e = np.frexp(a)                            # a = m 2^e, m in [0.5, 1)
    q = np.maximum(e - 1, -14)                    # binade of a, floored at the normal minimum
    n = np.rint(np.ldexp(a, 10 - q)).astype(np.int64)   # significand in units of the spacing
    # n in [0, 2048]; 2048 carries into the next binade
    carry = n >= 2048
    q = np.where(carry, q + 1, q)
    n = np.where(carry, n >> 1, n)
    normal = n >= 1024
    field = np.where(normal, q + 15, 0)
    bits = np.where(normal, (field << 10) | (n - 1024), n)
    bits = np.where(field >= 31, 0x7C00, bits)
    return (sign | bits).astype(np.uint16)


def ulp_f16(bits) -> np.ndarray:
    """Unit in the last place of a binary16 value: 2^(e - 25) for exponent
    field e, 2^-24 in the subnormal range and at zero."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    e = (b >> 10) & 31
    return np.ldexp(1.0, np.maximum(e, 1) - 25)


def e2m1_to_f64(code) -> np.ndarray:
    """OCP MX FP4 E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.

    Exponent field 0 is subnormal: value = mantissa * 1/2. Otherwise
    value = 2^(e-1) * (1 + mantissa/2). No infinities or NaNs.
    """
    c = np.asarray(code, dtype=np.int64)
    sign = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, np.ldexp(1.0 + m * 0.5, (e - 1)))
    return np.where(sign == 1, -mag, mag).astype(np.float64)


def e4m3_to_f64(byte) -> np.ndarray:
    """OCP FP8 E4M3: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.

    Exponent field 0 is subnormal: value = 2^-6 * m/8. Exponent 15 with
    mantissa 7 is NaN (the only NaN pattern); there are no infinities.
    """
    b = np.asarray(byte, dtype=np.int64)
    sign = (b >> 7) & 1
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag).astype(np.float64)


def unpack_e2m1(packed, H: int) -> np.ndarray:
    """[V, H/2] bytes -> [V, H] codes; element 2i is the low nibble of byte i."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (H,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def nvfp4_weight_f64(packed, scale_bytes, H: int) -> np.ndarray:
    """Dequantised NVFP4 weight w[v, k] = e2m1(code[v, k]) * e4m3(scale[v, k // 16]).

    The per-tensor scale g is not folded in here (it is applied to the sum).
    The product of a 2-bit and a 4-bit significand is exact in binary64.
    """
    codes = unpack_e2m1(packed, H)
    s = e4m3_to_f64(scale_bytes)
    return e2m1_to_f64(codes) * np.repeat(s, 16, axis=-1)


def f32_to_bf16_rne(x) -> np.ndarray:
    """binary32 -> bf16 bits, round to nearest, ties to even (NaN stays quiet)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    is_nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    r = np.where(is_nan, (u >> 16) | 0x40, r)
    return r.astype(np.uint16)


def f64_to_f32_round_to_odd(x) -> np.ndarray:
    """binary64 -> binary32 with rounding to odd: exact values stay, inexact
    ones take the neighbour whose last significand bit is 1.
    Finite inputs within binary32 range only."""
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)                      # nearest-even
    back = f.astype(np.float64)
    inexact = back != x
    # the binary32 neighbour toward zero
    toward0 = np.where(np.abs(back) > np.abs(x), np.nextafter(f, np.float32(0.0)), f)
    bits = toward0.view(np.uint32)
    bits = np.where(inexact, bits | np.uint32(1), bits)
    return bits.astype(np.uint32).view(np.float32)


def f64_to_bf16_correct(x) -> np.ndarray:
    """binary64 -> bf16 bits, correctly rounded (nearest even) from binary64.

    Round to odd into binary32 (24 >= 8 + 2 bits), then nearest-even into
    bf16; by Boldo and Melquiond (2008) the result equals direct rounding."""
    return f32_to_bf16_rne(f64_to_f32_round_to_odd(x))


def ulp_bf16(bits) -> np.ndarray:
    """Unit in the last place of a bf16 value: 2^(e - 7) for exponent e,
    2^-133 in the subnormal range and at zero."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    e = (b >> 7) & 0xFF
    return np.ldexp(1.0, np.maximum(e, 1) - 127 - 7)


# ----------------------------------------------------------------------------
# The projection.
# ----------------------------------------------------------------------------


_DECODE = {"bf16": bf16_to_f64, "f16": f16_to_f64}


def dot_f64(h_bits, w_bits, in_dtype: str = "bf16"):
    """S[m, v] = sum_k h[m, k] * w[v, k] and A[m, v] = sum_k |h[m, k] * w[v, k]|,
    both in binary64, for bf16 or fp16 ("f16") inputs of one type. Every
    bf16 x bf16 (8 x 8 significant bits) and fp16 x fp16 (11 x 11) product is
    exact in binary64, so the only rounding is that of the binary64 sums
    (relative 2^-53 per add)."""
    dec = _DECODE[in_dtype]
    return _dot_pair(dec(h_bits), dec(w_bits))


def _dot_pair(hf, wf):
    S = hf @ wf.T
    A = np.abs(hf) @ np.abs(wf).T
    return S, A


def logits_f32(S, alpha: float, bias=None) -> np.ndarray:
    """fp32 logits from binary64 dot products, in the unfused order: round the
    projection to fp32, multiply by alpha in fp32, then add the fp32 bias in
    fp32 (no fused multiply-add)."""
    a = np.float32(alpha)
    r = np.asarray(S, dtype=np.float64).astype(np.float32)
    r = (r * a).astype(np.float32)
    if bias is not None:
        r = (r + np.asarray(bias, dtype=np.float32)).astype(np.float32)
    return r


def logits_bf16(S, alpha: float, bias=None) -> np.ndarray:
    """bf16 logits (bits): alpha*S (+ bias) in binary64, correctly rounded."""
    y = np.float64(np.float32(alpha)) * np.asarray(S, dtype=np.float64)
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float32).astype(np.float64)
    return f64_to_bf16_correct(y)


def logits_f16(S, alpha: float, bias=None) -> np.ndarray:
    """fp16 logits (bits): alpha*S (+ bias) in binary64, correctly rounded."""
    y = np.float64(np.float32(alpha)) * np.asarray(S, dtype=np.float64)
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float32).astype(np.float64)
    return f64_to_f16_correct(y)


def lmhead_logits(h_bits, w_bits, alpha: float, bias=None, out_dtype: str = "f32",
                  in_dtype: str = "bf16"):
    """Reference logits for hidden [M, H] and weight [V, H], both bf16 or both
    fp16 (in_dtype "bf16" / "f16", given as uint16 bit patterns).

    Returns (logits, A): logits are fp32 values for out_dtype "f32", or bf16 /
    fp16 bit patterns (uint16) for "bf16" / "f16"; A = sum_k |h*w| for the
    tolerance."""
    S, A = dot_f64(h_bits, w_bits, in_dtype)
    if out_dtype == "f32":
        return logits_f32(S, alpha, bias), A
    if out_dtype == "bf16":
        return logits_bf16(S, alpha, bias), A
    if out_dtype == "f16":
        return logits_f16(S, alpha, bias), A
    raise ValueError(out_dtype)


def lmhead_logits_nvfp4(h_bits, packed, scale_bytes, g: float, alpha: float = 1.0, bias=None):
    """Reference bf16 logits (bits) of the W4A16 NVFP4 head, and A for the
    tolerance: y = g * alpha * S (+ bias) in binary64 with S the exact-product
    binary64 dot of the bf16 hidden with the dequantised weight, correctly
    rounded to bf16. g and alpha are taken at their binary32 values."""
    hf = bf16_to_f64(h_bits)
    H = hf.shape[-1]
    wf = nvfp4_weight_f64(packed, scale_bytes, H)
    S, A = _dot_pair(hf, wf)
    ga = np.float64(np.float32(g)) * np.float64(np.float32(alpha))
    y = ga * S
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float32).astype(np.float64)
    return f64_to_bf16_correct(y), A


# ----------------------------------------------------------------------------
# Row reduction of the logits.
# ----------------------------------------------------------------------------


def row_reduce(x):
    """Softmax quantities of each row of fp32 logits x [M, V]:
    (max, argmax, sumexp) with max the largest value (fp32), argmax the lowest
    column holding it (numpy's argmax returns the first occurrence), and
    sumexp = sum_v exp(x[m, v] - max) in binary64, so that the row's
    log-sum-exp is max + log(sumexp).

    Greedy selection with ties going to the lowest index is the stable
    descending order of tokenspeed PR 720 (summary and review thread); the
    softmax of the logits is the acceptance distribution of vLLM PR 49120
    (section Purpose)."""
    x = np.asarray(x, dtype=np.float32)
    idx = np.argmax(x, axis=1)
    mx = x[np.arange(x.shape[0]), idx]
    s = np.exp(x.astype(np.float64) - mx.astype(np.float64)[:, None]).sum(axis=1)
    return mx, idx.astype(np.int64), s


def lmhead_rowreduce(h_bits, w_bits, alpha: float, bias=None, in_dtype: str = "bf16"):
    """Row reduction of the fp32 logits of ``lmhead_logits``: returns
    (max, argmax, sumexp, logits, A)."""
    S, A = dot_f64(h_bits, w_bits, in_dtype)
    x = logits_f32(S, alpha, bias)
    mx, idx, s = row_reduce(x)
    return mx, idx, s, x, A


# ----------------------------------------------------------------------------
# BF16 -> NVFP4 quantisation of a head (the step before the NVFP4 projection).
# ----------------------------------------------------------------------------

E2M1_MAX = 6.0
E4M3_MAX = 448.0


def f32_to_e4m3_rne(s) -> np.ndarray:
    """Non-negative binary32 values -> OCP E4M3 bytes, round to nearest even,
    saturating at 448 (0x7E). |s| lies in the binade [2^e, 2^(e+1)) with
    e >= -6 (the subnormals share the spacing of the lowest binade), where
    E4M3 keeps 4 significant bits: spacing 2^(e-3)."""
    s = np.asarray(s, dtype=np.float32).astype(np.float64)    # exact widening
    assert np.all(s >= 0)
    _, fe = np.frexp(s)
    e = np.maximum(fe - 1, -6)
    n = np.rint(np.ldexp(s, 3 - e))                            # nearest even, in [0, 16]
    carry = n >= 16
    e = np.where(carry, e + 1, e)
    n = np.where(carry, 8, n).astype(np.int64)
    sub = n < 8                                                # only at e == -6
    field = np.where(sub, 0, e + 7)
    code = np.where(sub, n, (field << 3) | (n - 8))
    over = (field > 15) | ((field == 15) & (n - 8 == 7)) | (s >= E4M3_MAX)
    return np.where(over, 0x7E, code).astype(np.uint8)


def e2m1_rne(x) -> np.ndarray:
    """Non-negative binary32 magnitudes -> E2M1 magnitude codes 0..7 (values 0,
    0.5, 1, 1.5, 2, 3, 4, 6), nearest with ties to the even code (the one
    whose mantissa bit is 0), saturating at 6."""
    x = np.asarray(x, dtype=np.float64)
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    d = np.abs(x[..., None] - grid)                            # distance to each value
    best = d.min(axis=-1, keepdims=True)
    cand = d == best                                           # one, or two at a tie
    even = (np.arange(8) % 2) == 0
    pick = np.where(cand & even, np.arange(8), 99).min(axis=-1)
    pick = np.where(cand.sum(axis=-1) == 1, np.argmax(cand, axis=-1), pick)
    return np.where(x >= E2M1_MAX, 7, pick).astype(np.uint8)


def quantize_nvfp4(w_bits, amax=None):
    """BF16 weight [V, H] (H % 16 == 0) -> (codes [V, H/2] u8, scales [V, H/16]
    u8, g fp32), every step an IEEE binary32 operation:

      amax = max |w|;  g = fl32(amax / 2688), or 1 when that is 0
      per block of 16:  s = fl32(bmax / fl32(6 g)),  byte = E4M3_RNE_sat(s),
                        d = fl32(e4m3(byte) * g)
      per element:      code = sign bit of w | E2M1_RNE_sat(fl32(|w| / d)), or
                        the sign bit alone when d == 0

    Two passes over the weight -- a per-tensor absolute maximum, then block
    quantisation -- as the metrale page's quantize_to_nvfp4 runs an absmax
    kernel and then an NVFP4 kernel (mtp_head/new_bf16_moe.rs source page,
    new_nvfp4_draft_moe). The constants put the largest block scale at E4M3's
    largest value (448) and the largest element at E2M1's (6).

    `amax`, when given, is the whole tensor's maximum, for quantising a subset
    of its rows."""
    w = bf16_to_f64(w_bits).astype(np.float32)                 # exact
    V, H = w.shape
    a = np.abs(w)
    if amax is None:
        amax = a.max() if a.size else np.float32(0)
    g = np.float32(amax) / np.float32(E2M1_MAX * E4M3_MAX)
    g = np.float32(1.0) if g == 0 else np.float32(g)
    blocks = a.reshape(V, H // 16, 16)
    bmax = blocks.max(axis=-1)
    s = (bmax / (np.float32(E2M1_MAX) * g)).astype(np.float32)
    scales = f32_to_e4m3_rne(s)
    d = (e4m3_to_f64(scales).astype(np.float32) * g).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        x = (blocks / d[..., None]).astype(np.float32)
    mag = np.where(d[..., None] == 0, 0, e2m1_rne(np.where(d[..., None] == 0, 0, x)))
    neg = np.signbit(w.reshape(V, H // 16, 16)).astype(np.uint8)   # -0 keeps its sign
    code = (mag.astype(np.uint8) | (neg << 3)).reshape(V, H)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, scales, np.float32(g)
