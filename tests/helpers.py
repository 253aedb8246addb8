"""Shared test helpers: golden-file parsing, exact rational rounding and the
parity tolerances. Nothing here computes logits."""
from __future__ import annotations

from fractions import Fraction
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parents[1]


def load_golden(name):
    """Parse a tests/golden fixture: '#' comments; 'key v1 v2 ...' lines; a
    repeated key gives one list per line."""
    out = {}
    for line in (ROOT / "tests" / "golden" / name).read_text().splitlines():
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, *vals = line.split()
        out.setdefault(key, []).append(vals)
    return out


def num(s: str) -> float:
    return float(int(s, 16)) if s.lower().startswith("0x") else float(s)


def f32_bits_to_bf16_bits_exact(values) -> np.ndarray:
    """bf16 bits of values that are exactly representable in bf16 (asserted)."""
    f = np.asarray(values, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


# ---------------------------------------------------------------------------
# Exact rational rounding to a binary format (round to nearest, ties to even),
# written from the IEEE 754 definition with integer arithmetic only.
# ---------------------------------------------------------------------------

def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_fraction(q: Fraction, p: int, emin: int) -> Fraction:
    """Nearest-even rounding of q to p significand bits, minimum normal
    exponent emin (gradual underflow below it). No overflow handling."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = max(_floor_log2(a), emin)
    quantum = Fraction(2) ** (e - p + 1)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * quantum


def rne32(q: Fraction) -> Fraction:
    return round_fraction(q, 24, -126)


def rne_bf16(q: Fraction) -> Fraction:
    return round_fraction(q, 8, -126)


# ---------------------------------------------------------------------------
# Parity tolerances.
# ---------------------------------------------------------------------------

def check_f32(gpu, ref, A, rel=2e-5, what=""):
    """|gpu - ref| <= rel * A + 1e-30 per element; returns (max ratio, exact fraction)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = rel * np.asarray(A, dtype=np.float64) + 1e-30
    err = np.abs(gpu - ref)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance, e.g. "
                             + ", ".join(f"{tuple(i)}: gpu={gpu[tuple(i)]!r} ref={ref[tuple(i)]!r} "
                                         f"bound={bound[tuple(i)]:.3g}" for i in idx))
    return float(np.max(err / bound)) if err.size else 0.0, float(np.mean(err == 0)) if err.size else 1.0


def bf16_bits_to_f64(bits):
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_bf16(gpu_bits, ref_bits, A, scale, ulp_fn, rel=2e-5, what=""):
    """bf16 parity: |gpu - ref| <= max(1 ulp(ref), rel*|scale|*A) per element
    (the second term covers cancellation near zero, where one bf16 ulp is
    smaller than any fp32-accumulation error). Returns the number of elements
    outside the strict 1-ulp bound, which the caller may report."""
    g = bf16_bits_to_f64(gpu_bits)
    r = bf16_bits_to_f64(ref_bits)
    ulp = ulp_fn(ref_bits)
    err = np.abs(g - r)
    bound = np.maximum(ulp, rel * abs(scale) * np.asarray(A, dtype=np.float64))
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} bf16 elements out of tolerance, e.g. "
                             + ", ".join(f"{tuple(i)}: gpu={g[tuple(i)]!r} ref={r[tuple(i)]!r}"
                                         for i in idx))
    return int(np.sum(err > ulp))


def check_f16(gpu_bits, ref_bits, A, scale, ulp_fn, rel=2e-5, what=""):
    """fp16 parity, the bound of ``check_bf16`` with fp16 ulps: |gpu - ref| <=
    max(1 ulp(ref), rel*|scale|*A); an infinite reference (overflow) must be
    met by the same infinity. Returns the count outside the strict 1-ulp bound."""
    g = np.asarray(gpu_bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    r = np.asarray(ref_bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    inf = np.isinf(r)
    if not np.array_equal(g[inf], r[inf]):
        raise AssertionError(f"{what}: overflow to infinity not matched")
    g, r = g[~inf], r[~inf]
    ulp = np.asarray(ulp_fn(ref_bits))[~inf]
    err = np.abs(g - r)
    bound = np.maximum(ulp, rel * abs(scale) * np.asarray(A, dtype=np.float64)[~inf])
    bad = ~(err <= bound)
    if bad.any():
        idx = np.flatnonzero(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} fp16 elements out of tolerance, e.g. "
                             + ", ".join(f"gpu={g[i]!r} ref={r[i]!r}" for i in idx))
    return int(np.sum(err > ulp))


# ---------------------------------------------------------------------------
# Row reduction.
# ---------------------------------------------------------------------------

U32 = 2.0 ** -24   # unit roundoff of binary32


def sumexp_bound(x, m, V):
    """Bound on |s_gpu - sum_v exp(x_v - m)| for a row reduced at fp32 from its
    fp32 logits x with maximum m, in the library's fixed order. Each
    exponential is 2^(d log2 e) for a rounded difference d: the difference,
    the product and the hardware exp2 (taken as within 2 ulp) give a relative
    error of at most 3u|d| + 4u. A term exp(x_v - m) is the block's
    exp(x_v - m_b) rescaled by factors exp(m_prev - m_next) whose differences
    add up to m_b - m, so its relative error is at most 3u|x_v - m| plus 4u
    per level; the sum passes through at most L = 4 + ceil(ceil(V/16) / 1024)
    + 6 + 4 levels (16-lane block sum, the combine thread's folds, the 64-lane
    and the 16-wave butterflies), each adding at most 4u more (multiply, add).
    Returned in binary64, per row."""
    x = np.asarray(x, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)[:, None]
    d = x - m
    e = np.exp(d)
    ncb = (V + 15) // 16
    L = 4 + (ncb + 1023) // 1024 + 6 + 4
    # a -inf logit (masked entry) contributes an exact 0
    per = np.where(e > 0, e * 3 * U32 * np.abs(np.where(e > 0, d, 0.0)), 0.0)
    return per.sum(axis=1) + e.sum(axis=1) * 8 * L * U32


def check_rowreduce_self(gmax, garg, gsum, x):
    """The GPU's row reduction against its own fp32 logits x [M, V]: max and
    argmax exactly (the lowest column of the maximum), sumexp within
    ``sumexp_bound``."""
    x = np.asarray(x, dtype=np.float32)
    idx = np.argmax(x, axis=1)
    mx = x[np.arange(x.shape[0]), idx]
    assert np.array_equal(np.asarray(gmax, np.float32), mx), \
        "row max differs from the maximum of the logits"   # by value: +0 == -0
    assert np.array_equal(np.asarray(garg, np.int64), idx), "argmax is not the lowest maximal column"
    ref = np.exp(x.astype(np.float64) - mx.astype(np.float64)[:, None]).sum(axis=1)
    err = np.abs(np.asarray(gsum, np.float64) - ref)
    bound = sumexp_bound(x, mx, x.shape[1])
    assert np.all(err <= bound), f"sumexp beyond its bound: max err/bound {np.max(err / bound):.3g}"
    return float(np.max(err / bound))


def check_rowreduce_oracle(gmax, garg, gsum, ref_max, ref_x, A, V, rel=2e-5):
    """The GPU's row reduction against the oracle's. With every logit within
    tol_v = rel*A_v + 1e-30 of the oracle's (the fp32 parity bound) and both
    max and log-sum-exp 1-Lipschitz in the largest coordinate change, the row
    max and log-sum-exp are within T = max_v tol_v (plus the sumexp rounding
    for the latter); the argmax column's oracle logit is within 2T of the
    oracle maximum."""
    T = (rel * np.asarray(A, np.float64) + 1e-30).max(axis=1)
    gmax = np.asarray(gmax, np.float64)
    assert np.all(np.abs(gmax - ref_max) <= T), "row max beyond tolerance"
    lse_gpu = gmax + np.log(np.asarray(gsum, np.float64))
    ref_x64 = np.asarray(ref_x, np.float64)
    ref_s = np.exp(ref_x64 - np.asarray(ref_max, np.float64)[:, None]).sum(axis=1)
    lse_ref = np.asarray(ref_max, np.float64) + np.log(ref_s)
    # sumexp rounding, relative, taken at the oracle's logits (within T of the GPU's)
    srel = sumexp_bound(ref_x, ref_max, V) / ref_s
    assert np.all(np.abs(lse_gpu - lse_ref) <= T * (1 + 1e-6) + 2 * srel + 1e-12), \
        "log-sum-exp beyond tolerance"
    rows = np.arange(ref_x64.shape[0])
    assert np.all(ref_x64[rows, np.asarray(garg)] >= np.asarray(ref_max) - 2 * T), \
        "argmax column is not within tolerance of the maximum"
