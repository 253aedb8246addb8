"""Pins of the CPU oracle to facts outside itself (no GPU needed).

Each test ties the oracle to something it does not contain: a hand-worked
example, exact rational arithmetic, an exact integer matmul, another
implementation of a number format (torch), a format table from its
specification, or a closed-form special case.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from helpers import (f32_bits_to_bf16_bits_exact, load_golden, num, rne32, rne_bf16,
                     round_fraction)


def _rows(g, key):
    return np.array([[num(x) for x in row] for row in g[key]], dtype=np.float64)


# ---------------------------------------------------------------------------
# Hand-computed examples (tests/golden).
# ---------------------------------------------------------------------------

def test_hand_example_fp32_and_bf16():
    g = load_golden("hand_2x3x4.txt")
    alpha = num(g["alpha"][0][0])
    h = f32_bits_to_bf16_bits_exact(_rows(g, "hidden"))
    w = f32_bits_to_bf16_bits_exact(_rows(g, "weight"))
    b = _rows(g, "bias")[0].astype(np.float32)
    S, A = oracle.dot_f64(h, w)
    assert np.array_equal(S, _rows(g, "dot"))
    assert np.array_equal(A, _rows(g, "absdot"))
    for bias, key in ((None, "nobias"), (b, "withbias")):
        want = _rows(g, key).astype(np.float32)
        got32, _ = oracle.lmhead_logits(h, w, alpha, bias, "f32")
        assert got32.dtype == np.float32
        assert np.array_equal(got32.view(np.uint32), want.view(np.uint32)), key
        got16, _ = oracle.lmhead_logits(h, w, alpha, bias, "bf16")
        assert np.array_equal(got16, f32_bits_to_bf16_bits_exact(want)), key


def test_hand_example_catches_transpose_and_sign():
    # The example is asymmetric enough that a transposed weight or a flipped
    # sign gives a different result: check the oracle really uses W^T.
    g = load_golden("hand_2x3x4.txt")
    h = _rows(g, "hidden")
    w = _rows(g, "weight")
    assert not np.array_equal(h @ w.T, _rows(g, "dot")[:, ::-1])
    S, _ = oracle.dot_f64(f32_bits_to_bf16_bits_exact(h), f32_bits_to_bf16_bits_exact(w))
    assert S[0, 2] == 3.875 and S[1, 1] == 1.125


def test_nvfp4_hand_example():
    g = load_golden("nvfp4_hand.txt")
    H = int(g["H"][0][0])
    h = f32_bits_to_bf16_bits_exact(_rows(g, "hidden"))
    codes = np.array([[int(x, 16) for x in row] for row in g["codes"]], dtype=np.uint8)
    scales = np.array([[int(x, 16) for x in row] for row in g["scales"]], dtype=np.uint8)
    gsc = num(g["g"][0][0])
    alpha = num(g["alpha"][0][0])
    wf = oracle.nvfp4_weight_f64(codes, scales, H)
    assert np.array_equal(oracle.bf16_to_f64(h) @ wf.T, _rows(g, "dot"))
    out, _ = oracle.lmhead_logits_nvfp4(h, codes, scales, gsc, alpha)
    want = np.array([[int(x, 16) for x in g["logits_bf16"][0]]], dtype=np.uint16)
    assert np.array_equal(out, want)


def test_nvfp4_nibble_order():
    # byte 0x72: element 0 (low nibble) is code 2 = 1.0, element 1 is code 7 = 6.0
    packed = np.array([[0x72]], dtype=np.uint8)
    assert oracle.unpack_e2m1(packed, 2).tolist() == [[2, 7]]
    one = np.array([[0x38]], dtype=np.uint8)                           # scale 1.0
    packed16 = np.zeros((1, 8), dtype=np.uint8)
    packed16[0, 0] = 0x72
    w = oracle.nvfp4_weight_f64(packed16, one, 16)
    assert w[0, 0] == 1.0 and w[0, 1] == 6.0 and np.all(w[0, 2:] == 0)


# ---------------------------------------------------------------------------
# Number formats against their specifications and torch.
# ---------------------------------------------------------------------------

def test_e2m1_matches_ocp_table():
    mags = [float(x) for x in load_golden("e2m1_ocp.txt")["magnitudes"][0]]
    vals = oracle.e2m1_to_f64(np.arange(16))
    assert vals[:8].tolist() == mags
    assert (-vals[8:]).tolist() == mags
    assert np.all(np.signbit(vals[8:]))


def test_e4m3_landmarks_and_torch_exhaustive():
    g = load_golden("e4m3_ocp.txt")
    for key, rows in g.items():
        byte = int(key, 16)
        want = float(rows[0][0])
        got = float(oracle.e4m3_to_f64(byte))
        if np.isnan(want):
            assert np.isnan(got)
        else:
            assert got == want and np.signbit(got) == np.signbit(want), hex(byte)
    ours = oracle.e4m3_to_f64(np.arange(256))
    theirs = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(ours, theirs, equal_nan=True)
    assert np.array_equal(np.signbit(ours), np.signbit(theirs))


def test_bf16_decode_exhaustive_vs_torch():
    bits = np.arange(65536, dtype=np.uint16)
    ours = oracle.bf16_to_f64(bits)
    theirs = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(ours, theirs, equal_nan=True)


def test_f32_to_bf16_rne_vs_torch():
    rng = np.random.default_rng(7)
    u = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    # force exact ties and near-ties
    u[:20000] = (u[:20000] & 0xFFFF0000) | 0x8000
    u[20000:40000] = (u[20000:40000] & 0xFFFF0000) | 0x7FFF
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    ours = oracle.f32_to_bf16_rne(f)
    theirs = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_f64_to_bf16_correct_rounding_vs_fractions():
    rng = np.random.default_rng(11)
    xs = list(rng.normal(0, 1, 3000) * np.exp2(rng.integers(-30, 30, 3000)))
    # values a hair above/below bf16 ties, where double rounding through fp32 would fail
    for k in range(300):
        base = Fraction(int(rng.integers(128, 256)), 128) * Fraction(2) ** int(rng.integers(-20, 20))
        tie = base + Fraction(1, 256) * Fraction(2) ** (_e(base))
        for d in (Fraction(1, 2**40), -Fraction(1, 2**40), 0):
            xs.append(float(tie + d * Fraction(2) ** _e(base)))
    xs = np.array(xs, dtype=np.float64)
    got = oracle.f64_to_bf16_correct(xs)
    want = np.array([_bf16_bits(rne_bf16(Fraction(float(x)))) for x in xs], dtype=np.uint16)
    assert np.array_equal(got, want)


def _e(q: Fraction) -> int:
    from helpers import _floor_log2
    return _floor_log2(abs(q))


def _bf16_bits(q: Fraction) -> int:
    return int(np.float32(float(q)).view(np.uint32) >> 16)


# ---------------------------------------------------------------------------
# Exact rational brute force on tiny random cases.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(40))
def test_bruteforce_vs_fractions(seed):
    rng = np.random.default_rng(seed)
    M, V = (int(x) for x in rng.integers(1, 4, 2))
    H = int(rng.integers(1, 9))
    hf = rng.normal(0, 1, (M, H)).astype(np.float32)
    wf = (rng.normal(0, 1, (V, H)) * np.exp2(rng.integers(-8, 3, (V, H)))).astype(np.float32)
    h = oracle.f32_to_bf16_rne(hf)
    w = oracle.f32_to_bf16_rne(wf)
    alpha = float(np.float32(rng.choice([1.0, 0.25, 1 / 3, 0.7, 1 / 16])))
    bias = rng.normal(0, 0.1, V).astype(np.float32) if seed % 2 else None
    hq = [[Fraction(float(x)) for x in row] for row in oracle.bf16_to_f64(h)]
    wq = [[Fraction(float(x)) for x in row] for row in oracle.bf16_to_f64(w)]
    got32, A = oracle.lmhead_logits(h, w, alpha, bias, "f32")
    got16, _ = oracle.lmhead_logits(h, w, alpha, bias, "bf16")
    for m in range(M):
        for v in range(V):
            S = sum(a * b for a, b in zip(hq[m], wq[v]))
            Aq = sum(abs(a * b) for a, b in zip(hq[m], wq[v]))
            assert abs(A[m, v] - float(Aq)) <= 1e-15 * float(Aq)
            # fp32 output: the unfused chain, every step rounded to binary32
            r = rne32(S)
            r = rne32(r * Fraction(alpha))
            if bias is not None:
                r = rne32(r + Fraction(float(bias[v])))
            assert got32[m, v] == np.float32(float(r)), (m, v)
            # bf16 output: exact value correctly rounded once
            y = Fraction(alpha) * S + (Fraction(float(bias[v])) if bias is not None else 0)
            assert got16[m, v] == _bf16_bits(rne_bf16(y)), (m, v)


def test_nvfp4_bruteforce_vs_fractions():
    rng = np.random.default_rng(5)
    M, V, H = 2, 3, 32
    h = oracle.f32_to_bf16_rne(rng.normal(0, 1, (M, H)).astype(np.float32))
    packed = rng.integers(0, 256, (V, H // 2), dtype=np.uint8)
    scales = rng.choice(np.r_[0x20:0x50], (V, H // 16)).astype(np.uint8)
    g, alpha = 0.01, 0.5
    got, _ = oracle.lmhead_logits_nvfp4(h, packed, scales, g, alpha)
    e2m1 = {0: 0, 1: Fraction(1, 2), 2: 1, 3: Fraction(3, 2), 4: 2, 5: 3, 6: 4, 7: 6}
    hq = [[Fraction(float(x)) for x in row] for row in oracle.bf16_to_f64(h)]
    for v in range(V):
        wv = []
        for k in range(H):
            byte = int(packed[v, k // 2])
            c = (byte & 0xF) if k % 2 == 0 else (byte >> 4)
            val = Fraction(e2m1[c & 7]) * (-1 if c & 8 else 1)
            sb = int(scales[v, k // 16])
            e, m = (sb >> 3) & 15, sb & 7
            s = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
            wv.append(val * s)
        for mi in range(M):
            S = sum(a * b for a, b in zip(hq[mi], wv))
            y = Fraction(float(np.float32(g))) * Fraction(float(np.float32(alpha))) * S
            assert got[mi, v] == _bf16_bits(rne_bf16(y))


# ---------------------------------------------------------------------------
# Exact arithmetic and closed-form special cases.
# ---------------------------------------------------------------------------

def test_integer_inputs_match_int64_matmul():
    import synth.workloads as wl
    M, V, H = 5, 37, 4096
    h = wl.int_hidden(9, M, H)
    w = wl.int_weight(9, V, H)
    hi = oracle.bf16_to_f64(h).astype(np.int64)
    wi = oracle.bf16_to_f64(w).astype(np.int64)
    exact = hi @ wi.T                         # integer matmul: exact
    for alpha in (1.0, 1 / 16, 0.125):
        got, _ = oracle.lmhead_logits(h, w, alpha, None, "f32")
        assert np.array_equal(got.astype(np.float64), exact * alpha)


def test_one_hot_weights_gather_hidden():
    rng = np.random.default_rng(3)
    M, H, V = 4, 64, 50
    h = oracle.f32_to_bf16_rne(rng.normal(0, 1, (M, H)).astype(np.float32))
    ks = rng.integers(0, H, V)
    w = np.zeros((V, H), dtype=np.uint16)
    w[np.arange(V), ks] = 0x3F80                   # bf16 1.0
    alpha = 0.7
    got, _ = oracle.lmhead_logits(h, w, alpha, None, "f32")
    hv = oracle.bf16_to_f64(h).astype(np.float32)
    want = (hv[:, ks] * np.float32(alpha)).astype(np.float32)
    assert np.array_equal(got, want)


def test_zero_hidden_gives_bias():
    rng = np.random.default_rng(4)
    h = np.zeros((3, 32), dtype=np.uint16)
    w = oracle.f32_to_bf16_rne(rng.normal(0, 0.02, (20, 32)).astype(np.float32))
    b = rng.normal(0, 0.1, 20).astype(np.float32)
    got, _ = oracle.lmhead_logits(h, w, 0.125, b, "f32")
    assert np.array_equal(got, np.broadcast_to(b, (3, 20)))


def test_alpha_one_is_plain_projection_and_fold_equals_unfused():
    # alpha = 1 is the plain projection rounded once; alpha != 1 applies one
    # more rounded multiply to that fp32 projection.
    rng = np.random.default_rng(12)
    h = oracle.f32_to_bf16_rne(rng.normal(0, 1, (3, 64)).astype(np.float32))
    w = oracle.f32_to_bf16_rne(rng.normal(0, 0.02, (9, 64)).astype(np.float32))
    S = oracle.bf16_to_f64(h) @ oracle.bf16_to_f64(w).T
    one, _ = oracle.lmhead_logits(h, w, 1.0, None, "f32")
    assert np.array_equal(one, S.astype(np.float32))
    third, _ = oracle.lmhead_logits(h, w, 1 / 3, None, "f32")
    assert np.array_equal(third, (one * np.float32(1 / 3)).astype(np.float32))


def test_ulp_bf16():
    assert oracle.ulp_bf16(np.uint16(0x3F80)) == 2.0 ** -7       # 1.0
    assert oracle.ulp_bf16(np.uint16(0x4000)) == 2.0 ** -6       # 2.0
    assert oracle.ulp_bf16(np.uint16(0xBF80)) == 2.0 ** -7       # -1.0
    assert oracle.ulp_bf16(np.uint16(0x0000)) == 2.0 ** -133


# ---------------------------------------------------------------------------
# fp16 inputs and outputs.
# ---------------------------------------------------------------------------

def _bits(g, key):
    return np.array([[int(x, 16) for x in row] for row in g[key]], dtype=np.uint16)


def rne_f16(q: Fraction) -> Fraction:
    return round_fraction(q, 11, -14)


def _f16_bits_of(q: Fraction, negative: bool) -> int:
    """binary16 bits of the rounded value q of an exact result with the given
    sign: +-inf past the largest finite value (nearest-even overflow), a
    signed zero when the result rounded to zero."""
    sign = 0x8000 if negative else 0
    if abs(q) >= 65520:          # 65504 + half its spacing: rounds past the largest finite
        return 0x7C00 | sign
    return int(np.float16(float(abs(q))).view(np.uint16)) | sign


def test_hand_example_f16():
    g = load_golden("hand_f16.txt")
    h, w = _bits(g, "hidden"), _bits(g, "weight")
    alpha = num(g["alpha"][0][0])
    b = _rows(g, "bias")[0].astype(np.float32)
    S, _ = oracle.dot_f64(h, w, "f16")
    assert np.array_equal(S, _rows(g, "dot"))
    for bias, key in ((None, "nobias"), (b, "withbias")):
        got32, _ = oracle.lmhead_logits(h, w, alpha, bias, "f32", in_dtype="f16")
        want32 = _rows(g, key + "_f32").astype(np.float32)
        assert np.array_equal(got32.view(np.uint32), want32.view(np.uint32)), key
        got16, _ = oracle.lmhead_logits(h, w, alpha, bias, "f16", in_dtype="f16")
        assert np.array_equal(got16, _bits(g, key + "_f16")), key
    # read as bf16 the same bits give other products: the input type matters
    S_bf, _ = oracle.dot_f64(h, w, "bf16")
    assert not np.array_equal(S_bf, S)


def test_f16_decode_exhaustive_vs_numpy():
    bits = np.arange(65536, dtype=np.uint16)
    ours = oracle.f16_to_f64(bits)
    theirs = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(ours, theirs, equal_nan=True)
    assert np.array_equal(np.signbit(ours), np.signbit(theirs))
    # landmarks of the format: 1, smallest subnormal, smallest normal, largest finite
    assert oracle.f16_to_f64(np.uint16(0x3C00)) == 1.0
    assert oracle.f16_to_f64(np.uint16(0x0001)) == 2.0 ** -24
    assert oracle.f16_to_f64(np.uint16(0x0400)) == 2.0 ** -14
    assert oracle.f16_to_f64(np.uint16(0x7BFF)) == 65504.0
    assert oracle.f16_to_f64(np.uint16(0xFC00)) == -np.inf


def test_f64_to_f16_correct_rounding_vs_fractions():
    rng = np.random.default_rng(13)
    xs = list(rng.normal(0, 1, 2000) * np.exp2(rng.integers(-28, 17, 2000)))
    # exact ties and their neighbours in normal and subnormal binades
    for _ in range(300):
        e = int(rng.integers(-24, 16))
        n = int(rng.integers(1024, 2048))
        tie = (Fraction(n) + Fraction(1, 2)) * Fraction(2) ** (max(e, -14) - 10)
        for d in (Fraction(1, 2**30), -Fraction(1, 2**30), 0):
            xs.append(float(tie + d * Fraction(2) ** e))
    # overflow threshold: 65504 + 16 is the tie between 65504 and 2^16
    xs += [65504.0, 65519.99, 65520.0, 65536.0, 1e6, -65520.0, -65519.0, 0.0, -0.0,
           2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -26, 3 * 2.0 ** -25]
    xs = np.array(xs, dtype=np.float64)
    got = oracle.f64_to_f16_correct(xs)
    want = np.array([_f16_bits_of(rne_f16(Fraction(float(x))), bool(np.signbit(x))) for x in xs],
                    dtype=np.uint16)
    assert np.array_equal(got, want)


def test_ulp_f16():
    assert oracle.ulp_f16(np.uint16(0x3C00)) == 2.0 ** -10     # 1.0
    assert oracle.ulp_f16(np.uint16(0x4000)) == 2.0 ** -9      # 2.0
    assert oracle.ulp_f16(np.uint16(0xBC00)) == 2.0 ** -10     # -1.0
    assert oracle.ulp_f16(np.uint16(0x7BFF)) == 32.0           # 65504
    assert oracle.ulp_f16(np.uint16(0x0001)) == 2.0 ** -24     # subnormal


@pytest.mark.parametrize("seed", range(20))
def test_bruteforce_f16_vs_fractions(seed):
    rng = np.random.default_rng(1000 + seed)
    M, V = (int(x) for x in rng.integers(1, 4, 2))
    H = int(rng.integers(1, 9))
    h = rng.normal(0, 1, (M, H)).astype(np.float16).view(np.uint16)
    w = (rng.normal(0, 1, (V, H)) * np.exp2(rng.integers(-12, 3, (V, H)))).astype(
        np.float16).view(np.uint16)
    alpha = float(np.float32(rng.choice([1.0, 0.25, 1 / 3, 0.7, 1 / 16])))
    bias = rng.normal(0, 0.1, V).astype(np.float32) if seed % 2 else None
    hq = [[Fraction(float(x)) for x in row] for row in h.view(np.float16)]
    wq = [[Fraction(float(x)) for x in row] for row in w.view(np.float16)]
    got32, A = oracle.lmhead_logits(h, w, alpha, bias, "f32", in_dtype="f16")
    got16, _ = oracle.lmhead_logits(h, w, alpha, bias, "f16", in_dtype="f16")
    for m in range(M):
        for v in range(V):
            S = sum(a * b for a, b in zip(hq[m], wq[v]))
            Aq = sum(abs(a * b) for a, b in zip(hq[m], wq[v]))
            assert abs(A[m, v] - float(Aq)) <= 1e-15 * float(Aq)
            r = rne32(S)
            r = rne32(r * Fraction(alpha))
            if bias is not None:
                r = rne32(r + Fraction(float(bias[v])))
            assert got32[m, v] == np.float32(float(r)), (m, v)
            y = Fraction(alpha) * S + (Fraction(float(bias[v])) if bias is not None else 0)
            # an exact zero sum is +0 in round-to-nearest
            assert got16[m, v] == _f16_bits_of(rne_f16(y), y < 0), (m, v)


def test_integer_f16_inputs_match_int64_matmul():
    import synth.workloads as wl
    M, V, H = 4, 29, 2048
    h = wl.int_hidden_f16(9, M, H)           # magnitudes up to 1000: not bf16 values
    w = wl.int_weight_f16(9, V, H)
    hi = h.view(np.float16).astype(np.int64)
    wi = w.view(np.float16).astype(np.int64)
    assert np.abs(hi).max() > 256
    exact = hi @ wi.T
    for alpha in (1.0, 0.125):
        got, _ = oracle.lmhead_logits(h, w, alpha, None, "f32", in_dtype="f16")
        want = (exact.astype(np.float32) * np.float32(alpha)).astype(np.float32)
        assert np.array_equal(got, want)


# ---------------------------------------------------------------------------
# Row reduction (max, lowest argmax, sum of exp(x - max)).
# ---------------------------------------------------------------------------

def test_rowreduce_hand_example():
    g = load_golden("rowreduce_hand.txt")
    h = f32_bits_to_bf16_bits_exact(_rows(g, "hidden"))
    w = f32_bits_to_bf16_bits_exact(_rows(g, "weight"))
    for a in g["alpha"][0]:
        alpha = num(a)
        mx, idx, s, x, _ = oracle.lmhead_rowreduce(h, w, alpha)
        want_m = np.array([num(v) for v in g[f"max_alpha{a}"][0]], dtype=np.float32)
        assert np.array_equal(mx.view(np.uint32), want_m.view(np.uint32)), a   # -0 kept
        assert list(idx) == [int(v) for v in g[f"argmax_alpha{a}"][0]], a
        want_s = np.array([num(v) for v in g[f"sumexp_alpha{a}"][0]])
        assert np.allclose(s, want_s, rtol=1e-14, atol=0), a


def test_rowreduce_vs_scipy_logsumexp():
    from scipy.special import logsumexp
    rng = np.random.default_rng(21)
    x = (rng.normal(0, 3, (50, 777))).astype(np.float32)
    x[7] = -100.0                              # a constant row
    x[8, [3, 400, 700]] = 50.0                 # ties far apart
    mx, idx, s = oracle.row_reduce(x)
    lse = mx.astype(np.float64) + np.log(s)
    want = logsumexp(x.astype(np.float64), axis=1)
    assert np.allclose(lse, want, rtol=1e-14, atol=1e-13)
    assert np.array_equal(mx, x.max(axis=1))
    assert idx[7] == 0 and s[7] == 777.0
    assert idx[8] == 3
    # every argmax holds the maximum, and no earlier column does
    for r in range(x.shape[0]):
        assert x[r, idx[r]] == mx[r] and np.all(x[r, :idx[r]] < mx[r])


def test_rowreduce_invariants():
    rng = np.random.default_rng(22)
    x = rng.integers(-30, 30, (20, 300)).astype(np.float32)   # integer rows: shifts are exact
    mx, idx, s = oracle.row_reduce(x)
    mx2, idx2, s2 = oracle.row_reduce(x + np.float32(1024))
    assert np.array_equal(mx2, mx + 1024) and np.array_equal(idx2, idx) and np.array_equal(s2, s)
    # reversing a row maps the lowest argmax to the highest tied column
    mr, ir, sr = oracle.row_reduce(x[:, ::-1])
    last = 299 - np.array([np.flatnonzero(row == row.max())[-1] for row in x])
    assert np.array_equal(ir, last) and np.array_equal(mr, mx)
    assert np.allclose(sr, s, rtol=1e-13)
    # one dominant column: sumexp -> 1
    y = np.full((1, 100), -1000.0, np.float32)
    y[0, 42] = 0.0
    assert oracle.row_reduce(y)[2][0] == 1.0 and oracle.row_reduce(y)[1][0] == 42


# ---------------------------------------------------------------------------
# BF16 -> NVFP4 quantisation.
# ---------------------------------------------------------------------------

def test_quantize_hand_example():
    g = load_golden("nvfp4_quant_hand.txt")
    w = f32_bits_to_bf16_bits_exact(_rows(g, "weight"))
    codes, scales, gs = oracle.quantize_nvfp4(w)
    assert gs == np.float32(num(g["g"][0][0]))
    assert list(scales[0]) == [int(x, 16) for x in g["scales"][0]]
    assert list(codes[0]) == [int(x, 16) for x in g["codes"][0]]


def test_e4m3_encoder_vs_torch():
    rng = np.random.default_rng(31)
    x = np.concatenate([rng.uniform(0, 448, 20000), np.exp2(rng.uniform(-12, 8.8, 20000)),
                        # exact ties between neighbouring E4M3 values
                        (oracle.e4m3_to_f64(np.arange(0, 126)) + oracle.e4m3_to_f64(np.arange(1, 127))) / 2
                        ]).astype(np.float32)
    x = x[x <= 448]
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.f32_to_e4m3_rne(x), want)
    assert oracle.f32_to_e4m3_rne(np.float32(1e6)) == 0x7E        # saturates


def test_e2m1_rounding_thresholds():
    # The same rounding written as thresholds: the midpoints between
    # neighbouring E2M1 values, a tie going to the code whose mantissa bit is 0.
    rng = np.random.default_rng(32)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    x = np.concatenate([rng.uniform(0, 8, 50000), mids, np.nextafter(mids, 0), np.nextafter(mids, 9),
                        [0.0, 6.0, 1e9]]).astype(np.float32)
    up_at_tie = np.array([False, True, False, True, False, True, False])   # tie -> the upper code is even
    want = sum(np.where(u, x >= m, x > m) for m, u in zip(mids, up_at_tie))
    assert np.array_equal(oracle.e2m1_rne(x), want.astype(np.uint8))


def _exact_nvfp4_head(rng, V, H, k):
    """A bf16 head whose every block is exactly e2m1 x e4m3 x g with g = 2^-k,
    each block holding a code-7 (6.0) element and one block scale 448: the
    quantiser must give back these codes and scales."""
    codes = rng.integers(0, 16, (V, H)).astype(np.uint8)
    codes[:, ::16] = rng.choice([7, 15], (V, H // 16))        # +-6 in every block
    scales = rng.integers(0x08, 0x7F, (V, H // 16)).astype(np.uint8)   # normal E4M3 values
    scales[0, 0] = 0x7E
    g = 2.0 ** -k
    w = oracle.e2m1_to_f64(codes) * np.repeat(oracle.e4m3_to_f64(scales), 16, axis=1) * g
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return f32_bits_to_bf16_bits_exact(w), packed, scales, g


def test_quantize_recovers_an_exact_nvfp4_head():
    rng = np.random.default_rng(33)
    w, packed, scales, g = _exact_nvfp4_head(rng, 7, 64, 12)
    c2, s2, g2 = oracle.quantize_nvfp4(w)
    assert g2 == np.float32(g) and np.array_equal(s2, scales)
    # a code for +-0 may come back with either sign bit: compare values
    assert np.array_equal(oracle.e2m1_to_f64(oracle.unpack_e2m1(c2, 64)),
                          oracle.e2m1_to_f64(oracle.unpack_e2m1(packed, 64)))


def test_quantize_scale_invariance_error_bound_and_zero():
    rng = np.random.default_rng(34)
    w = oracle.f32_to_bf16_rne(rng.normal(0, 0.02, (9, 96)).astype(np.float32))
    c, s, g = oracle.quantize_nvfp4(w)
    w2 = f32_bits_to_bf16_bits_exact(oracle.bf16_to_f64(w) * 4)      # exact
    c2, s2, g2 = oracle.quantize_nvfp4(w2)
    assert np.array_equal(c, c2) and np.array_equal(s, s2) and g2 == np.float32(4 * g)
    # every element is within half an E2M1 spacing (in units of its block's
    # scale d), or saturated at 6 when it exceeds 6 d
    wf = oracle.bf16_to_f64(w)
    d = np.repeat(oracle.e4m3_to_f64(s) * np.float64(g), 16, axis=1)
    q = oracle.e2m1_to_f64(oracle.unpack_e2m1(c, 96))
    x = np.abs(wf) / d
    half = np.where(x < 2, 0.25, np.where(x < 4, 0.5, 1.0)) * (1 + 1e-6)
    assert np.all((np.abs(np.abs(q) - x) <= half) | ((x > 6) & (np.abs(q) == 6)))
    assert np.all(np.sign(q) * np.sign(wf) >= 0)
    z, zs, zg = oracle.quantize_nvfp4(np.zeros((2, 32), np.uint16))
    assert zg == 1.0 and not z.any() and not zs.any()
