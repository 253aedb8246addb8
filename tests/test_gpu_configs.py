"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: the oracle checks sampled outputs (all rows x a column
sample that includes the ragged vocabulary tail), integer-valued inputs are
checked bit for bit at every full shape, and the row-invariance contract is
checked bit for bit across row counts, row orders, target/draft calls and
vocabulary sub-ranges."""
import math

import numpy as np
import pytest
import torch

import lm_head_logits_amd as L
import oracle
import synth.workloads as wl
from gpu_util import DEV, bf16_dev, f16_dev, f32_dev, host_bits, host_f32, say, u8_dev
from helpers import check_bf16, check_f32

pytestmark = pytest.mark.gpu


def col_sample(V, n=1536, seed=0):
    rng = np.random.default_rng(seed)
    cols = np.concatenate([np.arange(16), rng.choice(V, n, replace=False), np.arange(V - 40, V)])
    return np.unique(cols)


def row_sample(M, n=48, seed=1):
    if M <= 256:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 1, M - 1], rng.choice(M, n, replace=False)]))


def ibits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


@pytest.fixture(scope="module")
def decode():
    w = wl.DECODE
    say("generate decode inputs H=4096 V=128256")
    h, W = wl.hidden(w), wl.weight(w)
    return w, h, W, bf16_dev(h), bf16_dev(W)


@pytest.fixture(scope="module")
def spec():
    w = wl.SPEC
    say("generate spec-decode inputs H=2048 V=151936")
    h, W, b = wl.hidden(w), wl.weight(w), wl.bias(w)
    return w, h, W, b, bf16_dev(h), bf16_dev(W), f32_dev(b)


@pytest.mark.parametrize("M", wl.DECODE.Ms)
@pytest.mark.parametrize("alpha", wl.DECODE.alphas)
def test_decode_parity(decode, M, alpha):
    w, h, W, hd, Wd = decode
    say(f"decode M={M} alpha={alpha}")
    got = host_f32(L.logits(hd[:M], Wd, alpha))
    cols = col_sample(w.V, seed=M)
    ref, A = oracle.lmhead_logits(h[:M], W[cols], alpha, None, "f32")
    ratio, exact = check_f32(got[:, cols], ref, A, what=f"decode M={M}")
    say(f"  max err/bound {ratio:.3f}, bit-exact fraction {exact:.3f}")


def test_prefill_parity():
    w = wl.PREFILL
    say("prefill M=2048 H=4096 V=151936")
    h, W = wl.hidden(w), wl.weight(w)
    alpha = w.alphas[0]
    out = L.logits(bf16_dev(h), bf16_dev(W), alpha)
    rows, cols = row_sample(w.M), col_sample(w.V, n=1024)
    got = host_f32(out[torch.as_tensor(rows, device=DEV)])
    ref, A = oracle.lmhead_logits(h[rows], W[cols], alpha, None, "f32")
    ratio, exact = check_f32(got[:, cols], ref, A, what="prefill")
    say(f"  max err/bound {ratio:.3f}, bit-exact fraction {exact:.3f}")
    hd, Wd = bf16_dev(h), bf16_dev(W)
    # bf16 logits (whole-row stores of 16-bit values): the oracle's on the
    # sample, and everywhere the fp32 logits rounded to nearest even
    o16 = L.logits(hd, Wd, alpha, None, torch.bfloat16)
    got16 = host_bits(o16[torch.as_tensor(rows, device=DEV)])[:, cols]
    ref16, _ = oracle.lmhead_logits(h[rows], W[cols], alpha, None, "bf16")
    check_bf16(got16, ref16, A, alpha, oracle.ulp_bf16, what="prefill bf16")
    assert torch.equal(ibits(o16), ibits(out.to(torch.bfloat16)))
    # rows of a shorter call (a ragged 256-row tile) equal the full call's
    part = L.logits(hd[:300].contiguous(), Wd, alpha)
    assert torch.equal(ibits(part), ibits(out[:300]))


@pytest.mark.parametrize("shape", [("decode", 64, 4096, 128256), ("prefill", 2048, 4096, 151936),
                                   ("spec", 128, 2048, 151936)])
def test_integer_inputs_exact_at_full_shape(shape):
    name, M, H, V = shape
    say(f"integer-exact {name} M={M} H={H} V={V}")
    h = wl.int_hidden(31, M, H)
    W = wl.int_weight(31, V, H)
    out = L.logits(bf16_dev(h), bf16_dev(W), 0.125)
    rows, cols = row_sample(M), col_sample(V, n=1024)
    got = host_bits(out[torch.as_tensor(rows, device=DEV)])[:, cols]
    ref, _ = oracle.lmhead_logits(h[rows], W[cols], 0.125, None, "f32")
    assert np.array_equal(got, ref.view(np.uint32))


def test_spec_target_parity(spec):
    w, h, W, b, hd, Wd, bd = spec
    say("spec-decode target M=128 with bias")
    alpha = w.alphas[0]
    got = host_f32(L.logits(hd, Wd, alpha, bd))
    cols = col_sample(w.V, seed=4)
    ref, A = oracle.lmhead_logits(h, W[cols], alpha, b[cols], "f32")
    ratio, exact = check_f32(got[:, cols], ref, A, what="spec")
    say(f"  max err/bound {ratio:.3f}, bit-exact fraction {exact:.3f}")


def test_spec_rows_invariant_across_row_counts(spec):
    w, h, W, b, hd, Wd, bd = spec
    alpha = w.alphas[0]
    full = L.logits(hd, Wd, alpha, bd)
    for M in range(1, w.M + 1):
        part = L.logits(hd[:M], Wd, alpha, bd)
        if not torch.equal(ibits(part), ibits(full[:M])):
            raise AssertionError(f"rows of the M={M} call differ from the M={w.M} call")
    say("  M = 1..128 all bit-identical prefixes (skinny <= 64 < tiled)")


def test_spec_rows_invariant_to_order_and_draft_gather(spec):
    w, h, W, b, hd, Wd, bd = spec
    alpha = w.alphas[0]
    target = L.logits(hd, Wd, alpha, bd)                    # 32 sequences x 4 tokens
    rev = L.logits(torch.flip(hd, [0]).contiguous(), Wd, alpha, bd)
    assert torch.equal(ibits(torch.flip(rev, [0])), ibits(target))
    for j in range(4):                                      # the draft call: one token per sequence
        idx = torch.arange(32, device=DEV) * 4 + j
        draft = L.logits(hd[idx].contiguous(), Wd, alpha, bd)
        assert torch.equal(ibits(draft), ibits(target[idx])), j


def test_spec_vocab_shard_equals_full(spec):
    # Column v's K order starts at ((v // 10240) * 5 mod (H / 256)) * 256, v
    # counted within the call: a vocabulary shard reproduces the full call's
    # columns bit for bit when its first column is a multiple of
    # 10240 * (H / 256) (5 and H / 256 = 8 coprime here), at any width,
    # ragged end included.
    w, h, W, b, hd, Wd, bd = spec
    alpha = w.alphas[0]
    full = L.logits(hd, Wd, alpha, bd)
    period = 10240 * (w.H // 256) // math.gcd(5, w.H // 256)
    for v0, v1 in ((0, 18992), (0, 10240 + 16), (period, period + 18992), (period, w.V)):
        part = L.logits(hd, Wd[v0:v1], alpha, bd[v0:v1])
        assert torch.equal(ibits(part), ibits(full[:, v0:v1])), (v0, v1)
        part32 = L.logits(hd[:32].contiguous(), Wd[v0:v1], alpha, bd[v0:v1])
        assert torch.equal(ibits(part32), ibits(full[:32, v0:v1])), (v0, v1)


@pytest.fixture(scope="module")
def nvfp4():
    w = wl.NVFP4
    say("generate NVFP4 inputs H=2048 V=151936")
    h, c, s = wl.hidden(w), wl.codes(w), wl.scales(w)
    return w, h, c, s, bf16_dev(h), u8_dev(c), u8_dev(s)


@pytest.mark.parametrize("M", wl.NVFP4.Ms)
def test_nvfp4_parity(nvfp4, M):
    w, h, c, s, hd, cd, sd = nvfp4
    say(f"nvfp4 M={M}")
    got = host_bits(L.logits_nvfp4(hd[:M], cd, sd, w.g, 1.0))
    cols = col_sample(w.V, seed=M)
    ref, A = oracle.lmhead_logits_nvfp4(h[:M], c[cols], s[cols], w.g, 1.0)
    strict = check_bf16(got[:, cols], ref, A, w.g, oracle.ulp_bf16, what=f"nvfp4 M={M}")
    say(f"  elements beyond 1 bf16 ulp (cancellation near zero): {strict} of {ref.size}")


def test_nvfp4_rows_invariant(nvfp4):
    w, h, c, s, hd, cd, sd = nvfp4
    full = L.logits_nvfp4(hd, cd, sd, w.g, 1.0)
    for M in (1, 2, 15, 16, 17, 63, 64, 65, 128, 255):
        part = L.logits_nvfp4(hd[:M].contiguous(), cd, sd, w.g, 1.0)
        assert torch.equal(ibits(part), ibits(full[:M])), M


@pytest.fixture(scope="module")
def f16():
    w = wl.F16
    say("generate fp16 inputs H=4096 V=128256")
    h, W = wl.hidden(w), wl.weight(w)
    return w, h, W, f16_dev(h), f16_dev(W)


@pytest.mark.parametrize("M", wl.F16.Ms)
def test_f16_parity(f16, M):
    w, h, W, hd, Wd = f16
    say(f"fp16 M={M}")
    alpha = w.alphas[0]
    out = L.logits(hd[:M], Wd, alpha)
    rows, cols = row_sample(M), col_sample(w.V, n=1024, seed=M)
    got = host_f32(out[torch.as_tensor(rows, device=DEV)])
    ref, A = oracle.lmhead_logits(h[rows], W[cols], alpha, None, "f32", in_dtype="f16")
    ratio, exact = check_f32(got[:, cols], ref, A, what=f"fp16 M={M}")
    say(f"  max err/bound {ratio:.3f}, bit-exact fraction {exact:.3f}")


def test_f16_rows_invariant(f16):
    w, h, W, hd, Wd = f16
    full = L.logits(hd, Wd, w.alphas[0])
    for M in (1, 7, 64, 65, 300):
        part = L.logits(hd[:M].contiguous(), Wd, w.alphas[0])
        assert torch.equal(ibits(part), ibits(full[:M])), M
