"""GPU parity of the fp16-input path (both inputs fp16, logits fp32 or fp16):
the hand example, ragged shapes on both kernels, exact integer inputs beyond
bf16's range, the epilogue identities, overflow, and the dtype contract.
Every call goes through the C ABI (lmhead_logits_ex, via the ctypes binding)."""
import numpy as np
import pytest
import torch

import lm_head_logits_amd as L
import oracle
import synth.workloads as wl
from gpu_util import DEV, bf16_dev, f16_dev, f32_dev, host_bits, host_f32, say
from helpers import check_f16, check_f32, load_golden, num

pytestmark = pytest.mark.gpu

PATHS = ("skinny", "tiled")


def _rand_f16(rng, shape, std):
    return rng.normal(0, std, shape).astype(np.float32).astype(np.float16).view(np.uint16)


def _bits(g, key):
    return np.array([[int(x, 16) for x in row] for row in g[key]], dtype=np.uint16)


def _rows(g, key):
    return np.array([[num(x) for x in row] for row in g[key]], dtype=np.float64)


@pytest.mark.parametrize("path", PATHS)
def test_hand_example_bitwise(path):
    g = load_golden("hand_f16.txt")
    say(f"fp16 hand example via {path}")
    h = np.zeros((1, 32), np.uint16)
    w = np.zeros((3, 32), np.uint16)
    h[:, :4] = _bits(g, "hidden")            # H = 4 zero-padded to one K-step
    w[:, :4] = _bits(g, "weight")
    alpha = num(g["alpha"][0][0])
    b = f32_dev(_rows(g, "bias")[0])
    for bias, key in ((None, "nobias"), (b, "withbias")):
        o32 = L.logits(f16_dev(h), f16_dev(w), alpha, bias, torch.float32, path=path)
        want = _rows(g, key + "_f32").astype(np.float32)
        assert np.array_equal(host_bits(o32), want.view(np.uint32)), key
        o16 = L.logits(f16_dev(h), f16_dev(w), alpha, bias, torch.float16, path=path)
        assert np.array_equal(host_bits(o16), _bits(g, key + "_f16")), key


SHAPES = [(1, 32, 1), (3, 32, 17), (5, 96, 1000), (16, 64, 4111), (63, 160, 333), (64, 128, 257),
          (65, 96, 129), (130, 224, 515), (200, 32, 2000), (7, 1024, 4097), (100, 64, 65601)]


@pytest.mark.parametrize("M,H,V", SHAPES)
def test_ragged_shapes_parity_and_paths_agree(M, H, V):
    rng = np.random.default_rng(M * 1000 + H + V + 7)
    say(f"fp16 ragged M={M} H={H} V={V}")
    h = _rand_f16(rng, (M, H), 1.0)
    W = _rand_f16(rng, (V, H), 0.02)
    bias = rng.normal(0, 0.1, V).astype(np.float32)
    alpha = 0.125
    hd, Wd, bd = f16_dev(h), f16_dev(W), f32_dev(bias)
    ref, A = oracle.lmhead_logits(h, W, alpha, bias, "f32", in_dtype="f16")
    outs = {p: L.logits(hd, Wd, alpha, bd, torch.float32, path=p) for p in PATHS}
    check_f32(host_f32(outs["skinny"]), ref, A, what="fp16 skinny")
    assert np.array_equal(host_bits(outs["skinny"]), host_bits(outs["tiled"])), \
        "skinny and tiled kernels must agree bit for bit"
    assert np.array_equal(host_bits(L.logits(hd, Wd, alpha, bd, torch.float32)),
                          host_bits(outs["skinny"]))
    ref16, _ = oracle.lmhead_logits(h, W, alpha, bias, "f16", in_dtype="f16")
    o16 = {p: L.logits(hd, Wd, alpha, bd, torch.float16, path=p) for p in PATHS}
    check_f16(host_bits(o16["tiled"]), ref16, A, alpha, oracle.ulp_f16, what="fp16 out")
    assert np.array_equal(host_bits(o16["skinny"]), host_bits(o16["tiled"]))


@pytest.mark.parametrize("H", [32, 96, 192])
@pytest.mark.parametrize("M", [1, 64])
def test_weight_stream_paths_match_tiled(M, H):
    rng = np.random.default_rng(M * 11 + H)
    V = 70001
    say(f"fp16 stream vs tiled M={M} H={H} V={V}")
    hd = f16_dev(_rand_f16(rng, (M, H), 1.0))
    Wd = f16_dev(_rand_f16(rng, (V, H), 0.02))
    a = L.logits(hd, Wd, 0.5, None, torch.float32, path="skinny")
    b = L.logits(hd, Wd, 0.5, None, torch.float32, path="tiled")
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_integer_inputs_are_exact():
    # |hidden| <= 1000 (past bf16's 8 significant bits), |weight| <= 4, H = 1024:
    # every partial sum stays below 2^24, so every summation order is exact.
    M, H, V = 37, 1024, 3001
    say("fp16 integer exact")
    h = wl.int_hidden_f16(21, M, H)
    W = wl.int_weight_f16(21, V, H)
    for alpha in (1.0, 0.0625):
        ref, _ = oracle.lmhead_logits(h, W, alpha, None, "f32", in_dtype="f16")
        for p in PATHS:
            got = L.logits(f16_dev(h), f16_dev(W), alpha, None, torch.float32, path=p)
            assert np.array_equal(host_bits(got), ref.view(np.uint32)), (p, alpha)


@pytest.mark.parametrize("path", PATHS)
def test_epilogue_identities_and_overflow(path):
    rng = np.random.default_rng(6)
    M, H, V = 48, 512, 3000
    say(f"fp16 epilogue via {path}")
    hd = f16_dev(_rand_f16(rng, (M, H), 1.0))
    Wd = f16_dev(_rand_f16(rng, (V, H), 0.02))
    base = L.logits(hd, Wd, 1.0, None, torch.float32, path=path)
    for a in (1 / 8, 1 / 3, 0.7):
        fused = L.logits(hd, Wd, a, None, torch.float32, path=path)
        unfused = base * torch.tensor(a, dtype=torch.float32, device=DEV)
        assert torch.equal(fused.view(torch.int32), unfused.view(torch.int32)), a
    b = f32_dev(rng.normal(0, 0.1, V))
    with_b = L.logits(hd, Wd, 0.7, b, torch.float32, path=path)
    # the fp16 output is the fp32 output rounded to nearest even
    o16 = L.logits(hd, Wd, 0.7, b, torch.float16, path=path)
    assert np.array_equal(host_bits(o16), host_f32(with_b).astype(np.float16).view(np.uint16))
    # logits past fp16's largest finite value become infinities of their sign
    big = L.logits(hd, Wd, 1e5, None, torch.float16, path=path)
    big32 = host_f32(L.logits(hd, Wd, 1e5, None, torch.float32, path=path))
    assert np.array_equal(host_bits(big), big32.astype(np.float16).view(np.uint16))
    assert np.isinf(big.float().cpu().numpy()).any()


def test_dtype_contract():
    say("fp16 dtype contract")
    rng = np.random.default_rng(9)
    h16 = f16_dev(_rand_f16(rng, (4, 64), 1.0))
    w16 = f16_dev(_rand_f16(rng, (100, 64), 0.02))
    hb = bf16_dev(np.zeros((4, 64), np.uint16))
    wb = bf16_dev(np.zeros((100, 64), np.uint16))
    sentinel = torch.full((4, 100), 7.0, device=DEV)
    with pytest.raises(L.NotHandled):            # mixed 16-bit input types
        L.logits(h16, wb, out=sentinel)
    with pytest.raises(L.NotHandled):
        L.logits(hb, w16, out=sentinel)
    with pytest.raises(L.NotHandled):            # fp32 inputs
        L.logits(h16.float(), w16.float(), out=sentinel)
    s16 = torch.full((4, 100), 7.0, device=DEV, dtype=torch.bfloat16)
    with pytest.raises(L.NotHandled):            # logits of the other 16-bit type
        L.logits(h16, w16, out_dtype=torch.bfloat16, out=s16)
    torch.cuda.synchronize()
    assert torch.all(sentinel == 7.0) and torch.all(s16 == 7.0)
