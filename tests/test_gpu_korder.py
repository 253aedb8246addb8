"""GPU tests of where each column's K reduction starts: the start is
((v // 10240) * 5 mod (H / 256)) * 256 for column v of the call (0 when
H % 256 != 0), and the chain of 32-element K-steps wraps around the row end.

An input built so that each logit reveals its order: one hidden row holds
+2^24, 1 and -2^24 at three K-steps (one nonzero product per K-step and
column, so the MFMA's own summation inside a step does not matter), and every
weight row is 1 there. In fp32 the 1 is absorbed when it is added to 2^24 and
kept when it is added to -2^24 or to 0 first, so the logit is 0 or 1 by the
order in which the chain meets the three steps. The expected logits come from
the stated rule, computed on the host in fp32. Then parity with the oracle and
kernel-to-kernel bit identity at shapes where several starts are in use."""
import numpy as np
import pytest
import torch

import lm_head_logits_amd as L
import oracle
from gpu_util import DEV, bf16_dev, f32_dev, host_bits, host_f32, say, u8_dev
from helpers import check_bf16, check_f32, f32_bits_to_bf16_bits_exact

pytestmark = pytest.mark.gpu

PATHS = ("skinny", "tiled")
GROUP = 10240
KSTEP = 32


def start_of(v, H):
    """The stated starting K element of column v (host restatement)."""
    if H % 256:
        return 0
    return ((v // GROUP) * 5 % (H // 256)) * 256


def chain_f32(products, H, start):
    """fp32 sum of {k: product} over the K-steps from `start`, wrapping."""
    nk = H // KSTEP
    acc = np.float32(0.0)
    for i in range(nk):
        s = (start // KSTEP + i) % nk
        for k, p in products.items():
            if k // KSTEP == s:
                acc = np.float32(acc + np.float32(p))
    return acc


# H = 1024: four 256-element quads; V: five groups, the last one ragged.
H_PIN, V_PIN = 1024, 4 * GROUP + 77
# Two probe rows whose logits together tell the four possible starts apart.
PROBES = ({0: 2.0 ** 24, 300: 1.0, 600: -(2.0 ** 24)},
          {300: 2.0 ** 24, 600: 1.0, 900: -(2.0 ** 24)})
KS = (0, 300, 600, 900)


def _pin_inputs(M):
    h = np.zeros((M, H_PIN), dtype=np.float32)
    rows = (0, 1, M - 2, M - 1) if M >= 4 else tuple(range(M))
    for i, r in enumerate(rows):
        for k, x in PROBES[i % 2].items():
            h[r, k] = x
    W = np.zeros((V_PIN, H_PIN), dtype=np.float32)
    W[:, list(KS)] = 1.0
    expect = np.zeros((M, V_PIN), dtype=np.float32)
    starts = np.array([start_of(v, H_PIN) for v in range(V_PIN)])
    for i, r in enumerate(rows):
        per_start = {s: chain_f32(PROBES[i % 2], H_PIN, s) for s in set(starts.tolist())}
        expect[r] = np.array([per_start[s] for s in starts], dtype=np.float32)
    return h, W, expect, rows


def test_pin_covers_every_start():
    # the probe rows' expected logits differ for each of the four starts
    pats = {tuple(chain_f32(p, H_PIN, s) for p in PROBES) for s in (0, 256, 512, 768)}
    assert len(pats) == 4


@pytest.mark.parametrize("M", [1, 40, 64, 65, 130])
def test_k_order_start_bf16_paths(M):
    say(f"K-order pin, bf16, M={M}")
    h, W, expect, rows = _pin_inputs(M)
    hd = bf16_dev(f32_bits_to_bf16_bits_exact(h))
    Wd = bf16_dev(f32_bits_to_bf16_bits_exact(W))
    for p in PATHS + ("auto",):
        got = host_f32(L.logits(hd, Wd, 1.0, None, torch.float32, path=p))
        assert np.array_equal(got, expect), (p, [int(np.sum(got[r] != expect[r])) for r in rows])


@pytest.mark.parametrize("M", [1, 40, 130])
def test_k_order_start_nvfp4(M):
    say(f"K-order pin, NVFP4, M={M}")
    h, W, expect, rows = _pin_inputs(M)
    hd = bf16_dev(f32_bits_to_bf16_bits_exact(h))
    codes = np.zeros((V_PIN, H_PIN // 2), dtype=np.uint8)
    codes[:, [k // 2 for k in KS]] = 0x02          # E2M1 code 2 = 1.0 in the low nibble (even k)
    scales = np.full((V_PIN, H_PIN // 16), 0x38, dtype=np.uint8)  # E4M3 1.0
    got = host_bits(L.logits_nvfp4(hd, u8_dev(codes), u8_dev(scales), 1.0, 1.0))
    ref = oracle.f32_to_bf16_rne(expect)            # 0 and 1 are exact in bf16
    assert np.array_equal(got, ref)


def test_k_order_start_nvfp4_generic_kernel():
    # scales at a 2-byte (not 16-byte) aligned address take the generic kernel
    say("K-order pin, NVFP4 generic kernel")
    M = 16
    h, W, expect, rows = _pin_inputs(M)
    hd = bf16_dev(f32_bits_to_bf16_bits_exact(h))
    codes = np.zeros((V_PIN, H_PIN // 2), dtype=np.uint8)
    codes[:, [k // 2 for k in KS]] = 0x02
    sc = u8_dev(np.full((V_PIN, H_PIN // 16), 0x38, dtype=np.uint8))
    big = torch.zeros(sc.numel() + 16, dtype=torch.uint8, device=DEV)
    shifted = big[2:2 + sc.numel()].view(V_PIN, H_PIN // 16)
    shifted.copy_(sc)
    got = host_bits(L.logits_nvfp4(hd, u8_dev(codes), shifted, 1.0, 1.0))
    assert np.array_equal(got, oracle.f32_to_bf16_rne(expect))


def _rand_bf16(rng, shape, std):
    return oracle.f32_to_bf16_rne(rng.normal(0, std, shape).astype(np.float32))


def _cols(V):
    # every group boundary, the ragged end, and a random sample
    rng = np.random.default_rng(V)
    b = [c for g in range(1, V // GROUP + 1) for c in (g * GROUP - 1, g * GROUP) if c < V]
    return np.unique(np.r_[np.arange(8), b, rng.choice(V, 400, replace=False), np.arange(V - 20, V)])


# several starts in use: H/256 = 2, 3, 4, 9 quads; V over two to four groups
@pytest.mark.parametrize("M,H,V", [(1, 512, 30001), (40, 768, 20483), (64, 1024, 10257),
                                   (65, 512, 30001), (130, 768, 20483), (200, 2304, 22000)])
def test_staggered_shapes_parity_and_paths_agree(M, H, V):
    rng = np.random.default_rng(M + H + V)
    say(f"staggered K order M={M} H={H} V={V}")
    h = _rand_bf16(rng, (M, H), 1.0)
    W = _rand_bf16(rng, (V, H), 0.02)
    bias = rng.normal(0, 0.1, V).astype(np.float32)
    cols = _cols(V)
    ref, A = oracle.lmhead_logits(h, W[cols], 0.125, bias[cols], "f32")
    hd, Wd, bd = bf16_dev(h), bf16_dev(W), f32_dev(bias)
    outs = {p: host_bits(L.logits(hd, Wd, 0.125, bd, torch.float32, path=p)) for p in PATHS}
    check_f32(outs["skinny"].view(np.float32)[:, cols], ref, A, what="staggered")
    assert np.array_equal(outs["skinny"], outs["tiled"])


@pytest.mark.parametrize("M,H,V", [(16, 512, 30001), (40, 768, 20483), (130, 1024, 10257)])
def test_staggered_nvfp4_parity_and_equals_bf16_path(M, H, V):
    rng = np.random.default_rng(M * 3 + H + V)
    say(f"staggered K order, NVFP4 M={M} H={H} V={V}")
    h = _rand_bf16(rng, (M, H), 1.0)
    codes = rng.integers(0, 256, (V, H // 2), dtype=np.uint8)
    scales = rng.choice(np.r_[0x30:0x4A], (V, H // 16)).astype(np.uint8)
    g, alpha = 0.01, 0.5
    cols = _cols(V)
    ref, A = oracle.lmhead_logits_nvfp4(h, codes[cols], scales[cols], g, alpha)
    got = host_bits(L.logits_nvfp4(bf16_dev(h), u8_dev(codes), u8_dev(scales), g, alpha))
    check_bf16(got[:, cols], ref, A, g * alpha, oracle.ulp_bf16, what="staggered nvfp4")
    wbits = f32_bits_to_bf16_bits_exact(oracle.nvfp4_weight_f64(codes, scales, H).astype(np.float32))
    s = float(np.float32(g) * np.float32(alpha))
    for p in PATHS:
        twin = L.logits(bf16_dev(h), bf16_dev(wbits), s, None, torch.bfloat16, path=p)
        assert np.array_equal(got, host_bits(twin)), p
