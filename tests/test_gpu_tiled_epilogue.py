"""The tiled kernel's two logits stores and its two loop tails. Rows of
16-byte aligned length (V % 8 == 0) leave through LDS as whole rows, except
in the work-group's last columns when they run past V; other widths are
stored block by block. The stage count's parity picks the loop tail of the
256-row tiles (one or two stages left, the last one full or a single K-step).
Every combination must give the oracle's values, the weight-streaming
kernel's bits, bf16 logits equal to the fp32 logits rounded to nearest even,
and rows that do not depend on M."""
import numpy as np
import pytest
import torch

import lm_head_logits_amd as L
import oracle
from gpu_util import bf16_dev, f16_dev, f32_dev, host_bits, host_f32, say
from helpers import check_f32

pytestmark = pytest.mark.gpu


def _rand(rng, shape, std, f16):
    x = rng.normal(0, std, shape).astype(np.float32)
    return x.astype(np.float16).view(np.uint16) if f16 else oracle.f32_to_bf16_rne(x)


# H: K-steps 2 (one full stage left), 3 (two left, the last a single K-step),
# 6 (one full stage after the loop), 7 (two left, the last a single K-step)
@pytest.mark.parametrize("H", [64, 96, 192, 224])
@pytest.mark.parametrize("V", [4104, 4100])
def test_tiled_stores_and_tails(H, V):
    rng = np.random.default_rng(H * 10007 + V)
    M = 300
    f16 = H == 96
    say(f"tiled epilogue and tails M={M} H={H} V={V} f16={f16}")
    h = _rand(rng, (M, H), 1.0, f16)
    W = _rand(rng, (V, H), 0.02, f16)
    b = rng.normal(0, 0.1, V).astype(np.float32)
    dev = f16_dev if f16 else bf16_dev
    hd, Wd, bd = dev(h), dev(W), f32_dev(b)
    t32 = L.logits(hd, Wd, 0.125, bd, torch.float32, path="tiled")
    s32 = L.logits(hd, Wd, 0.125, bd, torch.float32, path="skinny")
    bits = host_bits(t32)
    assert np.array_equal(bits, host_bits(s32)), "tiled and weight-streaming kernels differ"
    ref, A = oracle.lmhead_logits(h, W, 0.125, b, "f32", in_dtype="f16" if f16 else "bf16")
    check_f32(host_f32(t32), ref, A, what=f"H={H} V={V} f16={f16}")
    dt16 = torch.float16 if f16 else torch.bfloat16
    t16 = host_bits(L.logits(hd, Wd, 0.125, bd, dt16, path="tiled"))
    f32v = bits.view(np.float32)
    want16 = f32v.astype(np.float16).view(np.uint16) if f16 else oracle.f32_to_bf16_rne(f32v)
    assert np.array_equal(t16, want16), "16-bit logits are not the fp32 logits rounded"
    for m in (129, 256, 257):
        part = host_bits(L.logits(hd[:m], Wd, 0.125, bd, torch.float32, path="tiled"))
        assert np.array_equal(part, bits[:m]), m
