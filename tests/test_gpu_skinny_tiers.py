"""The weight-streaming kernel's launch tiers for vocabularies with few
16-column blocks per compute unit: four waves with an eight-stage ring (up to
4 blocks per CU), eight waves with eight stages (up to 8), sixteen waves with
four stages (up to 16), then sixteen waves with two stages. Every tier must
give the tiled kernel's bits and the oracle's values within tolerance, with H
shorter than the ring, H % 64 == 32 (a last stage of one K-step) and H longer
than the ring, and the same row-reduction partials."""
import numpy as np
import pytest
import torch

import lm_head_logits_amd as L
import oracle
from gpu_util import bf16_dev, f32_dev, host_bits, host_f32, say
from helpers import check_f32

pytestmark = pytest.mark.gpu


def _rand_bf16(rng, shape, std):
    return oracle.f32_to_bf16_rne(rng.normal(0, std, shape).astype(np.float32))


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


# blocks per CU -> tier: 1, 3.5 (4 waves x 8 stages), 6 (8 x 8), 12 (16 x 4), 20 (16 x 2, two blocks)
@pytest.mark.parametrize("per_cu", [1, 3.5, 6, 12, 20])
@pytest.mark.parametrize("H", [96, 160, 544])
def test_tier_equals_tiled_and_oracle(per_cu, H):
    V = int(per_cu * _cus() * 16) + 5
    rng = np.random.default_rng(int(per_cu * 10) + H)
    Mmax = 37
    say(f"skinny tiers: {per_cu} blocks per CU, V={V}, H={H}")
    W = _rand_bf16(rng, (V, H), 0.02)
    h = _rand_bf16(rng, (Mmax, H), 1.0)
    b = rng.normal(0, 0.1, V).astype(np.float32)
    Wd, hd, bd = bf16_dev(W), bf16_dev(h), f32_dev(b)
    cols = np.unique(np.r_[0, V - 1, rng.integers(0, V, 200)])
    for M in (1, 37):
        sk = L.logits(hd[:M], Wd, 0.125, bd, torch.float32, path="skinny")
        ti = L.logits(hd[:M], Wd, 0.125, bd, torch.float32, path="tiled")
        assert np.array_equal(host_bits(sk), host_bits(ti)), (M, V, H)
        ref, A = oracle.lmhead_logits(h[:M], W[cols], 0.125, b[cols], "f32")
        check_f32(host_f32(sk)[:, cols], ref, A, what=f"tier V={V} H={H} M={M}")
        mx, am, se, _ = L.logits_rowreduce(hd[:M], Wd, 0.125, bd, path="skinny")
        mx2, am2, se2, _ = L.logits_rowreduce(hd[:M], Wd, 0.125, bd, path="tiled")
        assert torch.equal(am, am2) and torch.equal(mx.view(torch.int32), mx2.view(torch.int32))
        assert torch.equal(se.view(torch.int32), se2.view(torch.int32))


@pytest.mark.parametrize("per_cu", [1, 6, 12])
def test_tier_rows_do_not_depend_on_M(per_cu):
    V, H = int(per_cu * _cus() * 16) + 3, 224
    rng = np.random.default_rng(7 + per_cu)
    say(f"skinny tiers: row invariance, V={V}")
    Wd = bf16_dev(_rand_bf16(rng, (V, H), 0.02))
    hd = bf16_dev(_rand_bf16(rng, (64, H), 1.0))
    full = host_bits(L.logits(hd, Wd, 0.5, None, torch.float32))
    for M in (1, 2, 17, 33, 63):
        assert np.array_equal(host_bits(L.logits(hd[:M], Wd, 0.5, None, torch.float32)), full[:M]), M
