"""GPU parity at the largest sizes the shape contract allows: V = 2^20 (the
largest vocabulary; the weight-streaming grid then holds several rounds of
work-groups and the row-combine kernel several load rounds), H = 65536 (the
largest row length: 2 MB per 16-row column block, 128 KB per hidden row), the
NVFP4 head at V = 2^20, and the row reduction at V = 2^20. Sampled columns
(the first, every group boundary, random ones and the last) against the
oracle; the kernels against each other bit for bit."""
import numpy as np
import pytest
import torch

import lm_head_logits_amd as L
import oracle
from gpu_util import bf16_dev, host_bits, host_f32, say, u8_dev
from helpers import check_bf16, check_f32, check_rowreduce_self

pytestmark = pytest.mark.gpu

PATHS = ("skinny", "tiled")
VMAX = 1 << 20
HMAX = 1 << 16


def _rand_bf16(rng, shape, std):
    # normal draws rounded to bf16, in slices (a few hundred MB at these sizes)
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(shape[0], -1)
    for a in range(0, shape[0], 65536):
        flat[a:a + 65536] = oracle.f32_to_bf16_rne(
            rng.normal(0, std, (min(65536, shape[0] - a),) + tuple(shape[1:])).astype(np.float32))
    return out


def _cols(V, n=300, seed=0):
    rng = np.random.default_rng(seed)
    b = [c for g in range(1, V // 10240 + 1) for c in (g * 10240 - 1, g * 10240) if c < V][:40]
    return np.unique(np.r_[np.arange(4), b, rng.choice(V, n, replace=False), np.arange(V - 8, V)])


@pytest.mark.parametrize("H", [256, 512])   # one K start; several (H / 256 = 2)
def test_largest_vocabulary(H):
    V = VMAX
    rng = np.random.default_rng(H)
    say(f"V = 2^20, H = {H}: generate the head")
    W = _rand_bf16(rng, (V, H), 0.02)
    Wd = bf16_dev(W)
    h = _rand_bf16(rng, (65, H), 1.0)
    hd = bf16_dev(h)
    cols = _cols(V, seed=H)
    for M in (1, 64, 65):
        say(f"  M={M}")
        outs = {p: host_bits(L.logits(hd[:M], Wd, 0.5, None, torch.float32, path=p)) for p in PATHS}
        assert np.array_equal(outs["skinny"], outs["tiled"]), M
        ref, A = oracle.lmhead_logits(h[:M], W[cols], 0.5, None, "f32")
        check_f32(outs["skinny"].view(np.float32)[:, cols], ref, 0.5 * A, what=f"V=2^20 M={M}")
    del Wd
    torch.cuda.empty_cache()


def test_longest_rows():
    # H = 65536 over two column groups (V > 10240): 256 K starts in the stagger
    H, V = HMAX, 10240 + 100
    rng = np.random.default_rng(7)
    say(f"H = 2^16, V = {V}: generate the head")
    W = _rand_bf16(rng, (V, H), 0.02)
    Wd = bf16_dev(W)
    h = _rand_bf16(rng, (65, H), 1.0)
    hd = bf16_dev(h)
    cols = _cols(V, n=120, seed=7)
    for M in (1, 65):
        say(f"  M={M}")
        outs = {p: host_bits(L.logits(hd[:M], Wd, 0.5, None, torch.float32, path=p)) for p in PATHS}
        assert np.array_equal(outs["skinny"], outs["tiled"]), M
        ref, A = oracle.lmhead_logits(h[:M], W[cols], 0.5, None, "f32")
        check_f32(outs["skinny"].view(np.float32)[:, cols], ref, 0.5 * A, what=f"H=2^16 M={M}")
    del Wd
    torch.cuda.empty_cache()


def test_nvfp4_largest_vocabulary():
    V, H = VMAX, 512
    rng = np.random.default_rng(11)
    say("NVFP4 V = 2^20, H = 512")
    codes = rng.integers(0, 256, (V, H // 2), dtype=np.uint8)
    scales = rng.choice(np.r_[0x30:0x4A], (V, H // 16)).astype(np.uint8)
    cd, sd = u8_dev(codes), u8_dev(scales)
    h = _rand_bf16(rng, (130, H), 1.0)
    hd = bf16_dev(h)
    cols = _cols(V, seed=11)
    full = None
    for M in (1, 40, 130):   # ring, register-streaming, tiled
        say(f"  M={M}")
        got = host_bits(L.logits_nvfp4(hd[:M].contiguous(), cd, sd, 0.01, 1.0))
        ref, A = oracle.lmhead_logits_nvfp4(h[:M], codes[cols], scales[cols], 0.01, 1.0)
        check_bf16(got[:, cols], ref, A, 0.01, oracle.ulp_bf16, what=f"nvfp4 V=2^20 M={M}")
        if full is None:
            full = host_bits(L.logits_nvfp4(hd, cd, sd, 0.01, 1.0))
        assert np.array_equal(got, full[:M]), M     # rows do not depend on the row count
    del cd, sd
    torch.cuda.empty_cache()


def test_rowreduce_largest_vocabulary():
    # 65536 column blocks per row: the combine kernel's threads loop over
    # several rounds of loads
    V, H, M = VMAX, 256, 24
    rng = np.random.default_rng(13)
    say("row reduction V = 2^20")
    Wd = bf16_dev(_rand_bf16(rng, (V, H), 0.02))
    hd = bf16_dev(_rand_bf16(rng, (M, H), 1.0))
    for p in PATHS:
        mx, am, se, lg = L.logits_rowreduce(hd, Wd, 0.5, write_logits=True, path=p)
        check_rowreduce_self(host_f32(mx), am.cpu().numpy(), host_f32(se), host_f32(lg))
    del Wd
    torch.cuda.empty_cache()
