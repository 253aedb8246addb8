"""GPU parity of the BF16 -> NVFP4 quantiser (lmhead_quantize_nvfp4): codes,
block scales and the per-tensor scale bit for bit against the oracle (integer
decisions taken in binary32 on both sides), on the hand example, ragged and
full-size heads, an exactly representable head and the all-zero head; and
the quantised head run through the NVFP4 projection."""
import numpy as np
import pytest
import torch

import lm_head_logits_amd as L
import oracle
import synth.workloads as wl
from gpu_util import DEV, bf16_dev, host_bits, say
from helpers import check_bf16, f32_bits_to_bf16_bits_exact, load_golden, num

pytestmark = pytest.mark.gpu


def _np(t):
    return t.detach().cpu().numpy()


def _rows(g, key):
    return np.array([[num(x) for x in row] for row in g[key]], dtype=np.float64)


def _check(w_bits, codes, scales, g, amax=None, what=""):
    rc, rs, rg = oracle.quantize_nvfp4(w_bits, amax)
    assert _np(g)[0] == rg, f"{what}: global scale {_np(g)[0]!r} != {rg!r}"
    assert np.array_equal(_np(scales), rs), f"{what}: block scales differ"
    bad = _np(codes) != rc
    assert not bad.any(), f"{what}: {int(bad.sum())} code bytes differ, first at {np.argwhere(bad)[0]}"


def test_hand_example():
    gg = load_golden("nvfp4_quant_hand.txt")
    say("quantise hand example")
    w = f32_bits_to_bf16_bits_exact(_rows(gg, "weight"))
    codes, scales, g = L.quantize_nvfp4(bf16_dev(w))
    assert _np(g)[0] == num(gg["g"][0][0])
    assert list(_np(scales)[0]) == [int(x, 16) for x in gg["scales"][0]]
    assert list(_np(codes)[0]) == [int(x, 16) for x in gg["codes"][0]]


@pytest.mark.parametrize("V,H", [(1, 32), (3, 64), (17, 96), (1000, 2048), (4097, 160), (333, 4096)])
def test_random_heads_bitwise(V, H):
    rng = np.random.default_rng(V * 7 + H)
    say(f"quantise V={V} H={H}")
    wf = rng.normal(0, 0.02, (V, H))
    wf[rng.random((V, H)) < 0.001] *= 50            # a few outliers spread the block scales
    wf[:, 16:32] *= 1e-6                            # blocks far below the tensor maximum
    w = oracle.f32_to_bf16_rne(wf.astype(np.float32))
    codes, scales, g = L.quantize_nvfp4(bf16_dev(w))
    _check(w, codes, scales, g, what=f"V={V} H={H}")


def test_exact_head_and_zero_head():
    rng = np.random.default_rng(35)
    say("quantise exact and zero heads")
    codes_in = rng.integers(0, 16, (50, 128)).astype(np.uint8)
    codes_in[:, ::16] = rng.choice([7, 15], (50, 8))
    sc_in = rng.integers(0x08, 0x7F, (50, 8)).astype(np.uint8)
    sc_in[3, 2] = 0x7E
    w = f32_bits_to_bf16_bits_exact(oracle.e2m1_to_f64(codes_in)
                                    * np.repeat(oracle.e4m3_to_f64(sc_in), 16, axis=1) * 2.0 ** -10)
    codes, scales, g = L.quantize_nvfp4(bf16_dev(w))
    assert _np(g)[0] == 2.0 ** -10 and np.array_equal(_np(scales), sc_in)
    got = oracle.e2m1_to_f64(oracle.unpack_e2m1(_np(codes), 128))
    assert np.array_equal(got, oracle.e2m1_to_f64(codes_in))
    _check(w, codes, scales, g, what="exact head")
    z = L.quantize_nvfp4(bf16_dev(np.zeros((20, 64), np.uint16)))
    assert _np(z[2])[0] == 1.0 and not _np(z[0]).any() and not _np(z[1]).any()


def test_full_nvfp4_head_and_projection():
    # The NVFP4 workload's head shape (V = 151936, H = 2048) drawn as a bf16
    # weight, quantised on the GPU; sampled rows checked against the oracle
    # (with the whole tensor's maximum), then the quantised head run through
    # the NVFP4 projection and checked like any NVFP4 head.
    w = wl.NVFP4
    say("quantise V=151936 H=2048")
    W = wl.bf16_head(w)
    Wd = bf16_dev(W)
    codes, scales, g = L.quantize_nvfp4(Wd)
    again = L.quantize_nvfp4(Wd)
    assert all(torch.equal(a, b) for a, b in zip((codes, scales, g), again))
    amax = np.float32(np.abs(oracle.bf16_to_f64(W)).max())
    rows = np.unique(np.concatenate([[0, 1, w.V - 1], np.random.default_rng(1).choice(w.V, 400)]))
    rc, rs, rg = oracle.quantize_nvfp4(W[rows], amax)
    assert _np(g)[0] == rg
    assert np.array_equal(_np(scales)[rows], rs) and np.array_equal(_np(codes)[rows], rc)
    h = wl.hidden(w, 16)
    gs = float(_np(g)[0])
    out = host_bits(L.logits_nvfp4(bf16_dev(h), codes, scales, gs))
    cols = rows
    ref, A = oracle.lmhead_logits_nvfp4(h, _np(codes)[cols], _np(scales)[cols], gs)
    check_bf16(out[:, cols], ref, A, gs, oracle.ulp_bf16, what="quantised head")


def test_concurrent_quantisation_on_streams():
    import threading
    rng = np.random.default_rng(36)
    say("quantise threads and streams")
    heads = [bf16_dev(oracle.f32_to_bf16_rne((rng.normal(0, 0.02 * (i + 1), (700 + 97 * i, 128)))
                                             .astype(np.float32))) for i in range(4)]
    serial = [[_np(t) for t in L.quantize_nvfp4(h)] for h in heads]
    torch.cuda.synchronize()
    outs, errors = [None] * 4, []

    def work(i):
        try:
            s = torch.cuda.Stream(device=DEV)
            with torch.cuda.stream(s):
                for _ in range(3):
                    r = L.quantize_nvfp4(heads[i], stream=s)
            s.synchronize()
            outs[i] = [_np(t) for t in r]
        except Exception as e:  # reported below, on the test's thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for a, b in zip(serial, outs):
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


@pytest.mark.parametrize("scale", [1e-37, 1e-30, 3e36, 1e37])
def test_extreme_ranges_bitwise(scale):
    # Heads whose per-tensor scale g or block scales d fall outside the range
    # of the reciprocal shortcut (subnormal g and d at 1e-37, d past 2^120 at
    # 3e36 and 1e37):
    # those blocks take the division itself; codes must still match.
    rng = np.random.default_rng(int(np.log10(scale) + 100))
    say(f"quantise at scale {scale:g}")
    wf = rng.normal(0, 1, (64, 96)) * scale
    w = oracle.f32_to_bf16_rne(wf.astype(np.float32))
    assert np.all(np.isfinite(oracle.bf16_to_f64(w)))
    codes, scales, g = L.quantize_nvfp4(bf16_dev(w))
    _check(w, codes, scales, g, what=f"scale {scale:g}")
