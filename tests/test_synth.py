"""The seeded input generator: published test vector, determinism, random
access, and the distributions the workloads ask for."""
import numpy as np
import torch

import synth
import synth.workloads as wl


def test_splitmix64_published_vector():
    # SplitMix64 started at state 1234567 (the reference sequence published
    # with the generator by S. Vigna).
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    assert [synth.splitmix64_at(1234567, i) for i in range(5)] == want


def test_thread_count_independent_and_random_access():
    a = synth.normal_bf16(7, 2, (300000,), std=0.02, threads=1)
    b = synth.normal_bf16(7, 2, (300000,), std=0.02, threads=8)
    assert np.array_equal(a, b)
    c = synth.normal_bf16(7, 2, (1000,), std=0.02, start=123456, threads=1)
    assert np.array_equal(a[123456:124456], c)
    d = synth.uniform_bytes(7, 4, (200000,), threads=5)
    e = synth.uniform_bytes(7, 4, (100,), start=99000, threads=1)
    assert np.array_equal(d[99000:99100], e)


def test_streams_and_seeds_differ():
    a = synth.normal_bf16(1, 1, (1000,))
    assert not np.array_equal(a, synth.normal_bf16(1, 2, (1000,)))
    assert not np.array_equal(a, synth.normal_bf16(2, 1, (1000,)))


def _bf16(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_normal_moments():
    x = _bf16(synth.normal_bf16(3, 1, (2_000_000,), std=0.02))
    assert abs(x.mean()) < 1e-4
    assert abs(x.std() - 0.02) < 2e-4
    # Gaussian tails: P(|z| > 3) = 0.0027
    assert 0.0022 < np.mean(np.abs(x) > 0.06) < 0.0032


def test_uniform_codes_and_scales():
    b = synth.uniform_bytes(5, 4, (400000,))
    nib = np.concatenate([b & 15, b >> 4])
    counts = np.bincount(nib, minlength=16) / nib.size
    assert np.all(np.abs(counts - 1 / 16) < 0.003)
    s = synth.uniform_e4m3(5, 5, (400000,), 0.25, 4.0)
    v = torch.from_numpy(s).view(torch.float8_e4m3fn).double().numpy()
    assert v.min() == 0.25 and v.max() == 4.0
    assert abs(v.mean() - 2.125) < 0.01
    # every byte is a normal, positive, finite E4M3 code
    assert np.all((s >> 3) & 15 > 0) and np.all(s < 0x7F)


def test_e4m3_generator_rounds_to_nearest():
    # the drawn E4M3 value is the nearest one to the fp32 uniform it came from
    s = synth.uniform_e4m3(9, 5, (50000,), 0.25, 4.0, threads=1)
    v = torch.from_numpy(s).view(torch.float8_e4m3fn).double().numpy()
    grid = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    grid = np.unique(grid[np.isfinite(grid) & (grid >= 0)])
    # regenerate the fp32 uniforms: same counter sequence, u in [0, 1)
    k = synth.key(9, 5)
    u = np.array([(synth.splitmix64_at(k, i) >> 11) * 2.0 ** -53 for i in range(2000)])
    x = np.float32(0.25 + 3.75 * u).astype(np.float64)
    near = grid[np.argmin(np.abs(grid[None, :] - x[:, None]), axis=1)]
    assert np.array_equal(v[:2000], near)


def test_integer_draws_are_integers_in_range():
    x = _bf16(synth.int_bf16(1, 1, (100000,), -4, 4))
    assert np.all(x == np.round(x)) and x.min() == -4 and x.max() == 4


def test_workload_prefix_property():
    w = wl.TINY
    h4 = wl.hidden(w, 4)
    h2 = wl.hidden(w, 2)
    assert np.array_equal(h4[:2], h2)
    assert np.array_equal(wl.hidden_rows(w, [3, 1]), h4[[3, 1]])
    full = wl.weight(w)
    assert np.array_equal(wl.weight_rows(w, 100, 7), full[100:107])


def test_nvfp4_byte_model():
    # NVFP4 reads 4 bits per weight plus one 8-bit scale per 16 weights:
    # 16 / 4.5 = 3.56x fewer bytes than bf16 (the "3.5x fewer bytes" the
    # metrale new_bf16_moe.rs page states for its NVFP4 experts).
    H, V = 2048, 151936
    bf16_bytes = V * H * 2
    nvfp4_bytes = V * H // 2 + V * H // 16
    assert abs(bf16_bytes / nvfp4_bytes - 3.5) < 0.1


def test_f16_generators():
    x = synth.normal_f16(3, 1, (1_000_000,), std=0.02).view(np.float16).astype(np.float64)
    assert abs(x.mean()) < 1e-4 and abs(x.std() - 0.02) < 2e-4
    # the fp16 draw is the fp32 draw rounded to nearest even
    f = synth.normal_f32(3, 1, (1000,), std=0.02)
    assert np.array_equal(synth.normal_f16(3, 1, (1000,), std=0.02), f.astype(np.float16).view(np.uint16))
    i = synth.int_f16(4, 1, (200000,), -1000, 1000).view(np.float16).astype(np.float64)
    assert i.min() == -1000 and i.max() == 1000 and np.all(i == np.round(i))
    assert np.array_equal(synth.int_f16(4, 1, (100,), -1000, 1000, start=500, threads=1),
                          synth.int_f16(4, 1, (600,), -1000, 1000, threads=3)[500:])
