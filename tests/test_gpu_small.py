"""GPU parity on small shapes: hand examples, the tiny workload, ragged and
degenerate shapes, the epilogue identities and the kernel-to-kernel bit
identity. Every call goes through the C ABI (via the ctypes binding)."""
import numpy as np
import pytest
import torch

import lm_head_logits_amd as L
import oracle
import synth.workloads as wl
from gpu_util import DEV, bf16_dev, f32_dev, host_bits, host_f32, say, u8_dev
from helpers import check_bf16, check_f32, f32_bits_to_bf16_bits_exact, load_golden, num

pytestmark = pytest.mark.gpu

PATHS = ("skinny", "tiled")


def _rand_bf16(rng, shape, std):
    return oracle.f32_to_bf16_rne(rng.normal(0, std, shape).astype(np.float32))


def _rows(g, key):
    return np.array([[num(x) for x in row] for row in g[key]], dtype=np.float64)


@pytest.mark.parametrize("path", PATHS)
def test_hand_example_bitwise(path):
    g = load_golden("hand_2x3x4.txt")
    say(f"hand 2x3x4 via {path}")
    alpha = num(g["alpha"][0][0])
    h = np.zeros((2, 32), dtype=np.uint16)
    w = np.zeros((3, 32), dtype=np.uint16)
    h[:, :4] = f32_bits_to_bf16_bits_exact(_rows(g, "hidden"))     # H = 4 zero-padded to one K-step
    w[:, :4] = f32_bits_to_bf16_bits_exact(_rows(g, "weight"))
    b = f32_dev(_rows(g, "bias")[0])
    for bias, key in ((None, "nobias"), (b, "withbias")):
        want = _rows(g, key).astype(np.float32)
        o32 = L.logits(bf16_dev(h), bf16_dev(w), alpha, bias, torch.float32, path=path)
        assert np.array_equal(host_bits(o32), want.view(np.uint32)), key
        o16 = L.logits(bf16_dev(h), bf16_dev(w), alpha, bias, torch.bfloat16, path=path)
        assert np.array_equal(host_bits(o16), f32_bits_to_bf16_bits_exact(want)), key


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("out", ("f32", "bf16"))
def test_tiny_workload_parity(path, out):
    w = wl.TINY
    say(f"tiny M=4 H=256 V=4096 via {path}, {out} out")
    h, W = wl.hidden(w), wl.weight(w)
    alpha = w.alphas[0]
    ref, A = oracle.lmhead_logits(h, W, alpha, None, out)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    got = L.logits(bf16_dev(h), bf16_dev(W), alpha, None, dt, path=path)
    if out == "f32":
        check_f32(host_f32(got), ref, A, what="tiny")
    else:
        check_bf16(host_bits(got), ref, A, alpha, oracle.ulp_bf16, what="tiny bf16")


# (M, H, V): ragged V, one K-step, an odd number of K-steps, the 64-row
# boundary, ragged M past it, V = 1.
# (100, 64, 65601): wide enough that the tiled kernel takes 160-column tiles,
# the last of them one column wide.
SHAPES = [(1, 32, 1), (3, 32, 17), (5, 96, 1000), (16, 64, 4111), (63, 160, 333), (64, 128, 257),
          (65, 96, 129), (130, 224, 515), (200, 32, 2000), (7, 1024, 4097), (100, 64, 65601)]


@pytest.mark.parametrize("M,H,V", SHAPES)
def test_ragged_shapes_parity_and_paths_agree(M, H, V):
    rng = np.random.default_rng(M * 1000 + H + V)
    say(f"ragged M={M} H={H} V={V}")
    h = _rand_bf16(rng, (M, H), 1.0)
    W = _rand_bf16(rng, (V, H), 0.02)
    bias = rng.normal(0, 0.1, V).astype(np.float32)
    alpha = 0.125
    ref, A = oracle.lmhead_logits(h, W, alpha, bias, "f32")
    hd, Wd, bd = bf16_dev(h), bf16_dev(W), f32_dev(bias)
    outs = {p: L.logits(hd, Wd, alpha, bd, torch.float32, path=p) for p in PATHS}
    check_f32(host_f32(outs["skinny"]), ref, A, what="skinny")
    assert np.array_equal(host_bits(outs["skinny"]), host_bits(outs["tiled"])), \
        "skinny and tiled kernels must agree bit for bit"
    auto = L.logits(hd, Wd, alpha, bd, torch.float32)
    assert np.array_equal(host_bits(auto), host_bits(outs["skinny"]))


# V = 70001: more column blocks than waves on a 256-CU part, so the
# weight-streaming kernel runs its direct-to-LDS path with two blocks per wave;
# H covers even and odd numbers of 64-element chunks and a final half chunk.
@pytest.mark.parametrize("H", [32, 64, 96, 160, 192, 320])
@pytest.mark.parametrize("M", [1, 20, 64])
def test_weight_stream_paths_match_tiled(M, H):
    rng = np.random.default_rng(M * 7 + H)
    V = 70001
    say(f"stream vs tiled M={M} H={H} V={V}")
    hd = bf16_dev(_rand_bf16(rng, (M, H), 1.0))
    Wd = bf16_dev(_rand_bf16(rng, (V, H), 0.02))
    a = L.logits(hd, Wd, 0.5, None, torch.float32, path="skinny")
    b = L.logits(hd, Wd, 0.5, None, torch.float32, path="tiled")
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_integer_inputs_are_exact_small():
    # |partial sums| <= 16 * H < 2^24: every summation order is exact, so the
    # GPU must equal the oracle bit for bit.
    M, H, V = 37, 1024, 3001
    say("integer exact small")
    h = wl.int_hidden(21, M, H)
    W = wl.int_weight(21, V, H)
    for alpha in (1.0, 0.0625):
        ref, _ = oracle.lmhead_logits(h, W, alpha, None, "f32")
        for p in PATHS:
            got = L.logits(bf16_dev(h), bf16_dev(W), alpha, None, torch.float32, path=p)
            assert np.array_equal(host_bits(got), ref.view(np.uint32)), (p, alpha)


@pytest.mark.parametrize("path", PATHS)
def test_alpha_fold_equals_unfused_multiply(path):
    rng = np.random.default_rng(5)
    M, H, V = 48, 512, 3000
    say(f"alpha fold via {path}")
    hd = bf16_dev(_rand_bf16(rng, (M, H), 1.0))
    Wd = bf16_dev(_rand_bf16(rng, (V, H), 0.02))
    base = L.logits(hd, Wd, 1.0, None, torch.float32, path=path)
    for a in (1 / 16, 1 / 8, 1 / 4, 1 / 3, 0.7):
        fused = L.logits(hd, Wd, a, None, torch.float32, path=path)
        unfused = base * torch.tensor(a, dtype=torch.float32, device=DEV)
        assert torch.equal(fused.view(torch.int32), unfused.view(torch.int32)), a
    # bias: a separately rounded add after the scaled projection
    b = f32_dev(rng.normal(0, 0.1, V))
    with_b = L.logits(hd, Wd, 0.7, b, torch.float32, path=path)
    scaled = L.logits(hd, Wd, 0.7, None, torch.float32, path=path)
    assert torch.equal(with_b.view(torch.int32), (scaled + b).view(torch.int32))
    # the bf16 output is the fp32 output rounded to nearest even
    o16 = L.logits(hd, Wd, 0.7, b, torch.bfloat16, path=path)
    assert np.array_equal(host_bits(o16), oracle.f32_to_bf16_rne(host_f32(with_b)))


@pytest.mark.parametrize("path", PATHS)
def test_zero_hidden_gives_bias_and_one_hot_gathers(path):
    rng = np.random.default_rng(8)
    M, H, V = 20, 256, 777
    say(f"zero hidden / one-hot via {path}")
    b = rng.normal(0, 0.1, V).astype(np.float32)
    W = _rand_bf16(rng, (V, H), 0.02)
    z = L.logits(bf16_dev(np.zeros((M, H), np.uint16)), bf16_dev(W), 0.125, f32_dev(b),
                 torch.float32, path=path)
    assert np.array_equal(host_bits(z), np.broadcast_to(b.view(np.uint32), (M, V)))
    h = _rand_bf16(rng, (M, H), 1.0)
    ks = rng.integers(0, H, V)
    onehot = np.zeros((V, H), np.uint16)
    onehot[np.arange(V), ks] = 0x3F80
    got = L.logits(bf16_dev(h), bf16_dev(onehot), 0.7, None, torch.float32, path=path)
    want = (oracle.bf16_to_f64(h).astype(np.float32)[:, ks] * np.float32(0.7)).astype(np.float32)
    assert np.array_equal(host_bits(got), want.view(np.uint32))


def test_m_zero_and_not_handled_launch_nothing():
    say("M=0 and H%32!=0")
    Wd = bf16_dev(np.zeros((10, 64), np.uint16))
    out = L.logits(bf16_dev(np.zeros((0, 64), np.uint16)), Wd)
    assert out.shape == (0, 10)
    sentinel = torch.full((3, 10), 7.0, device=DEV)
    with pytest.raises(L.NotHandled):
        L.logits(bf16_dev(np.zeros((3, 48), np.uint16)), bf16_dev(np.zeros((10, 48), np.uint16)),
                 out=sentinel)
    torch.cuda.synchronize()
    assert torch.all(sentinel == 7.0)


def test_run_to_run_identical():
    rng = np.random.default_rng(2)
    say("run to run")
    hd = bf16_dev(_rand_bf16(rng, (100, 512), 1.0))
    Wd = bf16_dev(_rand_bf16(rng, (5000, 512), 0.02))
    for p in PATHS:
        a = L.logits(hd, Wd, 0.3, None, path=p)
        b = L.logits(hd, Wd, 0.3, None, path=p)
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_concurrent_calls_on_several_streams_and_threads():
    # The library keeps no per-call state: calls from several host threads,
    # each on its own stream, give the same bits as the calls made one by one.
    import threading
    rng = np.random.default_rng(3)
    say("threads and streams")
    hd = bf16_dev(_rand_bf16(rng, (64, 256), 1.0))
    Wd = bf16_dev(_rand_bf16(rng, (7000, 256), 0.02))
    Ms = [1, 5, 17, 64, 40, 3, 64, 33]
    serial = [L.logits(hd[:m], Wd, 0.25, None, path=("skinny" if i % 2 else "tiled"))
              for i, m in enumerate(Ms)]
    torch.cuda.synchronize()
    outs = [None] * len(Ms)
    errors = []

    def work(i):
        try:
            s = torch.cuda.Stream(device=DEV)
            with torch.cuda.stream(s):
                o = torch.empty((Ms[i], 7000), device=DEV, dtype=torch.float32)
                for _ in range(3):
                    L.logits(hd[:Ms[i]], Wd, 0.25, None, out=o,
                             path=("skinny" if i % 2 else "tiled"), stream=s)
            s.synchronize()
            outs[i] = o
        except Exception as e:  # reported below, on the test's thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(Ms))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for a, b in zip(serial, outs):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


# ----------------------------------------------------------------------------
# NVFP4
# ----------------------------------------------------------------------------

def test_nvfp4_hand_example():
    g = load_golden("nvfp4_hand.txt")
    say("nvfp4 hand example")
    h = f32_bits_to_bf16_bits_exact(_rows(g, "hidden"))
    codes = np.array([[int(x, 16) for x in row] for row in g["codes"]], dtype=np.uint8)
    scales = np.array([[int(x, 16) for x in row] for row in g["scales"]], dtype=np.uint8)
    out = L.logits_nvfp4(bf16_dev(h), u8_dev(codes), u8_dev(scales), num(g["g"][0][0]),
                         num(g["alpha"][0][0]))
    want = np.array([[int(x, 16) for x in g["logits_bf16"][0]]], dtype=np.uint16)
    assert np.array_equal(host_bits(out), want)


def test_nvfp4_nibble_order_on_gpu():
    say("nvfp4 nibble order")
    codes = np.zeros((2, 16), np.uint8)
    codes[:, 0] = 0x72                       # element 0 -> 1.0, element 1 -> 6.0
    scales = np.full((2, 2), 0x38, np.uint8)  # 1.0
    for e, want in ((0, 0x3F80), (1, 0x40C0)):
        h = np.zeros((1, 32), np.uint16)
        h[0, e] = 0x3F80
        out = L.logits_nvfp4(bf16_dev(h), u8_dev(codes), u8_dev(scales), 1.0)
        assert host_bits(out)[0, 0] == want


# M <= 64 runs the weight-streaming NVFP4 kernel, M > 64 the tiled kernel with
# the decode in its B stage (128-row tiles: 129 and 300 leave ragged tiles;
# H = 96 and 160 end in a half stage).
# H = 2176 and 4096 (M <= 64) cross the streaming kernel's block-scale segment
# of 2048 elements, which it reloads into LDS inside its K loop.
@pytest.mark.parametrize("M,H,V", [(1, 32, 1), (4, 64, 100), (64, 256, 1000), (65, 96, 333),
                                   (129, 160, 515), (200, 512, 2049), (300, 128, 1000),
                                   (3, 2176, 700), (33, 4096, 1500), (64, 2304, 333)])
def test_nvfp4_parity_and_equals_bf16_path(M, H, V):
    rng = np.random.default_rng(M + H + V)
    say(f"nvfp4 M={M} H={H} V={V}")
    h = _rand_bf16(rng, (M, H), 1.0)
    codes = rng.integers(0, 256, (V, H // 2), dtype=np.uint8)
    scales = rng.choice(np.r_[0x30:0x4A], (V, H // 16)).astype(np.uint8)
    bias = rng.normal(0, 0.1, V).astype(np.float32)
    g, alpha = 0.01, 0.5
    for b in (None, bias):
        ref, A = oracle.lmhead_logits_nvfp4(h, codes, scales, g, alpha, b)
        bd = f32_dev(b) if b is not None else None
        got = L.logits_nvfp4(bf16_dev(h), u8_dev(codes), u8_dev(scales), g, alpha, bd)
        check_bf16(host_bits(got), ref, A, g * alpha, oracle.ulp_bf16, what="nvfp4")
        # the same chain on the dequantised weight through the bf16 entry point
        wdeq = oracle.nvfp4_weight_f64(codes, scales, H).astype(np.float32)
        wbits = f32_bits_to_bf16_bits_exact(wdeq)
        s = float(np.float32(g) * np.float32(alpha))
        for p in PATHS:
            twin = L.logits(bf16_dev(h), bf16_dev(wbits), s, bd, torch.bfloat16, path=p)
            assert np.array_equal(host_bits(got), host_bits(twin)), p


def test_nvfp4_misaligned_scales_take_the_generic_kernel():
    # Scales at an address that is 2 but not 8 bytes aligned take the generic
    # NVFP4 kernel: the same chain, the same bits as an aligned copy.
    rng = np.random.default_rng(23)
    M, H, V = 16, 256, 900
    say("nvfp4 misaligned scales")
    h = bf16_dev(_rand_bf16(rng, (M, H), 1.0))
    codes = u8_dev(rng.integers(0, 256, (V, H // 2), dtype=np.uint8))
    sc = rng.choice(np.r_[0x30:0x4A], (V, H // 16)).astype(np.uint8)
    aligned = u8_dev(sc)
    big = torch.zeros(V * (H // 16) + 16, dtype=torch.uint8, device=DEV)
    shifted = big[2:2 + V * (H // 16)].view(V, H // 16)
    shifted.copy_(aligned)
    assert shifted.data_ptr() % 8 == 2
    a = L.logits_nvfp4(h, codes, aligned, 0.01)
    b = L.logits_nvfp4(h, codes, shifted, 0.01)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# Hidden rows of extreme magnitude through the M <= 32 NVFP4 kernel: typical
# rows, rows scaled by 2^-60, 2^10 and 2^-100, zeros and signed zeros, one
# value of 1e-30 beside O(1) values, one of 40000, one bf16 subnormal. The
# bits must be those of the bf16 chain on the dequantised head (both bf16
# paths) and within the oracle's bound.
_EXTREME_CASES = ("normal", "x2^-60", "x2^10", "zeros", "signed_zero", "tiny", "big", "subnormal",
               "x2^-100")


@pytest.mark.parametrize("M", [1, 5, 20, 32])
@pytest.mark.parametrize("case", _EXTREME_CASES)
def test_nvfp4_ring_extreme_hidden_equals_bf16_chain(M, case):
    H, V = 1024, 700
    rng = np.random.default_rng(7 * M + len(case))
    say(f"nvfp4 ring extreme hidden {case} M={M}")
    x = rng.normal(0, 1, (M, H))
    if case == "x2^-60":
        x = x * 2.0 ** -60
    elif case == "x2^10":
        x = x * 2.0 ** 10
    elif case == "x2^-100":
        x = x * 2.0 ** -100
    elif case == "zeros":
        x[:] = 0.0
        x[M // 2, 3] = 1.5
    elif case == "signed_zero":
        x[:, ::3] = -0.0
        x[:, 1::3] = 0.0
    elif case == "tiny":
        x[M - 1, H // 2] = 1e-30
    elif case == "big":
        x[0, 5] = 40000.0
    h = oracle.f32_to_bf16_rne(x.astype(np.float32))
    if case == "subnormal":
        h[M - 1, 7] = 0x0001
    codes = rng.integers(0, 256, (V, H // 2), dtype=np.uint8)
    scales = rng.choice(np.r_[0x30:0x4A], (V, H // 16)).astype(np.uint8)
    g, alpha = 0.01, 0.5
    got = host_bits(L.logits_nvfp4(bf16_dev(h), u8_dev(codes), u8_dev(scales), g, alpha))
    ref, A = oracle.lmhead_logits_nvfp4(h, codes, scales, g, alpha, None)
    check_bf16(got, ref, A, g * alpha, oracle.ulp_bf16, what=f"nvfp4 {case}")
    wbits = f32_bits_to_bf16_bits_exact(oracle.nvfp4_weight_f64(codes, scales, H).astype(np.float32))
    s = float(np.float32(g) * np.float32(alpha))
    for p in PATHS:
        twin = L.logits(bf16_dev(h), bf16_dev(wbits), s, None, torch.bfloat16, path=p)
        assert np.array_equal(got, host_bits(twin)), (case, p)


def test_hip_graph_capture_and_replay():
    # The entry points allocate, free and synchronise nothing, so they can be
    # captured in a HIP graph (the decode loop of a server). Every replay,
    # with eager work and synchronisations between replays, must give the
    # eager results bit for bit.
    rng = np.random.default_rng(17)
    say("graph capture")
    M, H, V = 40, 512, 6000
    hd = bf16_dev(_rand_bf16(rng, (M, H), 1.0))
    Wd = bf16_dev(_rand_bf16(rng, (V, H), 0.02))
    bd = f32_dev(rng.normal(0, 0.1, V))
    h2 = bf16_dev(_rand_bf16(rng, (150, H), 1.0))
    codes = u8_dev(rng.integers(0, 256, (V, H // 2), dtype=np.uint8))
    scales = u8_dev(rng.choice(np.r_[0x28:0x48], (V, H // 16)).astype(np.uint8))
    ws = torch.empty(L.rowreduce_workspace_bytes(M, V), dtype=torch.uint8, device=DEV)
    outs = {
        "skinny": torch.empty((M, V), device=DEV),
        "tiled": torch.empty((150, V), device=DEV),
        "nvfp4": torch.empty((M, V), device=DEV, dtype=torch.bfloat16),
    }

    def run():
        L.logits(hd, Wd, 0.25, bd, out=outs["skinny"])
        L.logits(h2, Wd, 0.25, bd, out=outs["tiled"])
        L.logits_nvfp4(hd, codes, scales, 0.01, out=outs["nvfp4"])
        return L.logits_rowreduce(hd, Wd, 0.25, bd, workspace=ws)[:3]

    eager_red = [t.clone() for t in run()]
    eager = {k: v.clone() for k, v in outs.items()}
    torch.cuda.synchronize()
    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()                                        # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        red = run()
    for rep in range(3):
        for v in outs.values():
            v.zero_()                                # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in outs:
            assert torch.equal(outs[k].view(torch.int16), eager[k].view(torch.int16)), (k, rep)
        for a, b in zip(red, eager_red):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), rep
