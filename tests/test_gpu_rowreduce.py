"""GPU parity of the row-reduction epilogue (lmhead_logits_rowreduce): per
row the largest logit, its lowest column and sum exp(x - max), computed in the
GEMM's epilogue. Checked exactly against the GPU's own fp32 logits (max,
argmax) and within a derived bound (sumexp), against the oracle through the
fp32 parity bound, bit for bit across kernels, row counts and row orders, and
on ties placed in different blocks, waves and tiles."""
import numpy as np
import pytest
import torch

import lm_head_logits_amd as L
import oracle
import synth.workloads as wl
from gpu_util import DEV, bf16_dev, f16_dev, f32_dev, host_bits, host_f32, say
from helpers import (check_rowreduce_oracle, check_rowreduce_self, f32_bits_to_bf16_bits_exact,
                     load_golden, num)

pytestmark = pytest.mark.gpu

PATHS = ("skinny", "tiled")


def _rand_bf16(rng, shape, std):
    return oracle.f32_to_bf16_rne(rng.normal(0, std, shape).astype(np.float32))


def _np(t):
    return t.detach().cpu().numpy()


def _rows(g, key):
    return np.array([[num(x) for x in row] for row in g[key]], dtype=np.float64)


@pytest.mark.parametrize("path", PATHS)
def test_hand_example(path):
    g = load_golden("rowreduce_hand.txt")
    say(f"rowreduce hand example via {path}")
    h = np.zeros((2, 32), np.uint16)
    w = np.zeros((6, 32), np.uint16)
    h[:, :2] = f32_bits_to_bf16_bits_exact(_rows(g, "hidden"))
    w[:, :2] = f32_bits_to_bf16_bits_exact(_rows(g, "weight"))
    for a in g["alpha"][0]:
        mx, am, se, _ = L.logits_rowreduce(bf16_dev(h), bf16_dev(w), num(a), path=path)
        want_m = np.array([num(v) for v in g[f"max_alpha{a}"][0]], dtype=np.float32)
        assert np.array_equal(_np(mx).view(np.uint32), want_m.view(np.uint32)), a
        assert list(_np(am)) == [int(v) for v in g[f"argmax_alpha{a}"][0]], a
        want_s = np.array([num(v) for v in g[f"sumexp_alpha{a}"][0]])
        assert np.allclose(_np(se), want_s, rtol=4e-7, atol=0), a


# (M, H, V, alpha, bias, fp16)
CASES = [(1, 32, 1, 1.0, False, False), (3, 64, 17, 0.5, True, False),
         (5, 96, 1000, -0.25, False, False), (16, 128, 4111, 0.125, True, False),
         (64, 256, 70001, 1.0, True, False), (65, 96, 515, 0.125, False, False),
         (130, 224, 4097, 0.7, True, False), (40, 160, 3001, 0.125, True, True)]


@pytest.mark.parametrize("M,H,V,alpha,has_bias,f16", CASES)
def test_parity_and_paths_agree(M, H, V, alpha, has_bias, f16):
    rng = np.random.default_rng(M * 31 + V)
    say(f"rowreduce M={M} H={H} V={V} alpha={alpha} bias={has_bias} fp16={f16}")
    if f16:
        h = rng.normal(0, 1, (M, H)).astype(np.float32).astype(np.float16).view(np.uint16)
        W = rng.normal(0, 0.02, (V, H)).astype(np.float32).astype(np.float16).view(np.uint16)
        hd, Wd, ind = f16_dev(h), f16_dev(W), "f16"
    else:
        h, W = _rand_bf16(rng, (M, H), 1.0), _rand_bf16(rng, (V, H), 0.02)
        hd, Wd, ind = bf16_dev(h), bf16_dev(W), "bf16"
    bias = rng.normal(0, 0.1, V).astype(np.float32) if has_bias else None
    bd = f32_dev(bias) if has_bias else None
    plain = host_f32(L.logits(hd, Wd, alpha, bd, torch.float32))
    res = {}
    for p in PATHS:
        mx, am, se, lg = L.logits_rowreduce(hd, Wd, alpha, bd, write_logits=True, path=p)
        res[p] = (_np(mx), _np(am), _np(se))
        # the logits written alongside are the plain call's, bit for bit
        assert np.array_equal(host_bits(lg), plain.view(np.uint32)), p
    for k in range(3):
        assert np.array_equal(res["skinny"][k].view(np.uint32), res["tiled"][k].view(np.uint32)), \
            "skinny and tiled row reductions must agree bit for bit"
    ratio = check_rowreduce_self(*res["tiled"], plain)
    ref_m, _, _, ref_x, A = oracle.lmhead_rowreduce(h, W, alpha, bias, ind)
    check_rowreduce_oracle(*res["tiled"], ref_m, ref_x, A, V)
    # 16-bit logits written alongside: the plain call's 16-bit logits, and the
    # reduction still over the fp32 epilogue values
    o16 = torch.float16 if f16 else torch.bfloat16
    mx, am, se, lg = L.logits_rowreduce(hd, Wd, alpha, bd, o16, write_logits=True)
    assert np.array_equal(host_bits(lg), host_bits(L.logits(hd, Wd, alpha, bd, o16)))
    assert np.array_equal(_np(mx).view(np.uint32), res["tiled"][0].view(np.uint32))
    assert np.array_equal(_np(se).view(np.uint32), res["tiled"][2].view(np.uint32))
    # without the logits: the same three results
    mx, am, se, lg = L.logits_rowreduce(hd, Wd, alpha, bd)
    assert lg is None
    assert np.array_equal(_np(mx), res["tiled"][0]) and np.array_equal(_np(am), res["tiled"][1])
    assert np.array_equal(_np(se), res["tiled"][2])
    say(f"  sumexp max err/bound {ratio:.3g}")


def test_ties_across_blocks_waves_and_tiles():
    # Integer inputs make the logits exact; copies of one weight row at
    # columns in different 16-column blocks, different waves of the
    # weight-streaming kernel and different tiles give exact ties.
    M, H, V = 70, 256, 70001
    say("rowreduce ties")
    h = wl.int_hidden(5, M, H)
    W = wl.int_weight(5, V, H, -2, 2)
    hv = oracle.bf16_to_f64(h)
    # a weight row that beats every other for every hidden row: 4 * sign(h)
    # is not available (rows differ), so give each tied column a large
    # multiple of hidden row 0's sign pattern and compare on row 0's logits.
    top = (np.sign(hv[0]) * 4).astype(np.float32)
    cols = [40000, 9, 69999, 4097, 33]
    for c in cols:
        W[c] = f32_bits_to_bf16_bits_exact(top)
    for p in PATHS:
        mx, am, se, _ = L.logits_rowreduce(bf16_dev(h), bf16_dev(W), 0.5, path=p)
        assert int(_np(am)[0]) == min(cols), p
    plain = host_f32(L.logits(bf16_dev(h), bf16_dev(W), 0.5))
    check_rowreduce_self(_np(mx), _np(am), _np(se), plain)


@pytest.mark.parametrize("path", PATHS)
def test_ties_inside_one_block(path):
    # Ties among columns of one 16-column block: within one lane's four
    # columns (4t .. 4t + 3) and across the four lanes that share a row of the
    # block, and a whole block of equal logits; integer inputs keep every
    # logit exact, so the lowest tied column must win in every row.
    M, H, V = 20, 64, 4133
    say(f"rowreduce ties inside one block via {path}")
    h = wl.int_hidden(9, M, H)
    W = wl.int_weight(9, V, H, -1, 1)
    hv = oracle.bf16_to_f64(h)
    top = f32_bits_to_bf16_bits_exact((np.sign(hv[0]) * 4).astype(np.float32))
    for c in (1030, 1031, 1033, 1037, 1045):       # block 64: lanes 1, 2, 3; one lane's pair
        W[c] = top
    W[3200:3216] = f32_bits_to_bf16_bits_exact((np.sign(hv[1]) * 4).astype(np.float32))
    mx, am, se, _ = L.logits_rowreduce(bf16_dev(h), bf16_dev(W), 0.25, path=path)
    am = _np(am)
    assert int(am[0]) == 1030 and int(am[1]) == 3200, (int(am[0]), int(am[1]))
    plain = host_f32(L.logits(bf16_dev(h), bf16_dev(W), 0.25, path=path))
    check_rowreduce_self(_np(mx), am, _np(se), plain)


def test_rows_invariant_across_counts_and_order():
    rng = np.random.default_rng(11)
    M, H, V = 130, 128, 20000
    say("rowreduce row invariance")
    hd = bf16_dev(_rand_bf16(rng, (M, H), 1.0))
    Wd = bf16_dev(_rand_bf16(rng, (V, H), 0.02))
    bd = f32_dev(rng.normal(0, 0.1, V))
    full = [_np(t) for t in L.logits_rowreduce(hd, Wd, 0.125, bd)[:3]]
    for m in (1, 2, 17, 63, 64, 65, 100, 129):
        part = [_np(t) for t in L.logits_rowreduce(hd[:m].contiguous(), Wd, 0.125, bd)[:3]]
        for a, b in zip(part, full):
            assert np.array_equal(a.view(np.uint32), b[:m].view(np.uint32)), m
    rev = [_np(t) for t in L.logits_rowreduce(torch.flip(hd, [0]).contiguous(), Wd, 0.125, bd)[:3]]
    for a, b in zip(rev, full):
        assert np.array_equal(a[::-1].view(np.uint32), b.view(np.uint32))


def test_workspace_and_empty():
    say("rowreduce workspace")
    hd = bf16_dev(np.zeros((4, 64), np.uint16))
    Wd = bf16_dev(np.zeros((100, 64), np.uint16))
    small = torch.empty(L.rowreduce_workspace_bytes(4, 100) - 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(L.LmHeadError):
        L.logits_rowreduce(hd, Wd, workspace=small)
    mx, am, se, _ = L.logits_rowreduce(hd[:0], Wd)
    assert mx.shape == (0,)
    # all-zero logits: max 0 at column 0, sumexp = V
    mx, am, se, _ = L.logits_rowreduce(hd, Wd)
    assert np.all(_np(mx) == 0) and np.all(_np(am) == 0) and np.all(_np(se) == 100.0)


def test_decode_shape_parity():
    # The decode head at its full size, M = 64: every row reduced on the GPU;
    # four rows recomputed by the oracle over the whole vocabulary.
    w = wl.DECODE
    say("rowreduce decode M=64 H=4096 V=128256")
    h, W = wl.hidden(w, 64), wl.weight(w)
    hd, Wd = bf16_dev(h), bf16_dev(W)
    alpha = w.alphas[1]
    mx, am, se, lg = L.logits_rowreduce(hd, Wd, alpha, write_logits=True)
    plain = host_f32(lg)
    ratio = check_rowreduce_self(_np(mx), _np(am), _np(se), plain)
    rows = np.array([0, 21, 42, 63])
    ref_m, _, _, ref_x, A = oracle.lmhead_rowreduce(h[rows], W, alpha)
    check_rowreduce_oracle(_np(mx)[rows], _np(am)[rows], _np(se)[rows], ref_m, ref_x, A, w.V)
    say(f"  sumexp max err/bound {ratio:.3g}")


def test_concurrent_calls_with_own_workspaces():
    # Calls from several host threads, each on its own stream with its own
    # workspace, give the bits of the same calls made one by one.
    import threading
    rng = np.random.default_rng(12)
    say("rowreduce threads and streams")
    hd = bf16_dev(_rand_bf16(rng, (96, 256), 1.0))
    Wd = bf16_dev(_rand_bf16(rng, (9000, 256), 0.02))
    Ms = [1, 7, 64, 96, 33, 65]
    serial = [[_np(t) for t in L.logits_rowreduce(hd[:m].contiguous(), Wd, 0.25)[:3]] for m in Ms]
    torch.cuda.synchronize()
    outs, errors = [None] * len(Ms), []

    def work(i):
        try:
            s = torch.cuda.Stream(device=DEV)
            with torch.cuda.stream(s):
                ws = torch.empty(L.rowreduce_workspace_bytes(Ms[i], 9000), dtype=torch.uint8, device=DEV)
                h = hd[:Ms[i]].contiguous()
                for _ in range(3):
                    r = L.logits_rowreduce(h, Wd, 0.25, workspace=ws, stream=s)
            s.synchronize()
            outs[i] = [_np(t) for t in r[:3]]
        except Exception as e:  # reported below, on the test's thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(Ms))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for a, b in zip(serial, outs):
        for x, y in zip(a, b):
            assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


def test_vocabulary_shards_fold_to_the_full_row():
    # The multi-GPU reading on one GPU: each of g vocabulary shards reduced by
    # its own call, the g triples folded in shard order with the combine
    # rule (larger maximum, ties to the lower global column, sums rescaled to
    # the new maximum). Maximum and argmax equal the one-call result exactly;
    # the sum of exponentials within the bound of its own fold order.
    rng = np.random.default_rng(14)
    M, H, V, g = 48, 256, 50000, 8
    say(f"rowreduce vocabulary shards g={g}")
    hd = bf16_dev(_rand_bf16(rng, (M, H), 1.0))
    Wd = bf16_dev(_rand_bf16(rng, (V, H), 0.02))
    mx, am, se, lg = L.logits_rowreduce(hd, Wd, 0.5, write_logits=True)
    bounds = np.linspace(0, V, g + 1).astype(int)
    m = np.full(M, -np.inf)
    s = np.zeros(M)
    idx = np.full(M, -1)
    for r in range(g):
        v0, v1 = bounds[r], bounds[r + 1]
        pm, pa, ps, _ = L.logits_rowreduce(hd, Wd[v0:v1].contiguous(), 0.5)
        pm, pa, ps = _np(pm).astype(np.float64), _np(pa) + v0, _np(ps).astype(np.float64)
        take = pm > m                                  # shards come in column order: ties keep the earlier
        new_m = np.where(take, pm, m)
        s = np.where(s == 0, 0, s * np.exp(m - new_m)) + ps * np.exp(pm - new_m)
        idx = np.where(take, pa, idx)
        m = new_m
    assert np.array_equal(m.astype(np.float32), _np(mx)) and np.array_equal(idx, _np(am))
    x = host_f32(lg)
    from helpers import sumexp_bound
    ref = np.exp(x.astype(np.float64) - x.max(axis=1, keepdims=True)).sum(axis=1)
    assert np.all(np.abs(s - ref) <= 2 * sumexp_bound(x, x.max(axis=1), V))


@pytest.mark.parametrize("path", PATHS)
def test_masked_blocks_minus_inf_bias(path):
    # A -inf bias masks vocabulary entries: whole 16-column blocks, part of a
    # block and the ragged last block. Masked entries contribute exp(-inf) = 0;
    # the result must match the reduction of the plain call's logits and the
    # oracle's, and be the same on both kernels.
    rng = np.random.default_rng(77)
    M, H, V = 37, 96, 4133
    say(f"rowreduce -inf bias via {path}")
    h, W = _rand_bf16(rng, (M, H), 1.0), _rand_bf16(rng, (V, H), 0.02)
    bias = rng.normal(0, 0.1, V).astype(np.float32)
    for lo, hi in ((16, 48), (1024, 1040), (100, 106), (4128, 4133), (2000, 2400)):
        bias[lo:hi] = -np.inf
    hd, Wd, bd = bf16_dev(h), bf16_dev(W), f32_dev(bias)
    mx, am, se, lg = L.logits_rowreduce(hd, Wd, 0.25, bd, write_logits=True, path=path)
    plain = host_f32(L.logits(hd, Wd, 0.25, bd, torch.float32))
    assert np.array_equal(host_bits(lg), plain.view(np.uint32))
    assert np.isneginf(plain[:, 20]).all()
    check_rowreduce_self(_np(mx), _np(am), _np(se), plain)
    ref_m, _, _, ref_x, A = oracle.lmhead_rowreduce(h, W, 0.25, bias)
    A = np.where(np.isfinite(ref_x), A, 0.0)
    check_rowreduce_oracle(_np(mx), _np(am), _np(se), ref_m, ref_x, A, V)
    other = "tiled" if path == "skinny" else "skinny"
    mx2, am2, se2, _ = L.logits_rowreduce(hd, Wd, 0.25, bd, path=other)
    for a, b in ((mx, mx2), (am, am2), (se, se2)):
        assert np.array_equal(_np(a).view(np.uint32), _np(b).view(np.uint32))


@pytest.mark.parametrize("path", PATHS)
def test_fully_masked_rows(path):
    # Every logit -inf: the row maximum is -inf, its lowest column 0, and the
    # sum 0 (the contract for rows with no finite logit).
    rng = np.random.default_rng(78)
    M, H, V = 5, 64, 300
    say(f"rowreduce all -inf via {path}")
    hd = bf16_dev(_rand_bf16(rng, (M, H), 1.0))
    Wd = bf16_dev(_rand_bf16(rng, (V, H), 0.02))
    bd = f32_dev(np.full(V, -np.inf, np.float32))
    mx, am, se, _ = L.logits_rowreduce(hd, Wd, 1.0, bd, path=path)
    assert np.isneginf(_np(mx)).all()
    assert np.all(_np(am) == 0) and np.all(_np(se) == 0.0)
