"""GPU parity on every output element at the workloads' full sizes, in the
launch configuration the benchmark times: the decode head at each row count
and both alphas, the spec-decode target and draft calls, the NVFP4 head at
each row count, and two complete 256-row tiles of the prefill call (the first
and the last). The oracle's binary64 dot products of a workload are taken once
and shared by its row counts and alphas (a row's dot products do not depend
on the other rows)."""
import numpy as np
import pytest
import torch

import lm_head_logits_amd as L
import oracle
import synth.workloads as wl
from gpu_util import DEV, bf16_dev, f32_dev, host_bits, host_f32, say, u8_dev
from helpers import check_bf16, check_f32

pytestmark = pytest.mark.gpu


def test_decode_full_output():
    w = wl.DECODE
    say("decode full output: generate H=4096 V=128256, oracle dots for 64 rows")
    h, W = wl.hidden(w), wl.weight(w)
    hd, Wd = bf16_dev(h), bf16_dev(W)
    S, A = oracle.dot_f64(h[:w.M], W)
    del W
    for alpha in w.alphas:
        for M in w.Ms:
            got = host_f32(L.logits(hd[:M], Wd, alpha))
            ref = oracle.logits_f32(S[:M], alpha)
            # the bound scaled by |alpha| (a power of two here): stricter
            # than 2e-5 sum|h w|, and the same ratio at either alpha
            ratio, exact = check_f32(got, ref, abs(alpha) * A[:M], what=f"decode M={M} alpha={alpha}")
            say(f"  M={M} alpha={alpha}: {got.size} elements, max err/bound {ratio:.3f}, "
                f"bit-exact {exact:.3f}")


def test_spec_full_output():
    w = wl.SPEC
    say("spec-decode full output: generate H=2048 V=151936, oracle dots for 128 rows")
    h, W, b = wl.hidden(w), wl.weight(w), wl.bias(w)
    hd, Wd, bd = bf16_dev(h), bf16_dev(W), f32_dev(b)
    alpha = w.alphas[0]
    S, A = oracle.dot_f64(h, W)
    del W
    ref = oracle.logits_f32(S, alpha, b)
    target = host_f32(L.logits(hd, Wd, alpha, bd))
    ratio, exact = check_f32(target, ref, A, what="spec target M=128")
    say(f"  target M=128: max err/bound {ratio:.3f}, bit-exact {exact:.3f}")
    # the draft call: one token of each of the 32 sequences (rows 4s + j)
    for j in (0, 3):
        idx = np.arange(32) * 4 + j
        draft = host_f32(L.logits(hd[torch.as_tensor(idx, device=DEV)].contiguous(), Wd, alpha, bd))
        ratio, _ = check_f32(draft, ref[idx], A[idx], what=f"spec draft M=32 j={j}")
        assert np.array_equal(draft.view(np.uint32), target[idx].view(np.uint32))
        say(f"  draft M=32 (token {j}): max err/bound {ratio:.3f}, equal to the target's rows")


def test_nvfp4_full_output():
    w = wl.NVFP4
    say("nvfp4 full output: generate H=2048 V=151936, oracle for 256 rows")
    h, c, s = wl.hidden(w), wl.codes(w), wl.scales(w)
    hd, cd, sd = bf16_dev(h), u8_dev(c), u8_dev(s)
    ref, A = oracle.lmhead_logits_nvfp4(h, c, s, w.g, 1.0)
    del c, s
    for M in w.Ms:
        got = host_bits(L.logits_nvfp4(hd[:M].contiguous(), cd, sd, w.g, 1.0))
        strict = check_bf16(got, ref[:M], A[:M], w.g, oracle.ulp_bf16, what=f"nvfp4 M={M}")
        say(f"  M={M}: {got.size} elements, beyond 1 bf16 ulp (cancellation near zero): {strict}")


def test_prefill_two_full_tiles():
    w = wl.PREFILL
    say("prefill full output of rows 0-255 and 1792-2047: generate H=4096 V=151936")
    h, W = wl.hidden(w), wl.weight(w)
    alpha = w.alphas[0]
    out = L.logits(bf16_dev(h), bf16_dev(W), alpha)
    rows = np.concatenate([np.arange(256), np.arange(w.M - 256, w.M)])
    got = host_f32(out[torch.as_tensor(rows, device=DEV)])
    del out
    S, A = oracle.dot_f64(h[rows], W)
    del W
    ratio, exact = check_f32(got, oracle.logits_f32(S, alpha), abs(alpha) * A, what="prefill tiles")
    say(f"  {got.size} elements, max err/bound {ratio:.3f}, bit-exact {exact:.3f}")
