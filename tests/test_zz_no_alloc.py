"""The row reduction without a workspace (lmhead_logits_rowreduce_noalloc):
called through the C ABI, its row maxima, argmaxes, sums of exponentials and
logits equal those of lmhead_logits_rowreduce with a caller workspace, bit
for bit, on two calls in a row on the library's one per-GPU buffer -- the
second with a smaller input, so stale partials of the first call would show
-- on both kernels, and a call past the buffer's size is refused."""
import ctypes

import numpy as np
import pytest
import torch

from lm_head_logits_amd import _lib
import oracle
from gpu_util import DEV, bf16_dev, f32_dev, host_bits, say

pytestmark = pytest.mark.gpu


def _rand_bf16(rng, shape, std):
    return oracle.f32_to_bf16_rne(rng.normal(0, std, shape).astype(np.float32))


def _rows(M):
    return (torch.empty(M, dtype=torch.float32, device=DEV),
            torch.empty(M, dtype=torch.int32, device=DEV),
            torch.empty(M, dtype=torch.float32, device=DEV))


def _call(noalloc, hd, Wd, M, H, V, alpha, bd, path):
    lib = _lib.load()
    out = torch.empty((M, V), dtype=torch.float32, device=DEV)
    rm, ra, rs = _rows(M)
    stream = torch.cuda.current_stream().cuda_stream
    bias = bd.data_ptr() if bd is not None else None
    if noalloc:
        st = lib.lmhead_logits_rowreduce_noalloc(
            hd.data_ptr(), M, H, Wd.data_ptr(), V, alpha, bias, _lib.LMHEAD_BF16, _lib.LMHEAD_F32,
            out.data_ptr(), rm.data_ptr(), ra.data_ptr(), rs.data_ptr(), stream, path)
    else:
        need = lib.lmhead_rowreduce_workspace_bytes(M, V)
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        st = lib.lmhead_logits_rowreduce(
            hd.data_ptr(), M, H, Wd.data_ptr(), V, alpha, bias, _lib.LMHEAD_BF16, _lib.LMHEAD_F32,
            out.data_ptr(), rm.data_ptr(), ra.data_ptr(), rs.data_ptr(), ws.data_ptr(), need,
            stream, path)
    assert st == _lib.OK, st
    torch.cuda.synchronize()
    return [host_bits(t) if t.dtype != torch.int32 else t.cpu().numpy() for t in (rm, ra, rs, out)]


# two calls in a row, the second smaller (rows and vocabulary): (M, H, V, bias)
SEQUENCES = [((64, 256, 40000, True), (3, 256, 999, False)),
             ((130, 192, 20001, False), (65, 192, 4100, True))]


@pytest.mark.parametrize("path", [_lib.PATH_AUTO, _lib.PATH_SKINNY, _lib.PATH_TILED])
@pytest.mark.parametrize("seq", SEQUENCES)
def test_noalloc_equals_workspace_call(seq, path):
    for k, (M, H, V, has_bias) in enumerate(seq):
        say(f"noalloc rowreduce call {k}: M={M} H={H} V={V} bias={has_bias} path={path}")
        rng = np.random.default_rng(1000 * M + V)
        hd = bf16_dev(_rand_bf16(rng, (M, H), 1.0))
        Wd = bf16_dev(_rand_bf16(rng, (V, H), 0.02))
        bd = f32_dev(rng.normal(0, 0.1, V).astype(np.float32)) if has_bias else None
        want = _call(False, hd, Wd, M, H, V, 0.125, bd, path)
        got = _call(True, hd, Wd, M, H, V, 0.125, bd, path)
        for name, g, w in zip(("max", "argmax", "sumexp", "logits"), got, want):
            assert np.array_equal(g, w), (k, name)


def test_noalloc_refuses_oversize_and_launches_nothing():
    lib = _lib.load()
    V = 151936
    M = _lib.NOALLOC_SCRATCH_BYTES // (16 * ((V + 15) // 16)) + 1
    say(f"noalloc oversize M={M} V={V}")
    rm, ra, rs = _rows(M)
    rm.fill_(7.0)
    fake = 1 << 20  # never dereferenced: the call is refused on the host
    st = lib.lmhead_logits_rowreduce_noalloc(fake, M, 64, fake, V, 1.0, None, _lib.LMHEAD_BF16,
                                             _lib.LMHEAD_F32, None, rm.data_ptr(), ra.data_ptr(),
                                             rs.data_ptr(), torch.cuda.current_stream().cuda_stream,
                                             _lib.PATH_AUTO)
    torch.cuda.synchronize()
    assert st == _lib.ERR_INVALID
    assert bool((rm == 7.0).all())
