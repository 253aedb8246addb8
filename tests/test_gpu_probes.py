"""The measurement probes of include/lmhead_probes.h (GPU): the HBM probe
reads every 16-byte piece of its buffer exactly once (the xor of what the
threads read equals the xor of the buffer), and the MFMA probe runs and
reports its operation count."""
import ctypes

import numpy as np
import pytest
import torch

import lm_head_logits_amd as L
from lm_head_logits_amd import _lib

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _sink(dtype):
    return torch.zeros(int(_lib.load_probes().lmhead_probe_grid()) * 256, dtype=dtype, device=DEV)


@pytest.mark.parametrize("nbytes", [16, 4096, (16 << 20) + 48, 3 * (1 << 20) + 16])
def test_hbm_probe_reads_every_piece_once(nbytes):
    print(f"hbm probe, {nbytes} bytes", flush=True)
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 1 << 32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to(DEV)
    sink = _sink(torch.int32)
    st = _lib.load_probes().lmhead_probe_hbm_read(buf.data_ptr(), nbytes, 1, sink.data_ptr(),
                                           torch.cuda.current_stream().cuda_stream)
    assert st == _lib.OK
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)


def test_hbm_probe_binding():
    buf = torch.ones(1 << 20, dtype=torch.float32, device=DEV)
    assert L.probe_hbm_read(buf) == 4 << 20
    torch.cuda.synchronize()


def test_mfma_probe_runs_and_counts_its_operations():
    sink = _sink(torch.float32)
    flops = ctypes.c_double(0.0)
    st = _lib.load_probes().lmhead_probe_mfma_bf16(50, 1, sink.data_ptr(),
                                            torch.cuda.current_stream().cuda_stream,
                                            ctypes.byref(flops))
    assert st == _lib.OK
    torch.cuda.synchronize()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert flops.value == 2 * cus * 4 * 50 * 16 * 2 * 16 * 16 * 32
    vals = sink[: 2 * cus * 256].cpu()
    assert torch.isfinite(vals).all() and (vals != 0).any()
    assert L.probe_mfma_bf16(10, DEV) == 2 * cus * 4 * 10 * 16 * 16384
    torch.cuda.synchronize()
