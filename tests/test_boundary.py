"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before touching the
device (no call here launches anything)."""
import ctypes
import re

import pytest

import lm_head_logits_amd as L
from lm_head_logits_amd import _lib
from helpers import ROOT

HEADER = ROOT / "include" / "lmhead.h"
PROBE_HEADER = ROOT / "include" / "lmhead_probes.h"


def declared_functions(header=HEADER):
    text = re.sub(r"/\*.*?\*/", "", header.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(lmhead_\w+)\s*\(", text)))


def test_header_declares_the_python_exports():
    assert declared_functions() == sorted(_lib.EXPORTS)
    assert declared_functions(PROBE_HEADER) == sorted(_lib.PROBE_EXPORTS)


def test_every_header_is_checked():
    assert sorted(p.name for p in (ROOT / "include").glob("*.h")) == ["lmhead.h", "lmhead_probes.h"]


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(str(_lib.lib_path()))
    for name in declared_functions():
        assert hasattr(lib, name), name
    # the measurement probes live in a library of their own
    for name in declared_functions(PROBE_HEADER):
        assert not hasattr(lib, name), name
    probes = ctypes.CDLL(str(_lib.probes_path()))
    for name in declared_functions(PROBE_HEADER):
        assert hasattr(probes, name), name


def test_probes_reject_bad_arguments_on_the_host():
    lib = _lib.load_probes()
    sink = ctypes.c_void_p(16)  # never dereferenced: every call below fails its host checks
    assert lib.lmhead_probe_hbm_read(None, 1024, 0, sink, None) == _lib.ERR_INVALID
    assert lib.lmhead_probe_hbm_read(ctypes.c_void_p(256), 1000, 0, sink, None) == _lib.ERR_INVALID
    assert lib.lmhead_probe_hbm_read(ctypes.c_void_p(8), 1024, 0, sink, None) == _lib.ERR_INVALID
    assert lib.lmhead_probe_hbm_read(ctypes.c_void_p(256), 1024, 0, None, None) == _lib.ERR_INVALID
    assert lib.lmhead_probe_mfma_bf16(0, 0, sink, None, None) == _lib.ERR_INVALID
    assert lib.lmhead_probe_mfma_bf16(10, 0, None, None, None) == _lib.ERR_INVALID


def test_status_strings_and_version():
    for s in (0, 1, -1, -2, -3):
        assert L.status_string(s) and L.status_string(s) != "unknown status"
    assert L.status_string(99) == "unknown status"
    assert re.fullmatch(r"\d+\.\d+\.\d+", L.version())


@pytest.mark.parametrize("M,H,V,ok", [
    (1, 4096, 128256, True), (64, 4096, 128256, True), (2048, 4096, 151936, True),
    (0, 32, 1, True), (5, 32, 1, True),
    (4, 4016, 4096, False),          # H % 32 != 0: outside the contract
    (4, 16, 4096, False),
    (-1, 4096, 10, False), (4, 0, 10, False), (4, 4096, 0, False),
    ((1 << 24) + 1, 32, 10, False),  # beyond LMHEAD_MAX_M
    (4, (1 << 16) + 32, 10, False),  # beyond LMHEAD_MAX_H
    (4, 32, (1 << 20) + 1, False),   # beyond LMHEAD_MAX_V
    (4, 32, 1 << 20, True),
    (1 << 24, 32, 1 << 19, False),   # M * V beyond 2^42
])
def test_shape_ok(M, H, V, ok):
    assert L.shape_ok(M, H, V) is ok
    assert L.shape_ok(M, H, V, nvfp4=True) is ok


def test_path_choice():
    assert L.path_for(1, 4096, 128256) == L.PATH_SKINNY
    assert L.path_for(64, 4096, 128256) == L.PATH_SKINNY
    assert L.path_for(65, 4096, 128256) == L.PATH_TILED
    assert L.path_for(2048, 4096, 151936) == L.PATH_TILED
    assert L.path_for(256, 2048, 151936, nvfp4=True) == L.PATH_NVFP4
    assert L.path_for(4, 4016, 4096) == L.PATH_NONE


FAKE = 1 << 20  # a 16-byte-aligned non-null address; never dereferenced on these paths


def call(hidden=FAKE, M=4, H=64, W=FAKE, V=100, alpha=1.0, bias=None, dt=0, out=FAKE, path=-2):
    return _lib.load().lmhead_logits_path(hidden, M, H, W, V, alpha, bias, dt, out, None, path)


def call4(hidden=FAKE, M=4, H=64, codes=FAKE, scales=FAKE, g=1.0, V=100, alpha=1.0, bias=None,
          out=FAKE):
    return _lib.load().lmhead_logits_nvfp4(hidden, M, H, codes, scales, g, V, alpha, bias, out,
                                           None)


def callx(hidden=FAKE, M=4, H=64, W=FAKE, V=100, alpha=1.0, bias=None, din=1, dout=0, out=FAKE,
          path=-2):
    return _lib.load().lmhead_logits_ex(hidden, M, H, W, V, alpha, bias, din, dout, out, None, path)


def test_dtype_pairs_of_the_general_entry_point():
    F32, BF16, F16 = _lib.LMHEAD_F32, _lib.LMHEAD_BF16, _lib.LMHEAD_F16
    NH, E = _lib.NOT_HANDLED, _lib.ERR_INVALID
    # supported pairs pass every host check (M = 0: nothing is launched)
    for din, dout in ((BF16, F32), (BF16, BF16), (F16, F32), (F16, F16)):
        assert callx(hidden=None, W=None, out=None, M=0, din=din, dout=dout) == _lib.OK
        assert callx(hidden=None, din=din, dout=dout) == E
    # fp32 inputs and mixed 16-bit types are the caller's fallback
    for din, dout in ((F32, F32), (BF16, F16), (F16, BF16)):
        assert callx(din=din, dout=dout) == NH
    assert callx(din=3) == E and callx(dout=-1) == E
    assert callx(path=_lib.PATH_NVFP4) == E
    # the bf16 entry points refuse fp16 logits
    assert call(dt=F16) == E


def test_m_zero_is_ok_and_launches_nothing():
    assert call(hidden=None, W=None, out=None, M=0) == _lib.OK
    assert call4(hidden=None, codes=None, scales=None, out=None, M=0) == _lib.OK


def test_invalid_arguments():
    E = _lib.ERR_INVALID
    assert call(hidden=None) == E
    assert call(W=None) == E
    assert call(out=None) == E
    assert call(M=-1) == E
    assert call(H=0) == E
    assert call(V=0) == E
    assert call(dt=2) == E
    assert call(path=7) == E
    assert call4(codes=None) == E
    assert call4(scales=None) == E


def test_not_handled_shape():
    assert call(H=48) == _lib.NOT_HANDLED
    assert call4(H=48) == _lib.NOT_HANDLED


def test_alignment():
    A = _lib.ERR_ALIGN
    assert call(hidden=FAKE + 8) == A
    assert call(W=FAKE + 2) == A
    assert call(out=FAKE + 4) == A
    assert call(bias=FAKE + 2) == A
    assert call4(codes=FAKE + 8) == A
    assert call4(scales=FAKE + 1) == A


def callr(hidden=FAKE, M=4, H=64, W=FAKE, V=100, alpha=1.0, bias=None, din=1, dout=0, out=None,
          rmax=FAKE, rarg=FAKE, rsum=FAKE, ws=FAKE, wsb=None, path=-2):
    wsb = 16 * M * ((V + 15) // 16) if wsb is None else wsb
    return _lib.load().lmhead_logits_rowreduce(hidden, M, H, W, V, alpha, bias, din, dout, out,
                                               rmax, rarg, rsum, ws, wsb, None, path)


def test_rowreduce_workspace_size():
    f = _lib.load().lmhead_rowreduce_workspace_bytes
    assert f(1, 1) == 16 and f(1, 16) == 16 and f(1, 17) == 32
    assert f(64, 128256) == 16 * 64 * 8016
    assert f(0, 100) == 0 and f(-1, 100) == 0 and f(4, 0) == 0


def test_rowreduce_host_checks():
    E, A = _lib.ERR_INVALID, _lib.ERR_ALIGN
    assert callr(M=0, hidden=None, W=None, rmax=None, rarg=None, rsum=None, ws=None) == _lib.OK
    for k in ("hidden", "W", "rmax", "rarg", "rsum", "ws"):
        assert callr(**{k: None}) == E, k
    assert callr(wsb=16 * 4 * 7 - 1) == E                 # workspace one byte short
    assert callr(ws=FAKE + 8) == A
    assert callr(rmax=FAKE + 2) == A and callr(rarg=FAKE + 1) == A and callr(rsum=FAKE + 3) == A
    assert callr(out=FAKE + 4) == A
    assert callr(H=48) == _lib.NOT_HANDLED
    assert callr(din=_lib.LMHEAD_F32) == _lib.NOT_HANDLED
    assert callr(dout=_lib.LMHEAD_F16) == _lib.NOT_HANDLED  # bf16 inputs, fp16 logits
    assert callr(path=_lib.PATH_NVFP4) == E


def callq(W=FAKE, V=100, H=64, codes=FAKE, scales=FAKE, g=FAKE, ws=FAKE, wsb=None):
    lib = _lib.load()
    wsb = lib.lmhead_quantize_nvfp4_workspace_bytes() if wsb is None else wsb
    return lib.lmhead_quantize_nvfp4(W, V, H, codes, scales, g, ws, wsb, None)


def test_quantize_host_checks():
    E, A = _lib.ERR_INVALID, _lib.ERR_ALIGN
    assert _lib.load().lmhead_quantize_nvfp4_workspace_bytes() >= 4
    for k in ("W", "codes", "scales", "g", "ws"):
        assert callq(**{k: None}) == E, k
    assert callq(wsb=3) == E
    assert callq(V=0) == E and callq(H=0) == E and callq(V=(1 << 20) + 1) == E
    assert callq(H=48) == _lib.NOT_HANDLED
    assert callq(W=FAKE + 8) == A and callq(codes=FAKE + 2) == A and callq(g=FAKE + 2) == A
    assert callq(ws=FAKE + 2) == A


def calln(hidden=FAKE, M=4, H=64, W=FAKE, V=100, alpha=1.0, bias=None, din=1, dout=0, out=None,
          rmax=FAKE, rarg=FAKE, rsum=FAKE, path=-2):
    return _lib.load().lmhead_logits_rowreduce_noalloc(hidden, M, H, W, V, alpha, bias, din, dout,
                                                       out, rmax, rarg, rsum, None, path)


def test_rowreduce_noalloc_host_checks():
    """Every rejection happens on the host, before the scratch buffer's device
    address is looked up (no call here touches a device)."""
    E, A = _lib.ERR_INVALID, _lib.ERR_ALIGN
    assert calln(M=0, hidden=None, W=None, rmax=None, rarg=None, rsum=None) == _lib.OK
    for k in ("hidden", "W", "rmax", "rarg", "rsum"):
        assert calln(**{k: None}) == E, k
    assert calln(rmax=FAKE + 2) == A and calln(rarg=FAKE + 1) == A and calln(rsum=FAKE + 3) == A
    assert calln(out=FAKE + 4) == A and calln(hidden=FAKE + 8) == A
    assert calln(H=48) == _lib.NOT_HANDLED
    assert calln(din=_lib.LMHEAD_F32) == _lib.NOT_HANDLED
    assert calln(path=_lib.PATH_NVFP4) == E
    # the partials must fit the library's buffer: 16 bytes per row and 16-column block
    cap = _lib.NOALLOC_SCRATCH_BYTES
    V = 151936
    per_row = 16 * ((V + 15) // 16)
    assert calln(M=cap // per_row + 1, V=V) == E
    assert calln(M=1, V=1 << 20, rmax=None) == E  # fits, but a NULL output is still rejected first


def test_noalloc_scratch_constant_matches_header():
    text = HEADER.read_text()
    m = re.search(r"#define LMHEAD_NOALLOC_SCRATCH_BYTES \(\(int64_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.NOALLOC_SCRATCH_BYTES
