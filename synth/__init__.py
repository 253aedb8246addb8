"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

This package draws inputs and nothing else: it holds none of the logits
projection's arithmetic. Every element is a pure function of
(seed, stream, index) -- SplitMix64 as a counter-based generator, Box-Muller
for normals -- so a slice of any tensor can be regenerated on its own and the
bytes do not depend on the thread count. See ``synth.c`` for the definitions.

Streams: each tensor of a workload draws from its own stream id (constants
below), so hidden, weight, bias, codes and scales never share random numbers.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "synth.c"
_LIB = _HERE / "libsynth.so"

STREAM_HIDDEN = 1
STREAM_WEIGHT = 2
STREAM_BIAS = 3
STREAM_CODES = 4
STREAM_SCALES = 5

_lib = None


def build(force: bool = True) -> Path:
    """Compile ``synth.c`` into ``libsynth.so`` next to it (gcc, -O2)."""
    if force or not _LIB.exists():
        tmp = _LIB.with_suffix(".so.tmp")
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
               "-o", str(tmp), str(_SRC), "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not _LIB.exists():
            build()
        lib = ctypes.CDLL(str(_LIB))
        u64, i32, dbl, vp = ctypes.c_uint64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        lib.synth_splitmix64_at.restype = u64
        lib.synth_splitmix64_at.argtypes = [u64, u64]
        lib.synth_key.restype = u64
        lib.synth_key.argtypes = [u64, u64]
        for name in ("synth_normal_bf16", "synth_normal_f32"):
            getattr(lib, name).restype = None
            getattr(lib, name).argtypes = [u64, u64, u64, u64, dbl, dbl, vp, i32]
        for name in ("synth_int_bf16", "synth_int_f32"):
            getattr(lib, name).restype = None
            getattr(lib, name).argtypes = [u64, u64, u64, u64, i32, i32, vp, i32]
        lib.synth_bytes.restype = None
        lib.synth_bytes.argtypes = [u64, u64, u64, u64, vp, i32]
        lib.synth_uniform_e4m3.restype = None
        lib.synth_uniform_e4m3.argtypes = [u64, u64, u64, u64, dbl, dbl, vp, i32]
        _lib = lib
    return _lib


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def _n(shape) -> int:
    return int(np.prod(shape, dtype=np.int64)) if len(shape) else 1


def splitmix64_at(key: int, i: int) -> int:
    return int(_load().synth_splitmix64_at(key, i))


def key(seed: int, stream: int) -> int:
    return int(_load().synth_key(seed, stream))


def normal_bf16(seed, stream, shape, std=1.0, mean=0.0, start=0, threads=None) -> np.ndarray:
    """bf16 bit patterns (uint16) of mean + std * N(0, 1)."""
    out = np.empty(shape, dtype=np.uint16)
    _load().synth_normal_bf16(seed, stream, start, _n(shape), float(mean), float(std),
                              out.ctypes.data, threads or default_threads())
    return out


def normal_f32(seed, stream, shape, std=1.0, mean=0.0, start=0, threads=None) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    _load().synth_normal_f32(seed, stream, start, _n(shape), float(mean), float(std),
                             out.ctypes.data, threads or default_threads())
    return out


def int_bf16(seed, stream, shape, lo, hi, start=0, threads=None) -> np.ndarray:
    """bf16 bit patterns of integers uniform in [lo, hi] (|lo|, |hi| <= 256: exact)."""
    assert -256 <= lo <= hi <= 256
    out = np.empty(shape, dtype=np.uint16)
    _load().synth_int_bf16(seed, stream, start, _n(shape), int(lo), int(hi), out.ctypes.data,
                           threads or default_threads())
    return out


def normal_f16(seed, stream, shape, std=1.0, mean=0.0, start=0, threads=None) -> np.ndarray:
    """fp16 bit patterns (uint16) of mean + std * N(0, 1): the binary32 draw of
    ``normal_f32`` rounded to binary16 by numpy (nearest even)."""
    return normal_f32(seed, stream, shape, std, mean, start, threads).astype(np.float16).view(np.uint16)


def int_f16(seed, stream, shape, lo, hi, start=0, threads=None) -> np.ndarray:
    """fp16 bit patterns of integers uniform in [lo, hi] (|lo|, |hi| <= 2048: exact)."""
    assert -2048 <= lo <= hi <= 2048
    f = np.empty(shape, dtype=np.float32)
    _load().synth_int_f32(seed, stream, start, _n(shape), int(lo), int(hi), f.ctypes.data,
                          threads or default_threads())
    return f.astype(np.float16).view(np.uint16)


def uniform_bytes(seed, stream, shape, start=0, threads=None) -> np.ndarray:
    out = np.empty(shape, dtype=np.uint8)
    _load().synth_bytes(seed, stream, start, _n(shape), out.ctypes.data, threads or default_threads())
    return out


def uniform_e4m3(seed, stream, shape, lo, hi, start=0, threads=None) -> np.ndarray:
    """OCP E4M3 bytes of fp32 uniforms in [lo, hi), rounded to nearest even."""
    out = np.empty(shape, dtype=np.uint8)
    _load().synth_uniform_e4m3(seed, stream, start, _n(shape), float(lo), float(hi),
                               out.ctypes.data, threads or default_threads())
    return out


def rows_of(gen, seed, stream, row_len, rows, **kw) -> np.ndarray:
    """Regenerate only the listed rows of a row-major [*, row_len] tensor."""
    rows = np.asarray(rows, dtype=np.int64)
    parts = [gen(seed, stream, (row_len,), start=int(r) * row_len, threads=1, **kw) for r in rows]
    return np.stack(parts) if parts else np.empty((0, row_len))
