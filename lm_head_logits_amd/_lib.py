"""ctypes declarations of the C ABI in include/lmhead.h (argument marshalling only).

Loading never falls back to anything: if the HIP library cannot be built or
loaded, importing fails loudly.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

from . import _build

LMHEAD_F32 = 0
LMHEAD_BF16 = 1
LMHEAD_F16 = 2

OK = 0
NOT_HANDLED = 1
ERR_INVALID = -1
ERR_ALIGN = -2
ERR_DEVICE = -3

PATH_NONE = -1
PATH_AUTO = -2
PATH_SKINNY = 0
PATH_TILED = 1
PATH_NVFP4 = 2

NOALLOC_SCRATCH_BYTES = 32 << 20  # LMHEAD_NOALLOC_SCRATCH_BYTES

EXPORTS = ("lmhead_logits", "lmhead_logits_path", "lmhead_logits_ex", "lmhead_logits_rowreduce",
           "lmhead_rowreduce_workspace_bytes", "lmhead_logits_rowreduce_noalloc", "lmhead_logits_nvfp4", "lmhead_quantize_nvfp4",
           "lmhead_quantize_nvfp4_workspace_bytes", "lmhead_shape_ok",
           "lmhead_path_for", "lmhead_status_string", "lmhead_version")
# include/lmhead_probes.h: measurement probes (not part of the projection),
# in a library of their own
PROBE_EXPORTS = ("lmhead_probe_grid", "lmhead_probe_hbm_read", "lmhead_probe_mfma_bf16")

_lib = None
_probes = None


def lib_path() -> Path:
    return _build.LIB


def probes_path() -> Path:
    return _build.PROBES_LIB


def load() -> ctypes.CDLL:
    """Load liblmhead.so (building it first only when no build exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not _build.LIB.exists():
        _build.build()
    lib = ctypes.CDLL(str(_build.LIB))
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    lib.lmhead_logits.restype = i32
    lib.lmhead_logits.argtypes = [vp, i64, i64, vp, i64, f32, vp, i32, vp, vp]
    lib.lmhead_logits_path.restype = i32
    lib.lmhead_logits_path.argtypes = [vp, i64, i64, vp, i64, f32, vp, i32, vp, vp, i32]
    lib.lmhead_logits_ex.restype = i32
    lib.lmhead_logits_ex.argtypes = [vp, i64, i64, vp, i64, f32, vp, i32, i32, vp, vp, i32]
    lib.lmhead_logits_rowreduce.restype = i32
    lib.lmhead_logits_rowreduce.argtypes = [vp, i64, i64, vp, i64, f32, vp, i32, i32, vp, vp, vp,
                                            vp, vp, ctypes.c_size_t, vp, i32]
    lib.lmhead_logits_rowreduce_noalloc.restype = i32
    lib.lmhead_logits_rowreduce_noalloc.argtypes = [vp, i64, i64, vp, i64, f32, vp, i32, i32, vp,
                                                    vp, vp, vp, vp, i32]
    lib.lmhead_rowreduce_workspace_bytes.restype = ctypes.c_size_t
    lib.lmhead_rowreduce_workspace_bytes.argtypes = [i64, i64]
    lib.lmhead_quantize_nvfp4.restype = i32
    lib.lmhead_quantize_nvfp4.argtypes = [vp, i64, i64, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.lmhead_quantize_nvfp4_workspace_bytes.restype = ctypes.c_size_t
    lib.lmhead_quantize_nvfp4_workspace_bytes.argtypes = []
    lib.lmhead_logits_nvfp4.restype = i32
    lib.lmhead_logits_nvfp4.argtypes = [vp, i64, i64, vp, vp, f32, i64, f32, vp, vp, vp]
    lib.lmhead_shape_ok.restype = i32
    lib.lmhead_shape_ok.argtypes = [i64, i64, i64, i32]
    lib.lmhead_path_for.restype = i32
    lib.lmhead_path_for.argtypes = [i64, i64, i64, i32]
    lib.lmhead_status_string.restype = ctypes.c_char_p
    lib.lmhead_status_string.argtypes = [i32]
    lib.lmhead_version.restype = ctypes.c_char_p
    lib.lmhead_version.argtypes = []
    _lib = lib
    return lib


def load_probes() -> ctypes.CDLL:
    """Load liblmhead_probes.so, the measurement probes (built with the
    projection's library when neither exists)."""
    global _probes
    if _probes is not None:
        return _probes
    if not _build.PROBES_LIB.exists():
        _build.build()
    lib = ctypes.CDLL(str(_build.PROBES_LIB))
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.lmhead_probe_grid.restype = i64
    lib.lmhead_probe_grid.argtypes = []
    lib.lmhead_probe_hbm_read.restype = i32
    lib.lmhead_probe_hbm_read.argtypes = [vp, ctypes.c_size_t, i32, vp, vp]
    lib.lmhead_probe_mfma_bf16.restype = i32
    lib.lmhead_probe_mfma_bf16.argtypes = [i64, i32, vp, vp, ctypes.POINTER(ctypes.c_double)]
    _probes = lib
    return lib
