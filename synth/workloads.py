"""The synthetic workloads: shapes, seeds and input distributions.

Only input recipes live here (which generator, which stream, which shape).
Nothing in this module computes logits.

Every tensor is row-major. A hidden tensor with M rows is the first M*H
elements of its stream, so the first rows of a large call and a small call
are the same bytes -- the property the row-invariance checks rely on.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import (STREAM_BIAS, STREAM_CODES, STREAM_HIDDEN, STREAM_SCALES, STREAM_WEIGHT,
               int_bf16, int_f16, normal_bf16, normal_f16, normal_f32, uniform_bytes,
               uniform_e4m3)

W_STD = 0.02      # weight draws N(0, 0.02): 0.02 read as the standard deviation
H_STD = 1.0       # hidden draws N(0, 1)
BIAS_STD = 0.1    # embedding bias draws N(0, 0.1)
SCALE_LO, SCALE_HI = 0.25, 4.0   # E4M3 block scales ~ U[0.25, 4], rounded to E4M3
NVFP4_G = 0.01    # per-tensor fp32 scale of the NVFP4 head (not a power of two)


@dataclass(frozen=True)
class Workload:
    name: str
    H: int
    V: int
    Ms: tuple
    alphas: tuple
    seed: int
    bias: bool = False
    out_dtype: str = "f32"          # "f32", or the input type
    in_dtype: str = "bf16"          # "bf16" or "f16" (hidden and weight alike)
    nvfp4: bool = False
    g: float = 1.0
    notes: str = field(default="", compare=False)

    @property
    def M(self) -> int:
        return max(self.Ms)


TINY = Workload("tiny", H=256, V=4096, Ms=(4,), alphas=(0.25,), seed=1,
                notes="M=4, H=256, V=4096, alpha=1/4, no bias, fp32 out")
DECODE = Workload("decode", H=4096, V=128256, Ms=(1, 2, 8, 32, 64), alphas=(1.0, 1.0 / 16), seed=2,
                  notes="weight-bandwidth-bound decode head, fp32 out")
PREFILL = Workload("prefill", H=4096, V=151936, Ms=(2048,), alphas=(1.0 / 8,), seed=3,
                   notes="compute-bound prefill/verify head, fp32 out")
SPEC = Workload("spec", H=2048, V=151936, Ms=(128,), alphas=(1.0 / 8,), seed=4, bias=True,
                notes="spec-decode target (32 x 4 rows) and draft (32 rows) sharing one head; "
                      "fp32 bias; fp32 out")
NVFP4 = Workload("nvfp4", H=2048, V=151936, Ms=(1, 16, 64, 256), alphas=(1.0,), seed=5,
                 out_dtype="bf16", nvfp4=True, g=NVFP4_G,
                 notes="W4A16 NVFP4 head, bf16 out, 64-row blocks")

F16 = Workload("f16", H=4096, V=128256, Ms=(1, 64, 2048), alphas=(1.0 / 8,), seed=6,
              in_dtype="f16",
              notes="fp16 hidden and weight (the fast path's other input type), fp32 out; "
                    "decode rows and one prefill batch")

ALL = {w.name: w for w in (TINY, DECODE, PREFILL, SPEC, NVFP4, F16)}


def _normal(w: Workload):
    return normal_f16 if w.in_dtype == "f16" else normal_bf16


def hidden(w: Workload, M: int | None = None) -> np.ndarray:
    """bf16 (or fp16) bits [M, H] of N(0, 1)."""
    M = w.M if M is None else M
    return _normal(w)(w.seed, STREAM_HIDDEN, (M, w.H), std=H_STD)


def hidden_rows(w: Workload, rows) -> np.ndarray:
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), w.H), dtype=np.uint16)
    for i, r in enumerate(rows):
        out[i] = _normal(w)(w.seed, STREAM_HIDDEN, (w.H,), std=H_STD, start=int(r) * w.H,
                            threads=1)
    return out


def weight(w: Workload) -> np.ndarray:
    """bf16 (or fp16) bits [V, H] of N(0, 0.02)."""
    return _normal(w)(w.seed, STREAM_WEIGHT, (w.V, w.H), std=W_STD)


def weight_rows(w: Workload, v0: int, nv: int) -> np.ndarray:
    """bf16 (or fp16) bits of weight rows [v0, v0 + nv) only."""
    return _normal(w)(w.seed, STREAM_WEIGHT, (nv, w.H), std=W_STD, start=v0 * w.H)


def bf16_head(w: Workload) -> np.ndarray:
    """bf16 bits [V, H] of N(0, 0.02) at the workload's head shape: the input
    of the BF16 -> NVFP4 quantiser."""
    return normal_bf16(w.seed, STREAM_WEIGHT, (w.V, w.H), std=W_STD)


def bias(w: Workload) -> np.ndarray | None:
    if not w.bias:
        return None
    return normal_f32(w.seed, STREAM_BIAS, (w.V,), std=BIAS_STD)


def codes(w: Workload, v0: int = 0, nv: int | None = None) -> np.ndarray:
    """Packed E2M1 codes [V, H/2]: every nibble uniform over the 16 codes."""
    nv = w.V - v0 if nv is None else nv
    return uniform_bytes(w.seed, STREAM_CODES, (nv, w.H // 2), start=v0 * (w.H // 2))


def scales(w: Workload, v0: int = 0, nv: int | None = None) -> np.ndarray:
    """E4M3 block scales [V, H/16] ~ RNE_E4M3(U[0.25, 4])."""
    nv = w.V - v0 if nv is None else nv
    return uniform_e4m3(w.seed, STREAM_SCALES, (nv, w.H // 16), SCALE_LO, SCALE_HI,
                        start=v0 * (w.H // 16))


def int_hidden(seed: int, M: int, H: int, lo: int = -4, hi: int = 4) -> np.ndarray:
    """Integer-valued bf16 hidden for exact-arithmetic checks."""
    return int_bf16(seed, STREAM_HIDDEN, (M, H), lo, hi)


def int_weight(seed: int, V: int, H: int, lo: int = -4, hi: int = 4) -> np.ndarray:
    return int_bf16(seed, STREAM_WEIGHT, (V, H), lo, hi)


def int_hidden_f16(seed: int, M: int, H: int, lo: int = -1000, hi: int = 1000) -> np.ndarray:
    """Integer-valued fp16 hidden; magnitudes past 256 are not bf16 values."""
    return int_f16(seed, STREAM_HIDDEN, (M, H), lo, hi)


def int_weight_f16(seed: int, V: int, H: int, lo: int = -4, hi: int = 4) -> np.ndarray:
    return int_f16(seed, STREAM_WEIGHT, (V, H), lo, hi)
