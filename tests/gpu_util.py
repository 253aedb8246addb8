"""Host <-> device plumbing for the GPU tests (no arithmetic of the method)."""
from __future__ import annotations

import numpy as np
import torch

DEV = "cuda:0"


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    """bf16 bit patterns (uint16) -> bf16 device tensor, same bytes."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def f16_dev(bits: np.ndarray) -> torch.Tensor:
    """fp16 bit patterns (uint16) -> fp16 device tensor, same bytes."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16).to(DEV)


def u8_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def f32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host array of its bit patterns (uint16 for bf16 and
    fp16, uint32 for fp32)."""
    t = t.detach().contiguous().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    raise TypeError(t.dtype)


def host_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def say(*a):
    print(*a, flush=True)
