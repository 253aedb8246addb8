"""LM-head logits on MI355X: a thin Python binding over the C ABI of liblmhead.so.

    logits[M, V] = alpha * (hidden[M, H] . W[V, H]^T) + bias[V]

Every step of the projection runs in the library's HIP kernels. This module
only checks tensor metadata, allocates the output through torch and passes
device pointers and torch's current HIP stream to the C functions of
include/lmhead.h. There is no fallback computation: when the library returns
LMHEAD_NOT_HANDLED the caller gets ``NotHandled`` and decides what to do.
"""
from __future__ import annotations

import contextlib
import ctypes

import torch

from . import _lib
from ._lib import (LMHEAD_BF16, LMHEAD_F16, LMHEAD_F32, NOT_HANDLED, OK, PATH_AUTO, PATH_NONE,
                   PATH_NVFP4, PATH_SKINNY, PATH_TILED)

__all__ = ["logits", "logits_rowreduce", "logits_rowreduce_noalloc", "rowreduce_workspace_bytes", "logits_nvfp4",
           "quantize_nvfp4", "shape_ok", "path_for", "status_string", "version",
           "LmHeadError", "NotHandled", "PATH_SKINNY", "PATH_TILED", "PATH_NVFP4", "PATH_AUTO",
           "PATH_NONE", "probe_hbm_read", "probe_mfma_bf16"]


class LmHeadError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class NotHandled(LmHeadError):
    """The shape lies outside the kernels' contract; nothing was launched."""


def status_string(status: int) -> str:
    return _lib.load().lmhead_status_string(int(status)).decode()


def version() -> str:
    return _lib.load().lmhead_version().decode()


def shape_ok(M: int, H: int, V: int, nvfp4: bool = False) -> bool:
    return bool(_lib.load().lmhead_shape_ok(M, H, V, int(nvfp4)))


def path_for(M: int, H: int, V: int, nvfp4: bool = False) -> int:
    return int(_lib.load().lmhead_path_for(M, H, V, int(nvfp4)))


def _check(status: int, where: str):
    if status == OK:
        return
    if status == NOT_HANDLED:
        raise NotHandled(status, where)
    raise LmHeadError(status, where)


# torch's current raw HIP stream of a device index, without building a Stream
# object per call (the public route below when this build lacks it)
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(device, stream):
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None:
        return _raw_stream(device.index if device.index is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(device).cuda_stream


_NO_SWITCH = contextlib.nullcontext()


def _device_ctx(device):
    """The library launches on the current device: make it `device`, switching
    (and switching back) only when it is another one."""
    idx = device.index if device.index is not None else torch.cuda.current_device()
    return _NO_SWITCH if torch.cuda.current_device() == idx else torch.cuda.device(idx)


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _same_device(*tensors):
    devs = {t.device for t in tensors if t is not None}
    if len(devs) != 1:  # the message only on failure: this runs on every call
        raise ValueError(f"all tensors must be on one device, got {sorted(map(str, devs))}")


_PATHS = {"auto": PATH_AUTO, "skinny": PATH_SKINNY, "tiled": PATH_TILED}


_DTYPES = {torch.float32: LMHEAD_F32, torch.bfloat16: LMHEAD_BF16, torch.float16: LMHEAD_F16}


def logits(hidden: torch.Tensor, weight: torch.Tensor, alpha: float = 1.0, bias=None,
           out_dtype=torch.float32, out: torch.Tensor | None = None, *, path: str = "auto",
           stream=None) -> torch.Tensor:
    """alpha * hidden @ weight.T (+ bias): [M, H] x [V, H] -> [M, V], both inputs
    bf16 or both fp16, accumulated at fp32, logits fp32 or of the input type
    (lmhead_logits_ex). Other dtype combinations raise NotHandled (nothing
    runs; the caller falls back)."""
    _need(hidden.is_cuda and weight.is_cuda, "hidden and weight must be device tensors")
    _need(hidden.dtype in _DTYPES and weight.dtype in _DTYPES and out_dtype in _DTYPES,
          "dtypes must be float32, bfloat16 or float16")
    _need(hidden.dim() == 2 and weight.dim() == 2, "hidden [M, H] and weight [V, H] are 2-D")
    _need(hidden.is_contiguous() and weight.is_contiguous(), "inputs must be contiguous")
    M, H = hidden.shape
    V, H2 = weight.shape
    if H != H2:
        raise ValueError(f"hidden has H={H}, weight has H={H2}")
    in_code = _DTYPES[hidden.dtype] if hidden.dtype == weight.dtype else LMHEAD_F32
    if bias is not None:
        _need(bias.is_cuda and bias.dtype == torch.float32 and bias.shape == (V,)
              and bias.is_contiguous(), "bias must be a contiguous fp32 device tensor [V]")
    if out is None:
        out = torch.empty((M, V), dtype=out_dtype, device=hidden.device)
    else:
        _need(out.is_cuda and out.dtype == out_dtype and out.shape == (M, V) and out.is_contiguous(),
              "out must be a contiguous [M, V] device tensor of out_dtype")
    _same_device(hidden, weight, bias, out)
    with _device_ctx(hidden.device):
        st = _lib.load().lmhead_logits_ex(
            hidden.data_ptr(), M, H, weight.data_ptr(), V, float(alpha),
            bias.data_ptr() if bias is not None else None, in_code, _DTYPES[out_dtype],
            out.data_ptr(), _stream_handle(hidden.device, stream), _PATHS[path])
    _check(st, "lmhead_logits_ex")
    return out


def rowreduce_workspace_bytes(M: int, V: int) -> int:
    return int(_lib.load().lmhead_rowreduce_workspace_bytes(M, V))


def logits_rowreduce(hidden: torch.Tensor, weight: torch.Tensor, alpha: float = 1.0, bias=None,
                     out_dtype=torch.float32, out: torch.Tensor | None = None, *,
                     write_logits: bool = False, workspace: torch.Tensor | None = None,
                     path: str = "auto", stream=None):
    """Row reduction of alpha * hidden @ weight.T (+ bias) inside the GEMM's
    epilogue (lmhead_logits_rowreduce): returns (row_max fp32 [M], row_argmax
    int32 [M], row_sumexp fp32 [M], logits or None). The logits [M, V] are
    written only when `out` is given or `write_logits` is true. `workspace`
    (a byte tensor of at least rowreduce_workspace_bytes(M, V)) is allocated
    here when not given."""
    _need(hidden.is_cuda and weight.is_cuda, "hidden and weight must be device tensors")
    _need(hidden.dtype in _DTYPES and weight.dtype in _DTYPES and out_dtype in _DTYPES,
          "dtypes must be float32, bfloat16 or float16")
    _need(hidden.dim() == 2 and weight.dim() == 2, "hidden [M, H] and weight [V, H] are 2-D")
    _need(hidden.is_contiguous() and weight.is_contiguous(), "inputs must be contiguous")
    M, H = hidden.shape
    V, H2 = weight.shape
    if H != H2:
        raise ValueError(f"hidden has H={H}, weight has H={H2}")
    in_code = _DTYPES[hidden.dtype] if hidden.dtype == weight.dtype else LMHEAD_F32
    dev = hidden.device
    if bias is not None:
        _need(bias.is_cuda and bias.dtype == torch.float32 and bias.shape == (V,)
              and bias.is_contiguous(), "bias must be a contiguous fp32 device tensor [V]")
    if out is None and write_logits:
        out = torch.empty((M, V), dtype=out_dtype, device=dev)
    if out is not None:
        _need(out.is_cuda and out.dtype == out_dtype and out.shape == (M, V) and out.is_contiguous(),
              "out must be a contiguous [M, V] device tensor of out_dtype")
    need = rowreduce_workspace_bytes(M, V)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _need(workspace.is_cuda and workspace.is_contiguous(), "workspace must be a contiguous device tensor")
    row_max = torch.empty(M, dtype=torch.float32, device=dev)
    row_argmax = torch.empty(M, dtype=torch.int32, device=dev)
    row_sumexp = torch.empty(M, dtype=torch.float32, device=dev)
    _same_device(hidden, weight, bias, out, workspace)
    with _device_ctx(dev):
        st = _lib.load().lmhead_logits_rowreduce(
            hidden.data_ptr(), M, H, weight.data_ptr(), V, float(alpha),
            bias.data_ptr() if bias is not None else None, in_code, _DTYPES[out_dtype],
            out.data_ptr() if out is not None else None, row_max.data_ptr(),
            row_argmax.data_ptr(), row_sumexp.data_ptr(), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), _stream_handle(dev, stream),
            _PATHS[path])
    _check(st, "lmhead_logits_rowreduce")
    return row_max, row_argmax, row_sumexp, out


def logits_rowreduce_noalloc(hidden: torch.Tensor, weight: torch.Tensor, alpha: float = 1.0,
                             bias=None, out_dtype=torch.float32, out: torch.Tensor | None = None,
                             *, row_max: torch.Tensor | None = None,
                             row_argmax: torch.Tensor | None = None,
                             row_sumexp: torch.Tensor | None = None, path: str = "auto",
                             stream=None):
    """logits_rowreduce without a workspace (lmhead_logits_rowreduce_noalloc):
    the partials go to the library's own per-GPU buffer. With `row_max`,
    `row_argmax`, `row_sumexp` (fp32, int32, fp32 [M]) and `out` given, this
    allocates nothing. Returns (row_max, row_argmax, row_sumexp, out or None)."""
    _need(hidden.is_cuda and weight.is_cuda, "hidden and weight must be device tensors")
    _need(hidden.dtype in _DTYPES and weight.dtype in _DTYPES and out_dtype in _DTYPES,
          "dtypes must be float32, bfloat16 or float16")
    _need(hidden.dim() == 2 and weight.dim() == 2, "hidden [M, H] and weight [V, H] are 2-D")
    _need(hidden.is_contiguous() and weight.is_contiguous(), "inputs must be contiguous")
    M, H = hidden.shape
    V, H2 = weight.shape
    if H != H2:
        raise ValueError(f"hidden has H={H}, weight has H={H2}")
    in_code = _DTYPES[hidden.dtype] if hidden.dtype == weight.dtype else LMHEAD_F32
    dev = hidden.device
    if bias is not None:
        _need(bias.is_cuda and bias.dtype == torch.float32 and bias.shape == (V,)
              and bias.is_contiguous(), "bias must be a contiguous fp32 device tensor [V]")
    if out is not None:
        _need(out.is_cuda and out.dtype == out_dtype and out.shape == (M, V) and out.is_contiguous(),
              "out must be a contiguous [M, V] device tensor of out_dtype")
    outs = []
    for t, dt in ((row_max, torch.float32), (row_argmax, torch.int32), (row_sumexp, torch.float32)):
        if t is None:
            t = torch.empty(M, dtype=dt, device=dev)
        if not (t.is_cuda and t.dtype == dt and t.shape == (M,) and t.is_contiguous()):
            raise ValueError(f"row outputs must be contiguous [M] device tensors of {dt}")
        outs.append(t)
    _same_device(hidden, weight, bias, out, *outs)
    with _device_ctx(dev):
        st = _lib.load().lmhead_logits_rowreduce_noalloc(
            hidden.data_ptr(), M, H, weight.data_ptr(), V, float(alpha),
            bias.data_ptr() if bias is not None else None, in_code, _DTYPES[out_dtype],
            out.data_ptr() if out is not None else None, outs[0].data_ptr(), outs[1].data_ptr(),
            outs[2].data_ptr(), _stream_handle(dev, stream), _PATHS[path])
    _check(st, "lmhead_logits_rowreduce_noalloc")
    return outs[0], outs[1], outs[2], out


def quantize_nvfp4(weight: torch.Tensor, *, workspace: torch.Tensor | None = None, stream=None):
    """BF16 [V, H] -> NVFP4 (lmhead_quantize_nvfp4): returns (codes uint8
    [V, H/2], scales uint8 [V, H/16], global_scale fp32 [1]), all on the
    weight's device; logits_nvfp4 takes float(global_scale)."""
    _need(weight.is_cuda and weight.dtype == torch.bfloat16 and weight.dim() == 2
          and weight.is_contiguous(), "weight must be a contiguous bf16 [V, H] device tensor")
    V, H = weight.shape
    dev = weight.device
    codes = torch.empty((V, H // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((V, H // 16), dtype=torch.uint8, device=dev)
    g = torch.empty(1, dtype=torch.float32, device=dev)
    need = int(_lib.load().lmhead_quantize_nvfp4_workspace_bytes())
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _need(workspace.is_cuda and workspace.is_contiguous(), "workspace must be a contiguous device tensor")
    _same_device(weight, workspace)
    with _device_ctx(dev):
        st = _lib.load().lmhead_quantize_nvfp4(
            weight.data_ptr(), V, H, codes.data_ptr(), scales.data_ptr(), g.data_ptr(),
            workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            _stream_handle(dev, stream))
    _check(st, "lmhead_quantize_nvfp4")
    return codes, scales, g


def logits_nvfp4(hidden: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                 global_scale: float, alpha: float = 1.0, bias=None,
                 out: torch.Tensor | None = None, *, stream=None) -> torch.Tensor:
    """NVFP4 W4A16 head: bf16 hidden [M, H], uint8 codes [V, H/2] (two E2M1 per
    byte, low nibble first), uint8 E4M3 scales [V, H/16], fp32 global scale ->
    bf16 logits [M, V] (lmhead_logits_nvfp4)."""
    _need(hidden.is_cuda and codes.is_cuda and scales.is_cuda, "inputs must be device tensors")
    _need(hidden.dtype == torch.bfloat16, "hidden must be bf16")
    _need(codes.dtype == torch.uint8 and scales.dtype == torch.uint8, "codes and scales are uint8")
    _need(hidden.is_contiguous() and codes.is_contiguous() and scales.is_contiguous(),
          "inputs must be contiguous")
    M, H = hidden.shape
    V = codes.shape[0]
    if not (codes.shape == (V, H // 2) and H % 2 == 0):
        raise ValueError(f"codes must be [V, H/2] = [{V}, {H // 2}]")
    _need(H % 16 == 0 and scales.shape == (V, H // 16), "scales must be [V, H/16]")
    if bias is not None:
        _need(bias.is_cuda and bias.dtype == torch.float32 and bias.shape == (V,)
              and bias.is_contiguous(), "bias must be a contiguous fp32 device tensor [V]")
    if out is None:
        out = torch.empty((M, V), dtype=torch.bfloat16, device=hidden.device)
    else:
        _need(out.is_cuda and out.dtype == torch.bfloat16 and out.shape == (M, V)
              and out.is_contiguous(), "out must be a contiguous bf16 [M, V] device tensor")
    _same_device(hidden, codes, scales, bias, out)
    with _device_ctx(hidden.device):
        st = _lib.load().lmhead_logits_nvfp4(
            hidden.data_ptr(), M, H, codes.data_ptr(), scales.data_ptr(), float(global_scale), V,
            float(alpha), bias.data_ptr() if bias is not None else None, out.data_ptr(),
            _stream_handle(hidden.device, stream))
    _check(st, "lmhead_logits_nvfp4")
    return out


# Load the HIP library now: a missing or broken build fails the import.
_lib.load()


# ---------------------------------------------------------------------------
# Measurement probes (include/lmhead_probes.h): not part of the projection.
# ---------------------------------------------------------------------------

def _probe_sink(device, dtype):
    n = int(_lib.load_probes().lmhead_probe_grid()) * 256
    return torch.empty(n, dtype=dtype, device=device)


def probe_hbm_read(buf: torch.Tensor, *, stream=None) -> int:
    """Enqueue one read of `buf`'s bytes (a contiguous CUDA tensor, 16-byte
    aligned, size a multiple of 16 bytes); returns the bytes read."""
    _need(buf.is_cuda and buf.is_contiguous(), "buf must be a contiguous CUDA tensor")
    nbytes = buf.numel() * buf.element_size()
    sink = _probe_sink(buf.device, torch.int32)
    st = _lib.load_probes().lmhead_probe_hbm_read(buf.data_ptr(), nbytes, 0, sink.data_ptr(),
                                           _stream_handle(buf.device, stream))
    _check(st, "lmhead_probe_hbm_read")
    return nbytes


def probe_mfma_bf16(iters: int, device="cuda", *, stream=None) -> float:
    """Enqueue the bf16 MFMA probe; returns the floating-point operations of the launch."""
    dev = torch.device(device)
    sink = _probe_sink(dev, torch.float32)
    flops = ctypes.c_double(0.0)
    st = _lib.load_probes().lmhead_probe_mfma_bf16(int(iters), 0, sink.data_ptr(),
                                            _stream_handle(dev, stream), ctypes.byref(flops))
    _check(st, "lmhead_probe_mfma_bf16")
    return flops.value
