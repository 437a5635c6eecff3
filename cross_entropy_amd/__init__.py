"""MI355X (gfx950) fused LM-head log-prob and entropy head.

Per token: logits z = h W^T over the whole vocabulary (never stored), lse,
logp = z[target] - lse and entropy = lse - sum softmax(z) z, and the
backward into dh and dW. All of it runs in the HIP library
``liblmhead_logps.so`` (C ABI in ``include/lmhead_logps.h``); this module
only checks torch tensors and passes their device pointers and the current
HIP stream. PyTorch provides device memory and streams, nothing else.

Entry points mirror the C ABI:
    lmhead_logps_workspace_bytes(N, H, V, chunk_size, with_backward)
    lmhead_logps_fwd(hidden, W, targets, chunk_size, logp, entropy, lse, workspace)
    lmhead_logps_bwd(hidden, W, targets, chunk_size, lse, entropy, g_logp, g_ent,
                     dh, dW, workspace)
    lmhead_logps_fwd_temp / lmhead_logps_bwd_temp   (the same with a temperature
                     after chunk_size: the head scores the logits divided by it)
and two allocating helpers, ``forward`` and ``backward`` (``temperature=``
selects the tempered calls).
"""
from __future__ import annotations

from typing import Optional, Tuple

from . import _native
from ._native import LmheadError, load, version  # noqa: F401

__all__ = [
    "LmheadError",
    "lmhead_logps_workspace_bytes",
    "lmhead_logps_fwd",
    "lmhead_logps_bwd",
    "lmhead_logps_fwd_temp",
    "lmhead_logps_bwd_temp",
    "forward",
    "backward",
    "version",
]


def _torch():
    import torch
    return torch


def _ptr(t, name, dtypes, device, numel=None, optional=False):
    torch = _torch()
    if t is None:
        if optional:
            return 0
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on a GPU, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return t.data_ptr()


def _bf16_types():
    torch = _torch()
    return (torch.bfloat16, torch.int16, torch.uint16)


def _stream(device, stream):
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def lmhead_logps_workspace_bytes(N: int, H: int, V: int, chunk_size: int, with_backward: bool = True) -> int:
    return _native.raw_workspace_bytes(N, H, V, chunk_size, with_backward)


def _shapes(hidden, W, targets):
    if hidden.dim() != 2 or W.dim() != 2 or hidden.shape[1] != W.shape[1]:
        raise ValueError(f"hidden [N,H] and W [V,H] must share H: {tuple(hidden.shape)} vs {tuple(W.shape)}")
    N, H = hidden.shape
    V = W.shape[0]
    if targets.numel() != N:
        raise ValueError(f"targets has {targets.numel()} entries, expected {N}")
    return int(N), int(H), int(V)


def _fwd_args(hidden, W, targets, chunk_size, logp, entropy, lse, workspace, stream):
    torch = _torch()
    N, H, V = _shapes(hidden, W, targets)
    dev = hidden.device
    ptrs = (
        _ptr(hidden, "hidden", _bf16_types(), dev),
        _ptr(W, "W", _bf16_types(), dev),
        _ptr(targets, "targets", (torch.int32,), dev),
        N, H, V, chunk_size,
    )
    outs = (
        _ptr(logp, "logp", (torch.float32,), dev, N),
        _ptr(entropy, "entropy", (torch.float32,), dev, N, optional=True),
        _ptr(lse, "lse", (torch.float32,), dev, N),
        _ptr(workspace, "workspace", (torch.uint8,), dev),
        workspace.numel(),
        _stream(dev, stream),
    )
    return ptrs, outs


def lmhead_logps_fwd(hidden, W, targets, chunk_size: int, logp, entropy, lse, workspace, stream=None) -> None:
    """Enqueue the forward on ``stream`` (default: torch's current stream)."""
    ptrs, outs = _fwd_args(hidden, W, targets, chunk_size, logp, entropy, lse, workspace, stream)
    _native.check(_native.raw_fwd(*ptrs, *outs))


def lmhead_logps_fwd_temp(hidden, W, targets, chunk_size: int, temperature: float, logp, entropy, lse, workspace,
                          stream=None) -> None:
    """Enqueue the tempered forward (logits / temperature) on ``stream``."""
    ptrs, outs = _fwd_args(hidden, W, targets, chunk_size, logp, entropy, lse, workspace, stream)
    _native.check(_native.raw_fwd_temp(*ptrs, temperature, *outs))


def _bwd_args(hidden, W, targets, chunk_size, lse, entropy, g_logp, g_ent, dh, dW, workspace, stream):
    torch = _torch()
    N, H, V = _shapes(hidden, W, targets)
    dev = hidden.device
    if tuple(dh.shape) != (N, H) or tuple(dW.shape) != (V, H):
        raise ValueError("dh must be [N,H] and dW [V,H]")
    ptrs = (
        _ptr(hidden, "hidden", _bf16_types(), dev),
        _ptr(W, "W", _bf16_types(), dev),
        _ptr(targets, "targets", (torch.int32,), dev),
        N, H, V, chunk_size,
    )
    rest = (
        _ptr(lse, "lse", (torch.float32,), dev, N),
        _ptr(entropy, "entropy", (torch.float32,), dev, N, optional=True),
        _ptr(g_logp, "g_logp", (torch.float32,), dev, N, optional=True),
        _ptr(g_ent, "g_ent", (torch.float32,), dev, N, optional=True),
        _ptr(dh, "dh", (torch.float32,), dev),
        _ptr(dW, "dW", (torch.float32,), dev),
        _ptr(workspace, "workspace", (torch.uint8,), dev),
        workspace.numel(),
        _stream(dev, stream),
    )
    return ptrs, rest


def lmhead_logps_bwd(hidden, W, targets, chunk_size: int, lse, entropy, g_logp, g_ent, dh, dW, workspace,
                     stream=None) -> None:
    """Enqueue the backward on ``stream`` (default: torch's current stream)."""
    ptrs, rest = _bwd_args(hidden, W, targets, chunk_size, lse, entropy, g_logp, g_ent, dh, dW, workspace, stream)
    _native.check(_native.raw_bwd(*ptrs, *rest))


def lmhead_logps_bwd_temp(hidden, W, targets, chunk_size: int, temperature: float, lse, entropy, g_logp, g_ent,
                          dh, dW, workspace, stream=None) -> None:
    """Enqueue the tempered backward on ``stream``; lse and entropy come from
    the tempered forward with the same temperature."""
    ptrs, rest = _bwd_args(hidden, W, targets, chunk_size, lse, entropy, g_logp, g_ent, dh, dW, workspace, stream)
    _native.check(_native.raw_bwd_temp(*ptrs, temperature, *rest))


def workspace_for(hidden, W, chunk_size: int, with_backward: bool = True):
    torch = _torch()
    N, H = hidden.shape
    V = W.shape[0]
    nbytes = lmhead_logps_workspace_bytes(N, H, V, chunk_size, with_backward)
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=hidden.device)


def forward(hidden, W, targets, chunk_size: int, with_entropy: bool = True, workspace=None,
            stream=None, temperature: Optional[float] = None) -> Tuple:
    """Allocate outputs (torch) and run the forward: (logp, entropy | None, lse).
    ``temperature`` (None: the untempered call) scores the logits divided by it."""
    torch = _torch()
    N = hidden.shape[0]
    dev = hidden.device
    logp = torch.empty(N, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    ent = torch.empty(N, dtype=torch.float32, device=dev) if with_entropy else None
    if workspace is None:
        workspace = workspace_for(hidden, W, chunk_size, with_backward=False)
    if temperature is None:
        lmhead_logps_fwd(hidden, W, targets, chunk_size, logp, ent, lse, workspace, stream)
    else:
        lmhead_logps_fwd_temp(hidden, W, targets, chunk_size, temperature, logp, ent, lse, workspace, stream)
    return logp, ent, lse


def backward(hidden, W, targets, chunk_size: int, lse, entropy, g_logp, g_ent: Optional = None,
             workspace=None, stream=None, temperature: Optional[float] = None) -> Tuple:
    """Allocate gradients (torch) and run the backward: (dh, dW), float32.
    ``temperature`` must match the forward that produced lse and entropy."""
    torch = _torch()
    N, H = hidden.shape
    V = W.shape[0]
    dev = hidden.device
    dh = torch.empty((N, H), dtype=torch.float32, device=dev)
    dW = torch.empty((V, H), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = workspace_for(hidden, W, chunk_size, with_backward=True)
    if temperature is None:
        lmhead_logps_bwd(hidden, W, targets, chunk_size, lse, entropy, g_logp, g_ent, dh, dW, workspace, stream)
    else:
        lmhead_logps_bwd_temp(hidden, W, targets, chunk_size, temperature, lse, entropy, g_logp, g_ent, dh, dW,
                              workspace, stream)
    return dh, dW
