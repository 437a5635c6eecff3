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
    lmhead_logps_bwd_ex  (tempered backward that can add into dh / dW)
    lmhead_logps_bwd_bf16  (the same writing bf16 dh / dW: float32 sums in the
                         workspace, each element rounded once)
    lmhead_logps_fwd_shard / lmhead_logps_merge_shards / lmhead_logps_bwd_shard
                         (the head over vocabulary shards, partials merged by log-sum-exp)
    lmhead_logps_fwd_noalloc  (tempered forward without a workspace, for callers
                         that cannot allocate; its scratch is a fixed device array)
two allocating helpers, ``forward`` and ``backward`` (``temperature=``
selects the tempered calls, ``dh=`` / ``dW=`` with ``accumulate=`` add into
caller buffers), and ``lmhead_logps``, a ``torch.autograd.Function`` front
end for training code.
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
    "lmhead_logps_bwd_ex",
    "lmhead_logps_bwd_bf16",
    "lmhead_logps_fwd_shard",
    "lmhead_logps_merge_shards",
    "lmhead_logps_bwd_shard",
    "lmhead_logps_fwd_noalloc",
    "lmhead_logps",
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


def lmhead_logps_workspace_bytes(N: int, H: int, V: int, chunk_size: int, with_backward=True) -> int:
    """Workspace bytes: with_backward False (forward only), True (forward and
    the float32-gradient backward) or "bf16" (also the bf16-gradient backward)."""
    return _native.raw_workspace_bytes(N, H, V, chunk_size, _ws_kind(with_backward))


def _ws_kind(with_backward) -> int:
    if with_backward == "bf16":
        return _native.WS_BWD_BF16
    if isinstance(with_backward, str):
        raise ValueError(f"with_backward must be a bool or 'bf16', got {with_backward!r}")
    return _native.WS_BWD if with_backward else _native.WS_FWD


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


def lmhead_logps_fwd_noalloc(hidden, W, targets, chunk_size: int, temperature: float, logp, entropy, lse,
                             stream=None) -> None:
    """Enqueue the tempered forward without a workspace (the library's fixed
    scratch array; calls that overlap on one GPU race)."""
    torch = _torch()
    N, H, V = _shapes(hidden, W, targets)
    dev = hidden.device
    _native.check(_native.raw_fwd_noalloc(
        _ptr(hidden, "hidden", _bf16_types(), dev), _ptr(W, "W", _bf16_types(), dev),
        _ptr(targets, "targets", (torch.int32,), dev), N, H, V, chunk_size, temperature,
        _ptr(logp, "logp", (torch.float32,), dev, N), _ptr(entropy, "entropy", (torch.float32,), dev, N, optional=True),
        _ptr(lse, "lse", (torch.float32,), dev, N), _stream(dev, stream)))


def _bwd_args(hidden, W, targets, chunk_size, lse, entropy, g_logp, g_ent, dh, dW, workspace, stream,
              grad_types=None):
    torch = _torch()
    if grad_types is None:
        grad_types = (torch.float32,)
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
        _ptr(dh, "dh", grad_types, dev),
        _ptr(dW, "dW", grad_types, dev),
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


def lmhead_logps_bwd_ex(hidden, W, targets, chunk_size: int, temperature: float, lse, entropy, g_logp, g_ent,
                        dh, dW, flags: int, workspace, stream=None) -> None:
    """Enqueue the backward with flags (``_native.BWD_ACCUMULATE_DH`` /
    ``BWD_ACCUMULATE_DW``: add into dh / dW instead of overwriting)."""
    ptrs, rest = _bwd_args(hidden, W, targets, chunk_size, lse, entropy, g_logp, g_ent, dh, dW, workspace, stream)
    _native.check(_native.raw_bwd_ex(*ptrs, temperature, *rest[:6], flags, *rest[6:]))


def lmhead_logps_bwd_bf16(hidden, W, targets, chunk_size: int, temperature: float, lse, entropy, g_logp, g_ent,
                          dh, dW, flags: int, workspace, stream=None) -> None:
    """Enqueue the backward writing bf16 gradients dh [N, H] / dW [V, H]
    (bfloat16 tensors); ``flags`` as for ``lmhead_logps_bwd_ex``; the
    workspace is sized with ``with_backward="bf16"``."""
    ptrs, rest = _bwd_args(hidden, W, targets, chunk_size, lse, entropy, g_logp, g_ent, dh, dW, workspace, stream,
                           grad_types=_bf16_types())
    _native.check(_native.raw_bwd_bf16(*ptrs, temperature, *rest[:6], flags, *rest[6:]))


def lmhead_logps_fwd_shard(hidden, W_shard, targets, vocab_offset: int, V_total: int, chunk_size: int,
                           temperature: float, partial, workspace, stream=None) -> None:
    """Enqueue one vocabulary shard's forward: partial f32 [N, 4] records."""
    torch = _torch()
    N, H, V = _shapes(hidden, W_shard, targets)
    dev = hidden.device
    _native.check(_native.raw_fwd_shard(
        _ptr(hidden, "hidden", _bf16_types(), dev), _ptr(W_shard, "W_shard", _bf16_types(), dev),
        _ptr(targets, "targets", (torch.int32,), dev), N, H, V, vocab_offset, V_total, chunk_size, temperature,
        _ptr(partial, "partial", (torch.float32,), dev, 4 * N), _ptr(workspace, "workspace", (torch.uint8,), dev),
        workspace.numel(), _stream(dev, stream)))


def lmhead_logps_merge_shards(partials, targets, V_total: int, temperature: float, logp, entropy, lse,
                              stream=None) -> None:
    """Merge shard records partials f32 [P, N, 4] (shard order) into logp / entropy / lse."""
    torch = _torch()
    if partials.dim() != 3 or partials.shape[2] != 4:
        raise ValueError("partials must be [P, N, 4]")
    P, N = int(partials.shape[0]), int(partials.shape[1])
    dev = partials.device
    _native.check(_native.raw_merge_shards(
        _ptr(partials, "partials", (torch.float32,), dev), P, _ptr(targets, "targets", (torch.int32,), dev, N),
        N, V_total, temperature, _ptr(logp, "logp", (torch.float32,), dev, N),
        _ptr(entropy, "entropy", (torch.float32,), dev, N, optional=True), _ptr(lse, "lse", (torch.float32,), dev, N),
        _stream(dev, stream)))


def lmhead_logps_bwd_shard(hidden, W_shard, targets, vocab_offset: int, V_total: int, chunk_size: int,
                           temperature: float, lse, entropy, g_logp, g_ent, dh, dW_shard, flags: int, workspace,
                           stream=None) -> None:
    """Enqueue one vocabulary shard's backward (dW_shard, and its part of dh)."""
    ptrs, rest = _bwd_args(hidden, W_shard, targets, chunk_size, lse, entropy, g_logp, g_ent, dh, dW_shard,
                           workspace, stream)
    hid, Wp, tg, N, H, V, C = ptrs
    _native.check(_native.raw_bwd_shard(hid, Wp, tg, N, H, V, vocab_offset, V_total, C, temperature, *rest[:6],
                                        flags, *rest[6:]))


def workspace_for(hidden, W, chunk_size: int, with_backward=True):
    """Allocate a workspace (uint8 tensor) for the given calls: with_backward
    False, True or "bf16" as for ``lmhead_logps_workspace_bytes``."""
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
             workspace=None, stream=None, temperature: Optional[float] = None, dh=None, dW=None,
             accumulate: bool = False, grad_dtype=None) -> Tuple:
    """Run the backward: (dh, dW), float32 (or bfloat16 with
    ``grad_dtype=torch.bfloat16``). Gradients are allocated unless ``dh`` /
    ``dW`` are given; with ``accumulate`` the given buffers are added into.
    ``temperature`` must match the forward that produced lse and entropy."""
    torch = _torch()
    N, H = hidden.shape
    V = W.shape[0]
    dev = hidden.device
    if grad_dtype is None:
        grad_dtype = dh.dtype if dh is not None else torch.float32
    if grad_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"grad_dtype must be float32 or bfloat16, got {grad_dtype}")
    if accumulate and (dh is None or dW is None):
        raise ValueError("accumulate needs both dh and dW buffers")
    if dh is None:
        dh = torch.empty((N, H), dtype=grad_dtype, device=dev)
    if dW is None:
        dW = torch.empty((V, H), dtype=grad_dtype, device=dev)
    if grad_dtype == torch.bfloat16:
        if workspace is None:
            workspace = workspace_for(hidden, W, chunk_size, with_backward="bf16")
        flags = (_native.BWD_ACCUMULATE_DH | _native.BWD_ACCUMULATE_DW) if accumulate else 0
        lmhead_logps_bwd_bf16(hidden, W, targets, chunk_size, 1.0 if temperature is None else temperature, lse,
                              entropy, g_logp, g_ent, dh, dW, flags, workspace, stream)
        return dh, dW
    if workspace is None:
        workspace = workspace_for(hidden, W, chunk_size, with_backward=True)
    if accumulate:
        flags = _native.BWD_ACCUMULATE_DH | _native.BWD_ACCUMULATE_DW
        lmhead_logps_bwd_ex(hidden, W, targets, chunk_size, 1.0 if temperature is None else temperature, lse,
                            entropy, g_logp, g_ent, dh, dW, flags, workspace, stream)
    elif temperature is None:
        lmhead_logps_bwd(hidden, W, targets, chunk_size, lse, entropy, g_logp, g_ent, dh, dW, workspace, stream)
    else:
        lmhead_logps_bwd_temp(hidden, W, targets, chunk_size, temperature, lse, entropy, g_logp, g_ent, dh, dW,
                              workspace, stream)
    return dh, dW


def _autograd_function():
    torch = _torch()

    class _LmheadLogps(torch.autograd.Function):
        """logp (and entropy) of the head with its backward through the
        library. The forward holds only its own small workspace (the split
        records) and keeps lse (and entropy) for the backward; the backward
        sizes its workspace when it runs and writes the gradients in the
        inputs' dtype directly (bf16 inputs: lmhead_logps_bwd_bf16, float32
        sums in the workspace, no float32 [N, H] / [V, H] gradient tensors
        and no cast)."""

        @staticmethod
        def forward(ctx, hidden, W, targets, chunk_size, temperature, with_entropy):
            logp, ent, lse = forward(hidden, W, targets, chunk_size, with_entropy=with_entropy,
                                     temperature=temperature)
            ctx.chunk_size = chunk_size
            ctx.temperature = temperature
            ctx.with_entropy = with_entropy
            saved = (hidden, W, targets, lse) + ((ent,) if with_entropy else ())
            ctx.save_for_backward(*saved)
            if with_entropy:
                return logp, ent
            return logp

        @staticmethod
        def backward(ctx, g_logp, g_ent=None):
            hidden, W, targets, lse = ctx.saved_tensors[:4]
            ent = ctx.saved_tensors[4] if ctx.with_entropy else None
            gl = None if g_logp is None else g_logp.detach().contiguous().float()
            ge = None if (g_ent is None or ent is None) else g_ent.detach().contiguous().float()
            bf16 = hidden.dtype == torch.bfloat16 and W.dtype == torch.bfloat16
            dh, dW = backward(hidden, W, targets, ctx.chunk_size, lse, ent if ge is not None else None, gl, ge,
                              temperature=ctx.temperature,
                              grad_dtype=torch.bfloat16 if bf16 else torch.float32)
            return (dh.to(hidden.dtype) if ctx.needs_input_grad[0] else None,
                    dW.to(W.dtype) if ctx.needs_input_grad[1] else None,
                    None, None, None, None)

    return _LmheadLogps


_FN = None


def lmhead_logps(hidden, W, targets, chunk_size: int, temperature: Optional[float] = None, with_entropy: bool = True):
    """Differentiable head for training code: returns ``(logp, entropy)``
    (or ``logp`` alone without entropy). ``hidden`` [N, H] and ``W`` [V, H]
    are bfloat16 tensors on one GPU; a backward through either output runs
    ``lmhead_logps_bwd`` on the saved lse / entropy (the logits are recomputed,
    never stored). Masked targets (outside [0, V)) give zeros."""
    global _FN
    if _FN is None:
        _FN = _autograd_function()
    return _FN.apply(hidden, W, targets, chunk_size, temperature, with_entropy)
