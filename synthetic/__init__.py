"""Seeded synthetic inputs for the LM-head log-prob / entropy head.

This module only draws random numbers and lays them out. It holds none of the
head's arithmetic, so both the fp64 oracle tests and the GPU path may use it.

The five workloads follow the shapes the pages measure on:

* the SkyRL issue "[tx] support long sequence" (section "4. Chunked LM Head"):
  Qwen3-4B-Instruct, batch 16 x sequence 4k, a 152k vocabulary, chunk 512;
* google/tunix pull request #2913 (pad-first packing and the fused sharded
  log-prob head): RL-trainer rows of 60,948 real tokens and 4,588 padding
  tokens, log-prob chunks of 4,096;
* google/tunix pull request #2876 ("Compile compute_chunked_logps at
  chunk_size > 1024 under context parallelism"): one context rank's share of a
  row at context 4, chunks 1,024 and 4,096.

No public dataset or checkpoint is used; every tensor is drawn here.

Seeds: numpy ``Generator(PCG64(seed))`` with ``seed = 1000 * config + stream``
(stream 0 hidden, 1 W, 2 targets, 3 g_logp, 4 g_ent, 5 segment cuts).
Floating values are drawn in float32 and rounded to bfloat16 with
round-to-nearest-even; bf16 tensors are returned as their uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "make_inputs",
    "make_cotangents",
    "sample_tokens",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: sizes plus the distributions its inputs use."""

    index: int            # 1-based workload number (seed base is 1000 * index)
    name: str
    N: int                # tokens (flattened batch x sequence)
    H: int                # hidden size
    V: int                # vocabulary size
    chunk_sizes: tuple    # chunk_size values the workload is run with
    hidden: str           # "normal" or "normal_rms1"
    w_std: float          # standard deviation of W entries
    n_pad_front: int = 0  # masked (target -1) tokens placed at the start
    n_segments: int = 1   # segments the real tokens are cut into

    @property
    def chunk_size(self) -> int:
        return self.chunk_sizes[0]


# Distribution notation N(0, s): s is the standard deviation.
WORKLOADS = {
    1: Workload(1, "tiny", 256, 256, 4096, (128,), "normal", 2.0 / np.sqrt(256.0)),
    2: Workload(2, "qwen3-4b-head-1seq", 4096, 2560, 151936, (512,), "normal_rms1", 0.02),
    3: Workload(3, "qwen3-4b-head-bs16x4096", 65536, 2560, 151936, (512,), "normal_rms1", 0.02),
    4: Workload(4, "context-rank-share", 15237, 4096, 151936, (1024, 4096), "normal", 0.02),
    5: Workload(5, "packed-row-pad-first", 65536, 2560, 151936, (4096,), "normal_rms1", 0.02,
                n_pad_front=4588, n_segments=8),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the uint16 bit patterns. NaN stays NaN (quiet bit forced)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint64(16)).astype(np.uint16) | np.uint16(0x0040))
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(workload_no: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * workload_no + stream))


def _normal_f32(rng: np.random.Generator, shape, std: float, block_rows: int = 4096) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    rows = shape[0]
    for r0 in range(0, rows, block_rows):
        r1 = min(rows, r0 + block_rows)
        out[r0:r1] = rng.standard_normal((r1 - r0,) + tuple(shape[1:]), dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def make_inputs(cfg: Workload, N: Optional[int] = None, seed_index: Optional[int] = None):
    """Draw (hidden_bits [N,H] u16, W_bits [V,H] u16, targets [N] i32).

    ``N`` may shrink the token count (the first N tokens of the workload's
    layout are not reproduced; a fresh draw of N tokens is made with the same
    recipe). ``seed_index`` overrides the seed base (default: the workload's).
    """
    idx = cfg.index if seed_index is None else seed_index
    n = cfg.N if N is None else int(N)
    H, V = cfg.H, cfg.V

    h = _normal_f32(_rng(idx, 0), (n, H), 1.0)
    if cfg.hidden == "normal_rms1":
        rms = np.sqrt(np.mean(np.square(h, dtype=np.float64), axis=1, keepdims=True))
        rms[rms == 0] = 1.0
        h = (h / rms.astype(np.float32)).astype(np.float32)
    h_bits = f32_to_bf16_bits(h)
    del h
    W_bits = f32_to_bf16_bits(_normal_f32(_rng(idx, 1), (V, H), cfg.w_std))

    t = _rng(idx, 2).integers(0, V, size=n, dtype=np.int64).astype(np.int32)
    pad = min(cfg.n_pad_front, n) if N is None or n == cfg.N else int(round(cfg.n_pad_front * n / cfg.N))
    if pad > 0:
        t[:pad] = -1
    return h_bits, W_bits, t


def segment_bounds(cfg: Workload, N: Optional[int] = None) -> np.ndarray:
    """Start offsets of the real-token segments (after the leading padding).

    The head itself does not read segments; they describe the packed-row
    layout (8 segments of random lengths after 4,588 leading padding tokens)."""
    n = cfg.N if N is None else int(N)
    pad = cfg.n_pad_front if n == cfg.N else int(round(cfg.n_pad_front * n / cfg.N))
    real = n - pad
    k = max(1, cfg.n_segments)
    cuts = np.sort(_rng(cfg.index, 5).choice(np.arange(1, max(2, real)), size=min(k - 1, max(0, real - 1)), replace=False))
    return np.concatenate([[pad], pad + cuts]).astype(np.int64)


def make_cotangents(cfg: Workload, N: Optional[int] = None, seed_index: Optional[int] = None):
    """Per-token cotangents: g_logp ~ N(0, 1), g_ent ~ N(0, 0.1), float32."""
    idx = cfg.index if seed_index is None else seed_index
    n = cfg.N if N is None else int(N)
    g_l = _rng(idx, 3).standard_normal(n, dtype=np.float32)
    g_e = (_rng(idx, 4).standard_normal(n, dtype=np.float32) * np.float32(0.1)).astype(np.float32)
    return g_l, g_e


def sample_tokens(targets: np.ndarray, count: int, seed: int = 7, include_masked: int = 0) -> np.ndarray:
    """A fixed, sorted sample of token indices: ``count`` unmasked tokens plus
    up to ``include_masked`` masked ones (target outside [0, V) is masked)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    valid = np.flatnonzero(targets >= 0)
    pick = rng.choice(valid, size=min(count, valid.size), replace=False)
    if include_masked:
        masked = np.flatnonzero(targets < 0)
        if masked.size:
            pick = np.concatenate([pick, rng.choice(masked, size=min(include_masked, masked.size), replace=False)])
    return np.sort(pick).astype(np.int64)
