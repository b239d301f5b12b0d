"""Seeded, counter-based synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module holds no arithmetic of the decode method itself: it only turns
(seed, tensor id, element index) into numbers of the shapes and value ranges the
compressed-KV decode consumes.  Every value is a pure function of its counter, so
the same tensor comes out identically on the CPU and on a GPU, in any chunking.

Integer source: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014; output mix constants as published in Vigna's
splitmix64.c).  The stream of tensor ``tid`` under ``seed`` has initial state
``K = mix64((seed << 32) | tid)``; its r-th draw is ``mix64(K + (r + 1) * GAMMA)``,
i.e. exactly the r-th output of a SplitMix64 generator started at ``K``.

Value shapes:
* ``normal``: Irwin-Hall(12) from the twelve 16-bit lanes of three draws,
  ``z = sum(u) / 2**16 - 6``: mean 0, variance 1, |z| <= 6, exact in fp32.
* ``kv rows``: ``z * g_c`` with ``g_c = 3.75`` on channels ``c % 64 == 7`` and 1
  elsewhere, rounded to bf16.  The largest |value| is 22.5, matching the
  RMSNorm'd maximum of about 22.6 that the V4.1-Flash report summary gives for
  the cached values (ailog.hnlab.kr page, FP4 KV paragraph).
* ``uniform01``: the top 24 bits of one draw divided by 2**24, exact in fp32.
"""
from __future__ import annotations

import torch

__all__ = [
    "draws",
    "normal",
    "uniform01",
    "bf16_normal",
    "kv_rows_bf16",
    "TID",
    "tid",
]

_MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB


def _s64(x: int) -> int:
    """Two's-complement int64 value of a 64-bit pattern."""
    x &= _MASK64
    return x - (1 << 64) if x >= (1 << 63) else x


def _lsr(z: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 bit patterns."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def _mix64_t(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _lsr(z, 30)) * _s64(_M1)
    z = (z ^ _lsr(z, 27)) * _s64(_M2)
    return z ^ _lsr(z, 31)


def _mix64_int(z: int) -> int:
    z &= _MASK64
    z = ((z ^ (z >> 30)) * _M1) & _MASK64
    z = ((z ^ (z >> 27)) * _M2) & _MASK64
    return z ^ (z >> 31)


def _key(seed: int, tensor_id: int) -> int:
    return _mix64_int(((seed & 0xFFFFFFFF) << 32) | (tensor_id & 0xFFFFFFFF))


def draws(seed: int, tensor_id: int, start: int, count: int, device="cpu") -> torch.Tensor:
    """64-bit draws r = start .. start+count-1 of stream (seed, tensor_id), as int64 patterns."""
    k = _key(seed, tensor_id)
    r = torch.arange(start + 1, start + count + 1, dtype=torch.int64, device=device)
    z = r * _s64(GAMMA) + _s64(k)
    return _mix64_t(z)


_CHUNK = 1 << 22


def _numel(shape) -> int:
    n = 1
    for s in shape:
        n *= int(s)
    return n


def normal(seed: int, tensor_id: int, shape, device="cpu") -> torch.Tensor:
    """Irwin-Hall(12) values, exact in fp32, element i using draws 3i, 3i+1, 3i+2."""
    n = _numel(shape)
    out = torch.empty(n, dtype=torch.float32, device=device)
    for s0 in range(0, n, _CHUNK):
        c = min(_CHUNK, n - s0)
        d = draws(seed, tensor_id, 3 * s0, 3 * c, device).view(c, 3)
        acc = torch.zeros(c, dtype=torch.int64, device=device)
        for j in range(3):
            x = d[:, j]
            for q in range(4):
                acc += (x >> (16 * q)) & 0xFFFF
        out[s0:s0 + c] = acc.to(torch.float32) * (1.0 / 65536.0) - 6.0
    return out.view(*shape)


def uniform01(seed: int, tensor_id: int, shape, device="cpu") -> torch.Tensor:
    """U[0,1) values k / 2**24, exact in fp32, element i using draw i."""
    n = _numel(shape)
    out = torch.empty(n, dtype=torch.float32, device=device)
    for s0 in range(0, n, _CHUNK):
        c = min(_CHUNK, n - s0)
        d = draws(seed, tensor_id, s0, c, device)
        out[s0:s0 + c] = _lsr(d, 40).to(torch.float32) * (1.0 / 16777216.0)
    return out.view(*shape)


def bf16_normal(seed: int, tensor_id: int, shape, device="cpu") -> torch.Tensor:
    """Irwin-Hall(12) values rounded to bf16 (round to nearest even)."""
    return normal(seed, tensor_id, shape, device).to(torch.bfloat16)


def kv_rows_bf16(seed: int, tensor_id: int, shape, device="cpu") -> torch.Tensor:
    """Shared-KV rows: Irwin-Hall(12) with gain 3.75 on channels c % 64 == 7, as bf16.

    ``shape[-1]`` is the row width (512 for main KV rows).  The gain keeps the
    largest magnitude at 22.5 so that the value range resembles RMSNorm'd
    activations with a few outlier channels.
    """
    z = normal(seed, tensor_id, shape, device)
    d = int(shape[-1])
    gain = torch.ones(d, dtype=torch.float32, device=device)
    gain[7::64] = 3.75
    return (z * gain).to(torch.bfloat16)


def distinct_indices(seed: int, tensor_id: int, n: int, m: int) -> "np.ndarray":
    """m distinct indices in [0, n), in a seeded random order: the first m of the stable
    argsort of draws 0 .. n-1 (a seeded permutation of range(n))."""
    import numpy as np
    d = draws(seed, tensor_id, 0, n).numpy()
    return np.argsort(d, kind="stable")[:m].astype(np.int64)


class TID:
    """Tensor-id roles; the id of a tensor is ``role * 256 + layer``."""

    Q = 1          # attention queries [B][Hq][512]
    Q_IDX = 2      # indexer queries [B][H_I][128]
    W_IDX = 3      # indexer head weights [B][H_I]
    IDX_KEYS = 4   # indexer keys [B][N_c][128]
    KV = 5         # shared-KV rows [B][W + N_c][512]
    POOL = 6       # candidate pools [B][n_pool] (one stream per query: layer = query)


def tid(role: int, layer: int = 0) -> int:
    return role * 256 + layer
