"""Output RoPE with position -i (oracle; test infrastructure only).

What is computed ("DeepSeek-V4 KV Cache 深度分析", section 五 "RoPE 的特殊处理": RoPE is
applied to the query, to the KV entries' last 64 dims, and to the core attention output
o_{t,i} with position -i; because each entry, used as the value too, carries its
absolute position R(j), rotating the output by R(-i) turns sum_j p_j R(j) e_j into
sum_j p_j R(j - i) e_j, i.e. relative positions).

Readings where the pages are silent: the rotation acts on the 64 RoPE dims (the last 64
of 512) as 32 planar rotations of consecutive pairs (2k, 2k+1), pair k turning by
angle position * theta_k with theta_k = base ** (-2k / 64); the base is a parameter.
Angles and rotations are in fp64.

Pins (tests/test_oracle_rope.py): R(0) is the identity; R(a) R(b) = R(a + b); pair norms
are kept; the pages' relative-position identity R(-i) R(j) = R(j - i); each pair equals
an explicit 2x2 rotation matrix; the no-RoPE dims are untouched.
"""
from __future__ import annotations

import numpy as np

ROPE_DIMS = 64
KV_DIM = 512


def rope_rotate(x, position, base: float) -> np.ndarray:
    """Rotate vectors x[..., 64] by RoPE at `position` (a scalar or broadcastable array)."""
    x = np.asarray(x, dtype=np.float64)
    k = np.arange(ROPE_DIMS // 2, dtype=np.float64)
    theta = np.asarray(base, dtype=np.float64) ** (-2.0 * k / ROPE_DIMS)
    ang = np.asarray(position, dtype=np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def output_rope(o, position, base: float) -> np.ndarray:
    """o[..., 512] attention output of a query at `position` -> R(-position) on its last 64 dims."""
    o = np.array(o, dtype=np.float64, copy=True)
    pos = np.asarray(position, dtype=np.float64)
    o[..., KV_DIM - ROPE_DIMS:] = rope_rotate(o[..., KV_DIM - ROPE_DIMS:], -pos, base)
    return o
