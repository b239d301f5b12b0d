"""Decode-step cache writes (oracle; test infrastructure only).

What is computed ("DeepSeek-V4 KV Cache 深度分析", section 二 "KV Cache 结构革命": a new
entry is quantised on its way into the cache, its 448 no-RoPE dims to E4M3 and its 64
RoPE dims kept as bf16; section 十一, the forward-flow diagram: the compressed row is then
written into the KV cache): every new row is encoded by the cache's format and stored
at its destination row of its own sequence.  Nothing else in the cache changes.

Readings: the window is a ring, so a new token's row goes to its ring slot, and a new
compressed entry j to row window + j (the caller names the rows); a destination outside
the sequence's rows writes nothing.

Pins (tests/test_oracle_cachewrite.py): writing every row of an array in order equals
encoding the whole array with the format's codec; rows not named keep their bytes;
out-of-range destinations write nothing; the order of the writes does not matter.
"""
from __future__ import annotations

import numpy as np

from . import formats


def encode_row(fmt: str, row_bits: np.ndarray):
    """One bf16 row (uint16 bits [dim]) -> (code bytes, scale bytes or None) in `fmt`."""
    if fmt == "bf16":
        return np.ascontiguousarray(row_bits).view(np.uint8).copy(), None
    if fmt == "mixed":
        return formats.mixed_quantize(row_bits[None])[0], None
    if fmt == "fp4":
        c, s = formats.fp4_quantize(formats.bf16_bits_to_f64(row_bits)[None])
        return c[0], s[0]
    raise ValueError(fmt)


def cache_write(fmt: str, codes, scales, x_bits, dst, n_rows: int):
    """Copies of (codes [B][stride][bytes], scales [B][stride][dim/16] or None) after
    writing rows x_bits [B][n][dim] (bf16 bits) to rows dst [B][n] of each sequence."""
    codes = np.array(codes, dtype=np.uint8, copy=True)
    scales = None if scales is None else np.array(scales, dtype=np.uint8, copy=True)
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    B, n = x_bits.shape[:2]
    for b in range(B):
        for i in range(n):
            d = int(dst[b][i])
            if d < 0 or d >= n_rows:
                continue
            c, s = encode_row(fmt, x_bits[b, i])
            codes[b, d] = c
            if s is not None:
                scales[b, d] = s
    return codes, scales
