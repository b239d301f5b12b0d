"""Storage formats of the compressed KV caches (oracle; test infrastructure only).

Sources
* Mixed shared-KV entry: 448 "nope" dims in FP8 plus 64 RoPE dims in BF16,
  576 bytes per entry ("DeepSeek-V4 KV Cache 深度分析", section 二 "KV Cache 结构革命",
  the entry-layout figure and the model.py write path; section 六 "精度配置",
  the S_kv table).  The FP8 cast is read as an unscaled OCP E4M3FN cast: the
  page's byte count (576) leaves no room for scale bytes.
* FP4 main KV: E2M1 values with one E4M3 scale per 16 channels and no global
  scale ("DeepSeek, KV 캐시를 토큰당 890바이트로 줄인 V4.1-Flash 공개", section
  핵심 내용; "KV cache 890 bajtów na token", section "Trzy mechanizmy zamiast
  jednej sztuczki").  The same block format stores FP4 indexer keys.
* Code points: OCP 8-bit floating point specification (E4M3FN: bias 7, no
  infinities, S.1111.111 is NaN, largest finite 448) and the OCP
  Microscaling specification (E2M1: bias 1, values 0, .5, 1, 1.5, 2, 3, 4, 6).

Rounding readings (the pages fix none of them)
* Encoding is round-to-nearest on the finite grid, ties to the even code, so
  magnitudes above the largest finite value saturate to it.  The sign is kept
  (a negative input that rounds to zero gives the negative-zero code).
* FP4 block: scale code = E4M3FN(amax / 6); if that scale decodes to 0 every
  code is 0; otherwise code_i = E2M1(x_i / scale).

Parity pins (tests/test_oracle_formats.py): exhaustive round trips over all
codes; brute-force nearest-value search over all 65,536 bf16 inputs; the FP4
format maximum 6 x 448 = 2688 printed on the V4.1-Flash page; the per-element
error bound |x - x_hat| <= scale.  The Hadamard rotation: bit-for-bit equal to the
dense Sylvester-matrix product (scipy) rounded the same way, exact rational
arithmetic on sample rows, a correctly rounded scale constant, norm preservation
and the involution property.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0
FP4_BLOCK = 16


# ---------------------------------------------------------------- E4M3FN

def e4m3_value(code) -> np.ndarray:
    """Real value of each E4M3FN code (NaN for the two NaN codes)."""
    c = np.asarray(code, dtype=np.int64) & 0xFF
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64)))
    mag = np.where((e == 0xF) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


# Finite non-negative grid: codes 0x00 .. 0x7E in increasing order of value.
_E4M3_CODES = np.arange(0x7F, dtype=np.int64)
_E4M3_GRID = e4m3_value(_E4M3_CODES)


def _nearest_even(mag: np.ndarray, grid: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """Index (code) of the grid point nearest to each |x|; ties go to the even code.

    ``grid`` is strictly increasing and starts at 0; inputs beyond its last point
    map to the last point.
    """
    hi = np.searchsorted(grid, mag, side="left")          # grid[hi-1] < mag <= grid[hi]
    hi = np.clip(hi, 1, len(grid) - 1)
    lo = hi - 1
    d_lo = mag - grid[lo]
    d_hi = grid[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(mag >= grid[-1], len(grid) - 1, idx)
    idx = np.where(mag <= 0.0, 0, idx)
    return codes[idx]


def e4m3_encode(x) -> np.ndarray:
    """E4M3FN code of each real x: nearest finite value, ties to even, saturating."""
    x = np.asarray(x, dtype=np.float64)
    code = _nearest_even(np.abs(x), _E4M3_GRID, _E4M3_CODES)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


# ---------------------------------------------------------------- E2M1

def e2m1_value(code) -> np.ndarray:
    """Real value of each E2M1 code (low 4 bits used)."""
    c = np.asarray(code, dtype=np.int64) & 0xF
    sign = np.where(c >> 3, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    mag = np.where(e == 0, m * 0.5, np.ldexp(1.0 + m / 2.0, (e - 1).astype(np.int64)))
    return sign * mag


_E2M1_CODES = np.arange(8, dtype=np.int64)
_E2M1_GRID = e2m1_value(_E2M1_CODES)


def e2m1_encode(x) -> np.ndarray:
    """E2M1 code of each real x: nearest value, ties to even, saturating at 6."""
    x = np.asarray(x, dtype=np.float64)
    code = _nearest_even(np.abs(x), _E2M1_GRID, _E2M1_CODES)
    return (code | np.where(np.signbit(x), 0x8, 0)).astype(np.uint8)


# ---------------------------------------------------------------- bf16

def bf16_bits_to_f64(bits) -> np.ndarray:
    """Value of bf16 bit patterns (uint16) as float64 (exact)."""
    b = np.asarray(bits).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """bf16 bit pattern of each value, round to nearest even.  Values are assumed finite.

    The value is first rounded to fp32 (exact for every input this project feeds
    it: bf16 values and their exact halves); the 16 dropped bits then decide the
    rounding.
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    low = u & 0xFFFF
    up = u >> 16
    rnd = (low > 0x8000) | ((low == 0x8000) & ((up & 1) == 1))
    return (up + rnd.astype(np.uint64)).astype(np.uint16)


# ---------------------------------------------------------------- FP4 block format

def fp4_quantize(x) -> tuple[np.ndarray, np.ndarray]:
    """FP4 block quantisation of rows ``x[..., dim]`` (dim % 16 == 0).

    Returns ``codes[..., dim/2]`` (element 2i in the low nibble of byte i) and
    ``scales[..., dim/16]`` (E4M3FN codes).
    """
    x = np.asarray(x, dtype=np.float64)
    dim = x.shape[-1]
    assert dim % FP4_BLOCK == 0
    blocks = x.reshape(*x.shape[:-1], dim // FP4_BLOCK, FP4_BLOCK)
    blocks = blocks.astype(np.float32).astype(np.float64)  # the codec's inputs are fp32 values
    amax = np.abs(blocks).max(axis=-1).astype(np.float32)
    # Both divisions are single correctly rounded fp32 divisions; the quotient is then
    # rounded to the E4M3 / E2M1 grid.
    scale_code = e4m3_encode((amax / np.float32(E2M1_MAX)).astype(np.float64))
    scale = e4m3_value(scale_code)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (blocks.astype(np.float32) / scale[..., None].astype(np.float32)).astype(np.float64)
    nib = e2m1_encode(ratio)
    nib = np.where((scale == 0.0)[..., None], 0, nib).astype(np.uint8)
    nib = nib.reshape(*x.shape[:-1], dim)
    codes = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    return codes, scale_code.astype(np.uint8)


def fp4_dequantize(codes, scales) -> np.ndarray:
    """Values of FP4 block rows: e2m1(code) * e4m3(scale of its 16-channel block)."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    dim = codes.shape[-1] * 2
    nib = np.empty(codes.shape[:-1] + (dim,), dtype=np.uint8)
    nib[..., 0::2] = codes & 0xF
    nib[..., 1::2] = codes >> 4
    v = e2m1_value(nib)
    s = np.repeat(e4m3_value(scales), FP4_BLOCK, axis=-1)
    return v * s


# ---------------------------------------------------------------- Hadamard-rotated FP4

HADAMARD_DIM = 128
# fp32(1 / sqrt(128)): the nearest fp32 value (pinned in tests/test_oracle_formats.py)
HADAMARD_SCALE_F32 = np.float32(1.0 / np.sqrt(HADAMARD_DIM))
# Largest spread, in binades, between the largest and the smallest nonzero magnitude of a
# bf16 row for which every partial sum of H x is exact in fp64: the terms are multiples of
# 2**(e_min - 7) and every sum stays below 128 * 2**(e_max + 1), so 38 + 7 + 1 + 7 = 53 bits.
HADAMARD_EXACT_SPAN = 38


def hadamard128_exact(x) -> np.ndarray:
    """H x for bf16 rows x[..., 128], H the 128 x 128 Sylvester Hadamard matrix, exactly.

    The fast Walsh-Hadamard transform in fp64: for h = 1, 2, ..., 64 every pair (i, i + h)
    with bit h of i clear becomes (y[i] + y[i+h], y[i] - y[i+h]).  Each row must hold bf16
    values whose nonzero magnitudes span at most HADAMARD_EXACT_SPAN binades; every sum is
    then exact (so any evaluation order gives the same result), and a row outside that range
    raises ValueError.
    """
    x = np.asarray(x, dtype=np.float64)
    assert x.shape[-1] == HADAMARD_DIM
    if not np.array_equal(bf16_bits_to_f64(f64_to_bf16_bits(x)), x):
        raise ValueError("hadamard128_exact takes bf16 values")
    a = np.abs(x)
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    e_max = np.where(a > 0, e, np.iinfo(np.int64).min).max(axis=-1)
    e_min = np.where(a > 0, e, np.iinfo(np.int64).max).min(axis=-1)
    span = np.where(e_max >= e_min, e_max - e_min, 0)
    if (span > HADAMARD_EXACT_SPAN).any():
        raise ValueError("a row spans more binades than H x can hold exactly in fp64")
    y = x.copy()
    lead = y.shape[:-1]
    h = 1
    while h < HADAMARD_DIM:
        v = y.reshape(*lead, HADAMARD_DIM // (2 * h), 2, h)
        lo, hi = v[..., 0, :], v[..., 1, :]
        y = np.stack([lo + hi, lo - hi], axis=-2).reshape(*lead, HADAMARD_DIM)
        h *= 2
    return y


def hadamard128_f32(x) -> np.ndarray:
    """bf16 rows x[..., 128] -> the fp32 values of their rotation H x / sqrt(128)
    ("DeepSeek-V4 KV Cache 深度分析", section 四, 结构: the indexer rotates its 128-wide vectors
    with a Hadamard transform before FP4 quantisation).

    The page names the rotation but not its arithmetic; the plain reading taken here is the
    product H x computed exactly (hadamard128_exact), rounded once to fp32 (nearest even),
    then one fp32 multiplication by fp32(1/sqrt(128)) (nearest even).
    """
    return hadamard128_exact(x).astype(np.float32) * HADAMARD_SCALE_F32


def fp4h_quantize(x_bf16_bits) -> tuple[np.ndarray, np.ndarray]:
    """bf16 rows [..., 128] -> FP4 block codes and scales of their Hadamard rotation."""
    rot = hadamard128_f32(bf16_bits_to_f64(x_bf16_bits))
    return fp4_quantize(rot.astype(np.float64))


# ---------------------------------------------------------------- mixed FP8 / BF16 row

NOPE_DIM = 448
ROPE_DIM = 64
MIXED_ROW_BYTES = NOPE_DIM + 2 * ROPE_DIM   # 576


def mixed_quantize(x_bf16_bits, nope_dim: int = NOPE_DIM) -> np.ndarray:
    """Mixed rows: E4M3FN(x[:nope]) then the bf16 bytes (little-endian) of x[nope:]."""
    bits = np.asarray(x_bf16_bits, dtype=np.uint16)
    vals = bf16_bits_to_f64(bits[..., :nope_dim])
    head = e4m3_encode(vals)
    tail = np.ascontiguousarray(bits[..., nope_dim:]).view(np.uint8)
    return np.concatenate([head, tail], axis=-1)


def mixed_dequantize(rows, dim: int = 512, nope_dim: int = NOPE_DIM) -> np.ndarray:
    rows = np.asarray(rows, dtype=np.uint8)
    head = e4m3_value(rows[..., :nope_dim])
    tail_bits = np.ascontiguousarray(rows[..., nope_dim:]).view(np.uint16)
    return np.concatenate([head, bf16_bits_to_f64(tail_bits)], axis=-1)
