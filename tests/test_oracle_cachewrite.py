"""Pins of the oracle's decode-step cache write (oracle/cachewrite.py)."""
import numpy as np
import pytest

from oracle import cachewrite as CW, formats as F

ROW_BYTES = {("bf16", 512): 1024, ("mixed", 512): 576, ("fp4", 512): 256, ("bf16", 128): 256,
             ("fp4", 128): 64}


def _bits(r, shape):
    return F.f64_to_bf16_bits(r.standard_normal(shape) * 3.0)


def _empty(fmt, dim, B, stride, fill=0xA5):
    codes = np.full((B, stride, ROW_BYTES[(fmt, dim)]), fill, dtype=np.uint8)
    scales = np.full((B, stride, dim // 16), fill, dtype=np.uint8) if fmt == "fp4" else None
    return codes, scales


def _bulk(fmt, bits):
    if fmt == "bf16":
        return np.ascontiguousarray(bits).view(np.uint8).reshape(bits.shape[:-1] + (-1,)), None
    if fmt == "mixed":
        return F.mixed_quantize(bits), None
    return F.fp4_quantize(F.bf16_bits_to_f64(bits))


@pytest.mark.parametrize("fmt,dim", list(ROW_BYTES))
def test_writing_every_row_in_order_is_the_bulk_codec(fmt, dim):
    r = np.random.default_rng(31)
    x = _bits(r, (2, 7, dim))
    codes, scales = _empty(fmt, dim, 2, 7)
    dst = np.tile(np.arange(7), (2, 1))
    got_c, got_s = CW.cache_write(fmt, codes, scales, x, dst, 7)
    ref_c, ref_s = _bulk(fmt, x)
    assert np.array_equal(got_c, ref_c)
    if fmt == "fp4":
        assert np.array_equal(got_s, ref_s)


@pytest.mark.parametrize("fmt,dim", list(ROW_BYTES))
def test_only_named_rows_change_and_order_does_not_matter(fmt, dim):
    r = np.random.default_rng(32)
    B, stride, n_rows, n = 3, 20, 16, 4
    x = _bits(r, (B, n, dim))
    codes, scales = _empty(fmt, dim, B, stride)
    dst = np.array([[3, 15, 0, 9], [16, -1, 7, 2], [5, 6, 1000, 4]])  # 16, -1, 1000: skipped
    c1, s1 = CW.cache_write(fmt, codes, scales, x, dst, n_rows)
    perm = np.array([2, 0, 3, 1])
    c2, s2 = CW.cache_write(fmt, codes, scales, x[:, perm], dst[:, perm], n_rows)
    assert np.array_equal(c1, c2)
    written = np.zeros((B, stride), dtype=bool)
    for b in range(B):
        for i in range(n):
            d = dst[b, i]
            if 0 <= d < n_rows:
                written[b, d] = True
                ref_c, ref_s = _bulk(fmt, x[b, i][None])
                assert np.array_equal(c1[b, d], ref_c[0])
                if fmt == "fp4":
                    assert np.array_equal(s1[b, d], ref_s[0])
    assert (c1[~written] == 0xA5).all()
    if fmt == "fp4":
        assert (s1[~written] == 0xA5).all()
    assert written.sum() == 9
