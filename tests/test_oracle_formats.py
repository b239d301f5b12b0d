"""Pins of the oracle's storage formats: OCP code points, exhaustive brute force, an
independent library cast, hand-worked blocks, and the FP4 maximum the pages print."""
import numpy as np
import pytest
import torch

from oracle import formats as F


def _all_bf16_finite():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = F.bf16_bits_to_f64(bits)
    keep = np.isfinite(vals)
    return bits[keep], vals[keep]


# ------------------------------------------------------------------ E4M3FN

def test_e4m3_code_points():
    assert F.e4m3_value(0x7E) == 448.0                  # largest finite
    assert F.e4m3_value(0x08) == 2.0 ** -6              # smallest normal
    assert F.e4m3_value(0x01) == 2.0 ** -9              # smallest subnormal
    assert F.e4m3_value(0x38) == 1.0                    # exponent field 7 = bias
    assert F.e4m3_value(0xB8) == -1.0
    assert np.isnan(F.e4m3_value(0x7F)) and np.isnan(F.e4m3_value(0xFF))
    v = F.e4m3_value(np.arange(256))
    assert np.isfinite(v).sum() == 254
    pos = F.e4m3_value(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)


def test_e4m3_matches_torch_cast_in_range():
    """torch's float8_e4m3fn cast (RNE) is an independent routine; it agrees wherever it
    does not overflow to NaN (|x| <= 464)."""
    bits, vals = _all_bf16_finite()
    keep = np.abs(vals) <= 464.0
    ours = F.e4m3_encode(vals[keep])
    ref = torch.from_numpy(vals[keep].astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_brute_force_all_bf16():
    """Every finite bf16 input up to 2**20: the code is the nearest finite value, ties to the
    even code, found by scanning all 254 finite codes (distances are exact in fp64 there).
    Larger inputs saturate to +-448."""
    bits, vals = _all_bf16_finite()
    big = np.abs(vals) > 2.0 ** 20
    assert np.all(F.e4m3_encode(vals[big]) == np.where(np.signbit(vals[big]), 0xFE, 0x7E))
    vals = vals[~big]
    codes = np.arange(256)
    cv = F.e4m3_value(codes)
    fin = np.isfinite(cv)
    ours = F.e4m3_encode(vals)
    # scan: distance to every finite code with the same sign bit as x
    for lo in range(0, len(vals), 8192):
        x = vals[lo:lo + 8192]
        neg = np.signbit(x)
        cand = np.where(fin[None, :] & ((codes[None, :] >= 0x80) == neg[:, None]), np.abs(x[:, None] - cv[None, :]), np.inf)
        best = cand.min(axis=1, keepdims=True)
        tie = cand == best
        even = tie & (codes[None, :] % 2 == 0)
        pick = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(tie, axis=1))
        assert np.array_equal(ours[lo:lo + 8192], pick.astype(np.uint8))


def test_e4m3_round_trip_and_saturation():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    assert np.array_equal(F.e4m3_encode(F.e4m3_value(codes)), codes.astype(np.uint8))
    assert F.e4m3_encode(1e6) == 0x7E and F.e4m3_encode(-1e6) == 0xFE
    assert F.e4m3_encode(-0.0) == 0x80 and F.e4m3_encode(-1e-9) == 0x80


# ------------------------------------------------------------------ E2M1

def test_e2m1_code_points():
    assert list(F.e2m1_value(np.arange(8))) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(F.e2m1_value(np.arange(8, 16))) == [-0.0, -0.5, -1, -1.5, -2, -3, -4, -6]


def test_e2m1_ties_to_even_and_saturation():
    x = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 100.0, 0.26, 4.9])
    want = np.array([0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 6.0, 0.5, 4.0])
    assert np.array_equal(F.e2m1_value(F.e2m1_encode(x)), want)
    assert np.array_equal(F.e2m1_value(F.e2m1_encode(-x)), -want)
    assert F.e2m1_encode(-0.0) == 0x8


# ------------------------------------------------------------------ FP4 block

def test_fp4_format_maximum_2688():
    """Largest FP4 block value: E2M1 6 times E4M3 448 = 2688 (V4.1-Flash news page, section 핵심 내용)."""
    codes = np.full((1, 8), 0x77, dtype=np.uint8)
    scales = np.full((1, 1), 0x7E, dtype=np.uint8)
    assert F.fp4_dequantize(codes, scales).max() == 2688.0
    x = np.full((1, 16), 2688.0)
    c, s = F.fp4_quantize(x)
    assert s[0, 0] == 0x7E and np.all(c == 0x77)


def test_fp4_hand_worked_block():
    # amax 6 -> scale E4M3(1.0) = 0x38; values on the E2M1 grid, two ties to even.
    x = np.array([[6, 3, 1.5, -0.75, 0.25, -6, 0, 2, 4, 1, 0.5, -1.5, 5, 3.5, -0.25, 1.75]], dtype=np.float64)
    c, s = F.fp4_quantize(x)
    assert s.tolist() == [[0x38]]
    nib = [int(b) & 0xF for b in c[0] for _ in (0,)] + []
    nibs = []
    for b in c[0]:
        nibs += [int(b) & 0xF, int(b) >> 4]
    #         6    3    1.5  -1(t) 0(t) -6   0    2    4    1    .5  -1.5  4(t) 4(t) -0   2(t)
    assert nibs == [0x7, 0x5, 0x3, 0xA, 0x0, 0xF, 0x0, 0x4, 0x6, 0x2, 0x1, 0xB, 0x6, 0x6, 0x8, 0x4]


def test_fp4_scale_rounding_and_zero_block():
    # amax 6.375 -> 6.375/6 = 1.0625 is a tie between 1.0 and 1.125 -> even code 0x38 (1.0);
    # the element 6.375 then saturates to 6.
    x = np.zeros((1, 16)); x[0, 3] = 6.375
    c, s = F.fp4_quantize(x)
    assert s[0, 0] == 0x38 and F.fp4_dequantize(c, s)[0, 3] == 6.0
    z = np.zeros((2, 32))
    c, s = F.fp4_quantize(z)
    assert np.all(c == 0) and np.all(s == 0)
    tiny = np.full((1, 16), 1e-6)                      # amax/6 below half the smallest subnormal
    c, s = F.fp4_quantize(tiny)
    assert np.all(s == 0) and np.all(c == 0)


def test_fp4_round_trip_idempotent():
    rng = np.random.default_rng(0)
    nib = rng.integers(0, 16, size=(64, 128))
    nib[:, ::16] = 0x7                                  # every block holds a +6, so amax/6 = scale
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales = rng.integers(0x08, 0x7F, size=(64, 8)).astype(np.uint8)
    scales[scales == 0x7F] = 0x7E
    v = F.fp4_dequantize(codes, scales)
    c2, s2 = F.fp4_quantize(v)
    assert np.array_equal(s2, scales)
    assert np.array_equal(F.fp4_dequantize(c2, s2), v)


def test_fp4_error_bound_on_seeded_rows():
    import seedgen
    x = seedgen.kv_rows_bf16(11, 5, (256, 512)).float().numpy().astype(np.float64)
    c, s = F.fp4_quantize(x)
    xh = F.fp4_dequantize(c, s)
    sc = np.repeat(F.e4m3_value(s), 16, axis=-1)
    assert np.all(np.abs(x - xh) <= sc)
    assert np.abs(x).max() <= 22.5                       # far from the 2688 ceiling: no saturation


# ------------------------------------------------------------------ mixed row

def test_mixed_row_layout():
    import seedgen
    x = seedgen.kv_rows_bf16(3, 5, (8, 512))
    bits = x.view(torch.int16).numpy().view(np.uint16)
    rows = F.mixed_quantize(bits)
    assert rows.shape == (8, 576)
    assert np.array_equal(rows[:, 448:].view(np.uint16), bits[:, 448:])
    ref = x[:, :448].float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(rows[:, :448], ref)
    back = F.mixed_dequantize(rows)
    assert np.array_equal(back[:, 448:], x[:, 448:].double().numpy())
    assert np.array_equal(back[:, :448], torch.from_numpy(ref).view(torch.float8_e4m3fn).double().numpy())


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    f = rng.standard_normal(100000).astype(np.float32) * np.float32(3.0)
    ours = F.f64_to_bf16_bits(f.astype(np.float64))
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# ------------------------------------------------------------------ Hadamard-rotated FP4

def _bf16_rows(rng, n, spread=1.0):
    """n random bf16 rows of 128 values, magnitudes spread over about `spread` decades."""
    x = rng.standard_normal((n, 128)) * 10.0 ** rng.uniform(-spread, spread, size=(n, 128))
    return F.bf16_bits_to_f64(F.f64_to_bf16_bits(x))


def test_hadamard_equals_the_sylvester_matrix_product_rounded_once():
    """The rotation is scipy's dense Sylvester matrix times x (exact in fp64 for these
    rows, whatever BLAS's summation order), rounded once to fp32, times fp32(1/sqrt(128))."""
    import scipy.linalg
    rng = np.random.default_rng(51)
    H = scipy.linalg.hadamard(128).astype(np.float64)
    for spread in (0.0, 1.0, 2.0, 2.5):
        x = _bf16_rows(rng, 64, spread)
        want = (x @ H.T).astype(np.float32) * np.float32(1.0 / np.sqrt(128))
        assert np.array_equal(F.hadamard128_f32(x).view(np.uint32), want.view(np.uint32))
    ints = rng.integers(-8, 9, size=(20, 128)).astype(np.float64)
    assert np.array_equal(F.hadamard128_exact(ints), ints @ H.T)


def test_hadamard_exact_product_matches_rational_arithmetic():
    """H x of sample rows summed in exact rationals: the fp64 transform loses nothing."""
    from fractions import Fraction
    import scipy.linalg
    rng = np.random.default_rng(55)
    H = scipy.linalg.hadamard(128)
    x = _bf16_rows(rng, 4, 2.0)
    x[0, :3] = [2.0 ** 20, 2.0 ** -17, -(2.0 ** -17)]   # a row near the exactness limit
    got = F.hadamard128_exact(x)
    for r in range(x.shape[0]):
        fx = [Fraction(float(v)) for v in x[r]]
        for i in (0, 1, 63, 64, 127):
            exact = sum((fx[j] if H[i, j] > 0 else -fx[j]) for j in range(128))
            assert Fraction(float(got[r, i])) == exact


def test_hadamard_scale_constant_is_correctly_rounded():
    """fp32(1/sqrt(128)) is the fp32 value nearest 1/sqrt(128): its half-ulp neighbours
    bracket 1/sqrt(128), checked by squaring in exact rationals."""
    from fractions import Fraction
    f = Fraction(float(F.HADAMARD_SCALE_F32))
    half_ulp = Fraction(1, 2 ** 28)          # values in [2^-4, 2^-3) have ulp 2^-27
    assert (f - half_ulp) ** 2 * 128 < 1 < (f + half_ulp) ** 2 * 128


def test_hadamard_rejects_rows_beyond_the_exact_range():
    x = np.zeros((1, 128))
    x[0, 0], x[0, 1] = 2.0 ** 30, 2.0 ** -10    # 40 binades apart
    with pytest.raises(ValueError):
        F.hadamard128_exact(x)
    x[0, 1] = 2.0 ** -8                          # 38 binades: still exact
    assert F.hadamard128_exact(x)[0, 0] == 2.0 ** 30 + 2.0 ** -8


def test_hadamard_fp32_butterfly_is_not_the_rotation():
    """An fp32 fast transform (one rounding per add) differs from the rotation on some of
    these rows: the pins above tell the two apart."""
    rng = np.random.default_rng(56)
    x = _bf16_rows(rng, 200, 2.0)
    y = x.astype(np.float32)
    h = 1
    while h < 128:
        v = y.reshape(200, 128 // (2 * h), 2, h)
        y = np.stack([v[..., 0, :] + v[..., 1, :], v[..., 0, :] - v[..., 1, :]], axis=-2).reshape(200, 128)
        h *= 2
    butterfly = y * np.float32(1.0 / np.sqrt(128))
    assert (butterfly != F.hadamard128_f32(x)).any()


def test_hadamard_is_orthonormal_and_an_involution():
    rng = np.random.default_rng(52)
    x = _bf16_rows(rng, 50)
    y = F.hadamard128_f32(x).astype(np.float64)
    assert np.allclose((y * y).sum(1), (x * x).sum(1), rtol=1e-5)                      # norms kept
    back = F.hadamard128_exact(F.bf16_bits_to_f64(F.f64_to_bf16_bits(y))) / np.sqrt(128)
    assert np.allclose(back, x, atol=1e-2 * np.abs(x).max())                          # R(R(x)) ~ x
    e = np.zeros((1, 128)); e[0, 37] = 1.0
    col = F.hadamard128_f32(e)[0] * np.sqrt(128)
    assert set(np.round(col).tolist()) == {-1.0, 1.0} and np.round(col[0]) == 1.0


def test_hadamard_is_within_the_two_roundings_of_the_exact_rotation():
    import scipy.linalg
    rng = np.random.default_rng(53)
    x = _bf16_rows(rng, 40, 1.0)
    exact = x @ scipy.linalg.hadamard(128).T / np.sqrt(128)
    bound = 2.0 ** -23 * np.abs(exact) + 2.0 ** -149
    assert (np.abs(F.hadamard128_f32(x) - exact) <= 1.5 * bound).all()


def test_fp4h_is_the_fp4_codec_of_the_rotation():
    rng = np.random.default_rng(54)
    bits = F.f64_to_bf16_bits(rng.standard_normal((30, 128)))
    c, s = F.fp4h_quantize(bits)
    c2, s2 = F.fp4_quantize(F.hadamard128_f32(F.bf16_bits_to_f64(bits)).astype(np.float64))
    assert np.array_equal(c, c2) and np.array_equal(s, s2)
    # halving the source halves the rotation exactly: same codes, scale one binade lower
    half = F.f64_to_bf16_bits(F.bf16_bits_to_f64(bits) / 2)
    ch, sh = F.fp4h_quantize(half)
    assert np.array_equal(F.fp4_dequantize(ch, sh) * 2, F.fp4_dequantize(c, s))
