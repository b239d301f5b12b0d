"""GPU codecs against the oracle, bit for bit: every finite bf16 value, hand-worked
ties, seeded rows, and the exact decode of every format; plus the generator's GPU
output against its CPU output."""
import numpy as np
import pytest
import torch

import compressed_sparse_kv_csa_amd as ck
import seedgen
from oracle import formats as OF

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _all_finite_bf16_rows(width):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = OF.bf16_bits_to_f64(bits)
    bits = bits[np.isfinite(vals)]
    pad = (-len(bits)) % width
    return np.concatenate([bits, np.zeros(pad, dtype=np.uint16)]).reshape(-1, width)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def test_fp8_exhaustive_all_bf16():
    print("case: E4M3 encode of every finite bf16 value", flush=True)
    x = _all_finite_bf16_rows(512)
    out = torch.empty((x.shape[0], 512), dtype=torch.uint8, device=DEV)
    ck.kv_quantize_fp8(_dev(x.view(np.int16)), x.shape[0], 512, 512, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), OF.e4m3_encode(OF.bf16_bits_to_f64(x)))


@pytest.mark.parametrize("rows", [1, 7, 1000])
def test_fp8_mixed_rows(rows):
    print(f"case: mixed rows={rows}", flush=True)
    x = seedgen.kv_rows_bf16(31, 5, (rows, 512)).view(torch.int16).numpy().view(np.uint16)
    out = torch.empty((rows, 576), dtype=torch.uint8, device=DEV)
    ck.kv_quantize_fp8(_dev(x.view(np.int16)), rows, 512, 448, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), OF.mixed_quantize(x))


def _fp4_check(bits):
    rows, dim = bits.shape
    codes = torch.empty((rows, dim // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty((rows, dim // 16), dtype=torch.uint8, device=DEV)
    ck.kv_quantize_fp4(_dev(bits.view(np.int16)), rows, dim, codes, scales)
    torch.cuda.synchronize()
    c_ref, s_ref = OF.fp4_quantize(OF.bf16_bits_to_f64(bits))
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    assert np.array_equal(codes.cpu().numpy(), c_ref)


def test_fp4_exhaustive_shuffled_blocks():
    print("case: FP4 blocks over every finite bf16 value (seeded shuffles)", flush=True)
    x = _all_finite_bf16_rows(512).reshape(-1)
    rng = np.random.default_rng(5)
    for _ in range(3):
        _fp4_check(rng.permutation(x).reshape(-1, 512))
    _fp4_check(x.reshape(-1, 512))


def test_fp4_small_magnitude_blocks():
    """Blocks whose scale lands in E4M3's subnormal range or rounds to zero."""
    print("case: FP4 small-magnitude blocks", flush=True)
    rng = np.random.default_rng(6)
    vals = rng.standard_normal((256, 128)) * np.exp2(rng.integers(-20, 0, size=(256, 1)))
    bits = OF.f64_to_bf16_bits(vals.astype(np.float32).astype(np.float64))
    _fp4_check(bits)


def test_fp4_hand_worked_ties():
    print("case: FP4 hand-worked ties", flush=True)
    row = np.array([6, 3, 1.5, -0.75, 0.25, -6, 0, 2, 4, 1, 0.5, -1.5, 5, 3.5, -0.25, 1.75] * 2)
    row2 = np.zeros(32); row2[3] = 6.375; row2[20] = -2688.0; row2[21] = 1.0
    bits = OF.f64_to_bf16_bits(np.stack([row, row2]))
    _fp4_check(bits)


@pytest.mark.parametrize("dim", [128, 512])
def test_fp4_seeded_rows(dim):
    print(f"case: FP4 seeded rows dim={dim}", flush=True)
    x = seedgen.kv_rows_bf16(32, 5, (777, dim)).view(torch.int16).numpy().view(np.uint16)
    _fp4_check(x)


@pytest.mark.parametrize("fmt", ["bf16", "mixed", "fp4"])
def test_dequantize_exact(fmt):
    print(f"case: dequantize {fmt}", flush=True)
    x = seedgen.kv_rows_bf16(33, 5, (300, 512)).view(torch.int16).numpy().view(np.uint16)
    out = torch.empty((300, 512), dtype=torch.int16, device=DEV)
    if fmt == "bf16":
        ck.kv_dequantize(ck.KV_BF16, _dev(x.view(np.int16)), None, 300, 512, out)
        ref = OF.bf16_bits_to_f64(x)
    elif fmt == "mixed":
        rows = OF.mixed_quantize(x)
        ck.kv_dequantize(ck.KV_FP8_MIXED, _dev(rows), None, 300, 512, out)
        ref = OF.mixed_dequantize(rows)
    else:
        c, s = OF.fp4_quantize(OF.bf16_bits_to_f64(x))
        ck.kv_dequantize(ck.KV_FP4, _dev(c), _dev(s), 300, 512, out)
        ref = OF.fp4_dequantize(c, s)
    torch.cuda.synchronize()
    got = OF.bf16_bits_to_f64(out.cpu().numpy().view(np.uint16))
    assert np.array_equal(got, ref)


def test_generator_gpu_matches_cpu():
    print("case: generator GPU vs CPU", flush=True)
    shape = (3, 5000, 128)
    assert torch.equal(seedgen.normal(9, 4, shape, DEV).cpu(), seedgen.normal(9, 4, shape))
    assert torch.equal(seedgen.uniform01(9, 3, (7, 64), DEV).cpu(), seedgen.uniform01(9, 3, (7, 64)))
    assert torch.equal(seedgen.kv_rows_bf16(9, 5, (2, 700, 512), DEV).cpu(),
                       seedgen.kv_rows_bf16(9, 5, (2, 700, 512)))
