"""HCA dense decode on the GPU against the oracle (max-abs 1e-2)."""
import math

import numpy as np
import pytest
import torch

import seedgen
from cases import attention_error, bf16_bits, encode_kv, oracle_hca
from gpu_helpers import run_hca

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,rows,hq,fmt", [
    (1, 128 + 64, 16, "bf16"),
    (2, 128 + 1000, 64, "bf16"),
    (2, 128 + 1000, 64, "mixed"),
    (3, 128 + 777, 32, "fp4"),
    (2, 20, 64, "bf16"),
    (1, 5000, 48, "mixed"),
    (2, 128 + 1000, 128, "mixed"),
    (2, 128 + 700, 128, "fp4"),
    # 2048 rows and more: 64-head workgroups, two blocks at 128 heads, one group of four at 16
    (1, 2500, 128, "fp4"),
    (2, 2100, 16, "bf16"),
])
def test_hca_parity(B, rows, hq, fmt):
    print(f"case: hca B={B} rows={rows} Hq={hq} kv={fmt}", flush=True)
    T = seedgen.TID
    q = bf16_bits(seedgen.bf16_normal(200 + rows, seedgen.tid(T.Q), (B, hq, 512)))
    kv = encode_kv(bf16_bits(seedgen.kv_rows_bf16(200 + rows, seedgen.tid(T.KV), (B, rows, 512))), fmt)
    scale = 1.0 / math.sqrt(512)
    ref = oracle_hca(q, kv, scale)
    out = run_hca(q, kv, scale, stride_pad=5)
    err, ok = attention_error(out, ref)
    print(f"max |out - oracle| = {err:.3e}  max |oracle| = {np.abs(ref).max():.3f}")
    assert ok, err


def test_hca_empty_sequence():
    print("case: hca with no rows", flush=True)
    q = bf16_bits(seedgen.bf16_normal(7, 1, (2, 16, 512)))
    kv = encode_kv(np.zeros((2, 0, 512), dtype=np.uint16), "bf16")
    out = run_hca(q, kv, 0.05)
    assert (out == 0).all()
