"""GPU parity of the decode-step cache write (kv_cache_write) against the oracle.

Seeded new rows are written into a cache whose bytes start as a seeded pattern; every
byte of the cache afterwards must equal the oracle's (oracle/cachewrite.py): the named
rows encoded by the format's codec, all other rows untouched, nothing written outside
the buffers."""
import numpy as np
import pytest
import torch

import compressed_sparse_kv_csa_amd as ck
import seedgen
from cases import bf16_bits
from gpu_helpers import Guarded
from oracle import cachewrite as CW

pytestmark = pytest.mark.gpu
FMT = {"bf16": ck.KV_BF16, "mixed": ck.KV_FP8_MIXED, "fp4": ck.KV_FP4}
ROW_BYTES = {("bf16", 512): 1024, ("mixed", 512): 576, ("fp4", 512): 256, ("bf16", 128): 256,
             ("fp4", 128): 64}


def _pattern(shape, seed):
    return (seedgen.draws(seed, 9, 0, int(np.prod(shape))).numpy() & 0xFF).astype(np.uint8).reshape(shape)


@pytest.mark.parametrize("fmt,dim", list(ROW_BYTES))
@pytest.mark.parametrize("B,n,n_rows,stride", [(3, 5, 300, 310), (1, 1, 8, 8), (4, 33, 1000, 1000)])
def test_cache_write_parity(fmt, dim, B, n, n_rows, stride):
    print(f"case: kv_cache_write {fmt} dim={dim} B={B} n={n} rows={n_rows} stride={stride}", flush=True)
    x = bf16_bits(seedgen.kv_rows_bf16(41, seedgen.tid(seedgen.TID.KV, 7), (B, n, dim)))
    dst = np.stack([seedgen.distinct_indices(42, seedgen.tid(seedgen.TID.POOL, b), n_rows + 8, n)
                    for b in range(B)]).astype(np.int32)
    dst[0, 0] = -3  # out of range on both sides: written nowhere
    codes0 = _pattern((B, stride, ROW_BYTES[(fmt, dim)]), 43)
    scales0 = _pattern((B, stride, dim // 16), 44) if fmt == "fp4" else None
    ref_c, ref_s = CW.cache_write(fmt, codes0, scales0, x, dst, n_rows)

    codes = Guarded(codes0.shape, torch.uint8)
    codes.t.copy_(torch.from_numpy(codes0))
    scales = None
    if fmt == "fp4":
        scales = Guarded(scales0.shape, torch.uint8)
        scales.t.copy_(torch.from_numpy(scales0))
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    dd = torch.from_numpy(dst).cuda()
    ck.kv_cache_write(FMT[fmt], dim, codes.t, scales.t if scales else None, stride, n_rows, B, n, xd, dd)
    torch.cuda.synchronize()
    assert codes.intact() and (scales is None or scales.intact())
    assert np.array_equal(codes.t.cpu().numpy(), ref_c)
    if fmt == "fp4":
        assert np.array_equal(scales.t.cpu().numpy(), ref_s)


def test_written_rows_feed_decode():
    """Rows written by kv_cache_write are the rows kv_quantize produces: a decode over a
    cache assembled row by row equals the decode over the bulk-encoded cache."""
    print("case: kv_cache_write then hca_decode", flush=True)
    B, rows, hq = 2, 96, 16
    kv16 = seedgen.kv_rows_bf16(45, seedgen.tid(seedgen.TID.KV, 8), (B, rows, 512), "cuda")
    bulk = torch.empty((B, rows, 576), dtype=torch.uint8, device="cuda")
    ck.kv_quantize_fp8(kv16, B * rows, 512, 448, bulk)
    built = torch.zeros_like(bulk)
    order = torch.from_numpy(np.stack([np.random.default_rng(b).permutation(rows) for b in range(B)])
                             .astype(np.int32)).cuda()
    src = torch.stack([kv16[b, order[b].long()] for b in range(B)]).contiguous()
    ck.kv_cache_write(ck.KV_FP8_MIXED, 512, built, None, rows, rows, B, rows, src, order)
    torch.cuda.synchronize()
    assert torch.equal(built, bulk)
    q = seedgen.bf16_normal(46, seedgen.tid(seedgen.TID.Q, 8), (B, hq, 512), "cuda")
    outs = []
    for cache in (bulk, built):
        out = torch.empty((B, hq, 512), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(max(ck.hca_decode_workspace_bytes(B, hq, rows), 256), dtype=torch.uint8, device="cuda")
        ck.hca_decode(B, hq, 512 ** -0.5, ck.cache(ck.KV_FP8_MIXED, cache, rows, rows), q, out, ws)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
