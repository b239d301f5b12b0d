"""GPU parity of the Hadamard-rotated FP4 indexer (CSAKV_IDX_FP4_HADAMARD) against the oracle.

Keys are written by idx_quantize_fp4_hadamard and must match the oracle's fp4h_quantize
byte for byte.  The indexer then rotates and FP4-quantises each query row itself; the
oracle scores with the same rotated, FP4-decoded queries (formats.fp4h_quantize), and the
keys are made tie-free for those queries, so the top-k sets must be identical."""
import numpy as np
import pytest
import torch

import compressed_sparse_kv_csa_amd as ck
import seedgen
from cases import DI, bf16_bits, topk_sets_equal
from gpu_helpers import Guarded, to_dev, workspace
from oracle import decode as OD, formats as F, tiefree

pytestmark = pytest.mark.gpu
T = seedgen.TID


def _fp4h_values(bits):
    return F.fp4_dequantize(*F.fp4h_quantize(bits))


def test_fp4h_codec_bytes():
    print("case: idx_quantize_fp4_hadamard bytes", flush=True)
    x = bf16_bits(seedgen.bf16_normal(61, seedgen.tid(T.IDX_KEYS, 3), (3000, DI)))
    x[0] = 0                                                     # zero row
    x[1] = F.f64_to_bf16_bits(np.where(np.arange(DI) == 5, 3.0e4, 0.0))   # one large entry
    x[2] = F.f64_to_bf16_bits(np.full(DI, 1e-3))                  # constant row
    x[3] = F.f64_to_bf16_bits(np.linspace(-300, 300, DI))
    ref_c, ref_s = F.fp4h_quantize(x)
    codes = Guarded((3000, 64), torch.uint8)
    scales = Guarded((3000, 8), torch.uint8)
    ck.idx_quantize_fp4_hadamard(to_dev(x.view(np.int16)), 3000, codes.t, scales.t)
    torch.cuda.synchronize()
    assert codes.intact() and scales.intact()
    assert np.array_equal(codes.t.cpu().numpy(), ref_c)
    assert np.array_equal(scales.t.cpu().numpy(), ref_s)


def make_case(seed, B, n_c, hi, top_k, layer=0, pool=None):
    keys = bf16_bits(seedgen.bf16_normal(seed, seedgen.tid(T.IDX_KEYS, layer), (B, n_c, DI)))
    qb = bf16_bits(seedgen.bf16_normal(seed, seedgen.tid(T.Q_IDX, layer), (B, hi, DI)))
    w = seedgen.uniform01(seed, seedgen.tid(T.W_IDX, layer), (B, hi)).numpy()
    qh = _fp4h_values(qb)                                          # the queries as scored
    wv = w.astype(np.float64)
    if pool is None:
        keys, _ = tiefree.make_tie_free(keys, qh, wv, top_k, "fp4h")
    else:
        for b in range(B):
            rows = np.unique(pool[b][(pool[b] >= 0) & (pool[b] < n_c)])
            adj, _ = tiefree.make_tie_free(keys[b][rows][None], qh[b][None], wv[b][None],
                                           min(top_k, len(rows)), "fp4h")
            keys[b][rows] = adj[0]
    codes, scales = F.fp4h_quantize(keys)
    kvals = F.fp4_dequantize(codes, scales)
    return dict(codes=codes, scales=scales, kvals=kvals, keys=keys, qb=qb, qh=qh, w=w, wv=wv)


def _cache(c, n_c):
    codes, scales = to_dev(c["codes"]), to_dev(c["scales"])
    return ck.cache(ck.IDX_FP4_HADAMARD, codes, n_c, n_c, scales), (codes, scales)


@pytest.mark.parametrize("seed,B,n_c,hi,k", [(62, 2, 5000, 64, 512), (63, 3, 9000, 40, 100),
                                              (64, 1, 4096 * 3 + 77, 16, 1024),
                                              (66, 2, 5000, 128, 2048)])
def test_fp4h_select_parity(seed, B, n_c, hi, k):
    print(f"case: fp4h select seed={seed} B={B} N_c={n_c} H_I={hi} k={k}", flush=True)
    c = make_case(seed, B, n_c, hi, k)
    expect = np.stack([OD.topk_indices(OD.indexer_scores(c["qh"][b], c["wv"][b], c["kvals"][b]), k)
                       for b in range(B)])
    idx, keep = _cache(c, n_c)
    p = ck.CsaParams(B, 64, hi, k, 128, ck.MODE_FULL, 1.0, 0)
    tk = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    ck.csa_select_topk(p, idx, to_dev(c["qb"].view(np.int16)), to_dev(c["w"]), tk,
                       workspace(ck.csa_select_topk_workspace_bytes(p, n_c)))
    torch.cuda.synchronize()
    assert topk_sets_equal(tk.cpu().numpy(), expect)


def test_fp4h_reindex_parity():
    print("case: fp4h reindex", flush=True)
    B, n_c, hi, n_pool, k = 2, 6000, 64, 1024, 300
    pool = np.stack([seedgen.distinct_indices(65, seedgen.tid(T.POOL, b), n_c, n_pool)
                     for b in range(B)])
    c = make_case(65, B, n_c, hi, k, layer=1, pool=pool)
    expect = np.stack([OD.reindex_topk(c["qh"][b], c["wv"][b], c["kvals"][b], pool[b], k)
                       for b in range(B)])
    idx, keep = _cache(c, n_c)
    p = ck.CsaParams(B, 0, hi, k, 0, ck.MODE_REINDEX, 1.0, 0)
    out = torch.empty((B, k), dtype=torch.int32, device="cuda")
    ck.csa_reindex_topk(p, idx, to_dev(c["qb"].view(np.int16)), to_dev(c["w"]),
                        to_dev(pool.astype(np.int32)), n_pool, out,
                        workspace(ck.csa_reindex_topk_workspace_bytes(p, n_pool)))
    torch.cuda.synchronize()
    assert topk_sets_equal(out.cpu().numpy(), expect)
