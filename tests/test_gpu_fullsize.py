"""Parity at the workloads' full sizes, in the launch configuration the bench times.

Each test runs the whole batch on the GPU and compares the queries the oracle checks
(all of them where the oracle finishes in seconds, a sample otherwise): top-k index
sets bit-exact (those queries' keys made tie-free), attention outputs within 1e-2."""
import numpy as np
import pytest
import torch

import compressed_sparse_kv_csa_amd as ck
from cases import attention_error, topk_sets_equal
from fullsize import (make_indexer, make_kv_cache, make_pool_tie_free, oracle_topk, query_bits,
                      reindex_query, run_decode, bf16_out, scale_of, DEV)
from oracle import decode as OD

pytestmark = [pytest.mark.gpu, pytest.mark.fullsize]


def _check_query(name, b, topk_gpu, out_gpu, sel, ref):
    assert topk_sets_equal(topk_gpu[b:b + 1], sel[None]), f"{name}: top-k set differs for query {b}"
    err, ok = attention_error(out_gpu[b], ref)
    print(f"{name} query {b}: max |out - oracle| = {err:.3e}", flush=True)
    assert ok, (name, b, err)


def _csa_full_layer(seed, B, n_c, W, hq, hi, k, kvf, idf, check, name):
    print(f"case: {name} seed={seed} B={B} Nc={n_c} W={W} Hq={hq} HI={hi} k={k} kv={kvf} idx={idf} "
          f"checked={check}", flush=True)
    ix = make_indexer(seed, 0, B, n_c, hi, k, idf, check)
    kv = make_kv_cache(seed, 0, B, W + n_c, kvf)
    q, qv = query_bits(seed, 0, B, hq)
    expect = {}
    for b in check:
        sel = oracle_topk(ix, b, k)
        rows = np.concatenate([np.arange(W), W + sel[sel >= 0]])
        expect[b] = (sel, OD.attention(qv[b], kv.put_oracle_rows(b, rows), scale_of()))
    p = ck.CsaParams(B, hq, hi, k, W, ck.MODE_FULL, scale_of(), 0)
    topk = torch.empty((B, k), dtype=torch.int32, device=DEV)
    out = bf16_out(run_decode(p, kv, ix, q, topk, n_c))
    tk = topk.cpu().numpy()
    for b in check:
        _check_query(name, b, tk, out, *expect[b])
    return topk, expect


def test_csa_pro_bf16_131k():
    # 131072-token context: 32768 entries, bf16 keys and rows, 32 query tokens
    _csa_full_layer(2, 32, 32768, 128, 64, 64, 512, "bf16", "bf16", list(range(32)), "csa_bf16_131k")


def test_csa_mixed_1m():
    # 1M-token context: 262144 entries, mixed FP8/BF16 rows, FP4 indexer keys, 4 tokens
    _csa_full_layer(4, 4, 262144, 128, 64, 64, 512, "mixed", "fp4", [0, 1, 2, 3], "csa_mixed_1m")


def test_csa2_stack_fp4_1m():
    # CSA2 stack: one Full layer (indexer + top-512) and five Reuse layers that attend with
    # its indices over their own FP4 caches; 8 tokens, every query checked.
    seed, B, n_c, W, hq, hi, k = 5, 8, 262144, 128, 64, 64, 512
    check = list(range(B))
    topk, expect = _csa_full_layer(seed, B, n_c, W, hq, hi, k, "fp4", "fp4", check, "csa2 full layer")
    for layer in range(1, 6):
        print(f"case: csa2 reuse layer {layer}", flush=True)
        kv = make_kv_cache(seed, layer, B, W + n_c, "fp4")
        q, qv = query_bits(seed, layer, B, hq)
        ref = {}
        for b in check:
            sel = expect[b][0]
            rows = np.concatenate([np.arange(W), W + sel[sel >= 0]])
            ref[b] = OD.attention(qv[b], kv.put_oracle_rows(b, rows), scale_of())
        p = ck.CsaParams(B, hq, 0, k, W, ck.MODE_REUSE, scale_of(), 0)
        out = bf16_out(run_decode(p, kv, None, q, topk, n_c))
        for b in check:
            err, ok = attention_error(out[b], ref[b])
            print(f"reuse layer {layer} query {b}: max |out - oracle| = {err:.3e}", flush=True)
            assert ok, (layer, b, err)
        del kv


def test_csa2_reindex_fp4_1m():
    # Hierarchical indexer at the CSA2 workload: the Full layer selects a 1024-row pool over
    # 262,144 FP4 keys; a Reindex layer re-ranks the pool with its own indexer query to 512
    # rows and attends (REUSE) over its own FP4 cache.  8 tokens, every query checked.
    seed, B, n_c, W, hq, hi, P, k = 5, 8, 262144, 128, 64, 64, 1024, 512
    check = list(range(B))
    print(f"case: csa2 reindex seed={seed} B={B} Nc={n_c} pool={P} k={k} checked={check}", flush=True)
    ix = make_indexer(seed, 0, B, n_c, hi, P, "fp4", check)
    p = ck.CsaParams(B, 0, hi, P, 0, ck.MODE_FULL, 1.0, 0)
    pool = torch.empty((B, P), dtype=torch.int32, device=DEV)
    ws = torch.empty(max(ck.csa_select_topk_workspace_bytes(p, n_c), 256), dtype=torch.uint8, device=DEV)
    ck.csa_select_topk(p, ix.cache, ix.q_idx, ix.w, pool, ws)
    torch.cuda.synchronize()
    pl = pool.cpu().numpy()
    for b in check:
        assert topk_sets_equal(pl[b:b + 1], oracle_topk(ix, b, P)[None]), f"pool of query {b}"
    qi1, w1, qv1, wv1 = reindex_query(seed, 1, B, hi)
    for b in check:
        make_pool_tie_free(ix, b, pl[b], qv1[b], wv1[b], k, "fp4")
    print("case: csa2 reindex layer 1 select", flush=True)
    pr = ck.CsaParams(B, 0, hi, k, 0, ck.MODE_REINDEX, 1.0, 0)
    tk = torch.empty((B, k), dtype=torch.int32, device=DEV)
    rws = torch.empty(ck.csa_reindex_topk_workspace_bytes(pr, P), dtype=torch.uint8, device=DEV)
    ck.csa_reindex_topk(pr, ix.cache, qi1, w1, pool, P, tk, rws)
    torch.cuda.synchronize()
    tkn = tk.cpu().numpy()
    sel = {}
    for b in check:
        sel[b] = OD.reindex_topk(qv1[b], wv1[b], ix.key_values[b], pl[b], k)
        assert topk_sets_equal(tkn[b:b + 1], sel[b][None]), f"reindexed top-k of query {b}"
    print("case: csa2 reindex layer 1 attention", flush=True)
    kv = make_kv_cache(seed, 1, B, W + n_c, "fp4")
    q, qv = query_bits(seed, 1, B, hq)
    ref = {}
    for b in check:
        rows = np.concatenate([np.arange(W), W + sel[b][sel[b] >= 0]])
        ref[b] = OD.attention(qv[b], kv.put_oracle_rows(b, rows), scale_of())
    out = bf16_out(run_decode(ck.CsaParams(B, hq, 0, k, W, ck.MODE_REUSE, scale_of(), 0), kv, None,
                              q, tk, n_c))
    for b in check:
        err, ok = attention_error(out[b], ref[b])
        print(f"reindex layer query {b}: max |out - oracle| = {err:.3e}", flush=True)
        assert ok, (b, err)


def test_csa_fp4h_mixed_1m():
    # The 1M mixed workload with Hadamard-rotated FP4 indexer keys (the indexer rotates and
    # FP4-quantises the queries itself); every query checked.
    _csa_full_layer(7, 4, 262144, 128, 64, 64, 512, "mixed", "fp4h", [0, 1, 2, 3], "csa fp4h mixed 1M")


def test_hca_1m():
    # HCA: 1M tokens at ratio 128 -> 8192 entries + 128 window rows, bf16, 16 tokens
    seed, B, rows, hq = 3, 16, 8192 + 128, 64
    print(f"case: hca seed={seed} B={B} rows={rows} Hq={hq}", flush=True)
    kv = make_kv_cache(seed, 0, B, rows, "bf16")
    q, qv = query_bits(seed, 0, B, hq)
    out = torch.empty((B, hq, 512), dtype=torch.int16, device=DEV)
    ws = torch.empty(max(ck.hca_decode_workspace_bytes(B, hq, rows), 256), dtype=torch.uint8, device=DEV)
    ck.hca_decode(B, hq, scale_of(), kv.descriptor(), q, out, ws)
    torch.cuda.synchronize()
    got = bf16_out(out)
    for b in range(B):
        vals = kv.put_oracle_rows(b, np.arange(rows))
        ref = OD.hca_decode_one(qv[b], vals, scale_of())
        err, ok = attention_error(got[b], ref)
        print(f"hca query {b}: max |out - oracle| = {err:.3e}", flush=True)
        assert ok, (b, err)
