"""GPU parity of CSA2 Reindex (csa_reindex_topk) against the oracle's reindex_topk.

Each case draws shared indexer keys, a candidate pool per query (distinct rows, with
empty slots in some cases) and a fresh indexer query.  The pool's keys are made
tie-free for that query (tests only: the unselected pool rows nearest the k-th score
are halved until every fp32 evaluation order gives the same set), quantised by the
oracle's codecs, and the oracle's top-k of the pool is the expected set.
"""
import numpy as np
import pytest
import torch

import compressed_sparse_kv_csa_amd as ck
import seedgen
from cases import (DI, IDX_FMTS, bf16_bits, encode_idx, indexer_query_values, make_csa_case,
                   topk_sets_equal)
from gpu_helpers import Guarded, to_dev, upload_idx, workspace
from oracle import decode as OD, formats as OF, tiefree

pytestmark = pytest.mark.gpu
T = seedgen.TID


def make_pool(seed, B, n_c, n_pool, n_empty=0):
    pools = []
    for b in range(B):
        rows = seedgen.distinct_indices(seed, seedgen.tid(T.POOL, b), n_c, n_pool - n_empty)
        empty = np.array([-1, n_c, n_c + 5, -1000][:n_empty] + [-1] * max(0, n_empty - 4))
        p = np.concatenate([rows, empty]).astype(np.int64)
        order = seedgen.distinct_indices(seed + 1, seedgen.tid(T.POOL, b), n_pool, n_pool)
        pools.append(p[order])
    return np.stack(pools)


def make_case(seed, B, n_c, hi, n_pool, top_k, fmt, n_empty=0, layer=1):
    keys = bf16_bits(seedgen.bf16_normal(seed, seedgen.tid(T.IDX_KEYS, 0), (B, n_c, DI)))
    qi = seedgen.bf16_normal(seed, seedgen.tid(T.Q_IDX, layer), (B, hi, DI))
    w = seedgen.uniform01(seed, seedgen.tid(T.W_IDX, layer), (B, hi)).numpy()
    pool = make_pool(seed, B, n_c, n_pool, n_empty)
    qv, wv = indexer_query_values(bf16_bits(qi), fmt), w.astype(np.float64)
    for b in range(B):  # tie-free inside the pool, for this query
        rows = np.unique(pool[b][(pool[b] >= 0) & (pool[b] < n_c)])
        adj, _ = tiefree.make_tie_free(keys[b][rows][None], qv[b][None], wv[b][None],
                                       min(top_k, len(rows)), fmt)
        keys[b][rows] = adj[0]
    idx = encode_idx(keys, fmt)
    expect = np.stack([OD.reindex_topk(qv[b], wv[b], idx.values[b], pool[b], top_k)
                       for b in range(B)])
    return dict(idx=idx, q_bits=bf16_bits(qi), w=w.astype(np.float32), pool=pool, expect=expect,
                B=B, n_c=n_c, hi=hi, n_pool=n_pool, top_k=top_k)


def run_reindex(c, stride_pad=0):
    p = ck.CsaParams(c["B"], 0, c["hi"], c["top_k"], 0, ck.MODE_REINDEX, 1.0, 0)
    idx, keep = upload_idx(c["idx"], stride_pad)
    pool = to_dev(c["pool"].astype(np.int32))
    out = Guarded((c["B"], c["top_k"]), torch.int32)
    ck.csa_reindex_topk(p, idx, to_dev(c["q_bits"].view(np.int16)), to_dev(c["w"]), pool,
                        c["n_pool"], out.t, workspace(ck.csa_reindex_topk_workspace_bytes(p, c["n_pool"])))
    torch.cuda.synchronize()
    assert out.intact(), "write outside the output buffer"
    return out.t.cpu().numpy()


def check(c, got):
    assert topk_sets_equal(got, c["expect"])
    for b in range(c["B"]):  # the kept rows come in pool order
        pos = {int(r): i for i, r in enumerate(c["pool"][b])}
        kept = [pos[int(r)] for r in got[b] if r >= 0]
        assert kept == sorted(kept)


CASES = [
    # seed, B, N_c, H_I, pool, k, key format, empty slots
    (301, 2, 5000, 64, 1024, 512, "bf16", 0),
    (302, 3, 3000, 48, 777, 100, "fp4", 9),
    (303, 2, 2000, 4, 16, 20, "bf16", 3),       # fewer pool rows than k: -1 padding
    (304, 1, 9000, 64, 4096, 1024, "fp4", 0),   # largest pool, k 1024
    (305, 2, 700, 20, 33, 1, "fp4", 1),
    (306, 2, 9000, 128, 4096, 2048, "fp4", 5),  # 128 indexer heads, the largest k
    (307, 1, 3000, 100, 2500, 2048, "bf16", 0),
]


@pytest.mark.parametrize("spec", CASES, ids=lambda s: "-".join(map(str, s)))
def test_reindex_parity(spec):
    seed, B, n_c, hi, n_pool, k, fmt, n_empty = spec
    print(f"case: reindex seed={seed} B={B} N_c={n_c} H_I={hi} pool={n_pool} k={k} {fmt}", flush=True)
    c = make_case(seed, B, n_c, hi, n_pool, k, fmt, n_empty)
    check(c, run_reindex(c, stride_pad=37))


def test_reindex_deterministic():
    print("case: reindex twice", flush=True)
    c = make_case(306, 2, 4000, 64, 1000, 300, "fp4")
    a, b = run_reindex(c), run_reindex(c)
    assert np.array_equal(a, b)
    check(c, a)


def test_reindex_of_the_full_pool_with_its_own_query_is_the_full_selection():
    """The Full layer's top-1024 pool, re-ranked with the Full layer's own query, gives
    exactly the Full layer's top-512 (both computed on the GPU)."""
    print("case: select top-1024, reindex own query to 512", flush=True)
    case = make_csa_case(307, 2, 30000, 128, 64, 64, 512, "bf16", "fp4")
    p = ck.CsaParams(case.B, case.hq, case.hi, 1024, case.window, ck.MODE_FULL, case.scale, 0)
    idx, keep = upload_idx(case.idx)
    qi, w = to_dev(case.q_idx_bits.view(np.int16)), to_dev(case.w)
    pool = torch.empty((case.B, 1024), dtype=torch.int32, device="cuda")
    ck.csa_select_topk(p, idx, qi, w, pool, workspace(ck.csa_select_topk_workspace_bytes(p, case.n_c)))
    pr = ck.CsaParams(case.B, 0, case.hi, 512, 0, ck.MODE_REINDEX, 1.0, 0)
    out = torch.empty((case.B, 512), dtype=torch.int32, device="cuda")
    ck.csa_reindex_topk(pr, idx, qi, w, pool, 1024, out,
                        workspace(ck.csa_reindex_topk_workspace_bytes(pr, 1024)))
    torch.cuda.synchronize()
    assert topk_sets_equal(out.cpu().numpy(), case.expect_topk)
