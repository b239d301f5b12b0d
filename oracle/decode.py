"""Decode-time attention over compressed KV caches (oracle; test infrastructure only).

What one query token computes, per the pages:
* CSA layer ("DeepSeek-V4 KV Cache 深度分析", section 三 "压缩机制详解" part 2,
  section 四 "索引器（Indexer）机制" and the section 十一 forward-flow diagram):
  the token's indexer query is scored against the indexer key of every
  compressed entry, the top-k entries are kept, and attention runs over the kept
  entries together with the most recent 128 uncompressed tokens (the sliding
  window).  Each cached entry serves as both key and value (section 五, the
  shared-KV remark).
* HCA layer (section 三 part 1): no selection; attention is dense over every
  compressed entry plus the window.
* CSA2 Reuse layers ("DeepSeek, KV 캐시를 토큰당 890바이트로 줄인 V4.1-Flash 공개",
  section 핵심 내용): attend with the top-512 indices an earlier layer chose.
* CSA2 Reindex layers (same section, and "KV cache 890 bajtów na token", section
  "Trzy mechanizmy zamiast jednej sztuczki"): a fresh indexer query re-ranks the
  candidate pool that the group's Full layer built over the shared indexer keys
  (the hierarchical sparse indexer), and the top-k of the pool is kept.

Readings where the pages are silent
* Indexer score: s_j = sum_h w_h * ReLU(q_h . k_j)  (the pages give no formula;
  this is the lightning-indexer form the decode workload fixes).
* Ties in the score: order by (score descending, index ascending).
* Window and selected entries share ONE softmax over their union; rows are not
  de-duplicated.  An empty row set gives a zero output.
* Softmax scale is a parameter (1/sqrt(512) by default).

Row layout of a sequence's shared-KV cache: ``[window rows | compressed rows]``;
top-k index j refers to compressed row j, i.e. cache row ``window + j``.

* Reindex pool: the Full layer's candidate rows (its own top-P, P >= k); entries that
  are negative or past N_c are empty, and a row listed twice counts once.  The pool
  size is a parameter (the pages give none).

Parity pins (tests/test_oracle_decode.py): brute-force per-element loops on tiny
shapes, permutation and scaling invariances, the H_I = 1 / w = 1 reduction to a
plain top-k of dot products, k >= N_c reducing CSA to dense attention, single-
row and identical-row attention; for Reindex, the whole-sequence pool reducing to
the Full selection, a pool holding the global top-k returning it, pool-order and
empty-entry invariance, and brute force over all subsets of a tiny pool.
"""
from __future__ import annotations

import numpy as np


def indexer_scores(q_idx, w_idx, keys) -> np.ndarray:
    """s[j] = sum_h w[h] * max(0, sum_c q_idx[h, c] * keys[j, c]), in fp64.

    q_idx: [H_I, d_I]; w_idx: [H_I]; keys: [N_c, d_I] -> [N_c].
    """
    q = np.asarray(q_idx, dtype=np.float64)
    w = np.asarray(w_idx, dtype=np.float64)
    k = np.asarray(keys, dtype=np.float64)
    dots = k @ q.T                       # [N_c, H_I]
    return np.maximum(dots, 0.0) @ w


def topk_indices(scores, k: int) -> np.ndarray:
    """Indices of the k largest scores, ordered by (score desc, index asc); -1 pads past N_c."""
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    order = np.lexsort((np.arange(n), -s))
    out = np.full(k, -1, dtype=np.int64)
    m = min(k, n)
    out[:m] = order[:m]
    return out


def reindex_topk(q_idx, w_idx, keys, pool, k: int) -> np.ndarray:
    """CSA2 Reindex: the k rows of the candidate pool with the largest scores under this
    layer's own indexer query, by (score desc, row index asc); -1 pads a short pool.

    keys: [N_c, d_I] decoded shared indexer keys; pool: compressed-row indices (empty
    when negative or >= N_c; repeats count once) -> [k] row indices.
    """
    keys = np.asarray(keys, dtype=np.float64)
    p = np.asarray(pool, dtype=np.int64).reshape(-1)
    rows = np.unique(p[(p >= 0) & (p < keys.shape[0])])
    s = indexer_scores(q_idx, w_idx, keys[rows])
    order = np.lexsort((rows, -s))
    out = np.full(k, -1, dtype=np.int64)
    m = min(k, rows.shape[0])
    out[:m] = rows[order[:m]]
    return out


def attention(q, rows, softmax_scale: float) -> np.ndarray:
    """Multi-query softmax attention where every row is both key and value.

    q: [H, D]; rows: [R, D] -> [H, D].  l = scale * q . e_r; p = softmax over r;
    o = sum_r p_r e_r.  R = 0 gives zeros.
    """
    q = np.asarray(q, dtype=np.float64)
    e = np.asarray(rows, dtype=np.float64)
    if e.shape[0] == 0:
        return np.zeros_like(q)
    logits = softmax_scale * (q @ e.T)                # [H, R]
    logits = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ e


def csa_rows(kv_rows, window: int, topk) -> np.ndarray:
    """The rows a CSA query attends to: all window rows, then the selected compressed rows."""
    kv = np.asarray(kv_rows, dtype=np.float64)
    sel = np.asarray(topk, dtype=np.int64)
    sel = sel[sel >= 0]
    return np.concatenate([kv[:window], kv[window + sel]], axis=0)


def csa_decode_one(q, q_idx, w_idx, idx_keys, kv_rows, window: int, top_k: int,
                   softmax_scale: float):
    """Full CSA decode for one query token -> (out [H_q, D] fp64, topk [top_k] int64).

    idx_keys: [N_c, d_I] decoded indexer keys; kv_rows: [window + N_c, D] decoded rows.
    """
    s = indexer_scores(q_idx, w_idx, idx_keys)
    sel = topk_indices(s, top_k)
    out = attention(q, csa_rows(kv_rows, window, sel), softmax_scale)
    return out, sel


def csa_reuse_one(q, kv_rows, window: int, topk, softmax_scale: float) -> np.ndarray:
    """CSA2 Reuse: attention over the window plus the given top-k compressed rows."""
    return attention(q, csa_rows(kv_rows, window, topk), softmax_scale)


def hca_decode_one(q, kv_rows, softmax_scale: float) -> np.ndarray:
    """HCA: dense attention over every row of the sequence (window and compressed)."""
    return attention(q, kv_rows, softmax_scale)
