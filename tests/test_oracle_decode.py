"""Pins of the oracle's indexer, top-k and attention: brute force on tiny inputs, closed
forms, reductions to textbook routines, and invariances that catch dropped terms,
wrong signs, wrong indices and transposed operands."""
import itertools
import math

import numpy as np
import pytest

from oracle import decode as D


def _rng(s=0):
    return np.random.default_rng(s)


# ------------------------------------------------------------------ indexer score

def test_score_brute_force_loops():
    r = _rng(1)
    q = r.standard_normal((3, 5)); w = r.uniform(0, 1, 3); k = r.standard_normal((7, 5))
    s = D.indexer_scores(q, w, k)
    for j in range(7):
        acc = 0.0
        for h in range(3):
            d = sum(q[h, c] * k[j, c] for c in range(5))
            acc += w[h] * (d if d > 0 else 0.0)
        assert math.isclose(s[j], acc, rel_tol=1e-12, abs_tol=1e-12)


def test_score_relu_and_sign():
    # one head, w = 2: s = 2 * max(q.k, 0); a key anti-aligned with q scores 0.
    q = np.array([[1.0, 2.0]]); w = np.array([2.0])
    k = np.array([[1.0, 1.0], [-1.0, -1.0], [0.5, 0.0]])
    assert D.indexer_scores(q, w, k).tolist() == [6.0, 0.0, 1.0]


def test_score_homogeneity_and_w_scaling():
    r = _rng(2)
    q = r.standard_normal((4, 8)); w = r.uniform(0, 1, 4); k = r.standard_normal((50, 8))
    s = D.indexer_scores(q, w, k)
    assert np.allclose(D.indexer_scores(q, w, 0.5 * k), 0.5 * s)
    assert np.allclose(D.indexer_scores(q, 3.0 * w, k), 3.0 * s)


# ------------------------------------------------------------------ top-k

def test_topk_single_head_is_textbook_topk():
    """H_I = 1, w = 1 and positive dots: the selection is the plain top-k of q.k (argsort)."""
    r = _rng(3)
    q = np.abs(r.standard_normal((1, 16))); k = np.abs(r.standard_normal((300, 16)))
    sel = D.topk_indices(D.indexer_scores(q, np.ones(1), k), 40)
    ref = np.argsort(-(k @ q[0]), kind="stable")[:40]
    assert set(sel.tolist()) == set(ref.tolist())


def test_topk_order_ties_padding():
    s = np.array([1.0, 3.0, 3.0, 2.0, 3.0])
    assert D.topk_indices(s, 3).tolist() == [1, 2, 4]
    assert D.topk_indices(s, 7).tolist() == [1, 2, 4, 3, 0, -1, -1]
    assert D.topk_indices(np.zeros(0), 2).tolist() == [-1, -1]


def test_topk_permutation_invariance():
    r = _rng(4)
    q = r.standard_normal((4, 8)); w = r.uniform(0, 1, 4); k = r.standard_normal((200, 8))
    perm = r.permutation(200)
    a = D.topk_indices(D.indexer_scores(q, w, k), 32)
    b = D.topk_indices(D.indexer_scores(q, w, k[perm]), 32)
    assert set(perm[b].tolist()) == set(a.tolist())


def test_topk_brute_force_subsets():
    """Tiny case: the chosen set maximises the total score over all C(8,3) subsets."""
    r = _rng(5)
    s = r.standard_normal(8)
    best = max(itertools.combinations(range(8), 3), key=lambda t: sum(s[i] for i in t))
    assert set(D.topk_indices(s, 3).tolist()) == set(best)


# ------------------------------------------------------------------ CSA2 reindex

def test_reindex_whole_sequence_pool_is_the_full_selection():
    """A pool of every row reduces Reindex to the Full layer's own selection."""
    r = _rng(21)
    q = r.standard_normal((6, 16)); w = r.uniform(0, 1, 6); k = r.standard_normal((500, 16))
    s = D.indexer_scores(q, w, k)
    for kk in (1, 37, 500, 520):
        got = D.reindex_topk(q, w, k, r.permutation(500), kk)
        assert got.tolist() == D.topk_indices(s, kk).tolist()


def test_reindex_pool_holding_the_global_topk_returns_it():
    """Whatever else the pool holds, the global top-k rows win inside it (row indices, not pool slots)."""
    r = _rng(22)
    q = r.standard_normal((4, 8)); w = r.uniform(0, 1, 4); k = r.standard_normal((1000, 8))
    top = D.topk_indices(D.indexer_scores(q, w, k), 24)
    others = r.choice(np.setdiff1d(np.arange(1000), top), 200, replace=False)
    pool = r.permutation(np.concatenate([top, others]))
    got = D.reindex_topk(q, w, k, pool, 24)
    assert set(got.tolist()) == set(top.tolist())


def test_reindex_pool_order_empty_entries_and_repeats():
    r = _rng(23)
    q = r.standard_normal((3, 8)); w = r.uniform(0, 1, 3); k = r.standard_normal((64, 8))
    pool = r.choice(64, 20, replace=False)
    ref = D.reindex_topk(q, w, k, pool, 8)
    noisy = np.concatenate([pool[::-1], [-1, 64, 1000, -7], pool[:5]])
    assert D.reindex_topk(q, w, k, noisy, 8).tolist() == ref.tolist()
    short = D.reindex_topk(q, w, k, pool, 25)   # k beyond the pool: all 20, then -1
    assert short[20:].tolist() == [-1] * 5
    assert set(short[:20].tolist()) == set(pool.tolist())
    assert D.reindex_topk(q, w, k, np.array([-1, -1]), 3).tolist() == [-1, -1, -1]


def test_reindex_brute_force_over_pool_subsets():
    """Tiny pools: the result maximises the summed score over every k-subset of the pool;
    with integer dots and equal scores, the lower row index wins."""
    r = _rng(24)
    q = r.standard_normal((2, 4)); w = r.uniform(0, 1, 2); k = r.standard_normal((40, 4))
    pool = r.choice(40, 9, replace=False)
    s = D.indexer_scores(q, w, k)
    best = max(itertools.combinations(pool.tolist(), 4), key=lambda t: sum(s[i] for i in t))
    assert set(D.reindex_topk(q, w, k, pool, 4).tolist()) == set(best)
    # H_I = 1, w = 1, integer keys: rows 3, 9 and 12 tie at the top score.
    qi = np.ones((1, 2)); ki = np.zeros((16, 2)); ki[[3, 9, 12]] = [2.0, 3.0]; ki[5] = [1.0, 1.0]
    assert D.reindex_topk(qi, np.ones(1), ki, [12, 5, 9, 3, 0], 2).tolist() == [3, 9]


# ------------------------------------------------------------------ attention

def test_attention_two_rows_closed_form():
    q = np.array([[1.0, 0.0]]); e = np.array([[2.0, 0.0], [0.0, 1.0]]); sc = 0.5
    # logits 1.0 and 0.0: weights e/(e+1), 1/(e+1)
    a = math.e / (math.e + 1.0)
    assert np.allclose(D.attention(q, e, sc), [[2.0 * a, 1.0 - a]])


def test_attention_zero_scale_is_mean_and_single_row():
    r = _rng(6)
    q = r.standard_normal((3, 4)); e = r.standard_normal((9, 4))
    assert np.allclose(D.attention(q, e, 0.0), np.tile(e.mean(0), (3, 1)))
    assert np.allclose(D.attention(q, e[:1], 0.7), np.tile(e[0], (3, 1)))
    same = np.tile(e[2], (5, 1))
    assert np.allclose(D.attention(q, same, 0.3), np.tile(e[2], (3, 1)))
    assert np.array_equal(D.attention(q, e[:0], 0.3), np.zeros((3, 4)))


def test_attention_head_independence_and_row_permutation():
    r = _rng(7)
    q = r.standard_normal((4, 6)); e = r.standard_normal((11, 6))
    o = D.attention(q, e, 0.4)
    assert np.allclose(o[2], D.attention(q[2:3], e, 0.4)[0])
    assert np.allclose(o, D.attention(q, e[r.permutation(11)], 0.4))


def test_attention_brute_force_loops():
    r = _rng(8)
    q = r.standard_normal((2, 3)); e = r.standard_normal((4, 3)); sc = 0.9
    o = D.attention(q, e, sc)
    for h in range(2):
        lg = [sc * sum(q[h, c] * e[j, c] for c in range(3)) for j in range(4)]
        z = [math.exp(x) for x in lg]
        for c in range(3):
            assert math.isclose(o[h, c], sum(z[j] * e[j, c] for j in range(4)) / sum(z), rel_tol=1e-12)


def test_duplicate_rows_count_twice():
    """Window and selected rows are not de-duplicated: a repeated row weighs double."""
    q = np.array([[0.0, 0.0]]); e = np.array([[1.0, 0.0], [0.0, 1.0]])
    kv = np.array([[1.0, 0.0], [1.0, 0.0], [0.0, 1.0]])       # window row 0 = compressed row 0
    out = D.csa_reuse_one(q, kv, 1, np.array([0, 1]), 1.0)
    assert np.allclose(out, [[2.0 / 3.0, 1.0 / 3.0]])


# ------------------------------------------------------------------ full CSA / HCA

def test_csa_with_k_ge_nc_equals_hca():
    r = _rng(9)
    W, Nc = 5, 12
    kv = r.standard_normal((W + Nc, 16)); q = r.standard_normal((4, 16))
    qi = r.standard_normal((2, 8)); w = r.uniform(0, 1, 2); keys = r.standard_normal((Nc, 8))
    out, sel = D.csa_decode_one(q, qi, w, keys, kv, W, 20, 0.25)
    assert sorted(sel[sel >= 0].tolist()) == list(range(Nc)) and (sel[Nc:] == -1).all()
    assert np.allclose(out, D.hca_decode_one(q, kv, 0.25))


def test_csa_selects_then_attends():
    """Rows outside window + top-k do not influence the output; the ones inside do."""
    r = _rng(10)
    W, Nc, k = 3, 20, 4
    kv = r.standard_normal((W + Nc, 8)); q = r.standard_normal((2, 8))
    qi = r.standard_normal((2, 8)); w = r.uniform(0, 1, 2); keys = r.standard_normal((Nc, 8))
    out, sel = D.csa_decode_one(q, qi, w, keys, kv, W, k, 0.5)
    unsel = [j for j in range(Nc) if j not in set(sel.tolist())]
    kv2 = kv.copy(); kv2[W + np.array(unsel)] = 100.0
    out2, sel2 = D.csa_decode_one(q, qi, w, keys, kv2, W, k, 0.5)
    assert np.array_equal(sel, sel2) and np.allclose(out, out2)
    kv3 = kv.copy(); kv3[W + sel[0]] += 1.0
    assert not np.allclose(out, D.csa_reuse_one(q, kv3, W, sel, 0.5))
    ref = D.attention(q, np.concatenate([kv[:W], kv[W + np.sort(sel)]]), 0.5)
    assert np.allclose(out, ref)
