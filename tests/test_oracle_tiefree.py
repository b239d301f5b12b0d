"""The tie-free certificate: after conditioning, fp32 scores in several evaluation orders
all select the oracle's set."""
import numpy as np
import torch

import seedgen
from oracle import decode as D, formats as F, tiefree


def _inputs(seed, B, Nc, H, d=128):
    keys = seedgen.bf16_normal(seed, seedgen.tid(seedgen.TID.IDX_KEYS), (B, Nc, d))
    q = seedgen.bf16_normal(seed, seedgen.tid(seedgen.TID.Q_IDX), (B, H, d)).double().numpy()
    w = seedgen.uniform01(seed, seedgen.tid(seedgen.TID.W_IDX), (B, H)).double().numpy()
    return keys.view(torch.int16).numpy().view(np.uint16), q, w


def _fp32_scores(q, w, kd, order):
    q32 = q.astype(np.float32); w32 = w.astype(np.float32); k32 = kd.astype(np.float32)
    if order == "matmul":
        dots = k32 @ q32.T
    else:
        idx = np.arange(q.shape[1])[::-1] if order == "reverse" else np.arange(q.shape[1])
        dots = np.zeros((kd.shape[0], q.shape[0]), dtype=np.float32)
        for c in idx:
            dots += np.outer(k32[:, c], q32[:, c]).astype(np.float32)
    r = np.maximum(dots, np.float32(0)) * w32[None, :]
    return r.sum(axis=1, dtype=np.float32)


def _check(fmt, seed, B, Nc, H, k):
    bits, q, w = _inputs(seed, B, Nc, H)
    adj, certs = tiefree.make_tie_free(bits, q, w, k, fmt)
    for b in range(B):
        vals = F.bf16_bits_to_f64(adj[b])
        kd = vals if fmt == "bf16" else F.fp4_dequantize(*F.fp4_quantize(vals))
        ref = set(D.topk_indices(D.indexer_scores(q[b], w[b], kd), k).tolist())
        for order in ("matmul", "forward", "reverse"):
            s32 = _fp32_scores(q[b], w[b], kd, order)
            got = set(np.argsort(-s32, kind="stable")[:k].tolist())
            assert got == ref, (fmt, b, order)
        c = certs[b]
        if c["zero_ties"]:  # positives certainly above 0, every other row certainly 0
            assert c["high_unselected"] == 0.0
            assert c["low_selected"] is None or c["low_selected"] > 0.0
            s32 = _fp32_scores(q[b], w[b], kd, "forward")
            assert np.count_nonzero(s32 > 0) < k and np.all(s32 >= 0)
        else:
            assert c["low_selected"] > c["high_unselected"]
    return certs


def test_tie_free_bf16_keys():
    _check("bf16", 21, 2, 3000, 8, 512)


def test_tie_free_fp4_keys():
    _check("fp4", 22, 2, 3000, 8, 512)


def test_tie_free_few_heads_and_small_nc():
    certs = _check("bf16", 23, 1, 1024, 4, 512)
    assert certs[0]["rows_halved"] >= 0
    bits, q, w = _inputs(24, 1, 100, 4)
    _, certs = tiefree.make_tie_free(bits, q, w, 512, "bf16")
    assert certs[0]["low_selected"] is None            # N_c <= k: everything is selected


def test_tie_free_zero_ties_with_few_heads():
    # Three indexer heads: about one row in eight scores exactly 0 (every head negative),
    # and top-2048 of 2118 rows reaches them.  The set is the positive rows plus the
    # lowest-index zero rows in every fp32 evaluation order.
    for fmt, seed in (("bf16", 25), ("fp4", 26)):
        certs = _check(fmt, seed, 2, 2118, 3, 2048)
        assert all(c["zero_ties"] for c in certs), certs


def test_certainly_zero_rows():
    q = np.array([[1.0, -2.0], [0.5, 0.5]])
    w = np.array([1.0, 0.0])
    kd = np.array([[-1.0, 1.0],     # head 0: -3, clearly negative; head 1 has weight 0
                   [0.0, 0.0],      # all products 0: exactly 0
                   [2.0, 1.0],      # head 0: 0 exactly, from nonzero terms: not certain
                   [1.0, 0.0]])     # head 0: +1
    assert tiefree.certainly_zero(q, w, kd).tolist() == [True, True, False, False]
