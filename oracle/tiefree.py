"""Tie-free conditioning of seeded indexer inputs (oracle side; tests only).

The top-k set is compared bit for bit, but a GPU accumulates the indexer score
in fp32 in an order of its own choosing.  This module certifies, per query, that
no fp32 evaluation order can change the set: every selected entry beats every
unselected one by more than the worst-case accumulation error.

Error bound: with exact products (a bf16 x bf16 product, and an FP4-decoded x
bf16 product, both fit in fp32) the fp32 value of
s_j = sum_h w_h ReLU(sum_c q_hc k_jc) differs from the exact one by at most
E_j = (d_I + H_I + 4) * 2**-23 * T_j,  T_j = sum_h |w_h| sum_c |q_hc k_jc|
for any summation order and for round-to-nearest or round-toward-zero adds
(the classical bound gamma_n * sum|terms| with unit 2**-23 and ReLU being
1-Lipschitz).

Procedure for a query: take S = the oracle's top-k set.  Any unselected j with
s_j + E_j >= min_{i in S}(s_i - E_i) has its source bf16 key row halved (exact in
bf16; the ReLU form makes the score halve as well), the row is re-encoded in the
cache format, and the check repeats until it holds.  The adjusted keys are then
the test input for both the oracle and the GPU.

Ties at zero.  With few indexer heads and k close to N_c the selection can reach the
rows whose score is 0 (every head's dot product negative), which halving cannot
separate.  A score is certainly 0 under any fp32 evaluation when each head with a
nonzero weight has a dot product d with d + (d_I + 2) * 2**-23 * sum_c |q_hc k_jc| <= 0:
the fp32 dot product is then <= 0, ReLU gives exactly 0, and the weighted sum of
zeros is exactly 0.  Equal scores go to the lower index (reading R3), so once every
row is either certainly positive (s_j - E_j > 0) or certainly 0, the set is the
positive rows plus the lowest-index zero rows on any evaluation.  When the selection's
lowest bound is not above 0, every other row (a score within its bound of 0) has its
source key row set to zero, which makes it certainly 0.
"""
from __future__ import annotations

import numpy as np

from . import formats
from .decode import indexer_scores, topk_indices


def _decode_keys(bits: np.ndarray, fmt: str) -> np.ndarray:
    vals = formats.bf16_bits_to_f64(bits)
    if fmt == "bf16":
        return vals
    if fmt == "fp4":
        codes, scales = formats.fp4_quantize(vals)
        return formats.fp4_dequantize(codes, scales)
    if fmt == "fp4h":  # FP4 codes of the Hadamard rotation (halving the source halves them too)
        codes, scales = formats.fp4h_quantize(bits)
        return formats.fp4_dequantize(codes, scales)
    raise ValueError(fmt)


def certainly_zero(q, w, kd) -> np.ndarray:
    """Rows whose score is exactly 0 under any fp32 evaluation order (see above)."""
    d_i = kd.shape[1]
    dots = kd @ q.T
    mags = np.abs(kd) @ np.abs(q).T
    ok = (dots + (d_i + 2) * 2.0 ** -23 * mags <= 0.0) | (w[None, :] == 0.0)
    return ok.all(axis=1)


def make_tie_free(key_bits, q_idx, w_idx, top_k: int, fmt: str, max_iter: int = 64):
    """Return (adjusted key bf16 bits [B][N_c][d_I], certificates list).

    key_bits: uint16 bf16 bit patterns [B][N_c][d_I]; q_idx: [B][H_I][d_I] values;
    w_idx: [B][H_I] values; fmt: "bf16", "fp4" or "fp4h" (the stored key format; with "fp4h"
    pass the queries as the indexer uses them, rotated and FP4-decoded).
    """
    keys = np.array(key_bits, dtype=np.uint16, copy=True)
    q_all = np.asarray(q_idx, dtype=np.float64)
    w_all = np.asarray(w_idx, dtype=np.float64)
    B, n_c, d_i = keys.shape
    h_i = q_all.shape[1]
    c_err = (d_i + h_i + 4) * 2.0 ** -23
    certs = []
    for b in range(B):
        q = q_all[b]
        w = w_all[b]
        kd = _decode_keys(keys[b], fmt)
        s = indexer_scores(q, w, kd)
        t = (np.abs(kd) @ np.abs(q).T) @ np.abs(w)
        halved = zeroed = 0
        for _ in range(max_iter):
            if n_c <= top_k:
                break
            sel = topk_indices(s, top_k)
            in_s = np.zeros(n_c, dtype=bool)
            in_s[sel] = True
            e = c_err * t
            lo = np.min(s[in_s] - e[in_s])
            if lo > 0.0:  # separate the unselected rows from the selected ones
                bad = np.nonzero((~in_s) & (s + e >= lo))[0]
                if bad.size == 0:
                    break
                keys[b, bad] = formats.f64_to_bf16_bits(formats.bf16_bits_to_f64(keys[b, bad]) * 0.5)
                halved += bad.size
            else:  # the selection reaches scores near 0: make every such row certainly 0
                bad = np.nonzero(~certainly_zero(q, w, kd) & (s - e <= 0.0))[0]
                if bad.size == 0:
                    break
                keys[b, bad] = 0
                zeroed += bad.size
            kd_bad = _decode_keys(keys[b, bad], fmt)
            kd[bad] = kd_bad
            s[bad] = indexer_scores(q, w, kd_bad)
            t[bad] = (np.abs(kd_bad) @ np.abs(q).T) @ np.abs(w)
        else:
            raise RuntimeError(f"query {b}: no tie-free certificate after {max_iter} rounds")
        if n_c > top_k:
            sel = topk_indices(s, top_k)
            in_s = np.zeros(n_c, dtype=bool)
            in_s[sel] = True
            e = c_err * t
            lo = float(np.min(s[in_s] - e[in_s]))
            if lo > 0.0:
                hi = float(np.max(s[~in_s] + e[~in_s]))
                certs.append({"query": b, "rows_halved": int(halved), "rows_zeroed": int(zeroed),
                              "zero_ties": False, "low_selected": lo, "high_unselected": hi})
            else:
                pos = s > 0.0
                if not (np.all(s[pos] - e[pos] > 0.0) and np.all(certainly_zero(q, w, kd)[~pos])):
                    raise RuntimeError(f"query {b}: rows neither certainly positive nor certainly 0")
                certs.append({"query": b, "rows_halved": int(halved), "rows_zeroed": int(zeroed),
                              "zero_ties": True,
                              "low_selected": float(np.min(s[pos] - e[pos])) if pos.any() else None,
                              "high_unselected": 0.0})
        else:
            certs.append({"query": b, "rows_halved": 0, "rows_zeroed": 0, "zero_ties": False,
                          "low_selected": None, "high_unselected": None})
    return keys, certs
