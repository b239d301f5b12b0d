"""The indexer's less common selection paths, against the oracle.

* A slice holding more winners than it sends (its bound lies above the k-th key): the
  merge must read that slice's stored scores again.
* A slice whose boundary histogram bin holds more keys than its candidate slots (many
  equal scores): the scan falls back to an exact top-cap for that slice.  Equal scores
  here are exact zeros (all-zero keys), which every evaluation order produces exactly,
  and are ordered by index on both sides, so no tie-free conditioning is needed."""
import math

import numpy as np
import pytest
import torch

import seedgen
from cases import (CsaCase, attention_error, bf16_bits, encode_idx, encode_kv, run_oracle_full,
                   topk_sets_equal, D, DI)
from gpu_helpers import run_csa
from oracle import tiefree

pytestmark = pytest.mark.gpu
T = seedgen.TID


def _case(seed, B, n_c, W, hq, hi, k, kvf, idf, edit_keys, tie_free=True):
    q = seedgen.bf16_normal(seed, seedgen.tid(T.Q), (B, hq, D))
    kv = encode_kv(bf16_bits(seedgen.kv_rows_bf16(seed, seedgen.tid(T.KV), (B, W + n_c, D))), kvf)
    qi = seedgen.bf16_normal(seed, seedgen.tid(T.Q_IDX), (B, hi, DI))
    w = seedgen.uniform01(seed, seedgen.tid(T.W_IDX), (B, hi)).numpy()
    keys = edit_keys(bf16_bits(seedgen.bf16_normal(seed, seedgen.tid(T.IDX_KEYS), (B, n_c, DI))))
    certs = []
    if tie_free:
        keys, certs = tiefree.make_tie_free(keys, qi.double().numpy(), w.astype(np.float64), k, idf)
    case = CsaCase(B, n_c, W, hq, hi, k, 1.0 / math.sqrt(D), bf16_bits(q), bf16_bits(qi),
                   w.astype(np.float32), kv, encode_idx(keys, idf), certs=certs)
    run_oracle_full(case)
    return case


def _check(case):
    topk, out = run_csa(case)
    assert topk_sets_equal(topk, case.expect_topk)
    err, ok = attention_error(out, case.expect_out)
    print(f"max |out - oracle| = {err:.3e}", flush=True)
    assert ok, err


@pytest.mark.parametrize("idf", ["bf16", "fp4"])
def test_winners_concentrated_in_one_slice(idf):
    # Keys of rows 8192..12287 (the third 4096-row slice) scaled by 4 (exact in bf16 and in
    # the FP4 block format): every one of the top-512 lies in that slice.
    def edit(bits):
        v = bits.copy()
        blk = v[:, 8192:12288]
        exp = (blk >> 7) & 0xFF
        nz = exp != 0
        blk[nz] = blk[nz] + np.uint16(2 << 7)  # exponent + 2 (no overflow: |x| <= 6)
        v[:, 8192:12288] = blk
        return v
    print(f"case: winners in one slice, idx={idf}", flush=True)
    case = _case(31, 2, 5 * 4096, 128, 64, 64, 512, "bf16", idf, edit)
    inside = (case.expect_topk >= 8192) & (case.expect_topk < 12288)
    assert inside.all(), "the construction must put every winner in one slice"
    _check(case)


@pytest.mark.parametrize("idf", ["bf16", "fp4"])
def test_many_equal_scores(idf):
    # Only rows 0..99 have nonzero keys; every other score is exactly 0, so the top-512 is
    # those 100 rows plus rows 100..511, and whole slices are one histogram bin.
    def edit(bits):
        v = bits.copy()
        v[:, 100:] = 0
        return v
    print(f"case: many equal scores, idx={idf}", flush=True)
    case = _case(32, 1, 9000, 128, 64, 64, 512, "bf16", idf, edit, tie_free=False)
    assert set(range(100, 512)) <= set(case.expect_topk[0].tolist())
    _check(case)
