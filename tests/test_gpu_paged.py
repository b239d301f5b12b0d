"""Paged caches (a page pool plus a per-sequence block table) against the same caches
laid out contiguously: the kernels compute on the same rows in the same order, so the
selected indices and the outputs must agree bit for bit; every case is also checked
against the oracle.  The pages are scattered over the pool in a seeded random order and
the pool holds spare pages filled with other data."""
import math

import numpy as np
import pytest
import torch

import compressed_sparse_kv_csa_amd as ck
from cases import (IDX_FMTS, KV_FMTS, attention_error, make_csa_case, oracle_hca,
                   topk_sets_equal)
import seedgen
from oracle import decode as OD, formats as OF
from cases import bf16_bits, encode_kv
from gpu_helpers import to_dev, workspace

pytestmark = pytest.mark.gpu

D = 512


def _paged(codes, scales, page_rows, seed):
    """[B][rows][...] arrays -> (pool codes, pool scales, table [B][pages per sequence])."""
    B, rows = codes.shape[:2]
    per_seq = -(-rows // page_rows)
    n_pages = B * per_seq + 3  # spare pages
    rng = np.random.default_rng(seed)
    perm = rng.permutation(n_pages)[:B * per_seq].reshape(B, per_seq).astype(np.int32)

    def scatter(a):
        pool = rng.integers(0, 256, size=(n_pages * page_rows,) + a.shape[2:], dtype=np.uint8)
        for b in range(B):
            for i in range(per_seq):
                r0, r1 = i * page_rows, min((i + 1) * page_rows, rows)
                p0 = perm[b, i] * page_rows
                pool[p0:p0 + r1 - r0] = a[b, r0:r1]
        return pool

    return scatter(codes), (scatter(scales) if scales is not None else None), perm


def _kv_cache(kv, page_rows, seed, lens=None):
    rows = kv.codes.shape[1]
    if page_rows == 0:
        flat = ck.cache(KV_FMTS[kv.fmt], to_dev(kv.codes), rows, None,
                        to_dev(kv.scales) if kv.scales is not None else None, seq_rows=lens)
        return flat
    pc, ps, tab = _paged(kv.codes, kv.scales, page_rows, seed)
    return ck.cache(KV_FMTS[kv.fmt], to_dev(pc), rows, 0, to_dev(ps) if ps is not None else None,
                    seq_rows=lens, block_table=to_dev(tab), page_rows=page_rows)


def _idx_cache(idx, page_rows, seed, lens=None):
    rows = idx.codes.shape[1]
    if page_rows == 0:
        return ck.cache(IDX_FMTS[idx.fmt], to_dev(idx.codes), rows, None,
                        to_dev(idx.scales) if idx.scales is not None else None, seq_rows=lens)
    pc, ps, tab = _paged(idx.codes, idx.scales, page_rows, seed)
    return ck.cache(IDX_FMTS[idx.fmt], to_dev(pc), rows, 0, to_dev(ps) if ps is not None else None,
                    seq_rows=lens, block_table=to_dev(tab), page_rows=page_rows)


def _csa(case, kvc, idxc):
    p = ck.CsaParams(case.B, case.hq, case.hi, case.top_k, case.window, ck.MODE_FULL, case.scale, 0)
    topk = torch.empty((case.B, case.top_k), dtype=torch.int32, device="cuda")
    out = torch.empty((case.B, case.hq, D), dtype=torch.bfloat16, device="cuda")
    ck.csa_decode(p, kvc, idxc, to_dev(case.q_bits.view(np.int16)),
                  to_dev(case.q_idx_bits.view(np.int16)), to_dev(case.w), topk, out,
                  workspace(ck.csa_decode_workspace_bytes(p, case.n_c)))
    torch.cuda.synchronize()
    return topk.cpu().numpy(), out.view(torch.int16).cpu().numpy()


# (seed, B, N_c, kv_fmt, idx_fmt, kv page rows, key page rows, top_k)
CASES = [
    (501, 3, 5000, "mixed", "fp4", 64, 16, 512),
    (502, 2, 9000, "bf16", "bf16", 256, 128, 512),
    (503, 2, 3001, "fp4", "fp4h", 16, 4096, 512),
    # a 2176-row list: the 64-head workgroups' paged kernel
    (508, 2, 5000, "mixed", "fp4", 32, 64, 2048),
]


@pytest.mark.parametrize("seed,B,n_c,kv_fmt,idx_fmt,kv_pr,idx_pr,top_k", CASES)
def test_csa_paged_matches_contiguous(seed, B, n_c, kv_fmt, idx_fmt, kv_pr, idx_pr, top_k):
    print(f"case: csa paged seed={seed} B={B} n_c={n_c} {kv_fmt}/{idx_fmt} pages {kv_pr}/{idx_pr}"
          f" k={top_k}", flush=True)
    case = make_csa_case(seed, B, n_c, 128, 64, 64, top_k, kv_fmt, idx_fmt)
    flat = _csa(case, _kv_cache(case.kv, 0, seed), _idx_cache(case.idx, 0, seed))
    paged = _csa(case, _kv_cache(case.kv, kv_pr, seed), _idx_cache(case.idx, idx_pr, seed + 1))
    assert (flat[0] == paged[0]).all(), "selected indices differ"
    assert (flat[1] == paged[1]).all(), "outputs differ"
    assert topk_sets_equal(paged[0], case.expect_topk)
    out = torch.from_numpy(paged[1]).view(torch.bfloat16).double().numpy()
    err, ok = attention_error(out, case.expect_out)
    assert ok, err


def test_csa_paged_varlen():
    # Paged caches with per-sequence lengths: the same as contiguous ones with them, and
    # each sequence's selection and output those of the oracle over its own rows (each
    # sequence's keys are tie-free over the rows it holds).
    from test_gpu_varlen import _varlen_case
    lens, cap, W = [6000, 2500, 100], 6000, 128
    c = _varlen_case(504, lens, cap, W, 64, 64, 512, "mixed", "fp4")
    kv_len = torch.tensor([W + n for n in lens], dtype=torch.int32, device="cuda")
    idx_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
    p = ck.CsaParams(3, 64, 64, 512, W, ck.MODE_FULL, 1.0 / math.sqrt(D), 0)
    res = []
    for kv_pr, idx_pr in ((0, 0), (32, 64)):
        kvc = _kv_cache(c["kv"], kv_pr, 504, kv_len)
        idxc = _idx_cache(c["idx"], idx_pr, 505, idx_len)
        topk = torch.empty((3, 512), dtype=torch.int32, device="cuda")
        out = torch.empty((3, 64, D), dtype=torch.bfloat16, device="cuda")
        ck.csa_decode(p, kvc, idxc, to_dev(c["q"].view(np.int16)), to_dev(c["qi"].view(np.int16)),
                      to_dev(c["w"]), topk, out, workspace(ck.csa_decode_workspace_bytes(p, cap)))
        torch.cuda.synchronize()
        res.append((topk.cpu().numpy(), out.view(torch.int16).cpu().numpy()))
    assert (res[0][0] == res[1][0]).all() and (res[0][1] == res[1][1]).all()
    qv, qiv = OF.bf16_bits_to_f64(c["q"]), OF.bf16_bits_to_f64(c["qi"])
    out = torch.from_numpy(res[1][1]).view(torch.bfloat16).double().numpy()
    for b, n in enumerate(lens):
        sel = OD.topk_indices(OD.indexer_scores(qiv[b], c["w"][b].astype(np.float64),
                                                c["idx"].values[b, :n]), 512)
        assert topk_sets_equal(res[1][0][b:b + 1], sel[None]), b
        ref = OD.attention(qv[b], OD.csa_rows(c["kv"].values[b, :W + n], W, sel), p.softmax_scale)
        err, ok = attention_error(out[b], ref)
        assert ok, (b, err)


@pytest.mark.parametrize("kv_fmt,pr", [("bf16", 128), ("mixed", 32), ("fp4", 16)])
def test_hca_paged(kv_fmt, pr):
    B, rows, hq = 3, 2500, 64
    T = seedgen.TID
    q = bf16_bits(seedgen.bf16_normal(506, seedgen.tid(T.Q), (B, hq, D)))
    kv = encode_kv(bf16_bits(seedgen.kv_rows_bf16(506, seedgen.tid(T.KV), (B, rows, D))), kv_fmt)
    scale = 1.0 / math.sqrt(D)
    outs = []
    for page_rows in (0, pr):
        kvc = _kv_cache(kv, page_rows, 506)
        out = torch.empty((B, hq, D), dtype=torch.bfloat16, device="cuda")
        ck.hca_decode(B, hq, scale, kvc, to_dev(q.view(np.int16)), out,
                      workspace(ck.hca_decode_workspace_bytes(B, hq, rows)))
        torch.cuda.synchronize()
        outs.append(out.view(torch.int16).cpu().numpy())
    assert (outs[0] == outs[1]).all()
    err, ok = attention_error(torch.from_numpy(outs[1]).view(torch.bfloat16).double().numpy(),
                              oracle_hca(q, kv, scale))
    assert ok, err


def test_reindex_paged():
    # A paged key cache gives the same Reindex selection as the contiguous one, and both are
    # the oracle's top-k of each query's pool (keys tie-free inside the pool).
    from test_gpu_reindex import make_case
    c = make_case(507, 2, 3000, 64, 1024, 128, "fp4", n_empty=5)
    p = ck.CsaParams(2, 0, 64, 128, 0, ck.MODE_REINDEX, 1.0, 0)
    pool = to_dev(c["pool"].astype(np.int32))
    got = []
    for pr in (0, 32):
        idxc = _idx_cache(c["idx"], pr, 507)
        topk = torch.empty((2, 128), dtype=torch.int32, device="cuda")
        ck.csa_reindex_topk(p, idxc, to_dev(c["q_bits"].view(np.int16)), to_dev(c["w"]), pool,
                            1024, topk, workspace(ck.csa_reindex_topk_workspace_bytes(p, 1024)))
        torch.cuda.synchronize()
        got.append(topk.cpu().numpy())
    assert (got[0] == got[1]).all()
    assert topk_sets_equal(got[1], c["expect"])
