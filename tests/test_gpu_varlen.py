"""Variable-length batches (per-sequence row counts in the cache descriptors) against the
oracle: each query selects among, and attends over, only the rows its own sequence
holds.  The oracle runs on each sequence's rows alone; the rows past a sequence's end
hold other data and must not be read.  Top-k index sets bit-exact (each sequence's keys
made tie-free over its own rows), attention outputs within 1e-2 max-abs."""
import math

import numpy as np
import pytest
import torch

import compressed_sparse_kv_csa_amd as ck
import seedgen
from cases import (IDX_FMTS, KV_FMTS, attention_error, bf16_bits, encode_idx, encode_kv,
                   indexer_query_values, topk_sets_equal)
from gpu_helpers import Guarded, to_dev, workspace
from oracle import decode as OD, formats as OF, tiefree

pytestmark = pytest.mark.gpu

D, DI = 512, 128


def _varlen_case(seed, lens, cap, window, hq, hi, top_k, kv_fmt, idx_fmt):
    """Capacity-sized caches; sequence b's first lens[b] keys are made tie-free."""
    T = seedgen.TID
    B = len(lens)
    q = bf16_bits(seedgen.bf16_normal(seed, seedgen.tid(T.Q), (B, hq, D)))
    qi = seedgen.bf16_normal(seed, seedgen.tid(T.Q_IDX), (B, hi, DI))
    w = seedgen.uniform01(seed, seedgen.tid(T.W_IDX), (B, hi)).numpy().astype(np.float64)
    keys = bf16_bits(seedgen.bf16_normal(seed, seedgen.tid(T.IDX_KEYS), (B, cap, DI))).copy()
    qv = indexer_query_values(bf16_bits(qi), idx_fmt)  # as the scores use them
    for b, n in enumerate(lens):
        m = max(0, min(n, cap))
        if m > 0:
            kb, _ = tiefree.make_tie_free(keys[b:b + 1, :m].copy(), qv[b:b + 1], w[b:b + 1], top_k,
                                          idx_fmt)
            keys[b, :m] = kb[0]
    kv_bits = bf16_bits(seedgen.kv_rows_bf16(seed, seedgen.tid(T.KV), (B, window + cap, D)))
    return dict(q=q, qi=bf16_bits(qi), w=w.astype(np.float32), kv=encode_kv(kv_bits, kv_fmt),
                idx=encode_idx(keys, idx_fmt))


def _lens_dev(lens):
    return torch.tensor(lens, dtype=torch.int32, device="cuda")


def _caches(c, lens, cap, window):
    kv, idx = c["kv"], c["idx"]
    kv_t = (to_dev(kv.codes), to_dev(kv.scales) if kv.scales is not None else None)
    idx_t = (to_dev(idx.codes), to_dev(idx.scales) if idx.scales is not None else None)
    kv_len = _lens_dev([window + n for n in lens])
    idx_len = _lens_dev(list(lens))
    kvc = ck.cache(KV_FMTS[kv.fmt], kv_t[0], window + cap, None, kv_t[1], seq_rows=kv_len)
    idxc = ck.cache(IDX_FMTS[idx.fmt], idx_t[0], cap, None, idx_t[1], seq_rows=idx_len)
    return kvc, idxc, (kv_t, idx_t, kv_len, idx_len)


# (seed, lens, capacity, window, H_q, H_I, top_k, kv_fmt, idx_fmt)
CASES = [
    # two slices at full length, one ragged inside the first slice, one empty
    (401, [5000, 2345, 0], 5000, 128, 64, 64, 512, "mixed", "fp4"),
    # shorter than k (-1 padding), exactly k, several slices
    (402, [300, 512, 9000], 9000, 128, 64, 64, 512, "bf16", "bf16"),
    # FP4 shared-KV, lengths around the 4096-row slice boundary
    (403, [4096, 4097, 4095], 4100, 128, 32, 16, 256, "fp4", "fp4"),
]


@pytest.mark.parametrize("seed,lens,cap,window,hq,hi,top_k,kv_fmt,idx_fmt", CASES)
def test_csa_varlen(seed, lens, cap, window, hq, hi, top_k, kv_fmt, idx_fmt):
    print(f"case: csa varlen seed={seed} lens={lens} cap={cap} {kv_fmt}/{idx_fmt}", flush=True)
    c = _varlen_case(seed, lens, cap, window, hq, hi, top_k, kv_fmt, idx_fmt)
    B, scale = len(lens), 1.0 / math.sqrt(D)
    kvc, idxc, keep = _caches(c, lens, cap, window)
    p = ck.CsaParams(B, hq, hi, top_k, window, ck.MODE_FULL, scale, 0)
    topk = Guarded((B, top_k), torch.int32)
    out = Guarded((B, hq, D), torch.int16)
    ws = workspace(ck.csa_decode_workspace_bytes(p, cap))
    ck.csa_decode(p, kvc, idxc, to_dev(c["q"].view(np.int16)), to_dev(c["qi"].view(np.int16)),
                  to_dev(c["w"]), topk.t, out.t, ws)
    torch.cuda.synchronize()
    assert topk.intact() and out.intact(), "write outside the output buffers"
    got_topk = topk.t.cpu().numpy()
    got = out.t.cpu().view(torch.bfloat16).double().numpy()
    qv, qiv = OF.bf16_bits_to_f64(c["q"]), OF.bf16_bits_to_f64(c["qi"])
    for b, n in enumerate(lens):
        o, sel = OD.csa_decode_one(qv[b], qiv[b], c["w"][b].astype(np.float64),
                                   c["idx"].values[b][:n], c["kv"].values[b][:window + n], window,
                                   top_k, scale)
        assert topk_sets_equal(got_topk[b:b + 1], sel[None]), f"top-k set of sequence {b}"
        err, ok = attention_error(got[b], o)
        print(f"  b={b} n={n}: max |out - oracle| = {err:.3e}")
        assert ok, (b, err)


def test_csa_varlen_select_matches_single():
    # A sequence's selection in a varlen batch equals its selection alone in a cache of
    # the same capacity (the same slices, candidates and order): the indices agree
    # element by element, so a sequence's neighbours in the batch do not matter.
    lens, cap, hi, top_k = [6000, 1000, 4500], 6000, 64, 512
    c = _varlen_case(404, lens, cap, 128, 16, hi, top_k, "bf16", "fp4")
    B = len(lens)
    _, idxc, keep = _caches(c, lens, cap, 128)
    p = ck.CsaParams(B, 16, hi, top_k, 128, ck.MODE_FULL, 1.0, 0)
    topk = torch.empty((B, top_k), dtype=torch.int32, device="cuda")
    qi, w = to_dev(c["qi"].view(np.int16)), to_dev(c["w"])
    ck.csa_select_topk(p, idxc, qi, w, topk, workspace(ck.csa_select_topk_workspace_bytes(p, cap)))
    torch.cuda.synchronize()
    batch = topk.cpu().numpy()
    idx = c["idx"]
    for b, n in enumerate(lens):
        p1 = ck.CsaParams(1, 16, hi, top_k, 128, ck.MODE_FULL, 1.0, 0)
        codes = to_dev(idx.codes[b:b + 1])
        scales = to_dev(idx.scales[b:b + 1]) if idx.scales is not None else None
        one = torch.empty((1, top_k), dtype=torch.int32, device="cuda")
        n_dev = _lens_dev([n])  # held until the call has run
        ck.csa_select_topk(p1, ck.cache(IDX_FMTS[idx.fmt], codes, cap, None, scales,
                                        seq_rows=n_dev),
                           qi[b:b + 1], w[b:b + 1], one,
                           workspace(ck.csa_select_topk_workspace_bytes(p1, cap)))
        torch.cuda.synchronize()
        assert (one.cpu().numpy()[0] == batch[b]).all(), f"sequence {b}"


def test_csa_varlen_lengths_clamped():
    # Lengths beyond the capacity act as the capacity; negative lengths as 0.
    lens_in, lens_eff, cap = [9999, -5], [3000, 0], 3000
    c = _varlen_case(405, lens_eff, cap, 64, 16, 8, 128, "bf16", "bf16")
    B, scale = 2, 1.0 / math.sqrt(D)
    kv, idx = c["kv"], c["idx"]
    kv_t, idx_t = to_dev(kv.codes), to_dev(idx.codes)
    kv_len = _lens_dev([64 + 9999, 64])   # clamped to the capacity; the window alone
    idx_len = _lens_dev(lens_in)
    kvc = ck.cache(KV_FMTS["bf16"], kv_t, 64 + cap, seq_rows=kv_len)
    idxc = ck.cache(IDX_FMTS["bf16"], idx_t, cap, seq_rows=idx_len)
    p = ck.CsaParams(B, 16, 8, 128, 64, ck.MODE_FULL, scale, 0)
    topk = torch.empty((B, 128), dtype=torch.int32, device="cuda")
    out = torch.empty((B, 16, D), dtype=torch.bfloat16, device="cuda")
    ck.csa_decode(p, kvc, idxc, to_dev(c["q"].view(np.int16)), to_dev(c["qi"].view(np.int16)),
                  to_dev(c["w"]), topk, out, workspace(ck.csa_decode_workspace_bytes(p, cap)))
    torch.cuda.synchronize()
    qv, qiv = OF.bf16_bits_to_f64(c["q"]), OF.bf16_bits_to_f64(c["qi"])
    got = out.double().cpu().numpy()
    for b, n in enumerate(lens_eff):
        o, sel = OD.csa_decode_one(qv[b], qiv[b], c["w"][b].astype(np.float64),
                                   idx.values[b][:n], kv.values[b][:64 + n], 64, 128, scale)
        assert topk_sets_equal(topk.cpu().numpy()[b:b + 1], sel[None])
        err, ok = attention_error(got[b], o)
        assert ok, (b, err)


@pytest.mark.parametrize("kv_fmt", ["bf16", "mixed", "fp4"])
def test_hca_varlen(kv_fmt):
    lens, cap, hq = [3000, 777, 0, 1], 3000, 64
    print(f"case: hca varlen lens={lens} {kv_fmt}", flush=True)
    T = seedgen.TID
    B, scale = len(lens), 1.0 / math.sqrt(D)
    q = bf16_bits(seedgen.bf16_normal(406, seedgen.tid(T.Q), (B, hq, D)))
    kv = encode_kv(bf16_bits(seedgen.kv_rows_bf16(406, seedgen.tid(T.KV), (B, cap, D))), kv_fmt)
    codes = to_dev(kv.codes)
    scales = to_dev(kv.scales) if kv.scales is not None else None
    lens_dev = _lens_dev(lens)  # held until the call has run
    kvc = ck.cache(KV_FMTS[kv_fmt], codes, cap, None, scales, seq_rows=lens_dev)
    out = Guarded((B, hq, D), torch.int16)
    ck.hca_decode(B, hq, scale, kvc, to_dev(q.view(np.int16)), out.t,
                  workspace(ck.hca_decode_workspace_bytes(B, hq, cap)))
    torch.cuda.synchronize()
    assert out.intact()
    got = out.t.cpu().view(torch.bfloat16).double().numpy()
    qv = OF.bf16_bits_to_f64(q)
    for b, n in enumerate(lens):
        ref = OD.hca_decode_one(qv[b], kv.values[b][:n], scale) if n > 0 else np.zeros((hq, D))
        err, ok = attention_error(got[b], ref)
        print(f"  b={b} n={n}: max |out - oracle| = {err:.3e}")
        assert ok, (b, err)


def test_reindex_varlen():
    # Pool rows at or past a sequence's length are empty slots.  The pool is every row of
    # the capacity, so each sequence's pool top-k is its (tie-free) full top-k.
    lens, cap, hi, top_k = [3000, 1500], 3000, 64, 128
    c = _varlen_case(407, lens, cap, 0, 16, hi, top_k, "bf16", "fp4")
    B = len(lens)
    rng = np.random.default_rng(407)
    pool = np.stack([rng.permutation(cap) for _ in range(B)]).astype(np.int32)
    _, idxc, keep = _caches(c, lens, cap, 0)
    p = ck.CsaParams(B, 0, hi, top_k, 0, ck.MODE_REINDEX, 1.0, 0)
    topk = torch.empty((B, top_k), dtype=torch.int32, device="cuda")
    ck.csa_reindex_topk(p, idxc, to_dev(c["qi"].view(np.int16)), to_dev(c["w"]), to_dev(pool),
                        cap, topk, workspace(ck.csa_reindex_topk_workspace_bytes(p, cap)))
    torch.cuda.synchronize()
    got = topk.cpu().numpy()
    qiv = OF.bf16_bits_to_f64(c["qi"])
    for b, n in enumerate(lens):
        want = OD.reindex_topk(qiv[b], c["w"][b].astype(np.float64), c["idx"].values[b][:n],
                               pool[b], top_k)
        assert topk_sets_equal(got[b:b + 1], np.asarray(want)[None]), f"sequence {b}"
