"""Scan workgroups that own several 4096-row slices, with sequences ending anywhere in them.

At B = 8 and 262,144 rows of capacity the indexer runs 32 workgroups per query, each
owning two slices: the key tiles of a slice are handed out to the workgroup's waves from
a counter, and a wave's next tiles after a slice's last are its first ones of the next
slice.  Per-sequence lengths put a sequence's end at a full slice, inside the second
slice of a workgroup, one row past a slice boundary, in the first slice, at one row and at
none, so workgroups have two, one or no slices with rows and ragged last slices.  The
oracle checks those sequences over their own rows only: top-k index sets bit-exact (keys
made tie-free over the sequence's rows), attention outputs within 1e-2 max-abs.  The
same batch through a paged cache (block tables with shuffled pages) must give identical
bytes."""
import numpy as np
import pytest
import torch

import compressed_sparse_kv_csa_amd as ck
import seedgen
from cases import D, DI, IDX_FMTS, KV_FMTS, attention_error, bf16_bits, topk_sets_equal
from fullsize import DEV, _dev, make_kv_cache, query_bits, scale_of
from oracle import decode as OD, formats as OF, tiefree

pytestmark = [pytest.mark.gpu, pytest.mark.fullsize]

T = seedgen.TID
SEED, B, CAP, W, HQ, HI, K = 61, 8, 262144, 128, 16, 64, 512
LENS = [262144, 261000, 200001, 131073, 8193, 4096, 1, 0]
CHECK = [1, 2, 3, 4, 6, 7]  # ragged in a second slice, in a first slice, one row past a
                            # boundary, a workgroup's first slice plus one row, one row, none


def _indexer(fmt):
    qi = seedgen.bf16_normal(SEED, seedgen.tid(T.Q_IDX), (B, HI, DI))
    w = seedgen.uniform01(SEED, seedgen.tid(T.W_IDX), (B, HI))
    keys = seedgen.bf16_normal(SEED, seedgen.tid(T.IDX_KEYS), (B, CAP, DI), DEV)
    codes = torch.empty((B, CAP, 64), dtype=torch.uint8, device=DEV)
    scales = torch.empty((B, CAP, 8), dtype=torch.uint8, device=DEV)
    ck.kv_quantize_fp4(keys, B * CAP, DI, codes, scales)
    qv, wv = qi.double().numpy(), w.double().numpy()
    values = {}
    for b in CHECK:  # tie-free over the sequence's own rows, stored with the oracle's codec
        n = LENS[b]
        if n == 0:
            values[b] = np.zeros((0, DI))
            continue
        adj, _ = tiefree.make_tie_free(bf16_bits(keys[b, :n])[None], qv[b:b + 1], wv[b:b + 1], K, fmt)
        c, s = OF.fp4_quantize(OF.bf16_bits_to_f64(adj[0]))
        codes[b, :n] = _dev(c)
        scales[b, :n] = _dev(s)
        values[b] = OF.fp4_dequantize(c, s)
    del keys
    return codes, scales, _dev(bf16_bits(qi).view(np.int16)), w.to(DEV), qv, wv, values


def _paged(t, page_rows, seed):
    """The same rows in a shuffled page pool: (pool, table [B][pages])."""
    rows = t.shape[1]
    assert rows % page_rows == 0
    n_pages = rows // page_rows
    perm = np.random.default_rng(seed).permutation(B * n_pages)
    table = torch.from_numpy(perm.reshape(B, n_pages).astype(np.int32)).to(DEV)
    pool = torch.empty((B * n_pages, page_rows) + tuple(t.shape[2:]), dtype=t.dtype, device=DEV)
    pool[table.flatten().long()] = t.reshape((B * n_pages, page_rows) + tuple(t.shape[2:]))
    return pool, table


def test_multi_slice_workgroups_varlen_and_paged():
    print(f"case: multi-slice scan B={B} cap={CAP} lens={LENS} HI={HI} k={K} fp4/fp4", flush=True)
    codes, scales, qi, w, qv, wv, key_values = _indexer("fp4")
    kv = make_kv_cache(SEED, 0, B, W + CAP, "fp4")
    q, qf = query_bits(SEED, 0, B, HQ)
    expect = {}
    for b in CHECK:
        n = LENS[b]
        sel = OD.topk_indices(OD.indexer_scores(qv[b], wv[b], key_values[b]), K) if n else np.full(K, -1)
        rows = np.concatenate([np.arange(W), W + sel[sel >= 0]]).astype(np.int64)
        expect[b] = (sel, OD.attention(qf[b], kv.put_oracle_rows(b, rows), scale_of()))
    kv_len = torch.tensor([W + n for n in LENS], dtype=torch.int32, device=DEV)
    idx_len = torch.tensor(LENS, dtype=torch.int32, device=DEV)
    p = ck.CsaParams(B, HQ, HI, K, W, ck.MODE_FULL, scale_of(), 0)
    ws = torch.empty(ck.csa_decode_workspace_bytes(p, CAP), dtype=torch.uint8, device=DEV)
    results = []
    for paged in (False, True):
        if paged:
            kc, kt = _paged(kv.codes, 128, SEED)  # W + CAP = 2049 pages of 128 rows
            ks, _ = _paged(kv.scales, 128, SEED)
            ic, it = _paged(codes, 8192, SEED + 1)
            isc, _ = _paged(scales, 8192, SEED + 1)
            kvc = ck.cache(KV_FMTS["fp4"], kc, W + CAP, 0, ks, seq_rows=kv_len, block_table=kt, page_rows=128)
            idxc = ck.cache(IDX_FMTS["fp4"], ic, CAP, 0, isc, seq_rows=idx_len, block_table=it, page_rows=8192)
        else:
            kvc = ck.cache(KV_FMTS["fp4"], kv.codes, W + CAP, None, kv.scales, seq_rows=kv_len)
            idxc = ck.cache(IDX_FMTS["fp4"], codes, CAP, None, scales, seq_rows=idx_len)
        topk = torch.empty((B, K), dtype=torch.int32, device=DEV)
        out = torch.empty((B, HQ, D), dtype=torch.int16, device=DEV)
        ck.csa_decode(p, kvc, idxc, q, qi, w, topk, out, ws)
        torch.cuda.synchronize()
        results.append((topk.cpu().numpy(), out.cpu().numpy()))
    assert np.array_equal(results[0][0], results[1][0]), "paged selection differs"
    assert np.array_equal(results[0][1], results[1][1]), "paged output differs"
    tk = results[0][0]
    got = torch.from_numpy(results[0][1]).view(torch.bfloat16).double().numpy()
    for b in CHECK:
        sel, ref = expect[b]
        assert topk_sets_equal(tk[b:b + 1], sel[None]), f"top-k set of sequence {b} (rows {LENS[b]})"
        err, ok = attention_error(got[b], ref)
        print(f"  b={b} rows={LENS[b]}: max |out - oracle| = {err:.3e}", flush=True)
        assert ok, (b, err)
