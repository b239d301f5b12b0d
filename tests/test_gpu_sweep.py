"""A seeded sweep of small CSA and HCA decode configurations on the GPU against the oracle.

The configurations are drawn once from a fixed generator over the whole supported
range: batch sizes, compressed lengths that are not multiples of the 16-row tile,
windows from none to 128, query heads 16..128, indexer heads 1..128, top-k from 1 to
2048 (some beyond N_c), and every pairing of main-KV and indexer-key formats.  Each
case is checked like the hand-picked ones: top-k index sets bit-exact (inputs made
tie-free), outputs within 1e-2 max-abs."""
import math

import numpy as np
import pytest
import torch

import compressed_sparse_kv_csa_amd as ck
import seedgen
from cases import (attention_error, bf16_bits, encode_kv, indexer_query_values, make_csa_case,
                   oracle_hca, topk_sets_equal)
from gpu_helpers import run_csa, to_dev, upload_kv, workspace

pytestmark = pytest.mark.gpu


def _csa_specs(n=48):
    g = np.random.default_rng(20261203)
    specs = []
    for i in range(n):
        B = int(g.choice([1, 2, 3, 5]))
        n_c = int(g.integers(1, 6000))
        W = int(g.choice([0, 1, 37, 128]))
        hq = int(g.choice([16, 32, 48, 64, 80, 128]))
        hi = int(g.choice([1, 3, 16, 17, 33, 64, 128]))
        k = int(g.choice([1, 5, 64, 333, 512, 1024, 2048]))
        kv = str(g.choice(["bf16", "mixed", "fp4"]))
        idx = str(g.choice(["bf16", "fp4", "fp4h"]))
        specs.append((3000 + i, B, n_c, W, hq, hi, k, kv, idx))
    return specs


def _hca_specs(n=12):
    g = np.random.default_rng(20261204)
    return [(3100 + i, int(g.choice([1, 2, 3, 7])), int(g.integers(1, 5000)),
             int(g.choice([16, 48, 64, 96, 128])), str(g.choice(["bf16", "mixed", "fp4"])))
            for i in range(n)]


@pytest.mark.parametrize("spec", _csa_specs(), ids=lambda s: "-".join(map(str, s)))
def test_csa_sweep(spec):
    seed, B, n_c, W, hq, hi, k, kvf, idf = spec
    print(f"case: csa sweep seed={seed} B={B} Nc={n_c} W={W} Hq={hq} HI={hi} k={k} kv={kvf} idx={idf}",
          flush=True)
    case = make_csa_case(seed, B, n_c, W, hq, hi, k, kvf, idf)
    topk, out = run_csa(case)
    assert topk_sets_equal(topk, case.expect_topk)
    err, ok = attention_error(out, case.expect_out)
    assert ok, err


@pytest.mark.parametrize("spec", _hca_specs(), ids=lambda s: "-".join(map(str, s)))
def test_hca_sweep(spec):
    seed, B, rows, hq, kvf = spec
    print(f"case: hca sweep seed={seed} B={B} rows={rows} Hq={hq} kv={kvf}", flush=True)
    T = seedgen.TID
    q_bits = bf16_bits(seedgen.bf16_normal(seed, seedgen.tid(T.Q), (B, hq, 512)))
    kv = encode_kv(bf16_bits(seedgen.kv_rows_bf16(seed, seedgen.tid(T.KV), (B, rows, 512))), kvf)
    kvc, keep = upload_kv(kv)
    out = torch.empty((B, hq, 512), dtype=torch.int16, device="cuda")
    ws = workspace(ck.hca_decode_workspace_bytes(B, hq, rows))
    scale = 1.0 / math.sqrt(512)
    ck.hca_decode(B, hq, scale, kvc, to_dev(q_bits.view(np.int16)), out, ws)
    torch.cuda.synchronize()
    got = out.cpu().view(torch.bfloat16).double().numpy()
    err, ok = attention_error(got, oracle_hca(q_bits, kv, scale))
    assert ok, err


def _paged_specs(n=12):
    g = np.random.default_rng(20261205)
    specs = []
    for i in range(n):
        B = int(g.choice([1, 2, 3]))
        cap = int(g.integers(200, 7000))
        # per-sequence lengths: full, ragged, short, or empty
        lens = [int(g.choice([cap, int(g.integers(1, cap + 1)), int(g.integers(1, 64)), 0])) for _ in range(B)]
        W = int(g.choice([0, 37, 128]))
        hq = int(g.choice([16, 64, 128]))
        hi = int(g.choice([3, 16, 64]))
        k = int(g.choice([1, 64, 512, 2048]))
        kv = str(g.choice(["bf16", "mixed", "fp4"]))
        idx = str(g.choice(["bf16", "fp4", "fp4h"]))
        kv_pr = int(g.choice([16, 32, 256, 4096]))
        idx_pr = int(g.choice([16, 64, 1024]))
        specs.append((3200 + i, tuple(lens), cap, W, hq, hi, k, kv, idx, kv_pr, idx_pr))
    return specs


@pytest.mark.parametrize("spec", _paged_specs(), ids=lambda s: "-".join(map(str, s)))
def test_paged_varlen_sweep(spec):
    """Paged caches with per-sequence lengths: the same result as contiguous caches with
    those lengths, bit for bit, and each sequence's selection and output the oracle's over
    the rows it holds."""
    from oracle import decode as OD, formats as OF
    from test_gpu_paged import _idx_cache, _kv_cache
    from test_gpu_varlen import _varlen_case
    seed, lens, cap, W, hq, hi, k, kvf, idf, kv_pr, idx_pr = spec
    print(f"case: paged varlen sweep seed={seed} lens={lens} cap={cap} W={W} Hq={hq} HI={hi} k={k} "
          f"kv={kvf} idx={idf} pages={kv_pr}/{idx_pr}", flush=True)
    B = len(lens)
    c = _varlen_case(seed, list(lens), cap, W, hq, hi, k, kvf, idf)
    kv_len = torch.tensor([W + n for n in lens], dtype=torch.int32, device="cuda")
    idx_len = torch.tensor(list(lens), dtype=torch.int32, device="cuda")
    p = ck.CsaParams(B, hq, hi, k, W, ck.MODE_FULL, 1.0 / math.sqrt(512), 0)
    res = []
    for kp, ip in ((0, 0), (kv_pr, idx_pr)):
        kvc = _kv_cache(c["kv"], kp, seed, kv_len)
        idxc = _idx_cache(c["idx"], ip, seed + 1, idx_len)
        topk = torch.empty((B, k), dtype=torch.int32, device="cuda")
        out = torch.empty((B, hq, 512), dtype=torch.bfloat16, device="cuda")
        ck.csa_decode(p, kvc, idxc, to_dev(c["q"].view(np.int16)), to_dev(c["qi"].view(np.int16)),
                      to_dev(c["w"]), topk, out, workspace(ck.csa_decode_workspace_bytes(p, cap)))
        torch.cuda.synchronize()
        res.append((topk.cpu().numpy(), out.view(torch.int16).cpu().numpy()))
    assert np.array_equal(res[0][0], res[1][0]), "selected indices differ"
    assert np.array_equal(res[0][1], res[1][1]), "outputs differ"
    qv = OF.bf16_bits_to_f64(c["q"])
    qiv = indexer_query_values(c["qi"], idf)
    out = torch.from_numpy(res[1][1]).view(torch.bfloat16).double().numpy()
    for b, n in enumerate(lens):
        sel = OD.topk_indices(OD.indexer_scores(qiv[b], c["w"][b].astype(np.float64),
                                                c["idx"].values[b, :n]), k)
        assert topk_sets_equal(res[1][0][b:b + 1], sel[None]), b
        ref = OD.attention(qv[b], OD.csa_rows(c["kv"].values[b, :W + n], W, sel), p.softmax_scale)
        err, ok = attention_error(out[b], ref)
        assert ok, (b, err)


def _reindex_specs(n=12):
    g = np.random.default_rng(20261206)
    specs = []
    for i in range(n):
        n_pool = int(g.choice([1, 16, 333, 1024, 4096]))
        n_c = int(g.integers(max(n_pool, 2), 9000))
        specs.append((3300 + i, int(g.choice([1, 2, 3])), n_c, int(g.choice([1, 3, 16, 64, 128])),
                      n_pool, int(g.choice([1, 20, 512, 2048])), str(g.choice(["bf16", "fp4", "fp4h"])),
                      int(g.choice([0, 0, 1, 7]))))
    return specs


@pytest.mark.parametrize("spec", _reindex_specs(), ids=lambda s: "-".join(map(str, s)))
def test_reindex_sweep(spec):
    from test_gpu_reindex import check, make_case, run_reindex
    seed, B, n_c, hi, n_pool, k, fmt, n_empty = spec
    n_empty = min(n_empty, n_pool - 1)
    print(f"case: reindex sweep seed={seed} B={B} Nc={n_c} HI={hi} pool={n_pool} k={k} {fmt} "
          f"empty={n_empty}", flush=True)
    c = make_case(seed, B, n_c, hi, n_pool, k, fmt, n_empty)
    check(c, run_reindex(c))
