"""CSA decode on the GPU against the oracle: top-k index sets bit-exact (inputs made
tie-free), attention outputs within 1e-2 max-abs (bf16 out, fp32 accumulation)."""
import numpy as np
import pytest

import compressed_sparse_kv_csa_amd as ck
from cases import attention_error, make_csa_case, oracle_reuse, topk_sets_equal
from gpu_helpers import run_csa

pytestmark = pytest.mark.gpu


def _check(case, topk, out):
    assert topk_sets_equal(topk, case.expect_topk)
    err, ok = attention_error(out, case.expect_out)
    print(f"max |out - oracle| = {err:.3e}  max |oracle| = {np.abs(case.expect_out).max():.3f}")
    assert ok, err


# (seed, B, N_c, window, H_q, H_I, top_k, kv_fmt, idx_fmt)
CASES = [
    # the tiny configuration: 4096 tokens -> 1024 entries, 16 q heads, 4 indexer heads
    (1, 1, 1024, 128, 16, 4, 512, "bf16", "bf16"),
    # several slices with a ragged tail, every storage combination
    (101, 3, 3001, 128, 64, 64, 512, "bf16", "bf16"),
    (102, 3, 3001, 128, 64, 64, 512, "mixed", "fp4"),
    (103, 3, 3001, 128, 64, 64, 512, "fp4", "fp4"),
    (104, 2, 3001, 128, 64, 64, 512, "bf16", "fp4"),
    (105, 2, 3001, 128, 64, 64, 512, "mixed", "bf16"),
    # many slices: the merge reads prefixes of 9 slices
    (106, 2, 9000, 128, 64, 64, 512, "mixed", "fp4"),
    # head counts that are not full tiles, small k
    (107, 2, 2500, 100, 32, 17, 100, "bf16", "bf16"),
    (108, 2, 2500, 64, 48, 1, 64, "fp4", "bf16"),
    # N_c < k (-1 padding), N_c == k, k == 1, no window
    (109, 2, 300, 128, 16, 4, 512, "bf16", "bf16"),
    (110, 1, 512, 128, 16, 4, 512, "mixed", "fp4"),
    (111, 2, 2000, 128, 16, 8, 1, "bf16", "fp4"),
    (112, 2, 1500, 0, 64, 64, 512, "bf16", "bf16"),
    # top_k 1024 (the V4-Pro configuration's value)
    (113, 1, 5000, 128, 64, 64, 1024, "fp4", "fp4"),
    # 128 query heads (V4-Pro's query), 128 and 80 indexer heads, top_k up to 2048
    (114, 2, 3001, 128, 128, 128, 512, "mixed", "fp4"),
    (115, 2, 6000, 128, 128, 80, 2048, "fp4", "bf16"),
    (116, 1, 9000, 128, 64, 64, 2048, "mixed", "fp4"),
    (117, 2, 5000, 128, 128, 128, 1024, "bf16", "fp4h"),
    # lists of 2048 rows and more run on the 64-head workgroups: bf16 rows there too
    (118, 2, 5000, 128, 64, 64, 2048, "bf16", "bf16"),
]


@pytest.mark.parametrize("spec", CASES, ids=lambda s: "-".join(map(str, s)))
def test_csa_full_parity(spec):
    seed, B, n_c, W, hq, hi, k, kvf, idf = spec
    print(f"case: csa FULL seed={seed} B={B} Nc={n_c} W={W} Hq={hq} HI={hi} k={k} kv={kvf} idx={idf}",
          flush=True)
    case = make_csa_case(seed, B, n_c, W, hq, hi, k, kvf, idf)
    topk, out = run_csa(case, stride_pad=3)
    _check(case, topk, out)


def test_csa_window_only():
    print("case: csa FULL with N_c = 0", flush=True)
    case = make_csa_case(120, 2, 0, 128, 16, 4, 512, "bf16", "bf16")
    topk, out = run_csa(case)
    assert (topk == -1).all()
    _check(case, topk, out)


def test_csa_reuse_equals_full():
    print("case: csa REUSE with FULL's indices", flush=True)
    case = make_csa_case(121, 2, 3001, 128, 64, 64, 512, "mixed", "fp4")
    topk, out = run_csa(case)
    _check(case, topk, out)
    _, out_r = run_csa(case, mode=ck.MODE_REUSE, topk_in=topk)
    assert np.array_equal(out_r, out)


@pytest.mark.parametrize("kvf", ["bf16", "mixed", "fp4"])
def test_csa_reuse_own_cache(kvf):
    """A Reuse layer attends over its own cache with another layer's indices, including
    padding (-1) and out-of-range entries, which are skipped."""
    print(f"case: csa REUSE own cache kv={kvf}", flush=True)
    full = make_csa_case(122, 2, 4000, 128, 64, 64, 512, "fp4", "fp4")
    layer = make_csa_case(122, 2, 4000, 128, 64, 64, 512, kvf, "fp4", layer=3, with_indexer=False,
                          expect=False)
    sel = full.expect_topk.copy()
    sel[0, 500:] = -1
    sel[1, 7] = 4000           # out of range: skipped
    _, out = run_csa(layer, mode=ck.MODE_REUSE, topk_in=sel)
    sel_ref = sel.copy(); sel_ref[1, 7] = -1
    ref = oracle_reuse(layer, sel_ref)
    err, ok = attention_error(out, ref)
    assert ok, err


def test_csa_deterministic():
    print("case: csa run-twice determinism", flush=True)
    case = make_csa_case(123, 2, 6000, 128, 64, 64, 512, "mixed", "fp4")
    (t1, o1), (t2, o2) = run_csa(case, repeat=2)
    assert np.array_equal(t1, t2) and np.array_equal(o1, o2)
    _check(case, t1, o1)


def test_csa_select_topk_matches_full():
    """The indexer stage alone writes the same index set, byte for byte, as FULL decode."""
    print("case: csa_select_topk vs FULL", flush=True)
    import torch
    from gpu_helpers import to_dev, upload_idx, workspace
    case = make_csa_case(124, 3, 70000, 128, 64, 64, 512, "bf16", "fp4")
    topk_full, out = run_csa(case)
    _check(case, topk_full, out)
    p = ck.CsaParams(case.B, case.hq, case.hi, case.top_k, case.window, ck.MODE_FULL, case.scale, 0)
    idx, keep = upload_idx(case.idx)
    tk = torch.full((case.B, case.top_k), -7, dtype=torch.int32, device="cuda")
    ws = workspace(ck.csa_select_topk_workspace_bytes(p, case.n_c))
    ck.csa_select_topk(p, idx, to_dev(case.q_idx_bits.view(np.int16)), to_dev(case.w), tk, ws)
    torch.cuda.synchronize()
    assert np.array_equal(tk.cpu().numpy(), topk_full)
    # the same through its two stages, scan then merge
    tk2 = torch.full((case.B, case.top_k), -7, dtype=torch.int32, device="cuda")
    ws.fill_(0x5A)
    ck.csa_select_scan(p, idx, to_dev(case.q_idx_bits.view(np.int16)), to_dev(case.w), ws)
    ck.csa_select_merge(p, idx, tk2, ws)
    torch.cuda.synchronize()
    assert np.array_equal(tk2.cpu().numpy(), topk_full)
