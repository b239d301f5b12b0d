"""csa_decode_noalloc (the library's own device scratch instead of a caller workspace)
against csa_decode with a workspace: the same kernels, so the same top-k sets and outputs
bit for bit, on two calls in a row (the second smaller than the first, so it reads
scratch the first one left), under a hipGraph, and the oracle's results."""
import numpy as np
import pytest
import torch

import compressed_sparse_kv_csa_amd as ck
from cases import attention_error, make_csa_case, topk_sets_equal
from gpu_helpers import Guarded, to_dev, upload_idx, upload_kv, workspace

pytestmark = pytest.mark.gpu


def _inputs(case):
    p = ck.CsaParams(case.B, case.hq, case.hi, case.top_k, case.window, ck.MODE_FULL, case.scale, 0)
    kv, k1 = upload_kv(case.kv)
    idx, k2 = upload_idx(case.idx)
    return p, kv, idx, (to_dev(case.q_bits.view(np.int16)), to_dev(case.q_idx_bits.view(np.int16)),
                        to_dev(case.w)), (k1, k2)


def _with_workspace(case):
    p, kv, idx, (q, qi, w), keep = _inputs(case)
    topk = torch.empty((case.B, case.top_k), dtype=torch.int32, device="cuda")
    out = torch.empty((case.B, case.hq, 512), dtype=torch.int16, device="cuda")
    ck.csa_decode(p, kv, idx, q, qi, w, topk, out, workspace(ck.csa_decode_workspace_bytes(p, case.n_c)))
    torch.cuda.synchronize()
    return topk.cpu().numpy(), out.cpu().numpy()


def _noalloc(case):
    p, kv, idx, (q, qi, w), keep = _inputs(case)
    assert ck.csa_decode_workspace_bytes(p, case.n_c) <= ck.csa_decode_noalloc_scratch_bytes()
    topk = Guarded((case.B, case.top_k), torch.int32)
    out = Guarded((case.B, case.hq, 512), torch.int16)
    ck.csa_decode_noalloc(p, kv, idx, q, qi, w, topk.t, out.t)
    torch.cuda.synchronize()
    assert topk.intact() and out.intact()
    return topk.t.cpu().numpy(), out.t.cpu().numpy()


def _check_oracle(case, topk, out):
    assert topk_sets_equal(topk, case.expect_topk)
    err, ok = attention_error(torch.from_numpy(out).view(torch.bfloat16).double().numpy(), case.expect_out)
    assert ok, err


def test_noalloc_equals_workspace_on_two_calls():
    print("case: csa_decode_noalloc, a large call then a smaller one", flush=True)
    big = make_csa_case(951, 3, 20000, 128, 64, 64, 512, "mixed", "fp4")
    small = make_csa_case(952, 1, 3001, 128, 32, 16, 256, "fp4", "bf16")
    for case in (big, small):
        ref = _with_workspace(case)
        got = _noalloc(case)
        assert np.array_equal(got[0], ref[0]), "top-k differs from csa_decode"
        assert np.array_equal(got[1], ref[1]), "output differs from csa_decode"
        _check_oracle(case, *got)


def test_noalloc_under_a_graph():
    print("case: csa_decode_noalloc captured in a hipGraph", flush=True)
    case = make_csa_case(953, 2, 9000, 128, 64, 64, 512, "bf16", "fp4")
    ref = _with_workspace(case)
    p, kv, idx, (q, qi, w), keep = _inputs(case)
    topk = torch.empty((case.B, case.top_k), dtype=torch.int32, device="cuda")
    out = torch.empty((case.B, case.hq, 512), dtype=torch.int16, device="cuda")
    cur = torch.cuda.current_stream
    ck.csa_decode_noalloc(p, kv, idx, q, qi, w, topk, out, stream=cur().cuda_stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        ck.csa_decode_noalloc(p, kv, idx, q, qi, w, topk, out, stream=cur().cuda_stream)
    for r in range(2):
        topk.fill_(-3)
        out.fill_(0x2222)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(topk.cpu().numpy(), ref[0]), r
        assert np.array_equal(out.cpu().numpy(), ref[1]), r


def test_noalloc_rejects_requests_beyond_the_scratch():
    # 32 sequences of 262,144 keys need more workspace than the 32 MiB scratch: rejected
    # before any launch (the pointers are never dereferenced)
    fake = 1 << 20
    p = ck.CsaParams(32, 64, 64, 512, 128, ck.MODE_FULL, 0.044, 0)
    n_c = 262144
    assert ck.csa_decode_workspace_bytes(p, n_c) > ck.csa_decode_noalloc_scratch_bytes()
    kv = ck.Cache(ck.KV_FP8_MIXED, 0, 128 + n_c, 128 + n_c, fake, None)
    idx = ck.Cache(ck.IDX_BF16, 0, n_c, n_c, fake, None)
    st = ck.csa_decode_noalloc(p, kv, idx, fake, fake, fake, fake, fake, stream=0, check=False)
    assert st == ck.ERR_WORKSPACE
    assert ck.csa_decode_noalloc_scratch_bytes() == 32 << 20
