"""Decode steps captured in a hipGraph (as the bench times them) and replayed several
times, with other eager work and synchronisations between the replays: every replay must
give the eager result bit for bit (the kernels are deterministic and the library records
no memset or allocation), and the eager result is the oracle's."""
import numpy as np
import pytest
import torch

import compressed_sparse_kv_csa_amd as ck
from cases import attention_error, make_csa_case, topk_sets_equal
from gpu_helpers import to_dev, upload_idx, upload_kv, workspace

pytestmark = pytest.mark.gpu


def _csa_inputs(case):
    p = ck.CsaParams(case.B, case.hq, case.hi, case.top_k, case.window, ck.MODE_FULL, case.scale, 0)
    kv, k1 = upload_kv(case.kv)
    idx, k2 = upload_idx(case.idx)
    t = dict(q=to_dev(case.q_bits.view(np.int16)), qi=to_dev(case.q_idx_bits.view(np.int16)),
             w=to_dev(case.w), topk=torch.empty((case.B, case.top_k), dtype=torch.int32, device="cuda"),
             out=torch.empty((case.B, case.hq, 512), dtype=torch.int16, device="cuda"),
             ws=workspace(ck.csa_decode_workspace_bytes(p, case.n_c)), keep=(k1, k2))
    return p, kv, idx, t


def _run(p, kv, idx, t, stream):
    ck.csa_decode(p, kv, idx, t["q"], t["qi"], t["w"], t["topk"], t["out"], t["ws"], stream=stream)


def test_csa_graph_replays_equal_eager():
    print("case: csa_decode in a hipGraph, 4 replays", flush=True)
    case = make_csa_case(901, 2, 9000, 128, 64, 64, 512, "mixed", "fp4")
    other = make_csa_case(902, 2, 5000, 128, 64, 64, 512, "fp4", "fp4", expect=False)
    p, kv, idx, t = _csa_inputs(case)
    po, kvo, idxo, to = _csa_inputs(other)
    cur = torch.cuda.current_stream
    _run(p, kv, idx, t, cur().cuda_stream)
    torch.cuda.synchronize()
    eager = (t["topk"].cpu().numpy().copy(), t["out"].cpu().numpy().copy())
    assert topk_sets_equal(eager[0], case.expect_topk)
    err, ok = attention_error(torch.from_numpy(eager[1]).view(torch.bfloat16).double().numpy(),
                              case.expect_out)
    assert ok, err
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        _run(p, kv, idx, t, cur().cuda_stream)
    for r in range(4):
        t["topk"].fill_(-5)
        t["out"].fill_(0x7BCD)
        t["ws"].fill_(0xA5)
        _run(po, kvo, idxo, to, cur().cuda_stream)          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(t["topk"].cpu().numpy(), eager[0]), f"replay {r}: top-k"
        assert np.array_equal(t["out"].cpu().numpy(), eager[1]), f"replay {r}: output"


def test_hca_graph_replays_equal_eager():
    print("case: hca_decode in a hipGraph, 3 replays", flush=True)
    import math
    import seedgen
    from cases import bf16_bits, encode_kv, oracle_hca
    T = seedgen.TID
    B, rows, hq = 3, 3000, 64
    q_bits = bf16_bits(seedgen.bf16_normal(903, seedgen.tid(T.Q), (B, hq, 512)))
    kv = encode_kv(bf16_bits(seedgen.kv_rows_bf16(903, seedgen.tid(T.KV), (B, rows, 512))), "fp4")
    kvc, keep = upload_kv(kv)
    q = to_dev(q_bits.view(np.int16))
    out = torch.empty((B, hq, 512), dtype=torch.int16, device="cuda")
    ws = workspace(ck.hca_decode_workspace_bytes(B, hq, rows))
    scale = 1.0 / math.sqrt(512)
    cur = torch.cuda.current_stream
    ck.hca_decode(B, hq, scale, kvc, q, out, ws, stream=cur().cuda_stream)
    torch.cuda.synchronize()
    eager = out.cpu().numpy().copy()
    err, ok = attention_error(torch.from_numpy(eager).view(torch.bfloat16).double().numpy(),
                              oracle_hca(q_bits, kv, scale))
    assert ok, err
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        ck.hca_decode(B, hq, scale, kvc, q, out, ws, stream=cur().cuda_stream)
    for r in range(3):
        out.fill_(0x1234)
        ws.fill_(0x3C)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), eager), f"replay {r}"
