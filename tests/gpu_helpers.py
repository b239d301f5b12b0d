"""Upload seeded cases to the GPU and run them through the C ABI (GPU tests only)."""
from __future__ import annotations

import numpy as np
import torch

import compressed_sparse_kv_csa_amd as ck
from cases import IDX_FMTS, KV_FMTS, CsaCase, IdxCache, KvCache

DEV = "cuda"
CANARY = 0x5A


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def padded_rows(a: np.ndarray, stride: int) -> np.ndarray:
    """[B][rows][...] -> [B][stride][...] with the extra rows filled with canary bytes."""
    B, rows = a.shape[:2]
    out = np.full((B, stride) + a.shape[2:], CANARY, dtype=a.dtype)
    out[:, :rows] = a
    return out


def upload_kv(kv: KvCache, stride_pad: int = 0):
    B, rows = kv.codes.shape[:2]
    stride = rows + stride_pad
    codes = to_dev(padded_rows(kv.codes, stride))
    scales = to_dev(padded_rows(kv.scales, stride)) if kv.scales is not None else None
    return ck.cache(KV_FMTS[kv.fmt], codes, rows, stride, scales), (codes, scales)


def upload_idx(idx: IdxCache, stride_pad: int = 0):
    B, rows = idx.codes.shape[:2]
    stride = rows + stride_pad
    codes = to_dev(padded_rows(idx.codes, stride))
    scales = to_dev(padded_rows(idx.scales, stride)) if idx.scales is not None else None
    return ck.cache(IDX_FMTS[idx.fmt], codes, rows, stride, scales), (codes, scales)


class Guarded:
    """A device buffer with canary bytes on both sides, to catch stray writes."""

    PAD = 4096

    def __init__(self, shape, dtype):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.raw = torch.full((n + 2 * self.PAD,), CANARY, dtype=torch.uint8, device=DEV)
        self.t = self.raw[self.PAD:self.PAD + n].view(dtype).view(*shape)

    def intact(self) -> bool:
        r = self.raw.cpu().numpy()
        return bool((r[:self.PAD] == CANARY).all() and (r[-self.PAD:] == CANARY).all())


def workspace(nbytes: int) -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=DEV)


def run_csa(case: CsaCase, mode: int = ck.MODE_FULL, topk_in: np.ndarray | None = None,
            stride_pad: int = 0, repeat: int = 1):
    p = ck.CsaParams(case.B, case.hq, case.hi if mode == ck.MODE_FULL else 0, case.top_k,
                     case.window, mode, case.scale, 0)
    kv, keep_kv = upload_kv(case.kv, stride_pad)
    q = to_dev(case.q_bits.view(np.int16))
    out = Guarded((case.B, case.hq, 512), torch.int16)
    topk = Guarded((case.B, case.top_k), torch.int32)
    if mode == ck.MODE_FULL:
        idx, keep_idx = upload_idx(case.idx, stride_pad)
        qi = to_dev(case.q_idx_bits.view(np.int16))
        w = to_dev(case.w)
    else:
        idx, keep_idx, qi, w = None, None, None, None
        topk.t.copy_(torch.from_numpy(np.ascontiguousarray(topk_in.astype(np.int32))))
    ws = workspace(ck.csa_decode_workspace_bytes(p, case.n_c))
    results = []
    for _ in range(repeat):
        ck.csa_decode(p, kv, idx, q, qi, w, topk.t, out.t, ws)
        torch.cuda.synchronize()
        results.append((topk.t.cpu().numpy().copy(), out.t.cpu().view(torch.bfloat16).double().numpy()))
    assert out.intact() and topk.intact(), "write outside the output buffers"
    if repeat == 1:
        return results[0]
    return results


def run_hca(q_bits: np.ndarray, kv: KvCache, scale: float, stride_pad: int = 0):
    B, hq = q_bits.shape[:2]
    kvc, keep = upload_kv(kv, stride_pad)
    q = to_dev(q_bits.view(np.int16))
    out = Guarded((B, hq, 512), torch.int16)
    ws = workspace(ck.hca_decode_workspace_bytes(B, hq, kv.codes.shape[1]))
    ck.hca_decode(B, hq, scale, kvc, q, out.t, ws)
    torch.cuda.synchronize()
    assert out.intact(), "write outside the output buffer"
    return out.t.cpu().view(torch.bfloat16).double().numpy()
