"""Workload-sized decode cases for the GPU parity tests, checked on sampled queries.

The workloads' caches are too large to build on the host, so the inputs are drawn on
the GPU with the same seeded generator (its device and host outputs are identical,
see test_seedgen / test_gpu_codecs) and quantised by the library's codecs.  Only the
inputs of the checked queries go through the oracle: their indexer keys are made
tie-free and quantised by the oracle's codecs, and every shared-KV row those queries
read (the window and the oracle's top-k) is re-encoded by the oracle's codecs and
written over the library-encoded row, so that the GPU and the oracle read identical
bytes.  Rows no checked query reads keep the library's encoding; the outputs of the
unchecked queries are not compared.  Expected values come from the oracle only.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

import compressed_sparse_kv_csa_amd as ck
import seedgen
from cases import D, DI, IDX_FMTS, KV_FMTS, bf16_bits
from oracle import decode as OD, formats as OF, tiefree

DEV = "cuda"
T = seedgen.TID
KV_ROW_BYTES = {"bf16": 1024, "mixed": 576, "fp4": 256}


def _dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def oracle_encode_kv(bits: np.ndarray, fmt: str):
    """bf16 rows [n][512] -> (codes [n][row bytes], scales [n][32] or None, values [n][512])."""
    if fmt == "bf16":
        return np.ascontiguousarray(bits).view(np.uint8).reshape(len(bits), -1), None, OF.bf16_bits_to_f64(bits)
    if fmt == "mixed":
        rows = OF.mixed_quantize(bits)
        return rows, None, OF.mixed_dequantize(rows)
    c, s = OF.fp4_quantize(OF.bf16_bits_to_f64(bits))
    return c, s, OF.fp4_dequantize(c, s)


@dataclass
class DevCache:
    fmt: str
    codes: torch.Tensor               # [B][rows][row bytes] uint8
    scales: torch.Tensor | None       # [B][rows][32] uint8 (fp4)
    bits: torch.Tensor                # [B][rows][512] bf16 source rows (device)

    def descriptor(self) -> ck.Cache:
        B, rows = self.codes.shape[:2]
        return ck.cache(KV_FMTS[self.fmt], self.codes, rows, rows, self.scales)

    def put_oracle_rows(self, b: int, rows: np.ndarray) -> np.ndarray:
        """Re-encode rows of sequence b with the oracle's codec, store them, return values."""
        bits = bf16_bits(self.bits[b, torch.from_numpy(rows).to(DEV)])
        codes, scales, vals = oracle_encode_kv(bits, self.fmt)
        idx = torch.from_numpy(rows).to(DEV)
        self.codes[b, idx] = _dev(codes)
        if scales is not None:
            self.scales[b, idx] = _dev(scales)
        return vals


def make_kv_cache(seed: int, layer: int, B: int, rows: int, fmt: str) -> DevCache:
    bits = seedgen.kv_rows_bf16(seed, seedgen.tid(T.KV, layer), (B, rows, D), DEV)
    if fmt == "bf16":
        codes = bits.contiguous().view(torch.uint8).view(B, rows, 1024)
        return DevCache(fmt, codes, None, bits)
    if fmt == "mixed":
        codes = torch.empty((B, rows, 576), dtype=torch.uint8, device=DEV)
        ck.kv_quantize_fp8(bits, B * rows, D, 448, codes)
        return DevCache(fmt, codes, None, bits)
    codes = torch.empty((B, rows, 256), dtype=torch.uint8, device=DEV)
    scales = torch.empty((B, rows, 32), dtype=torch.uint8, device=DEV)
    ck.kv_quantize_fp4(bits, B * rows, D, codes, scales)
    return DevCache(fmt, codes, scales, bits)


@dataclass
class IndexerInputs:
    cache: ck.Cache
    keep: tuple
    q_idx: torch.Tensor      # [B][H_I][128] bf16 (device)
    w: torch.Tensor          # [B][H_I] fp32 (device)
    key_values: dict         # checked query -> [N_c][128] fp64 (oracle-decoded stored keys)
    q_idx_values: np.ndarray  # [B][H_I][128] fp64
    w_values: np.ndarray      # [B][H_I] fp64
    certs: list
    key_bits: dict            # checked query -> [N_c][128] bf16 source bits of the stored keys


def make_indexer(seed: int, layer: int, B: int, n_c: int, hi: int, top_k: int, fmt: str,
                 check: list[int]) -> IndexerInputs:
    qi = seedgen.bf16_normal(seed, seedgen.tid(T.Q_IDX, layer), (B, hi, DI))
    w = seedgen.uniform01(seed, seedgen.tid(T.W_IDX, layer), (B, hi))
    keys = seedgen.bf16_normal(seed, seedgen.tid(T.IDX_KEYS, layer), (B, n_c, DI), DEV)
    qv = qi.double().numpy()
    if fmt == "fp4h":  # the queries as the indexer scores them: rotated, FP4, decoded
        qv = OF.fp4_dequantize(*OF.fp4h_quantize(bf16_bits(qi)))
    wv = w.double().numpy()
    chk = np.array(check)
    sub = bf16_bits(keys[torch.from_numpy(chk).to(DEV)])
    adj, certs = tiefree.make_tie_free(sub, qv[chk], wv[chk], top_k, fmt)
    key_values = {}
    if fmt == "bf16":
        keys[torch.from_numpy(chk).to(DEV)] = _dev(adj.view(np.int16)).view(torch.bfloat16)
        for i, b in enumerate(check):
            key_values[b] = OF.bf16_bits_to_f64(adj[i])
        codes = keys.contiguous().view(torch.uint8).view(B, n_c, 256)
        cache = ck.cache(IDX_FMTS[fmt], codes, n_c, n_c)
        keep = (codes,)
    else:
        codes = torch.empty((B, n_c, 64), dtype=torch.uint8, device=DEV)
        scales = torch.empty((B, n_c, 8), dtype=torch.uint8, device=DEV)
        if fmt == "fp4h":
            ck.idx_quantize_fp4_hadamard(keys, B * n_c, codes, scales)
        else:
            ck.kv_quantize_fp4(keys, B * n_c, DI, codes, scales)
        for i, b in enumerate(check):
            c, s = (OF.fp4h_quantize(adj[i]) if fmt == "fp4h"
                    else OF.fp4_quantize(OF.bf16_bits_to_f64(adj[i])))
            codes[b] = _dev(c)
            scales[b] = _dev(s)
            key_values[b] = OF.fp4_dequantize(c, s)
        cache = ck.cache(IDX_FMTS[fmt], codes, n_c, n_c, scales)
        keep = (codes, scales)
    del keys
    return IndexerInputs(cache, keep, _dev(bf16_bits(qi).view(np.int16)), w.to(DEV), key_values,
                         qv, wv, certs, {b: adj[i] for i, b in enumerate(check)})


def reindex_query(seed: int, layer: int, B: int, hi: int):
    """A Reindex layer's indexer query and head weights: device tensors and fp64 values."""
    qi = seedgen.bf16_normal(seed, seedgen.tid(T.Q_IDX, layer), (B, hi, DI))
    w = seedgen.uniform01(seed, seedgen.tid(T.W_IDX, layer), (B, hi))
    return (_dev(bf16_bits(qi).view(np.int16)), w.to(DEV), qi.double().numpy(),
            w.double().numpy())


def make_pool_tie_free(ix: IndexerInputs, b: int, pool_rows: np.ndarray, qv: np.ndarray,
                       wv: np.ndarray, top_k: int, fmt: str):
    """Make query b's keys tie-free inside its pool for a Reindex query (halving pool rows
    as needed), and store the re-encoded rows in the device cache and the oracle's view."""
    rows = np.sort(pool_rows[pool_rows >= 0])
    adj, _ = tiefree.make_tie_free(ix.key_bits[b][rows][None], qv[None], wv[None], top_k, fmt)
    ix.key_bits[b][rows] = adj[0]
    idx = torch.from_numpy(rows).to(DEV)
    if fmt == "bf16":
        ix.keep[0][b, idx] = _dev(np.ascontiguousarray(adj[0]).view(np.uint8).reshape(len(rows), 256))
        ix.key_values[b][rows] = OF.bf16_bits_to_f64(adj[0])
    else:
        c, s = OF.fp4_quantize(OF.bf16_bits_to_f64(adj[0]))
        ix.keep[0][b, idx] = _dev(c)
        ix.keep[1][b, idx] = _dev(s)
        ix.key_values[b][rows] = OF.fp4_dequantize(c, s)


def oracle_topk(ix: IndexerInputs, b: int, top_k: int) -> np.ndarray:
    return OD.topk_indices(OD.indexer_scores(ix.q_idx_values[b], ix.w_values[b], ix.key_values[b]), top_k)


def query_bits(seed: int, layer: int, B: int, hq: int):
    q = seedgen.bf16_normal(seed, seedgen.tid(T.Q, layer), (B, hq, D))
    return _dev(bf16_bits(q).view(np.int16)), OF.bf16_bits_to_f64(bf16_bits(q))


def run_decode(p: ck.CsaParams, kv: DevCache, ix: IndexerInputs | None, q: torch.Tensor,
               topk: torch.Tensor, n_c: int) -> torch.Tensor:
    out = torch.empty((p.batch, p.n_q_heads, D), dtype=torch.int16, device=DEV)
    ws = torch.empty(max(ck.csa_decode_workspace_bytes(p, n_c), 256), dtype=torch.uint8, device=DEV)
    if ix is None:
        ck.csa_decode(p, kv.descriptor(), None, q, None, None, topk, out, ws)
    else:
        ck.csa_decode(p, kv.descriptor(), ix.cache, q, ix.q_idx, ix.w, topk, out, ws)
    torch.cuda.synchronize()
    return out


def bf16_out(out: torch.Tensor) -> np.ndarray:
    return out.cpu().view(torch.bfloat16).double().numpy()


def scale_of(dim: int = D) -> float:
    return 1.0 / math.sqrt(dim)
