"""Seeded decode cases shared by the parity tests.

A case holds the inputs of one csa_decode / hca_decode call as host arrays, built
from the seeded generator; the indexer keys are made tie-free and every cache is
quantised by the oracle, so both the oracle and the GPU read identical bytes.  The
expected values come from the oracle only.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

import seedgen
from oracle import decode as OD, formats as OF, tiefree

KV_FMTS = {"bf16": 0, "mixed": 1, "fp4": 2}
IDX_FMTS = {"bf16": 0, "fp4": 1, "fp4h": 2}
D, DI = 512, 128


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@dataclass
class KvCache:
    fmt: str
    codes: np.ndarray            # [B][rows][row_bytes] uint8
    scales: np.ndarray | None    # [B][rows][32] uint8 (fp4)
    values: np.ndarray           # [B][rows][512] decoded fp64


@dataclass
class IdxCache:
    fmt: str
    codes: np.ndarray            # [B][N_c][bytes] uint8
    scales: np.ndarray | None
    values: np.ndarray           # [B][N_c][128] decoded fp64


def encode_kv(bits: np.ndarray, fmt: str) -> KvCache:
    """bits: [B][rows][512] bf16 patterns -> cache bytes + decoded values (oracle codecs)."""
    if fmt == "bf16":
        return KvCache(fmt, np.ascontiguousarray(bits).view(np.uint8), None, OF.bf16_bits_to_f64(bits))
    if fmt == "mixed":
        rows = OF.mixed_quantize(bits)
        return KvCache(fmt, rows, None, OF.mixed_dequantize(rows))
    if fmt == "fp4":
        c, s = OF.fp4_quantize(OF.bf16_bits_to_f64(bits))
        return KvCache(fmt, c, s, OF.fp4_dequantize(c, s))
    raise ValueError(fmt)


def encode_idx(bits: np.ndarray, fmt: str) -> IdxCache:
    if fmt == "bf16":
        return IdxCache(fmt, np.ascontiguousarray(bits).view(np.uint8), None, OF.bf16_bits_to_f64(bits))
    if fmt == "fp4h":  # FP4 codes of each row's Hadamard rotation
        c, s = OF.fp4h_quantize(bits)
    else:
        c, s = OF.fp4_quantize(OF.bf16_bits_to_f64(bits))
    return IdxCache(fmt, c, s, OF.fp4_dequantize(c, s))


def indexer_query_values(q_idx_bits: np.ndarray, fmt: str) -> np.ndarray:
    """The indexer queries as the scores use them: bf16 values, or for Hadamard-rotated FP4
    keys the FP4-decoded rotation of each query row."""
    if fmt == "fp4h":
        return OF.fp4_dequantize(*OF.fp4h_quantize(q_idx_bits))
    return OF.bf16_bits_to_f64(q_idx_bits)


@dataclass
class CsaCase:
    B: int
    n_c: int
    window: int
    hq: int
    hi: int
    top_k: int
    scale: float
    q_bits: np.ndarray
    q_idx_bits: np.ndarray | None
    w: np.ndarray | None
    kv: KvCache
    idx: IdxCache | None
    expect_topk: np.ndarray | None = None     # [B][top_k] oracle order
    expect_out: np.ndarray | None = None      # [B][hq][512] fp64
    certs: list = field(default_factory=list)


def make_csa_case(seed: int, B: int, n_c: int, window: int, hq: int, hi: int, top_k: int,
                  kv_fmt: str, idx_fmt: str, layer: int = 0, with_indexer: bool = True,
                  expect: bool = True) -> CsaCase:
    T = seedgen.TID
    q = seedgen.bf16_normal(seed, seedgen.tid(T.Q, layer), (B, hq, D))
    kv_bits = bf16_bits(seedgen.kv_rows_bf16(seed, seedgen.tid(T.KV, layer), (B, window + n_c, D)))
    kv = encode_kv(kv_bits, kv_fmt)
    scale = 1.0 / math.sqrt(D)
    case = CsaCase(B, n_c, window, hq, hi, top_k, scale, bf16_bits(q), None, None, kv, None)
    if with_indexer:
        qi = seedgen.bf16_normal(seed, seedgen.tid(T.Q_IDX, layer), (B, hi, DI))
        w = seedgen.uniform01(seed, seedgen.tid(T.W_IDX, layer), (B, hi)).numpy()
        keys = bf16_bits(seedgen.bf16_normal(seed, seedgen.tid(T.IDX_KEYS, layer), (B, n_c, DI)))
        case.q_idx_bits = bf16_bits(qi)
        qi_vals = indexer_query_values(case.q_idx_bits, idx_fmt)
        keys, certs = tiefree.make_tie_free(keys, qi_vals, w.astype(np.float64), top_k, idx_fmt)
        case.w = w.astype(np.float32)
        case.idx = encode_idx(keys, idx_fmt)
        case.certs = certs
    if expect and with_indexer:
        run_oracle_full(case)
    return case


def run_oracle_full(case: CsaCase):
    qv = OF.bf16_bits_to_f64(case.q_bits)
    qiv = indexer_query_values(case.q_idx_bits, case.idx.fmt)
    outs, tks = [], []
    for b in range(case.B):
        o, sel = OD.csa_decode_one(qv[b], qiv[b], case.w[b].astype(np.float64), case.idx.values[b],
                                   case.kv.values[b], case.window, case.top_k, case.scale)
        outs.append(o)
        tks.append(sel)
    case.expect_out = np.stack(outs)
    case.expect_topk = np.stack(tks)


def oracle_reuse(case: CsaCase, topk: np.ndarray) -> np.ndarray:
    qv = OF.bf16_bits_to_f64(case.q_bits)
    return np.stack([OD.csa_reuse_one(qv[b], case.kv.values[b], case.window, topk[b], case.scale)
                     for b in range(case.B)])


def oracle_hca(q_bits: np.ndarray, kv: KvCache, scale: float) -> np.ndarray:
    qv = OF.bf16_bits_to_f64(q_bits)
    return np.stack([OD.hca_decode_one(qv[b], kv.values[b], scale) for b in range(q_bits.shape[0])])


def topk_sets_equal(got: np.ndarray, want: np.ndarray) -> bool:
    for g, w in zip(got, want):
        if sorted(int(x) for x in g if x >= 0) != sorted(int(x) for x in w if x >= 0):
            return False
        if (g < 0).sum() != (w < 0).sum():
            return False
    return True


ATOL = 1e-2


def attention_error(out: np.ndarray, ref: np.ndarray) -> tuple[float, bool]:
    """Max-abs error and whether every element meets the bar.

    The bar is max-abs 1e-2.  Where |ref| >= 4 (only in few-row edge cases) bf16 itself
    cannot hold the result to 1e-2 - its half-ulp there is 2**(floor(log2|ref|) - 8) -
    so that half-ulp is added to the allowance for those elements.
    """
    a = np.abs(ref)
    hulp = np.where(a >= 4.0, np.exp2(np.floor(np.log2(np.maximum(a, 1e-30))) - 8), 0.0)
    err = np.abs(out - ref)
    return float(err.max()) if err.size else 0.0, bool((err <= ATOL + hulp).all())
