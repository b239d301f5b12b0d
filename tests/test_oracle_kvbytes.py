"""Pins of the oracle's KV-cache byte accounting to every consistent figure the pages print."""
import json
import os

import pytest

from oracle import kvbytes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_cache_bytes.json")
MIB = 1 << 20
GIB = 1 << 30
UNIT = {"B": 1, "MiB": MIB, "GiB": GIB}

# Model descriptions; byte sizes per row follow from the dims, not from the oracle.
MODELS = {
    # MLA (V3): one 576-dim row of bf16 per token per layer, 61 layers, no window.
    "v3_mla": dict(n_csa=61, n_hca=0, csa_ratio=1, window=0, s_kv=(512 + 64) * 2, s_idx=0, count_window=0),
    # DSA (V3.2): MLA row plus a 128-dim bf16 indexer key.
    "v32_dsa": dict(n_csa=61, n_hca=0, csa_ratio=1, window=0, s_kv=(512 + 64) * 2, s_idx=128 * 2, count_window=0),
    # V4-Pro, 30 CSA + 31 HCA, per-token accounting without window rows.
    "v4_pro_bf16_nowin": dict(n_csa=30, n_hca=31, s_kv=512 * 2, s_idx=128 * 2, count_window=0),
    # V4-Pro with the window counted once per layer.
    "v4_pro_bf16": dict(n_csa=30, n_hca=31, s_kv=512 * 2, s_idx=128 * 2, count_window=1),
    "v4_pro_mixed": dict(n_csa=30, n_hca=31, s_kv=448 + 64 * 2, s_idx=128 // 2, count_window=1),
    # V4-Flash: 21 CSA + 20 HCA + 2 pure sliding-window layers (padded runtime size).
    "v4_flash_nowin": dict(n_csa=21, n_hca=20, s_kv=512 * 2, s_idx=128 * 2, count_window=0, n_swa=2,
                           swa_layer_bytes=2 * 1 * 128 * 2 * (128 + 256)),
}


def _field(model, field, seq_len, entry):
    if model == "swa_layer":
        return kvbytes.swa_layer_bytes(1, 128, 2, 128, pad=entry["pad"])
    if model.startswith("ratio_v32_over_"):
        num = kvbytes.kv_cache_bytes(seq_len, **MODELS["v32_dsa"])["total"]
        den = kvbytes.kv_cache_bytes(seq_len, **MODELS[model[len("ratio_v32_over_"):]])["total"]
        return num / den
    r = kvbytes.kv_cache_bytes(seq_len, **MODELS[model])
    p = MODELS[model]
    n_c = seq_len // p.get("csa_ratio", 4)
    n_h = seq_len // p.get("hca_ratio", 128)
    derived = {
        "per_token_layer": r["csa_per_layer"] // max(1, seq_len),
        "csa_compressed_per_layer": n_c * p["s_kv"],
        "hca_compressed_per_layer": n_h * p["s_kv"],
        "csa_indexer_per_layer": n_c * p["s_idx"],
        "window_per_layer": p.get("window", 128) * p["s_kv"],
        "csa_total": p["n_csa"] * r["csa_per_layer"],
        "hca_total": p["n_hca"] * r["hca_per_layer"],
        "csa_windows": p["n_csa"] * 128 * p["s_kv"],
        "hca_windows": p["n_hca"] * 128 * p["s_kv"],
    }
    if field.startswith("pct:"):
        return 100.0 * r[field[4:]] / r["total"]
    if field in derived:
        return derived[field]
    return r[field]


def _pins():
    with open(GOLDEN, encoding="utf-8") as f:
        return json.load(f)["pins"]


@pytest.mark.parametrize("entry", _pins(), ids=lambda e: f"{e['model']}:{e['field']}:{e['figure']}")
def test_printed_figure(entry):
    v = _field(entry["model"], entry["field"], entry.get("seq_len", 0), entry)
    unit = entry["unit"]
    if unit in UNIT:
        v = v / UNIT[unit]
    tol = 0.5 * 10.0 ** (-entry["decimals"]) + 1e-9
    assert abs(v - entry["value"]) <= tol, (entry["cite"], entry["figure"], v)


def test_exact_totals_1m():
    """The exact byte totals behind the 9.62 GiB and 4.83 GiB labels."""
    n = 1 << 20
    assert kvbytes.kv_cache_bytes(n, **MODELS["v4_pro_bf16"])["total"] == 10_334_371_840
    assert kvbytes.kv_cache_bytes(n, **MODELS["v4_pro_mixed"])["total"] == 5_183_938_560
    assert kvbytes.kv_cache_bytes(n, **MODELS["v4_pro_bf16_nowin"])["total"] == 9848 * MIB


def test_window_count_readings():
    """Counting the window 0, 1 or 2 times shifts each layer by exactly window * S_kv."""
    n = 1 << 20
    base = dict(MODELS["v4_pro_bf16"])
    t = [kvbytes.kv_cache_bytes(n, **{**base, "count_window": c})["total"] for c in (0, 1, 2)]
    assert t[1] - t[0] == t[2] - t[1] == 61 * 128 * 1024


def test_scale_bytes_reading():
    """FP4 scale bytes (one per 16 dims) are not in the pages' 64-byte indexer row: counting
    them adds exactly the `scales` figure, which is one byte per 16 dims of every FP4 row."""
    n = 1 << 20
    kw = dict(MODELS["v4_pro_mixed"], s_idx_scales=128 // 16)
    t0 = kvbytes.kv_cache_bytes(n, **kw)
    t1 = kvbytes.kv_cache_bytes(n, **kw, count_scales=1)
    assert t0["total"] == 5_183_938_560                      # the 4.83 GiB figure is unchanged
    assert t0["scales"] == t1["scales"] == 30 * (n // 4) * 8
    assert t1["total"] - t0["total"] == t0["scales"]
    fp4 = dict(n_csa=30, n_hca=31, s_kv=256, s_kv_scales=32, s_idx=64, s_idx_scales=8)
    r = kvbytes.kv_cache_bytes(n, **fp4, count_window=1)
    assert r["scales"] == 30 * ((n // 4) * 40 + 128 * 32) + 31 * ((n // 128) + 128) * 32
