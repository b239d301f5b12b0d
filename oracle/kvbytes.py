"""KV-cache size accounting in closed form (oracle; test infrastructure only).

The closed form is the per-layer formula of "DeepSeek-V4 KV Cache 深度分析",
section 七 "总 KV Cache 计算公式":
    PerCSA = (N/4 + w) * S_kv + (N/4) * S_idx,   PerHCA = (N/128 + w) * S_kv,
    Total  = N_CSA * PerCSA + N_HCA * PerHCA,
with the row sizes S_kv, S_idx of section 六 "精度配置" (bf16: 1024 / 256 bytes;
mixed: 576 / 64 bytes).

The pages disagree on how the sliding window is counted, so it is a parameter:
* ``count_window=0``: not at all (the per-token figures 320 B and 8 B of
  "DeepSeek V4 의 정확한 KV 캐시 사용량 분석");
* ``count_window=1``: once per layer (the section 七 formula and the printed
  calculator output, 320.12 MiB per CSA layer);
* ``count_window=2``: twice per layer (the calculator code of the appendix as
  written, which adds the window inside the shared-KV term and again as SWA).
Pure sliding-window layers (V4-Flash's first two layers) add
``n_swa * swa_layer_bytes``.

MLA (V3) and DSA (V3.2) caches are the special case ratio 1, no window: S_kv =
(512 + 64) * 2 and, for V3.2, an extra 128 * 2 indexer bytes.

FP4 rows carry one E4M3 scale byte per 16 channels besides their codes; section 六
counts the FP4 indexer row as 64 bytes, without them.  ``s_kv_scales`` / ``s_idx_scales``
are those scale bytes per row; ``count_scales=1`` adds them to every row (and so to
``total``), and ``scales`` reports the cache's scale bytes either way.

Parity pins (tests/test_oracle_kvbytes.py and tests/golden/kv_cache_bytes.json):
every byte total the pages print that the closed form reproduces.
"""
from __future__ import annotations


def kv_cache_bytes(seq_len: int, *, n_csa: int, n_hca: int, csa_ratio: int = 4,
                   hca_ratio: int = 128, window: int = 128, s_kv: int = 1024,
                   s_idx: int = 256, count_window: int = 1, n_swa: int = 0,
                   swa_layer_bytes: int = 0, s_kv_scales: int = 0, s_idx_scales: int = 0,
                   count_scales: int = 0) -> dict:
    n_c = seq_len // csa_ratio if n_csa else 0
    n_h = seq_len // hca_ratio if n_hca else 0
    scales = (n_csa * (n_c * (s_kv_scales + s_idx_scales) + count_window * window * s_kv_scales)
              + n_hca * (n_h + count_window * window) * s_kv_scales)
    if count_scales:
        s_kv, s_idx = s_kv + s_kv_scales, s_idx + s_idx_scales
    win = count_window * window * s_kv
    csa_shared = n_c * s_kv
    csa_index = n_c * s_idx
    per_csa = csa_shared + csa_index + win
    per_hca = n_h * s_kv + win
    total = n_csa * per_csa + n_hca * per_hca + n_swa * swa_layer_bytes
    return {
        "csa_per_layer": per_csa,
        "hca_per_layer": per_hca,
        "csa_shared_kv": n_csa * csa_shared,
        "csa_indexer": n_csa * csa_index,
        "hca_shared_kv": n_hca * n_h * s_kv,
        "windows": (n_csa + n_hca) * win,
        "swa_layers": n_swa * swa_layer_bytes,
        "scales": scales,
        "total": total,
    }


def swa_layer_bytes(n_head_kv: int, head_dim: int, precision: int, window: int,
                    pad: int = 0) -> int:
    """Bytes of one pure sliding-window layer: K and V for (window + pad) tokens.

    ("DeepSeek V4 의 정확한 KV 캐시 사용량 분석", the V4-Flash paragraph: window 128,
    and a 256-token pad in one runtime's implementation.)
    """
    return 2 * n_head_kv * head_dim * precision * (window + pad)


# Presets named by the model and storage they describe.
V4_PRO = dict(n_csa=30, n_hca=31)
V4_FLASH = dict(n_csa=21, n_hca=20)
BF16_ROWS = dict(s_kv=512 * 2, s_idx=128 * 2)
MIXED_ROWS = dict(s_kv=448 * 1 + 64 * 2, s_idx=128 // 2)
