"""The C ABI on the host: the library loads, exports every entry point the header
declares, its byte accounting matches the oracle, and invalid calls are rejected
before anything is launched (no device needed for any of these)."""
import ctypes
import os
import re

import pytest

import compressed_sparse_kv_csa_amd as ck
from oracle import kvbytes

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "csakv.h")


def _declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s+\**([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_binding_names():
    assert _declared_functions() == sorted(ck.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(ck.lib_path())
    for name in _declared_functions():
        assert hasattr(L, name), name


def _spec(**kw):
    base = dict(n_csa=30, n_hca=31, n_swa=0, csa_ratio=4, hca_ratio=128, window=128, kv_dim=512,
                rope_dim=64, idx_dim=128, kv_fmt=ck.KV_BF16, idx_fmt=ck.IDX_BF16, count_window=1,
                count_scales=0, reserved=0, swa_layer_bytes=0)
    base.update(kw)
    return ck.KvCacheSpec(**base)


# (library spec, oracle row bytes) pairs; row bytes follow from the format definitions:
# bf16 2 B per dim; mixed 448 E4M3 + 64 bf16 = 576 B; FP4 half a byte per dim in codes and
# one scale byte per 16 dims (512 dims: 256 + 32; 128 dims: 64 + 8).
FP4_KV = dict(s_kv=256, s_kv_scales=32)
FP4_IDX = dict(s_idx=64, s_idx_scales=8)
FORMATS = [
    (dict(kv_fmt=ck.KV_BF16, idx_fmt=ck.IDX_BF16), dict(s_kv=1024, s_idx=256)),
    (dict(kv_fmt=ck.KV_FP8_MIXED, idx_fmt=ck.IDX_FP4), dict(s_kv=576, **FP4_IDX)),
    (dict(kv_fmt=ck.KV_FP8_MIXED, idx_fmt=ck.IDX_FP4, count_scales=1),
     dict(s_kv=576, **FP4_IDX, count_scales=1)),
    (dict(kv_fmt=ck.KV_FP4, idx_fmt=ck.IDX_FP4, count_scales=1), dict(**FP4_KV, **FP4_IDX, count_scales=1)),
    (dict(kv_fmt=ck.KV_FP4, idx_fmt=ck.IDX_FP4), dict(**FP4_KV, **FP4_IDX)),
    (dict(kv_fmt=ck.KV_FP8_MIXED, idx_fmt=ck.IDX_FP4_HADAMARD), dict(s_kv=576, **FP4_IDX)),
    (dict(kv_fmt=ck.KV_FP4, idx_fmt=ck.IDX_FP4_HADAMARD, count_scales=1),
     dict(**FP4_KV, **FP4_IDX, count_scales=1)),
]


@pytest.mark.parametrize("lib_kw,orc_kw", FORMATS)
@pytest.mark.parametrize("count_window", [0, 1, 2])
@pytest.mark.parametrize("seq_len", [0, 1, 4097, 131072, 1 << 20])
def test_kv_cache_bytes_matches_oracle(lib_kw, orc_kw, count_window, seq_len):
    total, br = ck.kv_cache_bytes(_spec(count_window=count_window, **lib_kw), seq_len)
    ref = kvbytes.kv_cache_bytes(seq_len, n_csa=30, n_hca=31, count_window=count_window, **orc_kw)
    assert total == ref["total"]
    for f in ("csa_per_layer", "hca_per_layer", "csa_shared_kv", "csa_indexer", "hca_shared_kv",
              "windows", "swa_layers", "scales"):
        assert getattr(br, f) == ref[f], f


def test_kv_cache_bytes_scales_are_what_counting_them_adds():
    """The scales field is exactly the difference counting the scale bytes makes."""
    for kw in (dict(kv_fmt=ck.KV_FP4, idx_fmt=ck.IDX_FP4), dict(kv_fmt=ck.KV_FP8_MIXED, idx_fmt=ck.IDX_FP4_HADAMARD),
               dict(kv_fmt=ck.KV_BF16, idx_fmt=ck.IDX_BF16)):
        for cw in (0, 1, 2):
            t0, b0 = ck.kv_cache_bytes(_spec(count_window=cw, count_scales=0, **kw), 1 << 20)
            t1, b1 = ck.kv_cache_bytes(_spec(count_window=cw, count_scales=1, **kw), 1 << 20)
            assert t1 - t0 == b0.scales == b1.scales
    # V4-Pro with FP4 indexer keys at 1M tokens: 30 CSA layers x 262,144 rows x 8 scale bytes
    _, br = ck.kv_cache_bytes(_spec(kv_fmt=ck.KV_FP8_MIXED, idx_fmt=ck.IDX_FP4_HADAMARD), 1 << 20)
    assert br.scales == 30 * 262144 * 8


def test_kv_cache_bytes_presets_and_invalid():
    mla = _spec(n_csa=61, n_hca=0, csa_ratio=1, window=0, kv_dim=576, idx_dim=0, count_window=0)
    assert ck.kv_cache_bytes(mla, 1 << 20)[0] == 1152 * 61 * (1 << 20)
    flash = _spec(n_csa=21, n_hca=20, n_swa=2, count_window=0,
                  swa_layer_bytes=kvbytes.swa_layer_bytes(1, 128, 2, 128, pad=256))
    assert ck.kv_cache_bytes(flash, 1 << 20)[0] == (320 * 21 + 8 * 20) * (1 << 20) + 2 * 196608
    assert ck.kv_cache_bytes(_spec(count_window=3), 10)[0] == 0
    assert ck.kv_cache_bytes(_spec(csa_ratio=0), 10)[0] == 0
    assert ck.kv_cache_bytes(_spec(kv_fmt=7), 10)[0] == 0
    assert ck.kv_cache_bytes(_spec(), -1)[0] == 0


def _params(**kw):
    base = dict(batch=1, n_q_heads=16, n_idx_heads=4, top_k=512, window=128, mode=ck.MODE_FULL,
                softmax_scale=0.044, reserved=0)
    base.update(kw)
    return ck.CsaParams(**base)


FAKE = 1 << 20  # an aligned, never-dereferenced address: every case below is rejected first


def _call(p, kv=None, idx=None, q=FAKE, qi=FAKE, w=FAKE, topk=FAKE, out=FAKE, ws=FAKE,
          ws_bytes=1 << 30):
    kv = kv or ck.Cache(ck.KV_BF16, 0, 128 + 1024, 128 + 1024, FAKE, None)
    return ck.csa_decode(p, kv, idx, q, qi, w, topk, out, ws, ws_bytes, stream=0, check=False)


IDX = ck.Cache(ck.IDX_BF16, 0, 1024, 1024, FAKE, None)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), ck.ERR_INVALID),
    (dict(top_k=0), ck.ERR_INVALID),
    (dict(top_k=2049), ck.ERR_UNSUPPORTED),
    (dict(n_q_heads=24), ck.ERR_UNSUPPORTED),
    (dict(n_q_heads=144), ck.ERR_UNSUPPORTED),
    (dict(n_idx_heads=129), ck.ERR_UNSUPPORTED),
    (dict(n_idx_heads=0), ck.ERR_INVALID),
    (dict(mode=5), ck.ERR_INVALID),
    (dict(window=-1), ck.ERR_INVALID),
    (dict(softmax_scale=float("nan")), ck.ERR_INVALID),
    (dict(reserved=1), ck.ERR_INVALID),
])
def test_csa_rejects_bad_params(kw, status):
    assert _call(_params(**kw), idx=IDX) == status


@pytest.mark.parametrize("kw", [dict(n_q_heads=128), dict(n_idx_heads=128), dict(top_k=2048),
                                dict(n_q_heads=128, n_idx_heads=65, top_k=1024)])
def test_csa_accepts_the_largest_shapes(kw):
    # accepted up to the workspace check: 128 heads of either kind, top_k 2048
    assert _call(_params(**kw), idx=IDX, ws_bytes=0) == ck.ERR_WORKSPACE
    assert ck.csa_decode_workspace_bytes(_params(**kw), 1024) > 0
    kv = ck.Cache(ck.KV_BF16, 0, 1000, 1000, FAKE, None)
    assert ck.hca_decode(1, 128, 0.04, kv, FAKE, FAKE, FAKE, 0, stream=0, check=False) == ck.ERR_WORKSPACE


def test_csa_rejects_bad_pointers_and_shapes():
    p = _params()
    assert _call(p, idx=IDX, q=FAKE + 2) == ck.ERR_INVALID                 # misaligned
    assert _call(p, idx=IDX, out=0) == ck.ERR_INVALID                      # null
    assert _call(p, idx=None) == ck.ERR_INVALID                            # FULL needs keys
    bad_rows = ck.Cache(ck.IDX_BF16, 0, 1000, 1000, FAKE, None)
    assert _call(p, idx=bad_rows) == ck.ERR_INVALID                        # keys != N_c rows
    fp4_no_scales = ck.Cache(ck.IDX_FP4, 0, 1024, 1024, FAKE, None)
    assert _call(p, idx=fp4_no_scales) == ck.ERR_INVALID
    bf16_with_scales = ck.Cache(ck.IDX_BF16, 0, 1024, 1024, FAKE, FAKE)
    assert _call(p, idx=bf16_with_scales) == ck.ERR_INVALID
    short = ck.Cache(ck.KV_BF16, 0, 100, 100, FAKE, None)                  # fewer rows than window
    assert _call(p, kv=short, idx=IDX) == ck.ERR_INVALID
    stride = ck.Cache(ck.KV_BF16, 0, 1152, 1000, FAKE, None)               # stride < rows
    assert _call(p, kv=stride, idx=IDX) == ck.ERR_INVALID
    lens_misaligned = ck.Cache(ck.IDX_BF16, 0, 1024, 1024, FAKE, None, FAKE + 2)
    assert _call(p, idx=lens_misaligned) == ck.ERR_INVALID                 # per-sequence lengths
    # paged layouts: pages of 2^k >= 16 rows, a table row covering n_rows, an aligned table
    for pr, ts, table in [(48, 32, FAKE), (8, 128, FAKE), (64, 15, FAKE), (64, 16, FAKE + 2)]:
        paged = ck.Cache(ck.IDX_BF16, 0, 1024, 0, FAKE, None, None, table, pr, ts)
        assert _call(p, idx=paged) == ck.ERR_INVALID, (pr, ts)
    pages_without_table = ck.Cache(ck.IDX_BF16, 0, 1024, 1024, FAKE, None, None, None, 64, 16)
    assert _call(p, idx=pages_without_table) == ck.ERR_INVALID
    paged_ok = ck.Cache(ck.IDX_BF16, 0, 1024, 0, FAKE, None, None, FAKE, 64, 16)
    assert _call(p, idx=paged_ok, ws_bytes=0) == ck.ERR_WORKSPACE          # accepted up to the workspace
    need = ck.csa_decode_workspace_bytes(p, 1024)
    assert need > 0
    assert _call(p, idx=IDX, ws_bytes=need - 1) == ck.ERR_WORKSPACE
    reuse = _params(mode=ck.MODE_REUSE, n_idx_heads=0)
    assert _call(reuse, idx=IDX) == ck.ERR_INVALID                         # REUSE takes no keys


def test_hca_and_codecs_reject_bad_arguments():
    kv = ck.Cache(ck.KV_BF16, 0, 1000, 1000, FAKE, None)
    assert ck.hca_decode(0, 64, 0.04, kv, FAKE, FAKE, FAKE, 1 << 30, stream=0, check=False) == ck.ERR_INVALID
    assert ck.hca_decode(1, 40, 0.04, kv, FAKE, FAKE, FAKE, 1 << 30, stream=0, check=False) == ck.ERR_UNSUPPORTED
    assert ck.hca_decode(1, 144, 0.04, kv, FAKE, FAKE, FAKE, 1 << 30, stream=0, check=False) == ck.ERR_UNSUPPORTED
    assert ck.hca_decode(1, 64, 0.04, kv, FAKE, FAKE, FAKE, 0, stream=0, check=False) == ck.ERR_WORKSPACE
    assert ck.kv_quantize_fp4(FAKE, 10, 100, FAKE, FAKE, stream=0, check=False) == ck.ERR_INVALID
    assert ck.kv_quantize_fp8(FAKE, 10, 512, 440, FAKE, stream=0, check=False) == ck.ERR_INVALID
    assert ck.kv_dequantize(1, FAKE, None, 10, 256, FAKE, stream=0, check=False) == ck.ERR_UNSUPPORTED
    assert ck.kv_dequantize(2, FAKE, None, 10, 512, FAKE, stream=0, check=False) == ck.ERR_INVALID
    assert ck.kv_dequantize(9, FAKE, None, 10, 512, FAKE, stream=0, check=False) == ck.ERR_INVALID
    assert ck.csakv_status_string(-2) == "unsupported shape or format"


def test_reindex_rejects_bad_arguments():
    p = _params(mode=ck.MODE_REINDEX)

    def call(p=p, idx=IDX, qi=FAKE, w=FAKE, pool=FAKE, n_pool=1024, topk=FAKE + 65536,
             ws=FAKE + (1 << 20), ws_bytes=None):
        if ws_bytes is None:
            ws_bytes = ck.csa_reindex_topk_workspace_bytes(p, n_pool)
        return ck.csa_reindex_topk(p, idx, qi, w, pool, n_pool, topk, ws, ws_bytes, stream=0,
                                   check=False)

    assert call(p=_params(mode=ck.MODE_FULL)) == ck.ERR_INVALID            # wrong mode
    assert ck.csa_decode_workspace_bytes(p, 1024) == 0                    # csa_decode has no REINDEX
    assert _call(p, idx=IDX) == ck.ERR_INVALID
    assert call(n_pool=0) == ck.ERR_INVALID
    assert call(n_pool=4097) == ck.ERR_UNSUPPORTED
    assert call(p=_params(mode=ck.MODE_REINDEX, top_k=2049)) == ck.ERR_UNSUPPORTED
    assert call(p=_params(mode=ck.MODE_REINDEX, n_idx_heads=129)) == ck.ERR_UNSUPPORTED
    assert call(p=_params(mode=ck.MODE_REINDEX, top_k=2048, n_idx_heads=128), ws_bytes=0) == ck.ERR_WORKSPACE
    assert call(p=_params(mode=ck.MODE_REINDEX, n_idx_heads=0)) == ck.ERR_INVALID
    assert call(pool=0) == ck.ERR_INVALID                                 # null
    assert call(qi=FAKE + 2) == ck.ERR_INVALID                            # misaligned
    assert call(idx=None) == ck.ERR_INVALID
    assert call(topk=FAKE + 1024) == ck.ERR_INVALID                       # output overlaps the pool
    huge = ck.Cache(ck.IDX_BF16, 0, 1 << 24, 1 << 24, FAKE, None)         # 4 GiB of keys
    assert call(idx=huge) == ck.ERR_UNSUPPORTED
    need = ck.csa_reindex_topk_workspace_bytes(p, 1024)
    assert need == 1024 * 8                                               # one key per slot
    assert ck.csa_reindex_topk_workspace_bytes(p, 0) == 0
    assert ck.csa_reindex_topk_workspace_bytes(_params(mode=ck.MODE_FULL), 1024) == 0
    assert call(ws_bytes=need - 1) == ck.ERR_WORKSPACE
    assert call(ws=0) == ck.ERR_INVALID                                   # null workspace
    assert call(ws=FAKE + 8) == ck.ERR_INVALID                            # misaligned workspace


def test_cache_write_rejects_bad_arguments():
    def call(fmt=ck.KV_BF16, dim=512, codes=FAKE, scales=None, stride=100, rows=100, B=1, n=2,
             x=FAKE, dst=FAKE):
        return ck.kv_cache_write(fmt, dim, codes, scales, stride, rows, B, n, x, dst, stream=0,
                                 check=False)

    assert call(fmt=3) == ck.ERR_INVALID
    assert call(dim=256) == ck.ERR_UNSUPPORTED
    assert call(fmt=ck.KV_FP8_MIXED, dim=128) == ck.ERR_UNSUPPORTED
    assert call(fmt=ck.KV_FP4) == ck.ERR_INVALID                  # FP4 needs scales
    assert call(scales=FAKE) == ck.ERR_INVALID                    # bf16 takes none
    assert call(B=0) == ck.ERR_INVALID
    assert call(stride=50) == ck.ERR_INVALID                      # stride < rows
    assert call(codes=0) == ck.ERR_INVALID
    assert call(x=FAKE + 2) == ck.ERR_INVALID                     # misaligned
    assert call(n=0, codes=0) == ck.OK                            # nothing to write


def test_rope_output_rejects_bad_arguments():
    def call(out=FAKE, B=2, H=64, pos=FAKE, base=10000.0):
        return ck.rope_output(out, B, H, pos, base, stream=0, check=False)

    assert call(B=0) == ck.ERR_INVALID
    assert call(H=0) == ck.ERR_INVALID
    assert call(base=0.0) == ck.ERR_INVALID
    assert call(base=float("inf")) == ck.ERR_INVALID
    assert call(out=0) == ck.ERR_INVALID
    assert call(pos=FAKE + 4) == ck.ERR_INVALID


# Golden figures of whole-model totals, reproduced from the library's presets alone (the
# printed figures come from the pages; the presets are the library's own table).
_PRESET_OF = {"v3_mla": (ck.PRESET_V3_MLA, {}), "v32_dsa": (ck.PRESET_V32_DSA, {}),
              "v4_pro_bf16": (ck.PRESET_V4_PRO_BF16, {}), "v4_pro_mixed": (ck.PRESET_V4_PRO_MIXED, {}),
              "v4_pro_bf16_nowin": (ck.PRESET_V4_PRO_BF16, {"count_window": 0}),
              "v4_flash_nowin": (ck.PRESET_V4_FLASH, {})}


def _golden_totals():
    import json
    with open(os.path.join(os.path.dirname(__file__), "golden", "kv_cache_bytes.json"), encoding="utf-8") as f:
        pins = json.load(f)["pins"]
    return [p for p in pins if p["field"] == "total" and p["model"] in _PRESET_OF]


@pytest.mark.parametrize("entry", _golden_totals(), ids=lambda e: f"{e['model']}:{e['figure']}")
def test_kv_cache_presets_reproduce_the_printed_totals(entry):
    preset, change = _PRESET_OF[entry["model"]]
    spec = ck.kv_cache_spec_preset(preset)
    for k, v in change.items():
        setattr(spec, k, v)
    total, _ = ck.kv_cache_bytes(spec, entry["seq_len"])
    unit = {"B": 1, "MiB": 1 << 20, "GiB": 1 << 30}[entry["unit"]]
    assert abs(total / unit - entry["value"]) <= 0.5 * 10.0 ** (-entry["decimals"]) + 1e-9, \
        (entry["cite"], entry["figure"], total / unit)


def test_kv_cache_presets_exact_and_invalid():
    n = 1 << 20
    assert ck.kv_cache_bytes(ck.kv_cache_spec_preset(ck.PRESET_V4_PRO_BF16), n)[0] == 10_334_371_840
    assert ck.kv_cache_bytes(ck.kv_cache_spec_preset(ck.PRESET_V4_PRO_MIXED), n)[0] == 5_183_938_560
    assert ck.kv_cache_bytes(ck.kv_cache_spec_preset(ck.PRESET_V3_MLA), n)[0] == 1152 * 61 * n
    assert ck.kv_cache_bytes(ck.kv_cache_spec_preset(ck.PRESET_V32_DSA), n)[0] == (1152 + 256) * 61 * n
    with pytest.raises(ck.CsakvError):
        ck.kv_cache_spec_preset(5)
    assert ck.lib().kv_cache_spec_preset(0, None) == ck.ERR_INVALID
