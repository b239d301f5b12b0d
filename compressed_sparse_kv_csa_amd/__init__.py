"""compressed_sparse_kv_csa_amd - decode attention over compressed sparse KV caches on MI355X.

Thin ctypes binding of the C ABI in ``include/csakv.h``: every function here has the
same name as its C entry point and only marshals arguments (tensor data pointers,
the current HIP stream, ctypes structs).  All computation happens in the HIP kernels
of ``libcsakv.so``; there is no Python or CPU fallback, and loading fails loudly if
the library has not been built (``python -m compressed_sparse_kv_csa_amd.build``).
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "CsakvError", "KV_BF16", "KV_FP8_MIXED", "KV_FP4", "IDX_BF16", "IDX_FP4", "IDX_FP4_HADAMARD",
    "MODE_FULL",
    "MODE_REUSE", "MODE_REINDEX", "CsaParams", "Cache", "KvCacheSpec", "KvCacheBreakdown", "lib", "lib_path",
    "cache", "csa_decode_workspace_bytes", "csa_decode", "csa_decode_noalloc",
    "csa_decode_noalloc_scratch_bytes", "csa_select_topk_workspace_bytes",
    "csa_select_topk", "csa_select_scan", "csa_select_merge", "csa_reindex_topk",
    "csa_reindex_topk_workspace_bytes", "hca_decode_workspace_bytes",
    "hca_decode", "rope_output", "kv_quantize_fp4", "kv_quantize_fp8", "idx_quantize_fp4_hadamard",
    "kv_cache_write", "kv_dequantize",
    "kv_cache_bytes", "kv_cache_spec_preset", "csakv_status_string", "EXPORTED_SYMBOLS",
    "PRESET_V4_PRO_BF16", "PRESET_V4_PRO_MIXED", "PRESET_V4_FLASH", "PRESET_V3_MLA", "PRESET_V32_DSA",
]

KV_BF16, KV_FP8_MIXED, KV_FP4 = 0, 1, 2
IDX_BF16, IDX_FP4, IDX_FP4_HADAMARD = 0, 1, 2
MODE_FULL, MODE_REUSE, MODE_REINDEX = 0, 1, 2
PRESET_V4_PRO_BF16, PRESET_V4_PRO_MIXED, PRESET_V4_FLASH, PRESET_V3_MLA, PRESET_V32_DSA = 0, 1, 2, 3, 4

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4

EXPORTED_SYMBOLS = (
    "csa_decode_workspace_bytes", "csa_decode", "csa_decode_noalloc",
    "csa_decode_noalloc_scratch_bytes", "csa_select_topk_workspace_bytes",
    "csa_select_topk", "csa_select_scan", "csa_select_merge", "csa_reindex_topk",
    "csa_reindex_topk_workspace_bytes",
    "hca_decode_workspace_bytes", "hca_decode", "rope_output", "kv_quantize_fp4", "kv_quantize_fp8", "idx_quantize_fp4_hadamard", "kv_cache_write",
    "kv_dequantize", "kv_cache_bytes", "kv_cache_spec_preset", "csakv_status_string",
)

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    """The in-tree libcsakv.so, or the library CSAKV_LIBRARY names (for example the
    host-sanitized build that tests load)."""
    return os.environ.get("CSAKV_LIBRARY") or os.path.join(_HERE, "libcsakv.so")


class CsakvError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {csakv_status_string(status)} (status {status})")
        self.status = status


class Cache(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("n_rows", ctypes.c_int64), ("seq_stride_rows", ctypes.c_int64),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("seq_rows", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("page_rows", ctypes.c_int32), ("table_stride", ctypes.c_int32)]


class CsaParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_idx_heads", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("window", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("reserved", ctypes.c_int32)]


class KvCacheSpec(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_csa", "n_hca", "n_swa", "csa_ratio", "hca_ratio", "window", "kv_dim", "rope_dim",
        "idx_dim", "kv_fmt", "idx_fmt", "count_window", "count_scales", "reserved")] + [
        ("swa_layer_bytes", ctypes.c_int64)]


class KvCacheBreakdown(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "csa_shared_kv", "csa_indexer", "hca_shared_kv", "windows", "swa_layers", "scales",
        "csa_per_layer", "hca_per_layer", "total")]


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded ``libcsakv.so`` (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m compressed_sparse_kv_csa_amd.build`")
        L = ctypes.CDLL(path)
        P, I32, I64, SZ, VP, F = (ctypes.POINTER, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                                  ctypes.c_void_p, ctypes.c_float)
        L.csa_decode_workspace_bytes.argtypes = [P(CsaParams), I64]
        L.csa_decode_workspace_bytes.restype = SZ
        L.csa_decode.argtypes = [P(CsaParams), P(Cache), P(Cache), VP, VP, VP, VP, VP, VP, SZ, VP]
        L.csa_decode.restype = I32
        L.csa_decode_noalloc.argtypes = [P(CsaParams), P(Cache), P(Cache), VP, VP, VP, VP, VP, VP]
        L.csa_decode_noalloc.restype = I32
        L.csa_decode_noalloc_scratch_bytes.argtypes = []
        L.csa_decode_noalloc_scratch_bytes.restype = SZ
        L.csa_select_topk_workspace_bytes.argtypes = [P(CsaParams), I64]
        L.csa_select_topk_workspace_bytes.restype = SZ
        L.csa_select_topk.argtypes = [P(CsaParams), P(Cache), VP, VP, VP, VP, SZ, VP]
        L.csa_select_topk.restype = I32
        L.csa_select_scan.argtypes = [P(CsaParams), P(Cache), VP, VP, VP, SZ, VP]
        L.csa_select_scan.restype = I32
        L.csa_select_merge.argtypes = [P(CsaParams), P(Cache), VP, VP, SZ, VP]
        L.csa_select_merge.restype = I32
        L.csa_reindex_topk.argtypes = [P(CsaParams), P(Cache), VP, VP, VP, I32, VP, VP, SZ, VP]
        L.csa_reindex_topk.restype = I32
        L.csa_reindex_topk_workspace_bytes.argtypes = [P(CsaParams), I32]
        L.csa_reindex_topk_workspace_bytes.restype = SZ
        L.hca_decode_workspace_bytes.argtypes = [I32, I32, I64]
        L.hca_decode_workspace_bytes.restype = SZ
        L.hca_decode.argtypes = [I32, I32, F, P(Cache), VP, VP, VP, SZ, VP]
        L.hca_decode.restype = I32
        L.kv_quantize_fp4.argtypes = [VP, I64, I32, VP, VP, VP]
        L.kv_quantize_fp4.restype = I32
        L.kv_quantize_fp8.argtypes = [VP, I64, I32, I32, VP, VP]
        L.kv_quantize_fp8.restype = I32
        L.rope_output.argtypes = [VP, I32, I32, VP, ctypes.c_double, VP]
        L.rope_output.restype = I32
        L.idx_quantize_fp4_hadamard.argtypes = [VP, I64, VP, VP, VP]
        L.idx_quantize_fp4_hadamard.restype = I32
        L.kv_cache_write.argtypes = [I32, I32, VP, VP, I64, I64, I32, I32, VP, VP, VP]
        L.kv_cache_write.restype = I32
        L.kv_dequantize.argtypes = [I32, VP, VP, I64, I32, VP, VP]
        L.kv_dequantize.restype = I32
        L.kv_cache_bytes.argtypes = [P(KvCacheSpec), I64, P(KvCacheBreakdown)]
        L.kv_cache_bytes.restype = ctypes.c_uint64
        L.kv_cache_spec_preset.argtypes = [I32, P(KvCacheSpec)]
        L.kv_cache_spec_preset.restype = I32
        L.csakv_status_string.argtypes = [I32]
        L.csakv_status_string.restype = ctypes.c_char_p
        _LIB = L
    return _LIB


# ------------------------------------------------------------------ marshalling helpers

def _ptr(t):
    """Device address of a tensor (or None / an int address)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, what: str):
    if status != OK:
        raise CsakvError(status, what)


def cache(fmt: int, codes, n_rows: int, seq_stride_rows: int | None = None, scales=None,
          seq_rows=None, block_table=None, page_rows: int = 0) -> Cache:
    """Cache descriptor for a tensor of B sequences (see ``csakv_cache`` in the header).

    ``seq_rows``: None, or a device int32 tensor [B] of per-sequence row counts.
    ``block_table``: None, or a device int32 tensor [B][table_stride] of page ids into the
    page pool held by ``codes``/``scales`` (``page_rows`` rows per page).  The descriptor
    keeps references to the tensors it points at, so they outlive it."""
    stride = int(n_rows if seq_stride_rows is None else seq_stride_rows)
    table_stride = int(block_table.shape[-1]) if block_table is not None else 0
    c = Cache(fmt, 0, int(n_rows), stride, _ptr(codes), _ptr(scales), _ptr(seq_rows),
              _ptr(block_table), int(page_rows), table_stride)
    c._tensors = (codes, scales, seq_rows, block_table)
    return c


def csakv_status_string(status: int) -> str:
    return lib().csakv_status_string(int(status)).decode()


def csa_decode_workspace_bytes(params: CsaParams, n_compressed: int) -> int:
    return int(lib().csa_decode_workspace_bytes(ctypes.byref(params), int(n_compressed)))


def csa_decode(params: CsaParams, kv: Cache, idx_keys: Cache | None, q, q_idx, w_idx, topk, out,
               workspace, workspace_bytes: int | None = None, stream=None, check: bool = True) -> int:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().csa_decode(ctypes.byref(params), ctypes.byref(kv),
                          ctypes.byref(idx_keys) if idx_keys is not None else None,
                          _ptr(q), _ptr(q_idx), _ptr(w_idx), _ptr(topk), _ptr(out), _ptr(workspace),
                          int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "csa_decode")
    return st


def csa_decode_noalloc(params: CsaParams, kv: Cache, idx_keys: Cache | None, q, q_idx, w_idx,
                       topk, out, stream=None, check: bool = True) -> int:
    st = lib().csa_decode_noalloc(ctypes.byref(params), ctypes.byref(kv),
                                  ctypes.byref(idx_keys) if idx_keys is not None else None,
                                  _ptr(q), _ptr(q_idx), _ptr(w_idx), _ptr(topk), _ptr(out),
                                  _stream(stream))
    if check:
        _check(st, "csa_decode_noalloc")
    return st


def csa_decode_noalloc_scratch_bytes() -> int:
    return int(lib().csa_decode_noalloc_scratch_bytes())


def csa_select_topk_workspace_bytes(params: CsaParams, n_compressed: int) -> int:
    return int(lib().csa_select_topk_workspace_bytes(ctypes.byref(params), int(n_compressed)))


def csa_select_topk(params: CsaParams, idx_keys: Cache, q_idx, w_idx, topk, workspace,
                    workspace_bytes: int | None = None, stream=None, check: bool = True) -> int:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().csa_select_topk(ctypes.byref(params), ctypes.byref(idx_keys), _ptr(q_idx),
                               _ptr(w_idx), _ptr(topk), _ptr(workspace), int(workspace_bytes),
                               _stream(stream))
    if check:
        _check(st, "csa_select_topk")
    return st


def csa_select_scan(params: CsaParams, idx_keys: Cache, q_idx, w_idx, workspace,
                    workspace_bytes: int | None = None, stream=None, check: bool = True) -> int:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().csa_select_scan(ctypes.byref(params), ctypes.byref(idx_keys), _ptr(q_idx),
                               _ptr(w_idx), _ptr(workspace), int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "csa_select_scan")
    return st


def csa_select_merge(params: CsaParams, idx_keys: Cache, topk, workspace,
                     workspace_bytes: int | None = None, stream=None, check: bool = True) -> int:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().csa_select_merge(ctypes.byref(params), ctypes.byref(idx_keys), _ptr(topk),
                                _ptr(workspace), int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "csa_select_merge")
    return st


def csa_reindex_topk_workspace_bytes(params: CsaParams, n_pool: int) -> int:
    return int(lib().csa_reindex_topk_workspace_bytes(ctypes.byref(params), int(n_pool)))


def csa_reindex_topk(params: CsaParams, idx_keys: Cache, q_idx, w_idx, pool, n_pool: int, topk,
                     workspace, workspace_bytes: int | None = None, stream=None,
                     check: bool = True) -> int:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    keys = ctypes.byref(idx_keys) if idx_keys is not None else None
    st = lib().csa_reindex_topk(ctypes.byref(params), keys, _ptr(q_idx),
                                _ptr(w_idx), _ptr(pool), int(n_pool), _ptr(topk),
                                _ptr(workspace), int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "csa_reindex_topk")
    return st


def hca_decode_workspace_bytes(batch: int, n_q_heads: int, n_rows: int) -> int:
    return int(lib().hca_decode_workspace_bytes(int(batch), int(n_q_heads), int(n_rows)))


def hca_decode(batch: int, n_q_heads: int, softmax_scale: float, kv: Cache, q, out, workspace,
               workspace_bytes: int | None = None, stream=None, check: bool = True) -> int:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().hca_decode(int(batch), int(n_q_heads), float(softmax_scale), ctypes.byref(kv),
                          _ptr(q), _ptr(out), _ptr(workspace), int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "hca_decode")
    return st


def kv_quantize_fp4(x, rows: int, dim: int, codes, scales, stream=None, check: bool = True) -> int:
    st = lib().kv_quantize_fp4(_ptr(x), int(rows), int(dim), _ptr(codes), _ptr(scales),
                               _stream(stream))
    if check:
        _check(st, "kv_quantize_fp4")
    return st


def kv_quantize_fp8(x, rows: int, dim: int, nope_dim: int, out, stream=None, check: bool = True) -> int:
    st = lib().kv_quantize_fp8(_ptr(x), int(rows), int(dim), int(nope_dim), _ptr(out),
                               _stream(stream))
    if check:
        _check(st, "kv_quantize_fp8")
    return st


def rope_output(out, batch: int, n_heads: int, positions, base: float, stream=None,
                check: bool = True) -> int:
    st = lib().rope_output(_ptr(out), int(batch), int(n_heads), _ptr(positions), float(base),
                           _stream(stream))
    if check:
        _check(st, "rope_output")
    return st


def idx_quantize_fp4_hadamard(x, rows: int, codes, scales, stream=None, check: bool = True) -> int:
    st = lib().idx_quantize_fp4_hadamard(_ptr(x), int(rows), _ptr(codes), _ptr(scales),
                                         _stream(stream))
    if check:
        _check(st, "idx_quantize_fp4_hadamard")
    return st


def kv_cache_write(fmt: int, dim: int, codes, scales, seq_stride_rows: int, n_rows: int, batch: int,
                   n: int, x, dst, stream=None, check: bool = True) -> int:
    st = lib().kv_cache_write(int(fmt), int(dim), _ptr(codes), _ptr(scales), int(seq_stride_rows),
                              int(n_rows), int(batch), int(n), _ptr(x), _ptr(dst), _stream(stream))
    if check:
        _check(st, "kv_cache_write")
    return st


def kv_dequantize(fmt: int, codes, scales, rows: int, dim: int, out, stream=None,
                  check: bool = True) -> int:
    st = lib().kv_dequantize(int(fmt), _ptr(codes), _ptr(scales), int(rows), int(dim), _ptr(out),
                             _stream(stream))
    if check:
        _check(st, "kv_dequantize")
    return st


def kv_cache_bytes(spec: KvCacheSpec, seq_len: int) -> tuple[int, KvCacheBreakdown]:
    out = KvCacheBreakdown()
    total = int(lib().kv_cache_bytes(ctypes.byref(spec), int(seq_len), ctypes.byref(out)))
    return total, out


def kv_cache_spec_preset(preset: int) -> KvCacheSpec:
    """The library's KvCacheSpec for a PRESET_* model (raises CsakvError for an unknown one)."""
    spec = KvCacheSpec()
    _check(lib().kv_cache_spec_preset(int(preset), ctypes.byref(spec)), "kv_cache_spec_preset")
    return spec
