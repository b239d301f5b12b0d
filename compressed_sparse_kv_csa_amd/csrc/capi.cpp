// C ABI of the csakv library: argument validation, workspace layout, dispatch.
// Every check runs on the host before any launch; a rejected call enqueues nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/csakv.h"
#include "csakv_launch.h"

namespace {

constexpr int kKvDim = 512;
constexpr int kNopeDim = 448;
constexpr int kIdxDim = 128;
constexpr size_t kWsAlign = 256;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

csakv_status hip_status(hipError_t e) { return e == hipSuccess ? CSAKV_OK : CSAKV_ERR_HIP; }

// Checks a cache descriptor: format, row counts, pointers and alignment.
csakv_status check_cache(const csakv_cache* c, bool is_kv) {
  if (!c || c->reserved != 0) return CSAKV_ERR_INVALID;
  const int nfmt = 3;  // csakv_kv_fmt, or csakv_idx_fmt
  if (c->fmt < 0 || c->fmt >= nfmt) return CSAKV_ERR_INVALID;
  if (c->n_rows < 0) return CSAKV_ERR_INVALID;
  if (c->block_table) {  // paged: power-of-two pages of at least 16 rows, a table row per sequence
    const int32_t pr = c->page_rows;
    if (pr < 16 || (pr & (pr - 1)) != 0 || !aligned(c->block_table, 4)) return CSAKV_ERR_INVALID;
    if ((int64_t)c->table_stride * pr < c->n_rows || c->table_stride < 0) return CSAKV_ERR_INVALID;
  } else {
    if (c->page_rows != 0 || c->table_stride != 0) return CSAKV_ERR_INVALID;
    if (c->seq_stride_rows < c->n_rows) return CSAKV_ERR_INVALID;
  }
  // A cache without rows may have null pointers; any pointer given must be aligned.
  const bool empty = c->n_rows == 0;
  if ((!empty && !c->codes) || !aligned(c->codes, 16)) return CSAKV_ERR_INVALID;
  if (!aligned(c->seq_rows, 4)) return CSAKV_ERR_INVALID;
  const bool fp4 = is_kv ? c->fmt == CSAKV_KV_FP4 : c->fmt != CSAKV_IDX_BF16;
  if (fp4) {
    if ((!empty && !c->scales) || !aligned(c->scales, 16)) return CSAKV_ERR_INVALID;
  } else if (c->scales) {
    return CSAKV_ERR_INVALID;
  }
  return CSAKV_OK;
}

// The paging descriptor of a validated cache.
csakv::Paging paging(const csakv_cache* c) {
  csakv::Paging pg{c->block_table, 0, c->table_stride};
  if (c->block_table)
    while ((1 << pg.page_shift) < c->page_rows) ++pg.page_shift;
  return pg;
}

struct CsaLayout {
  csakv::IndexerPlan idx;
  csakv::AttnPlan attn;
  size_t idx_bytes, attn_offset, total;
};

CsaLayout csa_layout(const csakv_csa_params* p, int64_t n_c) {
  CsaLayout L{};
  L.idx_bytes = 0;
  if (p->mode == CSAKV_MODE_FULL) {
    L.idx = csakv::plan_indexer(p->batch, n_c, p->top_k);
    L.idx_bytes = round_up(csakv::indexer_workspace_bytes(p->batch, L.idx), kWsAlign);
  }
  L.attn = csakv::plan_attention(p->batch, (int64_t)p->window + p->top_k, true, p->n_q_heads);
  L.attn_offset = L.idx_bytes;
  L.total = L.idx_bytes + round_up(csakv::attention_workspace_bytes(p->batch, p->n_q_heads, L.attn), kWsAlign);
  return L;
}

// Parameters the indexer stage reads (FULL mode).
csakv_status check_select_params(const csakv_csa_params* p) {
  if (p->reserved != 0 || p->batch < 1 || p->top_k < 1 || p->n_idx_heads < 1)
    return CSAKV_ERR_INVALID;
  if (p->top_k > csakv::kMaxTopK || p->n_idx_heads > csakv::kMaxHeads) return CSAKV_ERR_UNSUPPORTED;
  return CSAKV_OK;
}

csakv_status check_csa_params(const csakv_csa_params* p) {
  if (!p || p->reserved != 0) return CSAKV_ERR_INVALID;
  if (p->batch < 1 || p->window < 0 || !std::isfinite(p->softmax_scale)) return CSAKV_ERR_INVALID;
  if (p->mode != CSAKV_MODE_FULL && p->mode != CSAKV_MODE_REUSE) return CSAKV_ERR_INVALID;
  if (p->top_k < 1 || p->n_q_heads < 1) return CSAKV_ERR_INVALID;
  if (p->top_k > csakv::kMaxTopK) return CSAKV_ERR_UNSUPPORTED;
  if (p->n_q_heads % 16 != 0 || p->n_q_heads > csakv::kMaxHeads) return CSAKV_ERR_UNSUPPORTED;
  if (p->mode == CSAKV_MODE_FULL) return check_select_params(p);
  return CSAKV_OK;
}

// ---- scratch of csa_decode_noalloc: one array in each GPU's memory, held until the process
// ends.  Host code never uses the array's name as an address: the device address of each
// GPU's copy comes from hipGetSymbolAddress on that GPU's first call and is kept per device.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_addr[kMaxDevices] = {};

// The current device's scratch address (looked up once per device, with it current).
csakv_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return CSAKV_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return CSAKV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CSAKV_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return CSAKV_OK;
}

}  // namespace

extern "C" {

const char* csakv_status_string(int32_t status) {
  switch (status) {
    case CSAKV_OK: return "ok";
    case CSAKV_ERR_INVALID: return "invalid argument";
    case CSAKV_ERR_UNSUPPORTED: return "unsupported shape or format";
    case CSAKV_ERR_WORKSPACE: return "workspace too small";
    case CSAKV_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

size_t csa_decode_workspace_bytes(const csakv_csa_params* p, int64_t n_compressed) {
  if (check_csa_params(p) != CSAKV_OK || n_compressed < 0) return 0;
  return csa_layout(p, n_compressed).total;
}

csakv_status csa_decode(const csakv_csa_params* p, const csakv_cache* kv,
                        const csakv_cache* idx_keys, const uint16_t* q, const uint16_t* q_idx,
                        const float* w_idx, int32_t* topk, uint16_t* out, void* workspace,
                        size_t workspace_bytes, void* stream) {
  csakv_status st = check_csa_params(p);
  if (st != CSAKV_OK) return st;
  if ((st = check_cache(kv, true)) != CSAKV_OK) return st;
  if (kv->n_rows < p->window) return CSAKV_ERR_INVALID;
  const int64_t n_c = kv->n_rows - p->window;
  if (kv->n_rows > INT32_MAX) return CSAKV_ERR_UNSUPPORTED;
  if (!q || !out || !topk || !aligned(q, 16) || !aligned(out, 16) || !aligned(topk, 4))
    return CSAKV_ERR_INVALID;
  const bool full = p->mode == CSAKV_MODE_FULL;
  if (full) {
    if ((st = check_cache(idx_keys, false)) != CSAKV_OK) return st;
    if (idx_keys->n_rows != n_c) return CSAKV_ERR_INVALID;
    if (!q_idx || !w_idx || !aligned(q_idx, 16) || !aligned(w_idx, 4)) return CSAKV_ERR_INVALID;
  } else if (idx_keys || q_idx || w_idx) {
    return CSAKV_ERR_INVALID;
  }
  const CsaLayout L = csa_layout(p, n_c);
  if (full && !csakv::indexer_supported(L.idx)) return CSAKV_ERR_UNSUPPORTED;
  if (!csakv::attention_supported(L.attn, kv->fmt, kv->n_rows)) return CSAKV_ERR_UNSUPPORTED;
  if (workspace_bytes < L.total) return CSAKV_ERR_WORKSPACE;
  if (L.total > 0 && (!workspace || !aligned(workspace, kWsAlign))) return CSAKV_ERR_INVALID;

  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  if (full) {
    hipError_t e = csakv::launch_indexer(
        idx_keys->fmt, static_cast<const uint8_t*>(idx_keys->codes), idx_keys->scales,
        idx_keys->seq_stride_rows, paging(idx_keys), n_c, idx_keys->seq_rows, q_idx, w_idx,
        p->batch, p->n_idx_heads, p->top_k, L.idx, ws, topk, s);
    if (e != hipSuccess) return CSAKV_ERR_HIP;
  }
  return hip_status(csakv::launch_attention(
      kv->fmt, true, static_cast<const uint8_t*>(kv->codes), kv->scales, kv->seq_stride_rows,
      paging(kv), kv->n_rows, kv->seq_rows, q, p->batch, p->n_q_heads, p->softmax_scale, topk,
      p->top_k,
      p->window, L.attn,
      ws + L.attn_offset, out, s));
}

csakv_status csa_decode_noalloc(const csakv_csa_params* p, const csakv_cache* kv,
                                const csakv_cache* idx_keys, const uint16_t* q,
                                const uint16_t* q_idx, const float* w_idx, int32_t* topk,
                                uint16_t* out, void* stream) {
  csakv_status st = check_csa_params(p);
  if (st != CSAKV_OK) return st;
  if ((st = check_cache(kv, true)) != CSAKV_OK) return st;
  if (kv->n_rows < p->window) return CSAKV_ERR_INVALID;
  const size_t need = csa_layout(p, kv->n_rows - p->window).total;
  if (need > kNoAllocScratchBytes) return CSAKV_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != CSAKV_OK) return st;
  return csa_decode(p, kv, idx_keys, q, q_idx, w_idx, topk, out, ws, kNoAllocScratchBytes, stream);
}

size_t csa_decode_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

size_t csa_select_topk_workspace_bytes(const csakv_csa_params* p, int64_t n_compressed) {
  if (!p || p->mode != CSAKV_MODE_FULL || check_select_params(p) != CSAKV_OK || n_compressed < 0)
    return 0;
  const csakv::IndexerPlan plan = csakv::plan_indexer(p->batch, n_compressed, p->top_k);
  return round_up(csakv::indexer_workspace_bytes(p->batch, plan), kWsAlign);
}

namespace {

// csa_select_topk and its two stages: validation, then the stages asked for.
csakv_status select_stages(const csakv_csa_params* p, const csakv_cache* idx_keys,
                           const uint16_t* q_idx, const float* w_idx, int32_t* topk,
                           void* workspace, size_t workspace_bytes, void* stream, int stages) {
  if (!p || p->mode != CSAKV_MODE_FULL) return CSAKV_ERR_INVALID;
  csakv_status st = check_select_params(p);
  if (st != CSAKV_OK) return st;
  if ((st = check_cache(idx_keys, false)) != CSAKV_OK) return st;
  if (idx_keys->n_rows > INT32_MAX) return CSAKV_ERR_UNSUPPORTED;
  const bool scan = stages & csakv::kStageScan, merge = stages & csakv::kStageMerge;
  if (scan && (!q_idx || !w_idx || !aligned(q_idx, 16) || !aligned(w_idx, 4)))
    return CSAKV_ERR_INVALID;
  if (merge && (!topk || !aligned(topk, 4))) return CSAKV_ERR_INVALID;
  const int64_t n_c = idx_keys->n_rows;
  const csakv::IndexerPlan plan = csakv::plan_indexer(p->batch, n_c, p->top_k);
  if (!csakv::indexer_supported(plan)) return CSAKV_ERR_UNSUPPORTED;
  const size_t need = round_up(csakv::indexer_workspace_bytes(p->batch, plan), kWsAlign);
  if (workspace_bytes < need) return CSAKV_ERR_WORKSPACE;
  if (need > 0 && (!workspace || !aligned(workspace, kWsAlign))) return CSAKV_ERR_INVALID;
  return hip_status(csakv::launch_indexer(
      idx_keys->fmt, static_cast<const uint8_t*>(idx_keys->codes), idx_keys->scales,
      idx_keys->seq_stride_rows, paging(idx_keys), n_c, idx_keys->seq_rows, q_idx, w_idx, p->batch,
      p->n_idx_heads, p->top_k, plan, workspace, topk, static_cast<hipStream_t>(stream), stages));
}

}  // namespace

csakv_status csa_select_topk(const csakv_csa_params* p, const csakv_cache* idx_keys,
                             const uint16_t* q_idx, const float* w_idx, int32_t* topk,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return select_stages(p, idx_keys, q_idx, w_idx, topk, workspace, workspace_bytes, stream,
                       csakv::kStageScan | csakv::kStageMerge);
}

csakv_status csa_select_scan(const csakv_csa_params* p, const csakv_cache* idx_keys,
                             const uint16_t* q_idx, const float* w_idx, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return select_stages(p, idx_keys, q_idx, w_idx, nullptr, workspace, workspace_bytes, stream,
                       csakv::kStageScan);
}

csakv_status csa_select_merge(const csakv_csa_params* p, const csakv_cache* idx_keys,
                              int32_t* topk, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return select_stages(p, idx_keys, nullptr, nullptr, topk, workspace, workspace_bytes, stream,
                       csakv::kStageMerge);
}

size_t csa_reindex_topk_workspace_bytes(const csakv_csa_params* p, int32_t n_pool) {
  if (!p || p->mode != CSAKV_MODE_REINDEX || check_select_params(p) != CSAKV_OK || n_pool < 1 ||
      n_pool > csakv::kMaxPool)
    return 0;
  return round_up(csakv::reindex_workspace_bytes(p->batch, n_pool), kWsAlign);
}

csakv_status csa_reindex_topk(const csakv_csa_params* p, const csakv_cache* idx_keys,
                              const uint16_t* q_idx, const float* w_idx, const int32_t* pool,
                              int32_t n_pool, int32_t* topk, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (!p || p->mode != CSAKV_MODE_REINDEX) return CSAKV_ERR_INVALID;
  csakv_status st = check_select_params(p);
  if (st != CSAKV_OK) return st;
  if ((st = check_cache(idx_keys, false)) != CSAKV_OK) return st;
  if (n_pool < 1) return CSAKV_ERR_INVALID;
  if (n_pool > csakv::kMaxPool) return CSAKV_ERR_UNSUPPORTED;
  if (!q_idx || !w_idx || !pool || !topk || !aligned(q_idx, 16) || !aligned(w_idx, 4) ||
      !aligned(pool, 4) || !aligned(topk, 4))
    return CSAKV_ERR_INVALID;
  const int64_t n_c = idx_keys->n_rows;
  if (n_c > INT32_MAX || !csakv::reindex_supported(idx_keys->fmt, n_c))
    return CSAKV_ERR_UNSUPPORTED;
  // The output must not overlap the pool it is computed from.
  const uintptr_t pb = reinterpret_cast<uintptr_t>(pool), tb = reinterpret_cast<uintptr_t>(topk);
  const uintptr_t pe = pb + (uintptr_t)p->batch * n_pool * 4, te = tb + (uintptr_t)p->batch * p->top_k * 4;
  if (pb < te && tb < pe) return CSAKV_ERR_INVALID;
  const size_t need = round_up(csakv::reindex_workspace_bytes(p->batch, n_pool), kWsAlign);
  if (workspace_bytes < need) return CSAKV_ERR_WORKSPACE;
  if (!workspace || !aligned(workspace, kWsAlign)) return CSAKV_ERR_INVALID;
  return hip_status(csakv::launch_reindex(
      idx_keys->fmt, static_cast<const uint8_t*>(idx_keys->codes), idx_keys->scales,
      idx_keys->seq_stride_rows, paging(idx_keys), n_c, idx_keys->seq_rows, q_idx, w_idx, p->batch,
      p->n_idx_heads, pool, n_pool,
      p->top_k, topk, workspace, static_cast<hipStream_t>(stream)));
}

size_t hca_decode_workspace_bytes(int32_t batch, int32_t n_q_heads, int64_t n_rows) {
  if (batch < 1 || n_q_heads < 1 || n_rows < 0) return 0;
  csakv::AttnPlan a = csakv::plan_attention(batch, n_rows, false, n_q_heads);
  return round_up(csakv::attention_workspace_bytes(batch, n_q_heads, a), kWsAlign);
}

csakv_status hca_decode(int32_t batch, int32_t n_q_heads, float softmax_scale,
                        const csakv_cache* kv, const uint16_t* q, uint16_t* out, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (batch < 1 || n_q_heads < 1 || !std::isfinite(softmax_scale)) return CSAKV_ERR_INVALID;
  if (n_q_heads % 16 != 0 || n_q_heads > csakv::kMaxHeads) return CSAKV_ERR_UNSUPPORTED;
  csakv_status st = check_cache(kv, true);
  if (st != CSAKV_OK) return st;
  if (!q || !out || !aligned(q, 16) || !aligned(out, 16)) return CSAKV_ERR_INVALID;
  if (kv->n_rows > INT32_MAX) return CSAKV_ERR_UNSUPPORTED;
  if (!csakv::attention_supported(csakv::plan_attention(batch, kv->n_rows, false, n_q_heads),
                                 kv->fmt, kv->n_rows))
    return CSAKV_ERR_UNSUPPORTED;
  const size_t need = hca_decode_workspace_bytes(batch, n_q_heads, kv->n_rows);
  if (workspace_bytes < need) return CSAKV_ERR_WORKSPACE;
  if (need > 0 && (!workspace || !aligned(workspace, kWsAlign))) return CSAKV_ERR_INVALID;
  csakv::AttnPlan a = csakv::plan_attention(batch, kv->n_rows, false, n_q_heads);
  return hip_status(csakv::launch_attention(
      kv->fmt, false, static_cast<const uint8_t*>(kv->codes), kv->scales, kv->seq_stride_rows,
      paging(kv), kv->n_rows, kv->seq_rows, q, batch, n_q_heads, softmax_scale, nullptr, 0, 0, a,
      workspace, out,
      static_cast<hipStream_t>(stream)));
}

csakv_status rope_output(uint16_t* out, int32_t batch, int32_t n_heads, const int64_t* positions,
                         double base, void* stream) {
  if (batch < 1 || n_heads < 1 || !std::isfinite(base) || base <= 0.0) return CSAKV_ERR_INVALID;
  if (!out || !positions || !aligned(out, 16) || !aligned(positions, 8)) return CSAKV_ERR_INVALID;
  return hip_status(csakv::launch_rope_output(out, batch, n_heads, positions, base,
                                              static_cast<hipStream_t>(stream)));
}

csakv_status idx_quantize_fp4_hadamard(const uint16_t* x, int64_t rows, uint8_t* codes,
                                       uint8_t* scales, void* stream) {
  if (rows < 0) return CSAKV_ERR_INVALID;
  if (rows == 0) return CSAKV_OK;
  if (!x || !codes || !scales || !aligned(x, 16) || !aligned(codes, 8)) return CSAKV_ERR_INVALID;
  return hip_status(
      csakv::launch_quantize_fp4h(x, rows, codes, scales, static_cast<hipStream_t>(stream)));
}

csakv_status kv_cache_write(int32_t fmt, int32_t dim, void* codes, uint8_t* scales,
                            int64_t seq_stride_rows, int64_t n_rows, int32_t batch, int32_t n,
                            const uint16_t* x, const int32_t* dst, void* stream) {
  if (fmt < CSAKV_KV_BF16 || fmt > CSAKV_KV_FP4) return CSAKV_ERR_INVALID;
  if (dim == kIdxDim) {
    if (fmt == CSAKV_KV_FP8_MIXED) return CSAKV_ERR_UNSUPPORTED;
  } else if (dim != kKvDim) {
    return CSAKV_ERR_UNSUPPORTED;
  }
  if (batch < 1 || n < 0 || n_rows < 0 || seq_stride_rows < n_rows) return CSAKV_ERR_INVALID;
  if (n == 0 || n_rows == 0) return CSAKV_OK;
  if (!codes || !x || !dst || !aligned(codes, 16) || !aligned(x, 16) || !aligned(dst, 4))
    return CSAKV_ERR_INVALID;
  if ((fmt == CSAKV_KV_FP4) != (scales != nullptr)) return CSAKV_ERR_INVALID;
  if (n_rows > INT32_MAX) return CSAKV_ERR_UNSUPPORTED;
  return hip_status(csakv::launch_cache_write(fmt, dim, codes, scales, seq_stride_rows, n_rows,
                                              batch, n, x, dst, static_cast<hipStream_t>(stream)));
}

csakv_status kv_quantize_fp4(const uint16_t* x, int64_t rows, int32_t dim, uint8_t* codes,
                             uint8_t* scales, void* stream) {
  if (rows < 0 || dim <= 0 || dim % 16 != 0) return CSAKV_ERR_INVALID;
  if (!x || !codes || !scales || !aligned(x, 16) || !aligned(codes, 8)) return CSAKV_ERR_INVALID;
  return hip_status(csakv::launch_quantize_fp4(x, rows, dim, codes, scales,
                                               static_cast<hipStream_t>(stream)));
}

csakv_status kv_quantize_fp8(const uint16_t* x, int64_t rows, int32_t dim, int32_t nope_dim,
                             uint8_t* out, void* stream) {
  if (rows < 0 || dim <= 0 || dim % 16 != 0 || nope_dim < 0 || nope_dim > dim ||
      nope_dim % 16 != 0)
    return CSAKV_ERR_INVALID;
  if (!x || !out || !aligned(x, 16) || !aligned(out, 16)) return CSAKV_ERR_INVALID;
  return hip_status(csakv::launch_quantize_fp8_mixed(x, rows, dim, nope_dim, out,
                                                     static_cast<hipStream_t>(stream)));
}

csakv_status kv_dequantize(int32_t fmt, const void* codes, const uint8_t* scales, int64_t rows,
                           int32_t dim, uint16_t* out, void* stream) {
  if (rows < 0 || dim <= 0 || dim % 16 != 0) return CSAKV_ERR_INVALID;
  if (!codes || !out || !aligned(codes, 16) || !aligned(out, 16)) return CSAKV_ERR_INVALID;
  int nope = 0;
  if (fmt == CSAKV_KV_BF16) {
    if (scales) return CSAKV_ERR_INVALID;
  } else if (fmt == CSAKV_KV_FP8_MIXED) {
    if (scales) return CSAKV_ERR_INVALID;
    if (dim != kKvDim) return CSAKV_ERR_UNSUPPORTED;
    nope = kNopeDim;
  } else if (fmt == CSAKV_KV_FP4) {
    if (!scales || !aligned(codes, 8)) return CSAKV_ERR_INVALID;
  } else {
    return CSAKV_ERR_INVALID;
  }
  return hip_status(csakv::launch_dequantize(fmt, codes, scales, rows, dim, nope, out,
                                             static_cast<hipStream_t>(stream)));
}

uint64_t kv_cache_bytes(const kv_cache_spec* sp, int64_t seq_len, kv_cache_breakdown* out) {
  if (!sp || seq_len < 0 || sp->reserved != 0) return 0;
  if (sp->n_csa < 0 || sp->n_hca < 0 || sp->n_swa < 0 || sp->csa_ratio < 1 || sp->hca_ratio < 1 ||
      sp->window < 0 || sp->kv_dim <= 0 || sp->rope_dim < 0 || sp->rope_dim > sp->kv_dim ||
      sp->idx_dim < 0 || sp->count_window < 0 || sp->count_window > 2 || sp->count_scales < 0 ||
      sp->count_scales > 1 || sp->swa_layer_bytes < 0)
    return 0;
  // Code bytes per row, and FP4 scale bytes per row (added to the row when count_scales).
  uint64_t s_kv, sc_kv = 0;
  switch (sp->kv_fmt) {
    case CSAKV_KV_BF16: s_kv = 2ull * sp->kv_dim; break;
    case CSAKV_KV_FP8_MIXED: s_kv = (uint64_t)(sp->kv_dim - sp->rope_dim) + 2ull * sp->rope_dim; break;
    case CSAKV_KV_FP4:
      if (sp->kv_dim % 16) return 0;
      s_kv = sp->kv_dim / 2;
      sc_kv = sp->kv_dim / 16;
      break;
    default: return 0;
  }
  uint64_t s_idx = 0, sc_idx = 0;
  if (sp->idx_dim > 0) {
    switch (sp->idx_fmt) {
      case CSAKV_IDX_BF16: s_idx = 2ull * sp->idx_dim; break;
      case CSAKV_IDX_FP4:
      case CSAKV_IDX_FP4_HADAMARD:  // the same bytes: codes of the rotated row, and scales
        if (sp->idx_dim % 16) return 0;
        s_idx = sp->idx_dim / 2;
        sc_idx = sp->idx_dim / 16;
        break;
      default: return 0;
    }
  }
  const uint64_t n = (uint64_t)seq_len;
  const uint64_t n_c = sp->n_csa ? n / sp->csa_ratio : 0;
  const uint64_t n_h = sp->n_hca ? n / sp->hca_ratio : 0;
  const uint64_t cw = (uint64_t)sp->count_window;
  kv_cache_breakdown r{};
  r.scales = sp->n_csa * (n_c * (sc_kv + sc_idx) + cw * sp->window * sc_kv) +
             sp->n_hca * (n_h + cw * sp->window) * sc_kv;
  if (sp->count_scales) {
    s_kv += sc_kv;
    s_idx += sc_idx;
  }
  const uint64_t win = cw * sp->window * s_kv;
  r.csa_per_layer = n_c * s_kv + n_c * s_idx + win;
  r.hca_per_layer = n_h * s_kv + win;
  r.csa_shared_kv = sp->n_csa * n_c * s_kv;
  r.csa_indexer = sp->n_csa * n_c * s_idx;
  r.hca_shared_kv = sp->n_hca * n_h * s_kv;
  r.windows = (uint64_t)(sp->n_csa + sp->n_hca) * win;
  r.swa_layers = (uint64_t)sp->n_swa * (uint64_t)sp->swa_layer_bytes;
  r.total = sp->n_csa * r.csa_per_layer + sp->n_hca * r.hca_per_layer + r.swa_layers;
  if (out) *out = r;
  return r.total;
}

csakv_status kv_cache_spec_preset(int32_t preset, kv_cache_spec* out) {
  if (!out) return CSAKV_ERR_INVALID;
  kv_cache_spec s{};
  // V4-Pro: 30 CSA + 31 HCA layers, 512-dim rows (64 of them RoPE), 128-dim indexer keys.
  s.n_csa = 30;
  s.n_hca = 31;
  s.csa_ratio = 4;
  s.hca_ratio = 128;
  s.window = 128;
  s.kv_dim = 512;
  s.rope_dim = 64;
  s.idx_dim = 128;
  s.kv_fmt = CSAKV_KV_BF16;
  s.idx_fmt = CSAKV_IDX_BF16;
  s.count_window = 1;
  switch (preset) {
    case CSAKV_PRESET_V4_PRO_BF16:
      break;
    case CSAKV_PRESET_V4_PRO_MIXED:
      s.kv_fmt = CSAKV_KV_FP8_MIXED;
      s.idx_fmt = CSAKV_IDX_FP4;
      break;
    case CSAKV_PRESET_V4_FLASH:
      s.n_csa = 21;
      s.n_hca = 20;
      s.n_swa = 2;
      s.count_window = 0;
      s.swa_layer_bytes = 2 * 128 * 2 * (128 + 256);  // K and V, one bf16 head, padded window
      break;
    case CSAKV_PRESET_V3_MLA:
    case CSAKV_PRESET_V32_DSA:
      s.n_csa = 61;  // every layer keeps one uncompressed row per token
      s.n_hca = 0;
      s.csa_ratio = 1;
      s.window = 0;
      s.kv_dim = 576;
      s.rope_dim = 64;
      s.idx_dim = preset == CSAKV_PRESET_V32_DSA ? 128 : 0;
      s.count_window = 0;
      break;
    default:
      return CSAKV_ERR_INVALID;
  }
  *out = s;
  return CSAKV_OK;
}

}  // extern "C"
