/*
 * csakv.h - decode-time attention over compressed sparse KV caches on MI355X (gfx950).
 *
 * The operation, as the source pages state it ("DeepSeek-V4 KV Cache 深度分析",
 * sections 三 "压缩机制详解", 四 "索引器（Indexer）机制" and the 十一 forward-flow
 * diagram):
 *   - CSA layers keep one 512-wide shared-KV entry per 4 tokens (448 no-RoPE dims,
 *     then 64 RoPE dims) plus a 128-wide indexer key per entry.  For each query
 *     token an indexer score picks the top-k compressed entries, and attention runs
 *     over those entries together with the most recent 128 uncompressed tokens
 *     (the sliding window).  Every entry is both key and value.
 *   - HCA layers keep one entry per 128 tokens and attend densely over all of them
 *     plus the window, without an indexer.
 *   - CSA2 "Reuse" layers ("DeepSeek, KV 캐시를 토큰당 890바이트로 줄인 V4.1-Flash 공개",
 *     section 핵심 내용; "KV cache 890 bajtów na token", section "Trzy mechanizmy
 *     zamiast jednej sztuczki") attend with the top-512 indices an earlier layer chose.
 * The pages give no formula for the indexer score; this library computes
 *     s_j = sum_h w_h * ReLU(q_h . k_j)
 * and keeps the k largest, ties broken toward the smaller index.
 *
 * Conventions shared by every entry point
 *   - All data pointers are DEVICE pointers into memory the caller owns (for
 *     example PyTorch tensors).  The library never allocates or frees device
 *     memory, keeps no pointer after a call returns and has no global state,
 *     except the fixed device scratch that csa_decode_noalloc alone uses.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     default stream).  No call synchronises.  Device faults surface at the
 *     caller's next synchronisation.
 *   - Every argument is checked on the host before anything is launched.  A
 *     rejected call returns CSAKV_ERR_INVALID, CSAKV_ERR_UNSUPPORTED or
 *     CSAKV_ERR_WORKSPACE and enqueues nothing.  A failed launch returns
 *     CSAKV_ERR_HIP.
 *   - bf16 tensors are passed as uint16_t bit patterns; every row is contiguous
 *     and little-endian.  Device pointers must be 16-byte aligned.
 *   - Calls that take a workspace need `workspace_bytes >= *_workspace_bytes(...)`;
 *     its contents need no initialisation and are scratch after the call.
 */
#ifndef CSAKV_H
#define CSAKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CSAKV_OK = 0,
  CSAKV_ERR_INVALID = -1,      /* null/misaligned pointer, bad size or shape      */
  CSAKV_ERR_UNSUPPORTED = -2,  /* valid request outside what the kernels support  */
  CSAKV_ERR_WORKSPACE = -3,    /* workspace smaller than *_workspace_bytes        */
  CSAKV_ERR_HIP = -4           /* a HIP launch reported an error                   */
} csakv_status;

/* Storage formats of 512-wide shared-KV rows ("DeepSeek-V4 KV Cache 深度分析", sections
 * 二 and 六; the V4.1-Flash pages for FP4).  Row bytes: BF16 1024; FP8_MIXED 576 =
 * 448 OCP E4M3FN bytes (unscaled) followed by the 64 RoPE dims as bf16; FP4 256 code
 * bytes (E2M1, element 2i in the low nibble of byte i) plus 32 scale bytes (one
 * E4M3FN scale per 16 channels) held in a separate scale plane. */
typedef enum { CSAKV_KV_BF16 = 0, CSAKV_KV_FP8_MIXED = 1, CSAKV_KV_FP4 = 2 } csakv_kv_fmt;

/* Storage formats of 128-wide indexer-key rows: BF16 256 bytes; FP4 64 code bytes
 * plus 8 scale bytes in a separate scale plane ("DeepSeek-V4 KV Cache 深度分析",
 * section 四: indexer keys are cached in FP4).  FP4_HADAMARD stores the same bytes for
 * the FP4 codes of each row's Hadamard rotation (section 四, 结构: a Hadamard rotation,
 * then FP4 quantisation over all 128 dims; written by idx_quantize_fp4_hadamard); with
 * it the indexer rotates and FP4-quantises each query row the same way before scoring,
 * so the QK product is FP4 x FP4 (decoded exactly, accumulated in fp32). */
typedef enum { CSAKV_IDX_BF16 = 0, CSAKV_IDX_FP4 = 1, CSAKV_IDX_FP4_HADAMARD = 2 } csakv_idx_fmt;

/* Layer modes of CSA2 ("DeepSeek, KV 캐시를 토큰당 890바이트로 줄인 V4.1-Flash 공개",
 * section 핵심 내용; "KV cache 890 bajtów na token", section "Trzy mechanizmy zamiast
 * jednej sztuczki"): FULL scores every compressed entry; REINDEX re-ranks the Full
 * layer's candidate pool with its own indexer query (csa_reindex_topk); REUSE attends
 * with indices chosen by an earlier layer.  csa_decode runs FULL or REUSE; a Reindex
 * layer is csa_reindex_topk followed by csa_decode in REUSE mode. */
typedef enum { CSAKV_MODE_FULL = 0, CSAKV_MODE_REUSE = 1, CSAKV_MODE_REINDEX = 2 } csakv_mode;

/* One cache tensor of B sequences.  Sequence b's row r starts at byte
 * (b * seq_stride_rows + r) * code_bytes(fmt) of `codes`; for FP4 its scales start
 * at byte (b * seq_stride_rows + r) * (dim / 16) of `scales` (NULL otherwise).
 * Shared-KV rows of a sequence are [window rows | compressed rows]: top-k index j
 * names row window + j.  A cache with n_rows == 0 may pass NULL pointers.
 * Variable lengths: with seq_rows == NULL every sequence holds n_rows rows; otherwise
 * seq_rows is a device array [B] of int32 and sequence b holds rows
 * [0, seq_rows[b]) (values are clamped to [0, n_rows], so n_rows is the capacity).
 * For a CSA layer the shared-KV lengths are window + N_c(b) and the indexer-key
 * lengths N_c(b); each query selects among, and attends over, its own rows only
 * (a sequence shorter than the window attends over the window rows it holds).
 * Paged layout (block_table != NULL): `codes` (and `scales`) hold a pool of pages of
 * page_rows rows each, page p's rows starting at row p * page_rows of the pool; row r
 * of sequence b lives at row r % page_rows of page block_table[b * table_stride +
 * r / page_rows].  page_rows is a multiple of 16; table_stride >= ceil(n_rows /
 * page_rows); seq_stride_rows is then unused; every page id a sequence's rows reach
 * must name a page of the pool, and the pool's codes (and scales) must span at most
 * 4 GiB - 256 bytes.  Decode-step writes into a paged pool go through kv_cache_write
 * with the pool viewed as one sequence and physical rows (page * page_rows + offset). */
typedef struct {
  int32_t fmt;              /* csakv_kv_fmt for shared-KV, csakv_idx_fmt for keys */
  int32_t reserved;         /* must be 0                                            */
  int64_t n_rows;           /* rows per sequence (the capacity with seq_rows)       */
  int64_t seq_stride_rows;  /* rows between consecutive sequences, >= n_rows        */
  const void* codes;
  const uint8_t* scales;
  const int32_t* seq_rows;  /* NULL, or [B] device int32 rows of each sequence      */
  const int32_t* block_table; /* NULL (contiguous), or [B][table_stride] page ids   */
  int32_t page_rows;        /* paged: rows per page (multiple of 16); else 0        */
  int32_t table_stride;     /* paged: page-table entries per sequence; else 0       */
} csakv_cache;

typedef struct {
  int32_t batch;            /* B >= 1 query tokens, one independent sequence each  */
  int32_t n_q_heads;        /* H_q: a multiple of 16, at most 128                    */
  int32_t n_idx_heads;      /* H_I: 1..128 (FULL mode)                              */
  int32_t top_k;            /* 1..2048                                              */
  int32_t window;           /* window rows at the start of each sequence, >= 0      */
  int32_t mode;             /* csakv_mode                                           */
  float softmax_scale;      /* logit scale, e.g. 1/sqrt(512)                        */
  int32_t reserved;         /* must be 0                                            */
} csakv_csa_params;

/* Head and selection limits follow the pages: V4-Pro's query projection yields 128 heads
 * of 512 ("DeepSeek-V4 KV Cache 深度分析", section 十一 forward-flow diagram), and its
 * indexer keeps the top 1024 (section 一 index_topk; 512 on the V4.1-Flash page); the
 * library accepts up to 128 heads of either kind and top_k up to 2048.  Calls beyond
 * them return CSAKV_ERR_UNSUPPORTED.  */

/* Bytes of workspace csa_decode needs for these parameters and N_c compressed rows. */
size_t csa_decode_workspace_bytes(const csakv_csa_params* p, int64_t n_compressed);

/* CSA decode for B query tokens (one layer).
 *   kv       shared-KV cache, n_rows = window + N_c, any csakv_kv_fmt.
 *   idx_keys FULL: indexer keys, n_rows = N_c, any csakv_idx_fmt; REUSE: NULL.
 *   q        [B][H_q][512] bf16 attention queries.
 *   q_idx    FULL: [B][H_I][128] bf16 indexer queries; REUSE: NULL.
 *   w_idx    FULL: [B][H_I] fp32 indexer head weights; REUSE: NULL.
 *   topk     [B][top_k] int32.  FULL writes the set of selected compressed-row
 *            indices (ties in score go to the lower index) in an unspecified but
 *            deterministic order; -1 pads when N_c < top_k.
 *            REUSE reads it (entries < 0 or >= N_c are skipped).
 *   out      [B][H_q][512] bf16: softmax(scale * q . e) weighted sum of the rows
 *            e in (window rows) + (selected rows), one softmax over their union.
 *            A query with no rows gets zeros.
 * Returns CSAKV_ERR_UNSUPPORTED for head/row dims other than 512 (KV) and 128
 * (indexer keys) implied by the formats, or for shapes beyond the limits above. */
csakv_status csa_decode(const csakv_csa_params* p, const csakv_cache* kv,
                        const csakv_cache* idx_keys, const uint16_t* q,
                        const uint16_t* q_idx, const float* w_idx, int32_t* topk,
                        uint16_t* out, void* workspace, size_t workspace_bytes,
                        void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): csa_decode with the library's own device
 * scratch in place of a caller workspace, arguments otherwise as csa_decode.  The scratch is
 * one array of csa_decode_noalloc_scratch_bytes() bytes (32 MiB) in the memory of each GPU
 * the library runs on, held until the process ends; its address is looked up on the first
 * call on each device.  The call allocates nothing: a request whose
 * csa_decode_workspace_bytes exceeds the scratch returns CSAKV_ERR_WORKSPACE before any
 * launch.  Every call on one GPU shares that GPU's scratch, which keeps the last call's
 * contents (nothing in it needs to start at zero): calls that overlap on one GPU (other
 * streams, other threads) race and must be serialised by the caller. */
csakv_status csa_decode_noalloc(const csakv_csa_params* p, const csakv_cache* kv,
                                const csakv_cache* idx_keys, const uint16_t* q,
                                const uint16_t* q_idx, const float* w_idx, int32_t* topk,
                                uint16_t* out, void* stream);
size_t csa_decode_noalloc_scratch_bytes(void);

/* Bytes of workspace csa_select_topk needs for these parameters and N_c rows. */
size_t csa_select_topk_workspace_bytes(const csakv_csa_params* p, int64_t n_compressed);

/* The indexer stage of a CSA Full layer alone ("DeepSeek-V4 KV Cache 深度分析", section
 * 四: the indexer query is scored against every compressed entry's key and the top-k
 * are kept): writes topk [B][top_k] exactly as csa_decode's FULL mode does, without
 * the attention.  p->mode must be CSAKV_MODE_FULL; p->n_q_heads and p->window are
 * not used.  idx_keys, q_idx, w_idx as for csa_decode. */
csakv_status csa_select_topk(const csakv_csa_params* p, const csakv_cache* idx_keys,
                             const uint16_t* q_idx, const float* w_idx, int32_t* topk,
                             void* workspace, size_t workspace_bytes, void* stream);

/* The two stages of csa_select_topk, for callers that schedule them apart (and to time
 * the scoring pass on its own).  csa_select_scan scores every key row and leaves, in the
 * workspace, each 4096-row slice's candidates (every key at or above a per-slice bound),
 * the bound and every row's score; csa_select_merge then writes topk exactly as
 * csa_select_topk does (it re-reads a slice's scores when its bound lies above the k-th
 * score).  Both take the arguments csa_select_topk takes, the same workspace (of
 * csa_select_topk_workspace_bytes bytes, unchanged between the two calls) and the same
 * p and idx_keys; run in this order on one stream, they equal one csa_select_topk call. */
csakv_status csa_select_scan(const csakv_csa_params* p, const csakv_cache* idx_keys,
                             const uint16_t* q_idx, const float* w_idx, void* workspace,
                             size_t workspace_bytes, void* stream);
csakv_status csa_select_merge(const csakv_csa_params* p, const csakv_cache* idx_keys,
                              int32_t* topk, void* workspace, size_t workspace_bytes,
                              void* stream);

/* CSA2 Reindex, the hierarchical sparse indexer ("DeepSeek, KV 캐시를 토큰당 890바이트로
 * 줄인 V4.1-Flash 공개", section 핵심 내용: a Reindex layer computes only a new query and
 * re-ranks; "KV cache 890 bajtów na token", section "Trzy mechanizmy zamiast jednej
 * sztuczki": deeper layers index only the candidate pool the group's Full layer built,
 * so their indexing cost no longer grows with the context).  For each query b, the rows
 * of pool[b] are scored with this layer's indexer query as s_j = sum_h w_h *
 * ReLU(q_h . k_j) over the shared indexer keys, and the top_k of the pool are kept.
 *   p         mode CSAKV_MODE_REINDEX; batch, n_idx_heads (1..128) and top_k
 *             (1..2048) are used, n_q_heads, window and softmax_scale are not.
 *   idx_keys  the shared indexer keys, n_rows = N_c, any csakv_idx_fmt; one sequence's
 *             keys (codes, and FP4 scales) must span at most 4 GiB - 256 bytes.
 *   q_idx     [B][H_I][128] bf16, this layer's indexer queries.
 *   w_idx     [B][H_I] fp32, this layer's head weights.
 *   pool      [B][n_pool] int32 compressed-row indices, 1 <= n_pool <= 4096, for
 *             example csa_select_topk's output with top_k = n_pool.  Entries < 0 or
 *             >= N_c are empty; the other entries of one query must be distinct.
 *   topk      [B][top_k] int32: the set of the top_k pool rows (ties in score go to
 *             the lower row index) in pool order; -1 pads when the pool holds fewer
 *             rows.  Must not overlap pool.
 *   workspace device memory of csa_reindex_topk_workspace_bytes(p, n_pool) bytes,
 *             256-byte aligned, overlapping no argument; it holds every pool slot's
 *             score between the call's two launches and may be reused once the call's
 *             work on `stream` has finished. */
csakv_status csa_reindex_topk(const csakv_csa_params* p, const csakv_cache* idx_keys,
                              const uint16_t* q_idx, const float* w_idx, const int32_t* pool,
                              int32_t n_pool, int32_t* topk, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Bytes of workspace csa_reindex_topk needs for p->batch queries of n_pool slots
 * (8 per slot, rounded up to 256); 0 when p or n_pool is invalid. */
size_t csa_reindex_topk_workspace_bytes(const csakv_csa_params* p, int32_t n_pool);

/* Bytes of workspace hca_decode needs for B sequences of n_rows rows each. */
size_t hca_decode_workspace_bytes(int32_t batch, int32_t n_q_heads, int64_t n_rows);

/* HCA decode ("DeepSeek-V4 KV Cache 深度分析", section 三 part 1): dense attention of
 * q [B][H_q][512] over every row of each sequence of `kv` (window and compressed
 * rows alike), out [B][H_q][512] bf16. */
csakv_status hca_decode(int32_t batch, int32_t n_q_heads, float softmax_scale,
                        const csakv_cache* kv, const uint16_t* q, uint16_t* out,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Output RoPE with position -i ("DeepSeek-V4 KV Cache 深度分析", section 五: the core
 * attention output o_{t,i} gets RoPE at position -i on its last 64 dims, which turns the
 * absolute positions R(j) that the entries carry into relative positions R(j - i)).
 * In place on out [B][n_heads][512] bf16 (for example csa_decode's or hca_decode's
 * output): for query b, pair (448 + 2k, 448 + 2k + 1), k < 32, of every head turns by
 * angle -positions[b] * base^(-2k/64), i.e. (x, y) -> (x cos - y sin, x sin + y cos).
 * positions [B] int64 (device).  base > 0 (the pages give none; 10000 is customary).
 * Angles, sines and cosines are fp64; the rotation is fp32, rounded to bf16 (nearest
 * even). */
csakv_status rope_output(uint16_t* out, int32_t batch, int32_t n_heads, const int64_t* positions,
                         double base, void* stream);

/* FP4 block quantisation of bf16 rows x [rows][dim] (dim % 16 == 0), the cache-write side
 * of the FP4 formats: FP4 E2M1 values with one E4M3 scale per 16 channels for the main KV
 * ("DeepSeek, KV 캐시를 토큰당 890바이트로 줄인 V4.1-Flash 공개", section 핵심 내용; "KV cache
 * 890 bajtów na token", section "Trzy mechanizmy zamiast jednej sztuczki") and FP4 indexer
 * keys ("DeepSeek-V4 KV Cache 深度分析", sections 四 and 六).  The pages fix neither
 * rounding; this library takes:
 * scale = E4M3FN(amax/6) per 16 channels (round to nearest even, saturating);
 * code  = E2M1(x / scale), or 0 for every element when the scale decodes to 0.
 * codes [rows][dim/2], scales [rows][dim/16].  x, codes and scales are device pointers
 * (x 16-byte aligned, codes 8-byte aligned); a negative row count or a dim that is not a
 * positive multiple of 16 returns CSAKV_ERR_INVALID. */
csakv_status kv_quantize_fp4(const uint16_t* x, int64_t rows, int32_t dim,
                             uint8_t* codes, uint8_t* scales, void* stream);

/* Mixed FP8/BF16 rows, the 576-byte shared-KV entry of "DeepSeek-V4 KV Cache 深度分析"
 * (section 二: the 448 no-RoPE dims are quantised to FP8 and the 64 RoPE dims kept in bf16
 * on the way into the cache; section 六: 448 + 64 x 2 = 576 bytes, no scale bytes):
 * out [rows][nope_dim + 2*(dim - nope_dim)] holds E4M3FN(x[0..nope_dim)) (round to nearest
 * even, saturating at 448; the pages give no scaling, so the cast is unscaled) followed by
 * the bf16 bytes of x[nope_dim..dim).  nope_dim % 16 == 0, dim % 16 == 0; x and out are
 * 16-byte aligned device pointers; other shapes return CSAKV_ERR_INVALID. */
csakv_status kv_quantize_fp8(const uint16_t* x, int64_t rows, int32_t dim,
                             int32_t nope_dim, uint8_t* out, void* stream);

/* Hadamard-rotated FP4 indexer keys ("DeepSeek-V4 KV Cache 深度分析", section 四, 结构):
 * each bf16 row x [rows][128] is rotated to H x / sqrt(128), H the Sylvester Hadamard
 * matrix: the product H x exactly (exact for rows whose nonzero magnitudes span at most 38
 * binades), rounded once to fp32, then multiplied once by fp32(1/sqrt(128)); the rotated
 * row is FP4-quantised as kv_quantize_fp4 does: codes [rows][64], scales [rows][8].  The rows of a
 * CSAKV_IDX_FP4_HADAMARD cache.  A decode-step write points codes / scales at the
 * destination row. */
csakv_status idx_quantize_fp4_hadamard(const uint16_t* x, int64_t rows, uint8_t* codes,
                                       uint8_t* scales, void* stream);

/* Decode-step cache write ("DeepSeek-V4 KV Cache 深度分析", section 二: a new entry is
 * quantised on its way into the cache, its 448 no-RoPE dims to E4M3 and its 64 RoPE
 * dims kept as bf16; section 十一: the compressed row is then written into the KV
 * cache).  The n new rows of each sequence, x [B][n][dim] bf16, are encoded in `fmt`
 * exactly as kv_quantize_fp8 / kv_quantize_fp4 do (bf16 rows are copied) and stored at
 * row dst[b][i] of sequence b: byte (b * seq_stride_rows + dst[b][i]) * code_bytes of
 * `codes`, and for FP4 byte (b * seq_stride_rows + dst[b][i]) * dim / 16 of `scales`.
 *   fmt, dim  a csakv_kv_fmt with dim 512 (shared-KV rows), or CSAKV_KV_BF16 /
 *             CSAKV_KV_FP4 with dim 128 (indexer-key rows: 256 B, or 64 code bytes
 *             plus 8 scale bytes).
 *   dst       [B][n] int32 rows: the ring slot of a new window token, or window + j for
 *             new compressed entry j.  An entry outside [0, n_rows) writes nothing; two
 *             entries naming one row of a sequence leave that row undefined.
 * batch >= 1, n >= 0, n_rows <= seq_stride_rows; the library only writes the named rows. */
csakv_status kv_cache_write(int32_t fmt, int32_t dim, void* codes, uint8_t* scales,
                            int64_t seq_stride_rows, int64_t n_rows, int32_t batch, int32_t n,
                            const uint16_t* x, const int32_t* dst, void* stream);

/* Decode rows of any KV format back to bf16, the read side of the formats above (sections
 * 二 and 六 of "DeepSeek-V4 KV Cache 深度分析" for the mixed row; the V4.1-Flash page, section
 * 핵심 내용, for FP4: value = E2M1 code x E4M3 scale).  Exact for every format (an E4M3 or
 * E2M1 x E4M3 value fits in bf16): fmt is csakv_kv_fmt; dim 512 for FP8_MIXED (nope 448),
 * dim % 16 == 0 otherwise; codes (scales for FP4 only, else NULL) and out [rows][dim] are
 * device pointers.  A mismatched scales pointer or shape returns CSAKV_ERR_INVALID, an
 * FP8_MIXED dim other than 512 CSAKV_ERR_UNSUPPORTED. */
csakv_status kv_dequantize(int32_t fmt, const void* codes, const uint8_t* scales,
                           int64_t rows, int32_t dim, uint16_t* out, void* stream);

/* KV-cache size in closed form ("DeepSeek-V4 KV Cache 深度分析", section 七):
 *   PerCSA = (N/csa_ratio + c_w*window) * S_kv + (N/csa_ratio) * S_idx
 *   PerHCA = (N/hca_ratio + c_w*window) * S_kv
 *   Total  = n_csa*PerCSA + n_hca*PerHCA + n_swa*swa_layer_bytes
 * where c_w = count_window (0, 1 or 2) and S_kv / S_idx are the row bytes of
 * kv_fmt / idx_fmt for kv_dim / idx_dim (FP4 scale bytes included iff count_scales;
 * FP8_MIXED keeps rope_dim dims in bf16).  idx_dim = 0 means no indexer; an MLA-style
 * layer is ratio 1, window 0, a BF16 row of kv_dim values.  Pure host arithmetic;
 * returns the total, fills `out` if non-NULL, and returns 0 for an invalid spec. */
typedef struct {
  int32_t n_csa, n_hca, n_swa;
  int32_t csa_ratio, hca_ratio, window;
  int32_t kv_dim, rope_dim, idx_dim;
  int32_t kv_fmt, idx_fmt;
  int32_t count_window, count_scales;
  int32_t reserved;
  int64_t swa_layer_bytes;
} kv_cache_spec;

/* `scales` holds the FP4 scale bytes of the whole cache (shared-KV, indexer and window
 * rows of every layer; 0 for formats without scales) whether or not count_scales adds them
 * to the row sizes: section 六 counts the FP4 indexer row as 64 bytes, which leaves them out. */
typedef struct {
  uint64_t csa_shared_kv, csa_indexer, hca_shared_kv, windows, swa_layers, scales;
  uint64_t csa_per_layer, hca_per_layer, total;
} kv_cache_breakdown;

uint64_t kv_cache_bytes(const kv_cache_spec* spec, int64_t seq_len, kv_cache_breakdown* out);

/* Model presets for kv_cache_bytes, each as the pages account for it:
 *   V4_PRO_BF16   30 CSA + 31 HCA layers (ratios 4 and 128), 512-dim bf16 rows, 128-dim bf16
 *                 indexer keys, the 128-row window counted once per layer
 *                 ("DeepSeek-V4 KV Cache 深度分析", 附录 calculator output, BF16 block; 八).
 *   V4_PRO_MIXED  the same with FP8_MIXED rows and FP4 indexer keys of 64 bytes (scale bytes
 *                 not counted) (the same appendix, mixed block; 六).
 *   V4_FLASH      21 CSA + 20 HCA bf16 layers without window rows, plus 2 sliding-window
 *                 layers of 196,608 bytes each (one 128-dim bf16 K/V head over a 128-token
 *                 window padded by 256) ("DeepSeek V4 의 정확한 KV 캐시 사용량 분석", PS
 *                 calculation, V4 Flash paragraphs).
 *   V3_MLA        61 MLA layers: one 576-dim bf16 row per token, no window, no indexer
 *                 (the same page, MLA paragraph).
 *   V32_DSA       V3_MLA plus a 128-dim bf16 indexer key per token (the same page, V3.2
 *                 paragraph).
 * Fills *out and returns CSAKV_OK; an unknown preset or a NULL out returns CSAKV_ERR_INVALID.
 * Pure host code. */
typedef enum {
  CSAKV_PRESET_V4_PRO_BF16 = 0,
  CSAKV_PRESET_V4_PRO_MIXED = 1,
  CSAKV_PRESET_V4_FLASH = 2,
  CSAKV_PRESET_V3_MLA = 3,
  CSAKV_PRESET_V32_DSA = 4
} csakv_preset;

csakv_status kv_cache_spec_preset(int32_t preset, kv_cache_spec* out);

/* Static, NUL-terminated description of a status code. */
const char* csakv_status_string(int32_t status);

#ifdef __cplusplus
}
#endif
#endif /* CSAKV_H */
