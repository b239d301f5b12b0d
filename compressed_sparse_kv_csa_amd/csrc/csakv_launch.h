// Host-side launchers of the csakv kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csakv {

// Paged cache layout: row r of sequence b lives at pool row
// table[b * table_stride + (r >> page_shift)] << page_shift | (r & (2^page_shift - 1)).
// table == nullptr: each sequence's rows are contiguous at its seq_stride offset.
struct Paging {
  const int32_t* table;
  int32_t page_shift;    // log2(rows per page), >= 4
  int32_t table_stride;  // table entries per sequence
};

// ------------------------------------------------------------------ codecs
hipError_t launch_quantize_fp4(const uint16_t* x, int64_t rows, int dim, uint8_t* codes,
                               uint8_t* scales, hipStream_t stream);
hipError_t launch_quantize_fp8_mixed(const uint16_t* x, int64_t rows, int dim, int nope,
                                     uint8_t* out, hipStream_t stream);
hipError_t launch_quantize_fp4h(const uint16_t* x, int64_t rows, uint8_t* codes, uint8_t* scales,
                                hipStream_t stream);
hipError_t launch_cache_write(int fmt, int dim, void* codes, uint8_t* scales, int64_t seq_stride,
                              int64_t n_rows, int batch, int n, const uint16_t* x,
                              const int32_t* dst, hipStream_t stream);
hipError_t launch_dequantize(int fmt, const void* codes, const uint8_t* scales, int64_t rows,
                             int dim, int nope, uint16_t* out, hipStream_t stream);

// ------------------------------------------------------------------ indexer + top-k
// Geometry of one indexer pass.
struct IndexerPlan {
  int64_t n_c;        // compressed rows per sequence
  int slice_rows;     // rows selected together (kSliceRows)
  int n_slices;       // slices per query
  int slices_per_wg;  // consecutive slices one scan workgroup owns
  int wg_per_query;   // scan workgroups per query
  int cap;            // candidate slots per slice
  int prefix;         // P: a slice sends at least its top-P keys
  int first;          // slots per slice the merge reads with the counts (a power of two)
};

constexpr int kSliceRows = 4096;
constexpr int kMaxTopK = 2048;
constexpr int kMaxHeads = 128;  // query heads (a multiple of 16) and indexer heads
constexpr int kMergeCap = 8192;
constexpr int kMergeFirstSlots = 4096;  // candidate slots a merge reads with the slice counts
constexpr int kMaxMergeSlices = 512;

// CSA2 reindex: pool slots per query, and the largest indexer-key byte count of one
// sequence (rows are addressed by 32-bit offsets inside a per-sequence buffer resource).
constexpr int kMaxPool = 4096;
constexpr uint32_t kReindexMaxSeqBytes = 0xFFFFFF00u;

bool reindex_supported(int key_fmt, int64_t n_c);
// seq_rows (here and below): NULL, or [B] device int32 rows of each sequence (clamped to
// [0, n_c] or [0, n_rows]).
// The workspace holds the selection key of every pool slot ([B][n_pool] uint64).
size_t reindex_workspace_bytes(int batch, int n_pool);
hipError_t launch_reindex(int key_fmt, const uint8_t* codes, const uint8_t* scales,
                          int64_t seq_stride, const Paging& pg, int64_t n_c, const int32_t* seq_rows,
                          const uint16_t* q_idx,
                          const float* w_idx, int batch, int n_heads, const int32_t* pool,
                          int n_pool, int top_k, int32_t* topk, void* workspace,
                          hipStream_t stream);

IndexerPlan plan_indexer(int batch, int64_t n_c, int top_k);
bool indexer_supported(const IndexerPlan& plan);
size_t indexer_workspace_bytes(int batch, const IndexerPlan& plan);

// The two stages of the indexer: the scan leaves each slice's candidates, bound and
// scores in the workspace; the merge reads them and writes topk.
constexpr int kStageScan = 1;
constexpr int kStageMerge = 2;

hipError_t launch_indexer(int key_fmt, const uint8_t* codes, const uint8_t* scales,
                          int64_t seq_stride, const Paging& pg, int64_t n_c, const int32_t* seq_rows,
                          const uint16_t* q_idx,
                          const float* w_idx, int batch, int n_heads, int top_k,
                          const IndexerPlan& plan, void* workspace, int32_t* topk,
                          hipStream_t stream, int stages = kStageScan | kStageMerge);

// ------------------------------------------------------------------ attention
struct AttnPlan {
  int64_t n_list;      // row positions per query (CSA: window + top_k; HCA: rows)
  int rows_per_chunk;  // multiple of 32
  int n_chunks;        // chunks per query
  bool wide;           // 64-head workgroups (long lists) instead of 16-head ones
};

constexpr int kMaxChunkRows = 1024;  // rows one attention workgroup walks
constexpr int kMaxChunks = 4096;     // chunks per query the combine merges
// Largest shared-KV byte count of one sequence (codes, and FP4 scales separately): rows
// are addressed by 32-bit offsets inside a per-sequence buffer resource.
constexpr uint32_t kAttnMaxSeqBytes = 0xFFFFFF00u;

AttnPlan plan_attention(int batch, int64_t n_list, bool csa, int n_heads);
bool attention_supported(const AttnPlan& plan, int kv_fmt, int64_t n_rows);
size_t attention_workspace_bytes(int batch, int n_heads, const AttnPlan& plan);

hipError_t launch_rope_output(uint16_t* out, int batch, int n_heads, const int64_t* positions,
                              double base, hipStream_t stream);
hipError_t launch_attention(int kv_fmt, bool csa, const uint8_t* codes, const uint8_t* scales,
                            int64_t seq_stride, const Paging& pg, int64_t n_rows,
                            const int32_t* seq_rows, const uint16_t* q, int batch,
                            int n_heads, float softmax_scale, const int32_t* topk, int top_k,
                            int window, const AttnPlan& plan, void* workspace, uint16_t* out,
                            hipStream_t stream);

}  // namespace csakv
