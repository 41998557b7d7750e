// Internal declarations shared by the library's translation units: the
// parameter blocks handed to each kernel family and their host launchers.
// Nothing here is part of the C ABI (include/pa.h is).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "pa.h"

namespace pa {

// Argument checks of the decode-row entry points (pa_decode and its
// variants): the descriptor, one row per request, the head ratio, pointers,
// alignment and scale.  Returns PA_OK or the status the entry point returns.
pa_status check_decode_call(const pa_desc* d, const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* page_table, const int32_t* seq_lens, float scale,
                            const void* out, const float* lse);

constexpr int kPageSize = 16;  // keys per page (the only page size built)
// Buffer resource word 3 for gfx9-family raw (unstructured) buffers.
constexpr int kBufferWord3 = 0x00020000;
// Requests the page-balanced decode handles in one call (its per-request page
// prefix lives in LDS).
constexpr int kMaxBalancedSeqs = 4096;
// Requests the mixed prefill/decode kernel handles in one call (each
// workgroup ranks them in LDS).
constexpr int kMaxMixedSeqs = 512;
// KV tiles per split that leaves every prefill row tile whole.
constexpr int kMixedUnsplit = 1 << 29;

// ---------------------------------------------------------------------------
// decode / split-K partition kernel
// ---------------------------------------------------------------------------
struct DecodeArgs {
  const void* q;            // [B, Hq, d]
  const void* k_pool;       // [NP, Hkv, P, d]
  const void* v_pool;
  const int32_t* page_table;  // [B, MP]
  const int32_t* seq_lens;    // [B]
  void* out;                // [B, Hq, d]     (unsplit)
  float* lse;               // [B, Hq] or null (unsplit)
  float* o_part;            // [B, Hq, S, d] (split) or [B + V - 1, Hq, d] (balanced)
  float* lse_part;          // [B, Hq, S]    (split) or [B + V - 1, Hq]    (balanced)
  int32_t* range_meta;      // balanced: [B, 2] first and last wave range of each request
  int32_t num_seqs, num_q_heads, num_kv_heads, max_pages_per_seq;
  int32_t num_pages;        // pool size; page ids are clamped into [0, num_pages)
  int32_t num_splits;       // S partitions per (request, KV head); balanced: V wave ranges
  int32_t write_partials;   // 1: write o_part/lse_part; 0: write out/lse (needs S == 1)
  float scale_log2;         // scale * log2(e)
};

// Query heads per KV head the decode kernels take: up to 16 for bf16 (the
// MFMA page step's query tile has 16 columns), up to 8 for fp32.  A group
// size that is not a power of two runs the kernel built for the next one,
// with the extra heads masked.  dtype: 0 = bf16, 1 = fp32.
bool decode_group_supported(int group, int dtype);
// Launchers return hipSuccess or the launch error.
// One workgroup per (request, KV head, split); bf16 runs the MFMA form of
// the page step, fp32 the VALU form.
hipError_t launch_decode(const DecodeArgs& a, int dtype, int head_dim, int group, hipStream_t s);
// The per-(request, KV head) kernel over a dense cache [B, Hkv, MP * P, d]
// (a.page_table unused; a.max_pages_per_seq = capacity in pages; unsplit).
hipError_t launch_decode_dense(const DecodeArgs& a, int dtype, int head_dim, int group, hipStream_t s);
// Page-balanced split: every KV head's flattened (request, page) sequence is
// cut into a.num_splits equal wave ranges (a.num_splits a multiple of 4).
// bf16 runs the MFMA form of the kernel, fp32 the VALU form.
hipError_t launch_decode_balanced(const DecodeArgs& a, int dtype, int head_dim, int group,
                                  hipStream_t s);

// ---------------------------------------------------------------------------
// direct (non-flash) paged decode: scores stored, then softmax, then values
// ---------------------------------------------------------------------------
struct DirectArgs {
  const void* q;            // [B, Hq, d]
  const void* k_pool;       // [NP, Hkv, P, d]
  const void* v_pool;
  const int32_t* page_table;  // [B, MP]
  const int32_t* seq_lens;    // [B]
  void* out;                // [B, Hq, d]
  float* lse;               // [B, Hq] or null
  float* scores;            // scratch [B, Hq, MP * P] fp32
  int32_t num_seqs, num_q_heads, num_kv_heads, max_pages_per_seq, num_pages;
  float scale_log2;
};

hipError_t launch_decode_direct(const DirectArgs& a, int dtype, int head_dim, int group, hipStream_t s);

// ---------------------------------------------------------------------------
// log-sum-exp merge of split partials
// ---------------------------------------------------------------------------
struct MergeArgs {
  const float* o_part;      // [rows, heads, S, d], or [rows + S - 1, heads, d] with range_meta
  const float* lse_part;    // [rows, heads, S],    or [rows + S - 1, heads]
  // null: fixed S partials per (row, head).  Otherwise [rows, 2]: row r's
  // partials sit in slots r + v for v in [meta[2r], meta[2r+1]].
  const int32_t* range_meta;
  void* out;                // [rows, heads, d]
  float* lse;               // [rows, heads] or null
  int32_t rows, heads, num_splits;
};

hipError_t launch_merge(const MergeArgs& a, int out_dtype, int head_dim, hipStream_t s);

// ---------------------------------------------------------------------------
// chunked prefill (bf16 MFMA)
// ---------------------------------------------------------------------------
struct PrefillArgs {
  const void* q;            // [total_q, Hq, d] bf16
  const void* k_pool;
  const void* v_pool;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int32_t* q_offsets;
  const int32_t* q_starts;  // [B+1] or null (derived on the device)
  void* out;                // [total_q, Hq, d] bf16
  float* lse;               // [total_q, Hq] or null
  float* part_o;            // split partials [units, S, tile_rows, d] (S > 1 only)
  float* part_lse;          // [units, S, tile_rows]
  int32_t num_seqs, num_q_heads, num_kv_heads, max_pages_per_seq;
  int32_t num_pages;
  int32_t tiles_per_seq;    // query tiles per (request, KV head) in the grid
  int32_t num_splits;       // S: key-range splits per query tile in the grid (1 = unsplit)
  int32_t kv_tiles_per_split;  // KV tiles one split covers
  float scale_log2;
};

// Rows of the packed (token, head-in-group) query tile one workgroup owns,
// and keys per KV tile.
int prefill_tile_rows(int head_dim);
int prefill_tile_keys();
hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int group, hipStream_t s);

// ---------------------------------------------------------------------------
// mixed prefill/decode batch in one launch (bf16; group in {1, 2, 4, 8})
// ---------------------------------------------------------------------------
// Upper bound on the work items of one KV head (prefill row tiles plus
// decode requests) of a batch with total_q query rows over num_seqs
// requests; the grid is this times Hkv, and surplus workgroups exit.
long long mixed_items_bound(long long total_q, int num_seqs, int group);
// Tiles are never split: the caller sets a.num_splits = 1 and
// a.kv_tiles_per_split = kMixedUnsplit; a.tiles_per_seq, a.part_o and
// a.part_lse are not used.
hipError_t launch_mixed(const PrefillArgs& a, int head_dim, int group, long long items_per_head,
                        hipStream_t s);

// ---------------------------------------------------------------------------
// KV append (new rows into their page slots)
// ---------------------------------------------------------------------------
struct AppendArgs {
  const void* k_new;        // [total_q, Hkv, d] rows by request then token
  const void* v_new;
  void* k_pool;             // [NP, Hkv, P, d]
  void* v_pool;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int32_t* q_offsets;
  const int32_t* q_starts;  // [B+1] or null (derived on the device)
  int32_t num_seqs, num_kv_heads, max_pages_per_seq, num_pages;
  int32_t head_bytes;       // d * element size (a multiple of 16)
  int32_t tiles_per_seq;    // row groups per request in the per-request grid
  int64_t total_rows;       // rows of k_new / v_new
};

int append_rows_per_wg();
hipError_t launch_append(const AppendArgs& a, hipStream_t s);

// Whole-page copies (K and V, every KV head) from src[i] to dst[i].
struct CopyPagesArgs {
  void* k_pool;             // [NP, Hkv, P, d]
  void* v_pool;
  const int32_t* src;       // [n] page ids
  const int32_t* dst;       // [n] page ids
  int32_t n, num_pages;
  int64_t page_bytes;       // Hkv * P * d * element size (a multiple of 16)
  int32_t slices;           // workgroups per page
};

hipError_t launch_copy_pages(const CopyPagesArgs& a, hipStream_t s);

// ---------------------------------------------------------------------------
// page gather (test hook)
// ---------------------------------------------------------------------------
struct GatherArgs {
  const void* k_pool;
  const void* v_pool;
  const int32_t* page_row;  // page_table + req * MP
  void* k_out;              // [seq_len, Hkv, d]
  void* v_out;
  int32_t seq_len, num_kv_heads, head_dim, elem_bytes;
  int32_t num_pages;        // page ids are clamped into [0, num_pages)
};

hipError_t launch_gather(const GatherArgs& a, hipStream_t s);

// ---------------------------------------------------------------------------
// read-bandwidth reference (measurement hook)
// ---------------------------------------------------------------------------
struct ReadBlocksArgs {
  const void* buf;          // buf_blocks blocks of block_bytes
  const int32_t* order;     // [nblocks] block ids; ids outside [0, buf_blocks) are skipped
  uint32_t* sink;           // XOR of every word read
  int64_t buf_blocks;
  int32_t nblocks, block_bytes;
};

constexpr int kReadBlocksGrid = 2048;   // workgroups of the read-bandwidth reference
hipError_t launch_read_blocks(const ReadBlocksArgs& a, hipStream_t s);

}  // namespace pa
