/*
 * pa.h -- paged attention for AMD Instinct MI355X (gfx950).
 *
 * Attention computed straight out of a paged KV cache: keys and values live
 * in a shared pool of fixed-size pages, every request owns an int32 page
 * table that maps its logical pages to physical pages, and the kernels read
 * the pages through that table while running online softmax, so neither a
 * contiguous copy of the keys nor a score matrix is ever materialized.  This
 * is the "Paged KV Cache" + "Paged FlashAttention" pair of the week-3
 * material in the tiny-llm source reading (yangyang233333.github.io) and in
 * "Build a vLLM from Scratch" (blog.mushroom.cv, Week 3).  Grouped-query
 * attention and the causal mask are the week-1 items of the same source
 * reading; split-K decode with a log-sum-exp merge is the Flash-Decoding item
 * (adv04) of the mini-vllm-tutorial advanced-series design.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All array arguments are DEVICE pointers owned by the caller.  The library
 *    never allocates or frees device memory and never synchronizes (except
 *    pa_validate_metadata, which is a debugging aid); the one piece of device
 *    memory it holds is the fixed scratch array of pa_decode_noalloc, which
 *    each device gets when the library is loaded.  All work is enqueued on
 *    `stream` (a hipStream_t; NULL = the null stream) and the call returns as
 *    soon as it is enqueued.
 *  - Errors are return codes; nothing aborts or throws across the ABI.
 *    PA_ERR_ARG: a null required pointer, a bad size or a misaligned pointer
 *    (all arrays must be 16-byte aligned).  PA_ERR_UNSUPPORTED: a valid but
 *    unimplemented shape (head_dim not 64/128, page_size not 16, fp32 prefill).
 *    PA_ERR_WORKSPACE: workspace smaller than the plan needs.  PA_ERR_HIP: a
 *    kernel launch failed.  PA_ERR_METADATA: pa_validate_metadata found a
 *    contract violation in the device arrays.  PA_ERR_NO_PAGES: the page pool
 *    has fewer free pages than a request needs (nothing was allocated).
 *  - Layouts (row-major, contiguous):
 *      q, out      [total_q, Hq, d]       rows ordered by request, then token
 *      lse         float32 [total_q, Hq]  natural log of sum_j exp(scale*q.k_j)
 *      k_pool,
 *      v_pool      [num_pages, Hkv, P, d] one (page, KV head) block of P*d
 *                                         elements is contiguous (4 KiB at
 *                                         d = 128 in bf16)
 *      page_table  int32 [B, max_pages_per_seq]
 *      seq_lens    int32 [B]  keys held by request r, this step's included
 *      q_offsets   int32 [B]  absolute position of request r's first query row
 *    Request r owns n_r = seq_lens[r] - q_offsets[r] query rows; its row i
 *    (position q_offsets[r] + i) sees keys 0 .. q_offsets[r] + i (causal).
 *    Query head h reads KV head h / (Hq / Hkv).  Logical key j of request r is
 *    slot j % P of physical page page_table[r][j / P].
 *  - Head ratio G = Hq / Hkv (Hkv must divide Hq): pa_prefill_chunk takes any
 *    G; the decode entry points take G <= 16 for bf16 and G <= 8 for fp32
 *    (a G that is not a power of two runs the kernel built for the next
 *    one, with the extra heads masked); pa_mixed_attention and
 *    pa_decode_direct take G in {1, 2, 4, 8}.  Other ratios return
 *    PA_ERR_UNSUPPORTED.
 *  - Device-array contract (checked only by pa_validate_metadata):
 *    1 <= seq_lens[r] <= max_pages_per_seq * P, 0 <= q_offsets[r] < seq_lens[r],
 *    sum_r n_r == total_q, and the first ceil(seq_lens[r] / P) entries of
 *    row r are in [0, num_pages).  Page-table entries past that, page slots
 *    past a request's last key, and unused pages may hold anything (-1, NaN):
 *    the kernels never let them reach the output.
 *  - bf16 is IEEE bfloat16; outputs are rounded to nearest even from float32
 *    accumulators.  fp32 I/O is accepted by the decode, split and merge paths.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_ARG = 1,
  PA_ERR_UNSUPPORTED = 2,
  PA_ERR_WORKSPACE = 3,
  PA_ERR_HIP = 4,
  PA_ERR_METADATA = 5,
  PA_ERR_NO_PAGES = 6
} pa_status;

typedef enum pa_dtype { PA_BF16 = 0, PA_F32 = 1 } pa_dtype;

/* Routes chosen by the dispatch guard. */
typedef enum pa_path {
  PA_PATH_DECODE = 0,          /* one workgroup per (request, KV head)                   */
  PA_PATH_DECODE_SPLIT = 1,    /* equal split-K partitions + log-sum-exp merge pass      */
  PA_PATH_PREFILL = 2,         /* query tiles through LDS-staged bf16 MFMA               */
  PA_PATH_DECODE_BALANCED = 3  /* page-balanced split-K (equal pages per wave) + merge   */
} pa_path;

/* Host scalars describing one call; everything the planner needs without
 * reading device memory. */
typedef struct pa_desc {
  int32_t num_seqs;          /* B: requests (rows of page_table/seq_lens/q_offsets) */
  int32_t num_q_heads;       /* Hq                                                  */
  int32_t num_kv_heads;      /* Hkv, divides Hq                                     */
  int32_t head_dim;          /* d: 64 or 128                                        */
  int32_t page_size;         /* P: 16                                               */
  int32_t num_pages;         /* pages in each pool                                  */
  int32_t max_pages_per_seq; /* row stride of page_table                            */
  int32_t total_q;           /* rows of q/out/lse                                   */
  int32_t max_seq_len;       /* host upper bound on seq_lens[r]                     */
  int32_t max_q_len;         /* host upper bound on n_r (1 for decode)              */
  int32_t dtype;             /* pa_dtype of q, the pools and out                    */
} pa_desc;

/* Output of the dispatch guard. */
typedef struct pa_plan_info {
  int32_t path;              /* pa_path                                             */
  int32_t num_splits;        /* S: partitions per request (1 unless split)          */
  int32_t grid_x;            /* workgroups the main kernel launches                 */
  int32_t reserved;
  uint64_t workspace_bytes;  /* bytes of scratch the route needs (0 if none)        */
} pa_plan_info;

/* Dispatch guard (pure host; reads no device memory).  Picks the route from
 * the query length and the context length, as the attention dispatch guard
 * of the tiny-llm source reading ("Prefill and decode need different
 * kernels") does: max_q_len > 1 -> PA_PATH_PREFILL.  Decode rows take
 * PA_PATH_DECODE_BALANCED when B <= 4096 and the contexts can hold at least
 * one page per wave (B * ceil(max_seq_len / P) >= num_splits): every KV
 * head's pages, taken in (request, page) order, are cut into num_splits
 * (= V) equal wave ranges, grid_x = Hkv * V / 4 workgroups (one resident
 * round: one per compute unit for bf16 with 2 * P * d * 2 >= 8192 bytes of
 * K and V per (page, KV head), else two), each wave writes a partial per
 * request it touches and a merge pass combines them by log-sum-exp.  Otherwise decode
 * runs one workgroup per (request, KV head), split into S equal partitions
 * (PA_PATH_DECODE_SPLIT) when B*Hkv workgroups would leave the chip's
 * cu_count compute units under-filled and the contexts are long enough.
 * cu_count <= 0 means "ask the current device" (falls back to 256). */
pa_status pa_plan(const pa_desc* desc, int32_t cu_count, pa_plan_info* plan);

/* Scratch bytes for split-K with num_splits partitions (the split-K
 * partition of long-sequence decode: "mini-vllm-tutorial advanced-series
 * design", section 4, Phase B, adv04 Flash-Decoding):
 * B*Hq*S*d float32 partial outputs + B*Hq*S float32 partial lse, each
 * 256-byte aligned.  Returns 0 for an invalid desc or num_splits < 1. */
size_t pa_workspace_bytes(const pa_desc* desc, int32_t num_splits);

/* Single-token decode read straight out of the paged cache: the attention
 * kernel walks the request's page table instead of a contiguous K/V copy,
 * with paging and online softmax in one kernel so no score row is stored
 * ("tiny-llm source reading", section "Paged KV Cache", the Paged
 * FlashAttention step; "Build a vLLM from Scratch", Week 3, Direct Paged
 * Attention + Paged FlashAttention).  It is the one-token step that the KV
 * cache leaves after prefill ("tiny-llm source reading", section "KV Cache
 * changes the shape of the computation"), grouped-query heads sharing each
 * K/V load (the same page's week-one GQA item).
 * Every request has exactly one query row (n_r = 1, so
 * total_q == B and q_offsets[r] == seq_lens[r] - 1; q_offsets may be NULL).
 * out [B, Hq, d] (dtype), lse float32 [B, Hq] (may be NULL).  The guard may
 * route through a split-K path, which needs `workspace` of at least
 * pa_plan(...).workspace_bytes bytes (else PA_ERR_WORKSPACE); workspace may be
 * NULL when the plan needs none.  The workspace contents after the call are
 * internal. */
pa_status pa_decode(const pa_desc* desc, const void* q, const void* k_pool, const void* v_pool,
                    const int32_t* page_table, const int32_t* seq_lens, const int32_t* q_offsets,
                    float scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                    void* stream);

/* pa_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same routes, kernels and results as pa_decode, with no workspace
 * argument.  The routes that need scratch use a fixed array of
 * PA_NOALLOC_SCRATCH_BYTES bytes of device memory that the library holds on
 * each device it runs on until the process ends; no call allocates or frees
 * anything.  A call whose plan needs more scratch than that (pa_plan's
 * workspace_bytes; for example more than about 900 requests at 64 query
 * heads and d = 128) returns PA_ERR_WORKSPACE and does nothing.  Every call
 * on one device shares that device's array, so calls that overlap on one
 * device (on different streams, or from different threads without ordering)
 * race and their results are undefined; calls ordered on one stream are
 * safe.  Argument errors as for pa_decode. */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
pa_status pa_decode_noalloc(const pa_desc* desc, const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* page_table, const int32_t* seq_lens,
                            const int32_t* q_offsets, float scale, void* out, float* lse,
                            void* stream);

/* Split-K decode with a caller-chosen partition count ("mini-vllm-tutorial
 * advanced-series design", section 4, Phase B, adv04 Flash-Decoding: a long
 * context is cut into partitions whose partial results are combined):
 * request r's ceil(seq_lens[r]/P) pages are cut into num_splits page-aligned
 * ranges of ceil(pages_r / num_splits) pages (trailing ranges may be empty).
 * Each (request, KV head, split) workgroup writes a normalized partial output
 * and its lse into `workspace`; a merge pass combines them by the log-sum-exp
 * rule and writes out and lse.  Same row contract as pa_decode.  Workspace
 * layout: o_part float32 [B, Hq, S, d] at offset 0, lse_part float32
 * [B, Hq, S] at the next 256-byte boundary; it holds the partials after the
 * call.  num_splits in [1, 256]. */
pa_status pa_split_merge(const pa_desc* desc, const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* page_table, const int32_t* seq_lens,
                         const int32_t* q_offsets, float scale, int32_t num_splits,
                         void* workspace, size_t workspace_bytes, void* out, float* lse,
                         void* stream);

/* Baselines for measuring what paging and online softmax cost (same row
 * contract and outputs as pa_decode; bf16 or fp32, d = 64 or 128; G as for
 * pa_decode, except pa_decode_direct: G in {1, 2, 4, 8}):
 *   pa_decode_dense:  the same fused (online-softmax) per-(request, KV head)
 *                     kernel over a dense cache k_cache, v_cache
 *                     [B, Hkv, MP * P, d] (MP = desc->max_pages_per_seq, the
 *                     capacity in pages; request r's first seq_lens[r] keys
 *                     of each KV head are contiguous), with no page table:
 *                     the dense KV cache the pages start from ("Build a vLLM
 *                     from Scratch", Week 2) before paging (Week 3).
 *   pa_decode_direct: attention read through the page table but not fused:
 *                     every score is stored (fp32) in `workspace` (at least
 *                     pa_direct_workspace_bytes(desc) = B * Hq * MP * P * 4
 *                     bytes), each head's row is turned into softmax weights
 *                     in place, then the values are summed: the direct paged
 *                     attention that "Build a vLLM from Scratch", Week 3,
 *                     names next to Paged FlashAttention. */
pa_status pa_decode_dense(const pa_desc* desc, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* seq_lens, float scale, void* out, float* lse, void* stream);
size_t pa_direct_workspace_bytes(const pa_desc* desc);
pa_status pa_decode_direct(const pa_desc* desc, const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* page_table, const int32_t* seq_lens, float scale, void* out,
                           float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Chunked prefill ("tiny-llm source reading", section "Chunked Prefill": a
 * long prompt is cut into bounded chunks that interleave with decode;
 * "Build a vLLM from Scratch", Week 3, Chunked Prefill, on the tiled
 * prefill attention of its Week 2; the matrix-shaped prefill kernel of the
 * tiny-llm source reading's "Prefill and decode need different kernels"):
 * request r's n_r query rows (a chunk of a prompt at prior
 * offset q_offsets[r]) attend causally to keys 0 .. q_offsets[r] + i, all of
 * them read from the pages (the chunk's own K/V already appended).  bf16
 * only.  The P V product runs in fp16 (weights rounded to fp16, V values
 * converted from bf16 exactly): V values must lie within fp16's range,
 * |v| <= 65504; a larger one becomes infinite.  q_starts: int32 [B+1]
 * exclusive prefix sum of n_r, or NULL to derive it on the device.  lse
 * may be NULL.  When the grid is small against the chip, the guard splits
 * long query tiles along their key range and merges the partials by
 * log-sum-exp; that needs `workspace` of at least
 * pa_plan(...).workspace_bytes bytes (PA_ERR_WORKSPACE if a smaller one is
 * given).  workspace = NULL runs every tile unsplit (always valid, slower on
 * unbalanced batches). */
pa_status pa_prefill_chunk(const pa_desc* desc, const void* q, const void* k_pool,
                           const void* v_pool, const int32_t* page_table, const int32_t* seq_lens,
                           const int32_t* q_offsets, const int32_t* q_starts, float scale,
                           void* out, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Mixed batch in one launch: one continuous-batching round whose requests
 * are in either phase (the tiny-llm source reading, "Continuous Batching":
 * one round carries prefill and decode requests side by side).  Request r
 * has n_r = seq_lens[r] - q_offsets[r] query rows, packed like
 * pa_prefill_chunk's q (q_starts as there, or NULL); n_r = 1 rows are
 * decoded and n_r > 1 chunks are prefilled, each with the same causal rule
 * as pa_prefill_chunk, and every row's out and lse land at its packed row.
 * The dispatch guard's choice ("Prefill and decode need different
 * kernels") is made per work item inside the kernel: each workgroup takes
 * either a 128-row prefill tile or a whole decode (request, KV head), so a
 * step needs one launch instead of a prefill launch, a decode launch and a
 * merge pass, and the MFMA-bound tiles and HBM-bound decode items run on
 * the chip at the same time.  bf16 only (prefill tiles as in
 * pa_prefill_chunk, V within fp16's range); d = 64 or 128; G in {1, 2, 4, 8};
 * B <= 512 (PA_ERR_UNSUPPORTED otherwise).  No workspace; prefill tiles are
 * never split along their keys, so a batch whose prefill is a few very
 * long chunks is better served by pa_prefill_chunk, which can split.
 * Requests with n_r <= 0 are skipped. */
pa_status pa_mixed_attention(const pa_desc* desc, const void* q, const void* k_pool,
                             const void* v_pool, const int32_t* page_table,
                             const int32_t* seq_lens, const int32_t* q_offsets,
                             const int32_t* q_starts, float scale, void* out, float* lse,
                             void* stream);

/* Append a step's new K and V rows into their page slots (the write that
 * precedes attention in every serving step: the "Paged KV Cache" section of
 * the tiny-llm source reading).  Request r contributes n_r = seq_lens[r] -
 * q_offsets[r] rows (seq_lens after this append), packed like q: k_new,
 * v_new [total_q, Hkv, d] of desc->dtype, rows by request then token.  Row i
 * of request r (position p = q_offsets[r] + i) is copied bit-exactly to
 * k_pool/v_pool[page_table[r][p / P], :, p % P, :].  q_starts: int32 [B+1]
 * exclusive prefix sum of n_r, or NULL to derive it on the device.  The
 * pages must already be in the table (pa_pool_reserve); rows whose page id
 * lies outside [0, num_pages) are skipped, never written elsewhere.  Rows of
 * different requests must map to different slots (requests own their pages).
 * Works for bf16 and fp32, d = 64 or 128. */
pa_status pa_append_kv(const pa_desc* desc, const void* k_new, const void* v_new,
                       const int32_t* page_table, const int32_t* seq_lens,
                       const int32_t* q_offsets, const int32_t* q_starts, void* k_pool,
                       void* v_pool, void* stream);

/* Host page allocator for the shared pool (pure host: no device memory, no
 * synchronization).  Pages are handed out on demand and returned when a
 * request finishes ("Paged KV Cache" in the tiny-llm source reading).  A page
 * may be held by several page tables at once (a shared prompt prefix, the
 * reference-count reuse of "mini-vllm-tutorial advanced-series design",
 * Phase C, adv05): it keeps one reference per holder and returns to the free
 * list when the last one is dropped.  Every call is all-or-nothing and
 * thread-safe.
 *   pa_pool_create:   a pool of num_pages free pages, ids 0 .. num_pages-1.
 *   pa_pool_alloc:    n free ids into ids[0..n), one reference each;
 *                     PA_ERR_NO_PAGES if fewer are free.
 *   pa_pool_free:     drop one reference per listed id; PA_ERR_ARG (nothing
 *                     changes) if an id is out of range or listed more often
 *                     than it is held.
 *   pa_pool_share:    add one reference per listed id (each must be held).
 *   pa_pool_refcount: references held on page id; -1 if out of range.
 *   pa_pool_reserve:  grow one request's host page-table row from old_len to
 *                     new_len keys: allocates the pages for logical pages
 *                     ceil(old_len/P) .. ceil(new_len/P)-1 into the row
 *                     (PA_ERR_ARG if that exceeds max_pages_per_seq).
 *   pa_pool_release:  drop the row's references on its ceil(len/P) pages and
 *                     set those entries to -1.
 *   pa_pool_fork:     start dst_row as a sharer of src_row's first
 *                     ceil(len/P) pages (a new request with the same prefix):
 *                     copies the ids and adds one reference each.
 *   pa_pool_cow:      before writing into logical page lp of a row: if the
 *                     row is the page's only holder, *old_id = *new_id = the
 *                     page and nothing changes; otherwise a free page
 *                     replaces it in the row (one reference moves over) and
 *                     *old_id, *new_id name the pair whose contents the caller
 *                     copies with pa_copy_pages before writing.
 *                     PA_ERR_NO_PAGES if no page is free.
 *   pa_pool_num_free: free pages, or -1 for a null pool. */
typedef struct pa_page_pool pa_page_pool;
pa_status pa_pool_create(int32_t num_pages, pa_page_pool** pool);
void pa_pool_destroy(pa_page_pool* pool);
int32_t pa_pool_num_free(pa_page_pool* pool);
int32_t pa_pool_refcount(pa_page_pool* pool, int32_t id);
pa_status pa_pool_alloc(pa_page_pool* pool, int32_t n, int32_t* ids);
pa_status pa_pool_free(pa_page_pool* pool, const int32_t* ids, int32_t n);
pa_status pa_pool_share(pa_page_pool* pool, const int32_t* ids, int32_t n);
pa_status pa_pool_reserve(pa_page_pool* pool, int32_t* page_table_row, int32_t max_pages_per_seq,
                          int32_t old_len, int32_t new_len, int32_t page_size);
pa_status pa_pool_release(pa_page_pool* pool, int32_t* page_table_row, int32_t max_pages_per_seq,
                          int32_t len, int32_t page_size);
pa_status pa_pool_fork(pa_page_pool* pool, const int32_t* src_row, int32_t* dst_row,
                       int32_t max_pages_per_seq, int32_t len, int32_t page_size);
pa_status pa_pool_cow(pa_page_pool* pool, int32_t* page_table_row, int32_t max_pages_per_seq,
                      int32_t logical_page, int32_t* old_id, int32_t* new_id);

/* Copy whole pages, K and V for every KV head, from src_ids[i] to
 * dst_ids[i] (device int32 arrays of n ids; bit-exact): the device half of
 * pa_pool_cow, the private copy a holder of a shared page takes before
 * writing ("mini-vllm-tutorial advanced-series design", Phase C, adv05).  A pair naming a page outside [0, num_pages), or the same
 * page twice, is skipped.  The dst pages must be distinct and none of them a
 * src page of the same call. */
pa_status pa_copy_pages(const pa_desc* desc, void* k_pool, void* v_pool, const int32_t* src_ids,
                        const int32_t* dst_ids, int32_t n, void* stream);

/* Log-sum-exp merge of split partials (the combine step of split-K decode,
 * "mini-vllm-tutorial advanced-series design", section 4, Phase B, adv04;
 * the merge pass on its own, a test hook).  o_part float32 [rows, heads, S, d], lse_part float32 [rows, heads, S]
 * (-inf marks an empty split) -> out [rows, heads, d] of out_dtype and
 * lse float32 [rows, heads] (may be NULL). */
pa_status pa_merge_partials(int32_t rows, int32_t heads, int32_t num_splits, int32_t head_dim,
                            const float* o_part, const float* lse_part, void* out,
                            int32_t out_dtype, float* lse, void* stream);

/* Copy request `req`'s first seq_len keys out of the pools into contiguous
 * k_out, v_out [seq_len, Hkv, d] (bit-exact; the page-table translation on
 * its own, a test hook).  This is the concatenation the attention kernels
 * avoid by reading pages through the table ("tiny-llm source reading",
 * section "Paged KV Cache").  seq_len is a host value. */
pa_status pa_gather_kv(const pa_desc* desc, const void* k_pool, const void* v_pool,
                       const int32_t* page_table, int32_t req, int32_t seq_len, void* k_out,
                       void* v_out, void* stream);

/* Measurement hook (not part of the attention path): the read rate of the
 * decode kernels' access pattern.  Reads nblocks blocks of block_bytes
 * (4096, 8192, 16384 or 32768) from buf (device, buf_blocks blocks, 16-byte
 * aligned), block j at byte offset order[j] * block_bytes (order: int32
 * device array; ids outside [0, buf_blocks) are skipped), with the loads
 * the decode kernels use for K and V (16 bytes per lane, nontemporal), and
 * XORs every 32-bit word read into *sink (device uint32; the caller zeroes
 * it).  A (page, KV head) K or V block is P * d * 2 = 4096 bytes at d = 128
 * in bf16, so 4096-byte blocks in a random order are what the decode route
 * reads: decode is bound by these reads ("tiny-llm source reading", section
 * "KV Cache changes the shape of the computation"), and its rate is
 * measured against this one as well as against the device's peak.
 * PA_ERR_ARG for a bad size or null pointer. */
pa_status pa_read_blocks(const void* buf, int64_t buf_blocks, const int32_t* order, int32_t nblocks,
                         int32_t block_bytes, uint32_t* sink, void* stream);

/* Debugging aid: copies the metadata to the host (synchronizing `stream`)
 * and checks the device-array contract above (the page table, context
 * lengths and offsets of the "Paged KV Cache" section of the tiny-llm
 * source reading).  q_offsets may be NULL (decode).  Returns PA_OK or
 * PA_ERR_METADATA.  With PA_DEBUG_VALIDATE set in the environment (to
 * anything but "0"; read once per process), pa_decode, pa_decode_noalloc,
 * pa_split_merge, pa_decode_direct, pa_prefill_chunk, pa_mixed_attention and
 * pa_append_kv run this check first and return its error instead of
 * launching; each call then synchronizes its stream, so the switch is for
 * debugging only. */
pa_status pa_validate_metadata(const pa_desc* desc, const int32_t* page_table,
                               const int32_t* seq_lens, const int32_t* q_offsets, void* stream);

/* Static string naming a status code. */
const char* pa_status_str(pa_status status);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
