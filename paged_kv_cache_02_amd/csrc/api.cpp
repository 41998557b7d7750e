// C-ABI entry points of the paged-attention library: argument checks, the
// dispatch guard, workspace carving and kernel launches on the caller's
// stream.  See include/pa.h for the contract of every function.
#include "pa.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <vector>

#include "pa_internal.h"

namespace {

// --------------------------------------------------------------------------
// dispatch-guard tuning constants
// --------------------------------------------------------------------------
// Page-balanced decode: workgroups of 4 waves per CU the grid is sized for,
// so the whole grid is one round and all of its waves carry equal page
// counts.  Each wave of the bf16 (MFMA) kernel keeps 3 pages of K and V in
// flight; its rate was best at about 96 KB in flight per CU (measured on
// the mixed step, Qwen3-4B and Qwen3-0.6B shapes, d = 128, and the long
// d = 64 one), so one workgroup per CU when a (page, KV head) block of K
// and V is 8 KB or more, else two (which every decode kernel instance can
// hold: two waves per SIMD).  The fp32 (VALU) kernel keeps two.
constexpr int kWavesPerDecodeWg = 4;
constexpr int kBlockBytesOneWg = 8192;
// Fallback equal-split decode (more than pa::kMaxBalancedSeqs requests, or too
// little work to spread): split until the grid holds about this many
// workgroups per CU, so that uneven context lengths still leave every CU busy.
constexpr int kTargetWgsPerCu = 8;
// A split must keep at least this many pages (4 per wave), or its fixed
// costs (q load, cross-wave merge, partial write) stop being small.
constexpr int kMinPagesPerSplit = 16;
constexpr int kMaxSplits = 64;
// Prefill: each workgroup already splits its key range between two wave
// groups; query tiles are additionally split across workgroups (partials +
// merge pass) only when the grid holds fewer workgroups than resident slots
// (one per CU); a split keeps at least kPrefillMinTiles KV tiles.
constexpr int kPrefillSlotsPerCu = 1;
constexpr int kPrefillUnitsPerSlot = 1;
constexpr int kPrefillMinTiles = 8;
constexpr int kMaxSplitsApi = 256;
constexpr int kDefaultCuCount = 256;
constexpr size_t kAlign = 256;

constexpr float kLog2e = 1.4426950408889634f;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int elem_bytes(int dtype) { return dtype == PA_BF16 ? 2 : 4; }

pa_status check_desc(const pa_desc* d) {
  if (d == nullptr) return PA_ERR_ARG;
  if (d->num_seqs < 0 || d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->head_dim <= 0 ||
      d->page_size <= 0 || d->num_pages <= 0 || d->max_pages_per_seq <= 0 || d->total_q < 0 ||
      d->max_seq_len < 0 || d->max_q_len < 0)
    return PA_ERR_ARG;
  if (d->num_q_heads % d->num_kv_heads != 0) return PA_ERR_ARG;
  if (d->dtype != PA_BF16 && d->dtype != PA_F32) return PA_ERR_ARG;
  if ((long long)d->max_seq_len > (long long)d->max_pages_per_seq * d->page_size) return PA_ERR_ARG;
  if (d->max_q_len > d->max_seq_len) return PA_ERR_ARG;
  if (d->head_dim != 64 && d->head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (d->page_size != pa::kPageSize) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return kDefaultCuCount;
  }
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    n = kDefaultCuCount;
  }
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace

namespace pa {
bool decode_group_supported(int group, int dtype) {
  // bf16 runs the MFMA page step, whose 16-column query tile holds up to 16
  // heads; the fp32 VALU kernels are built for up to 8
  return group >= 1 && group <= (dtype == PA_BF16 ? 16 : 8);
}

// Checks shared by the decode-row entry points (declared in pa_internal.h).
pa_status check_decode_call(const pa_desc* d, const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* page_table, const int32_t* seq_lens, float scale,
                            const void* out, const float* lse) {
  pa_status st = check_desc(d);
  if (st != PA_OK) return st;
  if (d->total_q != d->num_seqs || d->max_q_len > 1) return PA_ERR_ARG;
  if (!pa::decode_group_supported(d->num_q_heads / d->num_kv_heads, d->dtype)) return PA_ERR_UNSUPPORTED;
  if (d->num_seqs == 0) return PA_OK;
  if (!q || !k_pool || !v_pool || !page_table || !seq_lens || !out) return PA_ERR_ARG;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out) ||
      !aligned4(page_table) || !aligned4(seq_lens) || (lse && !aligned4(lse)))
    return PA_ERR_ARG;
  if (out == q) return PA_ERR_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return PA_ERR_ARG;
  return PA_OK;
}
}  // namespace pa

namespace {
using pa::check_decode_call;

// Debugging switch: with PA_DEBUG_VALIDATE set in the environment (to
// anything but "0"), every call that reads a page table first checks the
// device metadata with pa_validate_metadata (a copy to the host and a
// synchronization of the caller's stream) and returns its error instead of
// launching.  The variable is read once per process.
bool debug_validate() {
  static const bool on = [] {
    const char* e = getenv("PA_DEBUG_VALIDATE");
    return e != nullptr && e[0] != '\0' && strcmp(e, "0") != 0;
  }();
  return on;
}

size_t partial_o_bytes(const pa_desc* d, int S) {
  return align_up((size_t)d->num_seqs * d->num_q_heads * (size_t)S * d->head_dim * sizeof(float));
}
size_t partial_lse_bytes(const pa_desc* d, int S) {
  return align_up((size_t)d->num_seqs * d->num_q_heads * (size_t)S * sizeof(float));
}

pa::DecodeArgs decode_args(const pa_desc* d, const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* page_table, const int32_t* seq_lens, float scale) {
  pa::DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.num_seqs = d->num_seqs;
  a.num_q_heads = d->num_q_heads;
  a.num_kv_heads = d->num_kv_heads;
  a.max_pages_per_seq = d->max_pages_per_seq;
  a.num_pages = d->num_pages;
  a.num_splits = 1;
  a.write_partials = 0;
  a.scale_log2 = scale * kLog2e;
  return a;
}

// Page-balanced decode: V wave ranges per KV head; workspace holds the
// partials of B + V - 1 slots and the [B, 2] range table.
int decode_wgs_per_cu(const pa_desc* d) {
  if (d->dtype != PA_BF16) return 2;
  const long long block = 2LL * d->page_size * d->head_dim * 2;
  return block >= kBlockBytesOneWg ? 1 : 2;
}
int balanced_ranges(const pa_desc* d, int cus) {
  long long wgs = (long long)cus * decode_wgs_per_cu(d) / d->num_kv_heads;
  if (wgs < 1) wgs = 1;
  if (wgs > (1 << 20)) wgs = 1 << 20;
  return (int)(wgs * kWavesPerDecodeWg);
}
size_t balanced_o_bytes(const pa_desc* d, int V) {
  return align_up(((size_t)d->num_seqs + V - 1) * d->num_q_heads * d->head_dim * sizeof(float));
}
size_t balanced_lse_bytes(const pa_desc* d, int V) {
  return align_up(((size_t)d->num_seqs + V - 1) * d->num_q_heads * sizeof(float));
}
size_t balanced_workspace_bytes(const pa_desc* d, int V) {
  return balanced_o_bytes(d, V) + balanced_lse_bytes(d, V) +
         align_up((size_t)d->num_seqs * 2 * sizeof(int32_t));
}

pa_status run_balanced(const pa_desc* d, pa::DecodeArgs a, int V, void* workspace, void* out,
                       float* lse, hipStream_t stream) {
  char* ws = reinterpret_cast<char*>(workspace);
  a.num_splits = V;
  a.write_partials = 1;
  a.o_part = reinterpret_cast<float*>(ws);
  a.lse_part = reinterpret_cast<float*>(ws + balanced_o_bytes(d, V));
  a.range_meta = reinterpret_cast<int32_t*>(ws + balanced_o_bytes(d, V) + balanced_lse_bytes(d, V));
  const int G = d->num_q_heads / d->num_kv_heads;
  if (pa::launch_decode_balanced(a, d->dtype, d->head_dim, G, stream) != hipSuccess)
    return PA_ERR_HIP;
  pa::MergeArgs m;
  m.o_part = a.o_part;
  m.lse_part = a.lse_part;
  m.range_meta = a.range_meta;
  m.out = out;
  m.lse = lse;
  m.rows = d->num_seqs;
  m.heads = d->num_q_heads;
  m.num_splits = V;
  if (pa::launch_merge(m, d->dtype, d->head_dim, stream) != hipSuccess) return PA_ERR_HIP;
  return PA_OK;
}

// Split launch + merge launch shared by pa_decode (guard-chosen S) and
// pa_split_merge (caller-chosen S).
pa_status run_split(const pa_desc* d, pa::DecodeArgs a, int S, void* workspace, void* out,
                    float* lse, hipStream_t stream) {
  float* o_part = reinterpret_cast<float*>(workspace);
  float* lse_part = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + partial_o_bytes(d, S));
  a.num_splits = S;
  a.write_partials = 1;
  a.o_part = o_part;
  a.lse_part = lse_part;
  const int G = d->num_q_heads / d->num_kv_heads;
  if (pa::launch_decode(a, d->dtype, d->head_dim, G, stream) != hipSuccess) return PA_ERR_HIP;
  pa::MergeArgs m;
  m.o_part = o_part;
  m.lse_part = lse_part;
  m.range_meta = nullptr;
  m.out = out;
  m.lse = lse;
  m.rows = d->num_seqs;
  m.heads = d->num_q_heads;
  m.num_splits = S;
  if (pa::launch_merge(m, d->dtype, d->head_dim, stream) != hipSuccess) return PA_ERR_HIP;
  return PA_OK;
}

// Chunked prefill: query tiles of packed (token, head-in-group) rows, each
// optionally split along its key range.
struct PrefillPlan {
  long long units;      // (request, query tile, KV head) triples in the grid
  int tiles_per_seq;
  int splits;           // S
  int kv_tiles_per_split;
};

PrefillPlan prefill_plan(const pa_desc* d, int cus) {
  PrefillPlan pp;
  const int G = d->num_q_heads / d->num_kv_heads;
  const int rows = pa::prefill_tile_rows(d->head_dim);
  pp.tiles_per_seq = (int)(((long long)d->max_q_len * G + rows - 1) / rows);
  pp.units = (long long)pp.tiles_per_seq * d->num_seqs * d->num_kv_heads;
  const int keys = pa::prefill_tile_keys();
  const int max_kv_tiles = (d->max_seq_len + keys - 1) / keys;
  const long long slots = (long long)kPrefillSlotsPerCu * cus;
  pp.splits = 1;
  pp.kv_tiles_per_split = max_kv_tiles > 0 ? max_kv_tiles : 1;
  if (pp.units > 0 && pp.units < (long long)kPrefillUnitsPerSlot * slots &&
      max_kv_tiles >= 2 * kPrefillMinTiles) {
    // aim for about kPrefillUnitsPerSlot splits of roughly half the longest
    // key range per slot
    long long want = (pp.units * max_kv_tiles + (long long)kPrefillUnitsPerSlot * slots - 1) /
                     ((long long)kPrefillUnitsPerSlot * slots);
    int kc = (int)(want < kPrefillMinTiles ? kPrefillMinTiles : want);
    int S = (max_kv_tiles + kc - 1) / kc;
    if (S > kMaxSplits) {
      S = kMaxSplits;
      kc = (max_kv_tiles + S - 1) / S;
    }
    if (S > 1) {
      pp.splits = S;
      pp.kv_tiles_per_split = kc;
    }
  }
  return pp;
}

size_t prefill_part_o_bytes(const pa_desc* d, const PrefillPlan& pp) {
  return align_up((size_t)pp.units * pp.splits * pa::prefill_tile_rows(d->head_dim) * d->head_dim *
                  sizeof(float));
}

size_t prefill_workspace_bytes(const pa_desc* d, const PrefillPlan& pp) {
  return prefill_part_o_bytes(d, pp) +
         align_up((size_t)pp.units * pp.splits * pa::prefill_tile_rows(d->head_dim) * sizeof(float));
}

}  // namespace

extern "C" {

const char* pa_status_str(pa_status s) {
  switch (s) {
    case PA_OK: return "PA_OK";
    case PA_ERR_ARG: return "PA_ERR_ARG: invalid argument";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: shape or dtype not built";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace too small";
    case PA_ERR_HIP: return "PA_ERR_HIP: kernel launch failed";
    case PA_ERR_METADATA: return "PA_ERR_METADATA: device metadata violates the contract";
    case PA_ERR_NO_PAGES: return "PA_ERR_NO_PAGES: the page pool has too few free pages";
  }
  return "unknown pa_status";
}

size_t pa_workspace_bytes(const pa_desc* d, int32_t num_splits) {
  if (check_desc(d) != PA_OK || num_splits < 1) return 0;
  return partial_o_bytes(d, num_splits) + partial_lse_bytes(d, num_splits);
}

pa_status pa_plan(const pa_desc* d, int32_t cu_count, pa_plan_info* plan) {
  pa_status st = check_desc(d);
  if (st != PA_OK) return st;
  if (plan == nullptr) return PA_ERR_ARG;
  memset(plan, 0, sizeof(*plan));
  const int cus = cu_count > 0 ? cu_count : device_cu_count();
  const int G = d->num_q_heads / d->num_kv_heads;
  if (d->max_q_len > 1) {
    if (d->dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
    PrefillPlan pp = prefill_plan(d, cus);
    plan->path = PA_PATH_PREFILL;
    plan->num_splits = pp.splits;
    plan->grid_x = (int32_t)(pp.units * pp.splits);
    plan->workspace_bytes = pp.splits > 1 ? prefill_workspace_bytes(d, pp) : 0;
    return PA_OK;
  }
  if (!pa::decode_group_supported(G, d->dtype)) return PA_ERR_UNSUPPORTED;
  const long long units = (long long)d->num_seqs * d->num_kv_heads;
  const int max_pages = (d->max_seq_len + d->page_size - 1) / d->page_size;
  const int V = balanced_ranges(d, cus);
  if (d->num_seqs <= pa::kMaxBalancedSeqs && (long long)d->num_seqs * max_pages >= V) {
    plan->path = PA_PATH_DECODE_BALANCED;
    plan->num_splits = V;
    plan->grid_x = (int32_t)((long long)d->num_kv_heads * (V / kWavesPerDecodeWg));
    plan->workspace_bytes = balanced_workspace_bytes(d, V);
    return PA_OK;
  }
  const long long target = (long long)kTargetWgsPerCu * cus;
  int S = 1;
  if (units > 0 && units < target) {
    long long want = (target + units - 1) / units;
    long long cap = max_pages / kMinPagesPerSplit;
    if (want > cap) want = cap;
    if (want > kMaxSplits) want = kMaxSplits;
    S = want >= 2 ? (int)want : 1;
  }
  plan->path = S > 1 ? PA_PATH_DECODE_SPLIT : PA_PATH_DECODE;
  plan->num_splits = S;
  plan->grid_x = (int32_t)(units * S);
  plan->workspace_bytes = S > 1 ? pa_workspace_bytes(d, S) : 0;
  return PA_OK;
}

pa_status pa_decode(const pa_desc* d, const void* q, const void* k_pool, const void* v_pool,
                    const int32_t* page_table, const int32_t* seq_lens, const int32_t* q_offsets,
                    float scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                    void* stream) {
  (void)q_offsets;  // decode rows sit at position seq_len - 1 by contract
  pa_status st = check_decode_call(d, q, k_pool, v_pool, page_table, seq_lens, scale, out, lse);
  if (st != PA_OK || d->num_seqs == 0) return st;
  if (debug_validate() && (st = pa_validate_metadata(d, page_table, seq_lens, nullptr, stream)) != PA_OK)
    return st;
  pa_plan_info plan;
  st = pa_plan(d, 0, &plan);
  if (st != PA_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  pa::DecodeArgs a = decode_args(d, q, k_pool, v_pool, page_table, seq_lens, scale);
  if (plan.path == PA_PATH_DECODE_BALANCED) {
    if (workspace == nullptr || workspace_bytes < plan.workspace_bytes || !aligned16(workspace))
      return PA_ERR_WORKSPACE;
    return run_balanced(d, a, plan.num_splits, workspace, out, lse, s);
  }
  if (plan.num_splits == 1) {
    a.out = out;
    a.lse = lse;
    const int G = d->num_q_heads / d->num_kv_heads;
    return pa::launch_decode(a, d->dtype, d->head_dim, G, s) == hipSuccess ? PA_OK : PA_ERR_HIP;
  }
  if (workspace == nullptr || workspace_bytes < plan.workspace_bytes || !aligned16(workspace))
    return PA_ERR_WORKSPACE;
  return run_split(d, a, plan.num_splits, workspace, out, lse, s);
}

pa_status pa_decode_dense(const pa_desc* d, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* seq_lens, float scale, void* out, float* lse, void* stream) {
  // the page-table check is satisfied with seq_lens: the dense kernel reads no table
  pa_status st = check_decode_call(d, q, k_cache, v_cache, seq_lens, seq_lens, scale, out, lse);
  if (st != PA_OK || d->num_seqs == 0) return st;
  pa::DecodeArgs a = decode_args(d, q, k_cache, v_cache, nullptr, seq_lens, scale);
  a.out = out;
  a.lse = lse;
  const int G = d->num_q_heads / d->num_kv_heads;
  return pa::launch_decode_dense(a, d->dtype, d->head_dim, G, reinterpret_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

size_t pa_direct_workspace_bytes(const pa_desc* d) {
  if (check_desc(d) != PA_OK) return 0;
  return align_up((size_t)d->num_seqs * d->num_q_heads * d->max_pages_per_seq * d->page_size *
                  sizeof(float));
}

pa_status pa_decode_direct(const pa_desc* d, const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* page_table, const int32_t* seq_lens, float scale, void* out,
                           float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  pa_status st = check_decode_call(d, q, k_pool, v_pool, page_table, seq_lens, scale, out, lse);
  if (st != PA_OK || d->num_seqs == 0) return st;
  if (debug_validate() && (st = pa_validate_metadata(d, page_table, seq_lens, nullptr, stream)) != PA_OK)
    return st;
  const int Gd = d->num_q_heads / d->num_kv_heads;
  if (!(Gd == 1 || Gd == 2 || Gd == 4 || Gd == 8)) return PA_ERR_UNSUPPORTED;
  if (workspace == nullptr || workspace_bytes < pa_direct_workspace_bytes(d) || !aligned16(workspace))
    return PA_ERR_WORKSPACE;
  pa::DirectArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.out = out;
  a.lse = lse;
  a.scores = reinterpret_cast<float*>(workspace);
  a.num_seqs = d->num_seqs;
  a.num_q_heads = d->num_q_heads;
  a.num_kv_heads = d->num_kv_heads;
  a.max_pages_per_seq = d->max_pages_per_seq;
  a.num_pages = d->num_pages;
  a.scale_log2 = scale * kLog2e;
  const int G = d->num_q_heads / d->num_kv_heads;
  return pa::launch_decode_direct(a, d->dtype, d->head_dim, G, reinterpret_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

pa_status pa_split_merge(const pa_desc* d, const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* page_table, const int32_t* seq_lens,
                         const int32_t* q_offsets, float scale, int32_t num_splits,
                         void* workspace, size_t workspace_bytes, void* out, float* lse,
                         void* stream) {
  (void)q_offsets;
  pa_status st = check_decode_call(d, q, k_pool, v_pool, page_table, seq_lens, scale, out, lse);
  if (st != PA_OK) return st;
  if (num_splits < 1 || num_splits > kMaxSplitsApi) return PA_ERR_ARG;
  if (d->num_seqs == 0) return PA_OK;
  if (debug_validate() && (st = pa_validate_metadata(d, page_table, seq_lens, nullptr, stream)) != PA_OK)
    return st;
  const size_t need = pa_workspace_bytes(d, num_splits);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return PA_ERR_WORKSPACE;
  pa::DecodeArgs a = decode_args(d, q, k_pool, v_pool, page_table, seq_lens, scale);
  return run_split(d, a, num_splits, workspace, out, lse, reinterpret_cast<hipStream_t>(stream));
}

pa_status pa_prefill_chunk(const pa_desc* d, const void* q, const void* k_pool,
                           const void* v_pool, const int32_t* page_table, const int32_t* seq_lens,
                           const int32_t* q_offsets, const int32_t* q_starts, float scale,
                           void* out, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream) {
  pa_status st = check_desc(d);
  if (st != PA_OK) return st;
  if (d->dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  const int G = d->num_q_heads / d->num_kv_heads;   // any ratio: rows pack (token, head) pairs
  if (d->num_seqs == 0 || d->total_q == 0) return PA_OK;
  if (!q || !k_pool || !v_pool || !page_table || !seq_lens || !q_offsets || !out) return PA_ERR_ARG;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out) ||
      !aligned4(page_table) || !aligned4(seq_lens) || !aligned4(q_offsets) ||
      (q_starts && !aligned4(q_starts)) || (lse && !aligned4(lse)))
    return PA_ERR_ARG;
  if (out == q) return PA_ERR_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return PA_ERR_ARG;
  if (d->max_q_len < 1) return PA_ERR_ARG;
  if (debug_validate() && (st = pa_validate_metadata(d, page_table, seq_lens, q_offsets, stream)) != PA_OK)
    return st;
  PrefillPlan pp = prefill_plan(d, device_cu_count());
  if (workspace == nullptr) {
    // no scratch: run every query tile over its whole key range
    pp.splits = 1;
    pp.kv_tiles_per_split = (d->max_seq_len + pa::prefill_tile_keys() - 1) / pa::prefill_tile_keys();
    if (pp.kv_tiles_per_split < 1) pp.kv_tiles_per_split = 1;
  } else if (pp.splits > 1 &&
             (workspace_bytes < prefill_workspace_bytes(d, pp) || !aligned16(workspace))) {
    return PA_ERR_WORKSPACE;
  }
  pa::PrefillArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.q_offsets = q_offsets;
  a.q_starts = q_starts;
  a.out = out;
  a.lse = lse;
  a.num_seqs = d->num_seqs;
  a.num_q_heads = d->num_q_heads;
  a.num_kv_heads = d->num_kv_heads;
  a.max_pages_per_seq = d->max_pages_per_seq;
  a.num_pages = d->num_pages;
  a.tiles_per_seq = pp.tiles_per_seq;
  a.num_splits = pp.splits;
  a.kv_tiles_per_split = pp.kv_tiles_per_split;
  if (pp.splits > 1) {
    a.part_o = reinterpret_cast<float*>(workspace);
    a.part_lse = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + prefill_part_o_bytes(d, pp));
  }
  a.scale_log2 = scale * kLog2e;
  const hipError_t e = pa::launch_prefill(a, d->head_dim, G, reinterpret_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return PA_ERR_UNSUPPORTED;
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_mixed_attention(const pa_desc* d, const void* q, const void* k_pool,
                             const void* v_pool, const int32_t* page_table, const int32_t* seq_lens,
                             const int32_t* q_offsets, const int32_t* q_starts, float scale,
                             void* out, float* lse, void* stream) {
  pa_status st = check_desc(d);
  if (st != PA_OK) return st;
  if (d->dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  const int G = d->num_q_heads / d->num_kv_heads;
  if (!(G == 1 || G == 2 || G == 4 || G == 8)) return PA_ERR_UNSUPPORTED;
  if (d->num_seqs > pa::kMaxMixedSeqs) return PA_ERR_UNSUPPORTED;
  if (d->num_seqs == 0 || d->total_q == 0) return PA_OK;
  if (!q || !k_pool || !v_pool || !page_table || !seq_lens || !q_offsets || !out) return PA_ERR_ARG;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out) ||
      !aligned4(page_table) || !aligned4(seq_lens) || !aligned4(q_offsets) ||
      (q_starts && !aligned4(q_starts)) || (lse && !aligned4(lse)))
    return PA_ERR_ARG;
  if (out == q) return PA_ERR_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return PA_ERR_ARG;
  if (d->max_q_len < 1) return PA_ERR_ARG;
  if (debug_validate() && (st = pa_validate_metadata(d, page_table, seq_lens, q_offsets, stream)) != PA_OK)
    return st;
  pa::PrefillArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.q_offsets = q_offsets;
  a.q_starts = q_starts;
  a.out = out;
  a.lse = lse;
  a.num_seqs = d->num_seqs;
  a.num_q_heads = d->num_q_heads;
  a.num_kv_heads = d->num_kv_heads;
  a.max_pages_per_seq = d->max_pages_per_seq;
  a.num_pages = d->num_pages;
  a.tiles_per_seq = 1;
  a.num_splits = 1;
  a.kv_tiles_per_split = pa::kMixedUnsplit;
  a.scale_log2 = scale * kLog2e;
  const long long items = pa::mixed_items_bound(d->total_q, d->num_seqs, G);
  const hipError_t e =
      pa::launch_mixed(a, d->head_dim, G, items, reinterpret_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return PA_ERR_UNSUPPORTED;
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_append_kv(const pa_desc* d, const void* k_new, const void* v_new,
                       const int32_t* page_table, const int32_t* seq_lens,
                       const int32_t* q_offsets, const int32_t* q_starts, void* k_pool,
                       void* v_pool, void* stream) {
  pa_status st = check_desc(d);
  if (st != PA_OK) return st;
  if (d->num_seqs == 0 || d->total_q == 0) return PA_OK;
  if (!k_new || !v_new || !page_table || !seq_lens || !q_offsets || !k_pool || !v_pool)
    return PA_ERR_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool) ||
      !aligned4(page_table) || !aligned4(seq_lens) || !aligned4(q_offsets) ||
      (q_starts && !aligned4(q_starts)))
    return PA_ERR_ARG;
  if (d->max_q_len < 1) return PA_ERR_ARG;
  if (debug_validate() && (st = pa_validate_metadata(d, page_table, seq_lens, q_offsets, stream)) != PA_OK)
    return st;
  pa::AppendArgs a;
  memset(&a, 0, sizeof(a));
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.q_offsets = q_offsets;
  a.q_starts = q_starts;
  a.num_seqs = d->num_seqs;
  a.num_kv_heads = d->num_kv_heads;
  a.max_pages_per_seq = d->max_pages_per_seq;
  a.num_pages = d->num_pages;
  a.head_bytes = d->head_dim * elem_bytes(d->dtype);
  const int rpw = pa::append_rows_per_wg();
  a.tiles_per_seq = (d->max_q_len + rpw - 1) / rpw;
  a.total_rows = d->total_q;
  return pa::launch_append(a, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? PA_OK
                                                                                    : PA_ERR_HIP;
}

pa_status pa_copy_pages(const pa_desc* d, void* k_pool, void* v_pool, const int32_t* src_ids,
                        const int32_t* dst_ids, int32_t n, void* stream) {
  pa_status st = check_desc(d);
  if (st != PA_OK) return st;
  if (n < 0) return PA_ERR_ARG;
  if (n == 0) return PA_OK;
  if (!k_pool || !v_pool || !src_ids || !dst_ids) return PA_ERR_ARG;
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned4(src_ids) || !aligned4(dst_ids))
    return PA_ERR_ARG;
  pa::CopyPagesArgs a;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.src = src_ids;
  a.dst = dst_ids;
  a.n = n;
  a.num_pages = d->num_pages;
  a.page_bytes = (int64_t)d->num_kv_heads * d->page_size * d->head_dim * elem_bytes(d->dtype);
  // enough workgroups to keep a few pages' copies spread over the chip
  a.slices = (int32_t)((a.page_bytes / 16 + 1023) / 1024);
  return pa::launch_copy_pages(a, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? PA_OK
                                                                                       : PA_ERR_HIP;
}

pa_status pa_merge_partials(int32_t rows, int32_t heads, int32_t num_splits, int32_t head_dim,
                            const float* o_part, const float* lse_part, void* out,
                            int32_t out_dtype, float* lse, void* stream) {
  if (rows < 0 || heads <= 0 || num_splits < 1 || num_splits > kMaxSplitsApi) return PA_ERR_ARG;
  if (out_dtype != PA_BF16 && out_dtype != PA_F32) return PA_ERR_ARG;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (rows == 0) return PA_OK;
  if (!o_part || !lse_part || !out) return PA_ERR_ARG;
  if (!aligned16(o_part) || !aligned4(lse_part) || !aligned16(out) || (lse && !aligned4(lse)))
    return PA_ERR_ARG;
  pa::MergeArgs m;
  m.o_part = o_part;
  m.lse_part = lse_part;
  m.range_meta = nullptr;
  m.out = out;
  m.lse = lse;
  m.rows = rows;
  m.heads = heads;
  m.num_splits = num_splits;
  return pa::launch_merge(m, out_dtype, head_dim, reinterpret_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

pa_status pa_gather_kv(const pa_desc* d, const void* k_pool, const void* v_pool,
                       const int32_t* page_table, int32_t req, int32_t seq_len, void* k_out,
                       void* v_out, void* stream) {
  pa_status st = check_desc(d);
  if (st != PA_OK) return st;
  if (req < 0 || req >= d->num_seqs || seq_len < 0 ||
      (long long)seq_len > (long long)d->max_pages_per_seq * d->page_size)
    return PA_ERR_ARG;
  if (seq_len == 0) return PA_OK;
  if (!k_pool || !v_pool || !page_table || !k_out || !v_out) return PA_ERR_ARG;
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_out) || !aligned16(v_out) ||
      !aligned4(page_table))
    return PA_ERR_ARG;
  pa::GatherArgs a;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.page_row = page_table + (size_t)req * d->max_pages_per_seq;
  a.k_out = k_out;
  a.v_out = v_out;
  a.seq_len = seq_len;
  a.num_kv_heads = d->num_kv_heads;
  a.head_dim = d->head_dim;
  a.elem_bytes = elem_bytes(d->dtype);
  a.num_pages = d->num_pages;
  return pa::launch_gather(a, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? PA_OK
                                                                                     : PA_ERR_HIP;
}

pa_status pa_read_blocks(const void* buf, int64_t buf_blocks, const int32_t* order, int32_t nblocks,
                         int32_t block_bytes, uint32_t* sink, void* stream) {
  if (!buf || !order || !sink || buf_blocks < 0 || nblocks < 0 || !aligned16(buf) || !aligned4(order) ||
      !aligned4(sink))
    return PA_ERR_ARG;
  if (!(block_bytes == 4096 || block_bytes == 8192 || block_bytes == 16384 || block_bytes == 32768))
    return PA_ERR_ARG;
  pa::ReadBlocksArgs a;
  a.buf = buf;
  a.order = order;
  a.sink = sink;
  a.buf_blocks = buf_blocks;
  a.nblocks = nblocks;
  a.block_bytes = block_bytes;
  return pa::launch_read_blocks(a, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_validate_metadata(const pa_desc* d, const int32_t* page_table,
                               const int32_t* seq_lens, const int32_t* q_offsets, void* stream) {
  pa_status st = check_desc(d);
  if (st != PA_OK) return st;
  const int B = d->num_seqs;
  if (B == 0) return PA_OK;
  if (!page_table || !seq_lens) return PA_ERR_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  std::vector<int32_t> pt((size_t)B * d->max_pages_per_seq), sl(B), qo(B);
  if (hipMemcpyAsync(pt.data(), page_table, pt.size() * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipMemcpyAsync(sl.data(), seq_lens, sl.size() * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
      (q_offsets &&
       hipMemcpyAsync(qo.data(), q_offsets, qo.size() * 4, hipMemcpyDeviceToHost, s) != hipSuccess) ||
      hipStreamSynchronize(s) != hipSuccess)
    return PA_ERR_HIP;
  long long total_q = 0;
  for (int r = 0; r < B; ++r) {
    const int L = sl[r];
    if (L < 1 || L > d->max_seq_len || (long long)L > (long long)d->max_pages_per_seq * d->page_size)
      return PA_ERR_METADATA;
    const int o = q_offsets ? qo[r] : L - 1;
    if (o < 0 || o >= L || L - o > (d->max_q_len > 0 ? d->max_q_len : 1)) return PA_ERR_METADATA;
    total_q += L - o;
    const int np = (L + d->page_size - 1) / d->page_size;
    for (int p = 0; p < np; ++p) {
      const int32_t id = pt[(size_t)r * d->max_pages_per_seq + p];
      if (id < 0 || id >= d->num_pages) return PA_ERR_METADATA;
    }
  }
  if (total_q != d->total_q) return PA_ERR_METADATA;
  return PA_OK;
}

}  // extern "C"
