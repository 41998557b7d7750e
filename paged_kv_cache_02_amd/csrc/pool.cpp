// Host-side page allocator for the shared KV pool.
//
// The pool hands out physical page ids on demand and takes them back when a
// request finishes, and a request's page-table row grows by whole pages as
// its sequence grows (tiny-llm source reading, section "Paged KV Cache": a
// pool of physical pages that are allocated on demand and returned when a
// request completes, plus a per-request logical sequence with its page
// table; "Build a vLLM from Scratch", Week 3: pages on demand instead of a
// contiguous reservation per request).
//
// Pages can be shared: several page tables may name the same physical page
// (a common prompt prefix), each holding one reference.  A page returns to
// the free list when its last reference is dropped, and a holder about to
// write into a shared page first takes a private copy (copy on write).  This
// is the reference-count form of prefix reuse ("mini-vllm-tutorial
// advanced-series design", Phase C, adv05, which sets radix-tree reuse with
// copy on write against the main series' hash plus reference counts); how a
// caller finds a shared prefix (hash or radix tree) is outside the pool.
// The attention kernels already read whatever page a table names, so
// sharing needs nothing from them.
//
// Free ids sit on a stack (the most recently freed page is reused first).
// Every call is all-or-nothing: a request that cannot be met changes
// nothing.  One mutex per pool makes the calls thread-safe.  Device memory is
// never touched: the page-table rows the helpers edit are host arrays the
// caller copies to the device, and the page contents a copy on write needs
// are moved by pa_copy_pages.
#include "pa.h"

#include <mutex>
#include <new>
#include <unordered_map>
#include <vector>

struct pa_page_pool {
  std::mutex mu;
  std::vector<int32_t> free_ids;
  std::vector<int32_t> refs;   // references held on each page; 0 = free
};

namespace {

int32_t pages_for(int32_t len, int32_t page_size) {
  return len <= 0 ? 0 : (int32_t)(((int64_t)len + page_size - 1) / page_size);
}

bool in_range(const pa_page_pool* p, int32_t id) { return id >= 0 && id < (int32_t)p->refs.size(); }

// Pops n ids (caller holds the lock and has checked n <= free count).
void pop_ids(pa_page_pool* p, int32_t n, int32_t* ids) {
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = p->free_ids.back();
    p->free_ids.pop_back();
    p->refs[id] = 1;
    ids[i] = id;
  }
}

// True if dropping one reference per occurrence of each id is possible:
// every id in range and listed no more often than it is held (caller holds
// the lock).
bool ids_releasable(const pa_page_pool* p, const int32_t* ids, int32_t n) {
  std::unordered_map<int32_t, int32_t> count;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (!in_range(p, id) || ++count[id] > p->refs[id]) return false;
  }
  return true;
}

// True if every id is in range and held (caller holds the lock).
bool ids_held(const pa_page_pool* p, const int32_t* ids, int32_t n) {
  for (int32_t i = 0; i < n; ++i)
    if (!in_range(p, ids[i]) || p->refs[ids[i]] <= 0) return false;
  return true;
}

void drop_ids(pa_page_pool* p, const int32_t* ids, int32_t n) {
  for (int32_t i = 0; i < n; ++i)
    if (--p->refs[ids[i]] == 0) p->free_ids.push_back(ids[i]);
}

bool row_args_ok(const int32_t* row, int32_t max_pages_per_seq, int32_t page_size) {
  return row != nullptr && max_pages_per_seq > 0 && page_size > 0;
}

}  // namespace

extern "C" {

pa_status pa_pool_create(int32_t num_pages, pa_page_pool** out) {
  if (out == nullptr) return PA_ERR_ARG;
  *out = nullptr;
  if (num_pages <= 0) return PA_ERR_ARG;
  pa_page_pool* p = new (std::nothrow) pa_page_pool;
  if (p == nullptr) return PA_ERR_ARG;
  p->free_ids.resize(num_pages);
  for (int32_t i = 0; i < num_pages; ++i) p->free_ids[i] = num_pages - 1 - i;   // pops 0, 1, 2, ...
  p->refs.assign(num_pages, 0);
  *out = p;
  return PA_OK;
}

void pa_pool_destroy(pa_page_pool* pool) { delete pool; }

int32_t pa_pool_num_free(pa_page_pool* pool) {
  if (pool == nullptr) return -1;
  std::lock_guard<std::mutex> lock(pool->mu);
  return (int32_t)pool->free_ids.size();
}

int32_t pa_pool_refcount(pa_page_pool* pool, int32_t id) {
  if (pool == nullptr) return -1;
  std::lock_guard<std::mutex> lock(pool->mu);
  return in_range(pool, id) ? pool->refs[id] : -1;
}

pa_status pa_pool_alloc(pa_page_pool* pool, int32_t n, int32_t* ids) {
  if (pool == nullptr || n < 0 || (n > 0 && ids == nullptr)) return PA_ERR_ARG;
  std::lock_guard<std::mutex> lock(pool->mu);
  if (n > (int32_t)pool->free_ids.size()) return PA_ERR_NO_PAGES;
  pop_ids(pool, n, ids);
  return PA_OK;
}

pa_status pa_pool_free(pa_page_pool* pool, const int32_t* ids, int32_t n) {
  if (pool == nullptr || n < 0 || (n > 0 && ids == nullptr)) return PA_ERR_ARG;
  std::lock_guard<std::mutex> lock(pool->mu);
  if (!ids_releasable(pool, ids, n)) return PA_ERR_ARG;
  drop_ids(pool, ids, n);
  return PA_OK;
}

pa_status pa_pool_share(pa_page_pool* pool, const int32_t* ids, int32_t n) {
  if (pool == nullptr || n < 0 || (n > 0 && ids == nullptr)) return PA_ERR_ARG;
  std::lock_guard<std::mutex> lock(pool->mu);
  if (!ids_held(pool, ids, n)) return PA_ERR_ARG;
  for (int32_t i = 0; i < n; ++i) ++pool->refs[ids[i]];
  return PA_OK;
}

pa_status pa_pool_reserve(pa_page_pool* pool, int32_t* page_table_row, int32_t max_pages_per_seq,
                          int32_t old_len, int32_t new_len, int32_t page_size) {
  if (pool == nullptr || !row_args_ok(page_table_row, max_pages_per_seq, page_size) || old_len < 0 ||
      new_len < old_len)
    return PA_ERR_ARG;
  const int32_t have = pages_for(old_len, page_size);
  const int32_t need = pages_for(new_len, page_size);
  if (need > max_pages_per_seq) return PA_ERR_ARG;
  if (need == have) return PA_OK;
  std::lock_guard<std::mutex> lock(pool->mu);
  if (need - have > (int32_t)pool->free_ids.size()) return PA_ERR_NO_PAGES;
  pop_ids(pool, need - have, page_table_row + have);
  return PA_OK;
}

pa_status pa_pool_release(pa_page_pool* pool, int32_t* page_table_row, int32_t max_pages_per_seq,
                          int32_t len, int32_t page_size) {
  if (pool == nullptr || !row_args_ok(page_table_row, max_pages_per_seq, page_size) || len < 0)
    return PA_ERR_ARG;
  const int32_t have = pages_for(len, page_size);
  if (have > max_pages_per_seq) return PA_ERR_ARG;
  std::lock_guard<std::mutex> lock(pool->mu);
  if (!ids_releasable(pool, page_table_row, have)) return PA_ERR_ARG;
  drop_ids(pool, page_table_row, have);
  for (int32_t i = 0; i < have; ++i) page_table_row[i] = -1;
  return PA_OK;
}

pa_status pa_pool_fork(pa_page_pool* pool, const int32_t* src_row, int32_t* dst_row,
                       int32_t max_pages_per_seq, int32_t len, int32_t page_size) {
  if (pool == nullptr || src_row == nullptr || !row_args_ok(dst_row, max_pages_per_seq, page_size) ||
      len < 0)
    return PA_ERR_ARG;
  const int32_t n = pages_for(len, page_size);
  if (n > max_pages_per_seq) return PA_ERR_ARG;
  std::lock_guard<std::mutex> lock(pool->mu);
  if (!ids_held(pool, src_row, n)) return PA_ERR_ARG;
  for (int32_t i = 0; i < n; ++i) {
    ++pool->refs[src_row[i]];
    dst_row[i] = src_row[i];
  }
  return PA_OK;
}

pa_status pa_pool_cow(pa_page_pool* pool, int32_t* page_table_row, int32_t max_pages_per_seq,
                      int32_t logical_page, int32_t* old_id, int32_t* new_id) {
  if (pool == nullptr || page_table_row == nullptr || max_pages_per_seq <= 0 || old_id == nullptr ||
      new_id == nullptr || logical_page < 0 || logical_page >= max_pages_per_seq)
    return PA_ERR_ARG;
  std::lock_guard<std::mutex> lock(pool->mu);
  const int32_t id = page_table_row[logical_page];
  if (!in_range(pool, id) || pool->refs[id] <= 0) return PA_ERR_ARG;
  if (pool->refs[id] == 1) {   // sole holder: write in place
    *old_id = id;
    *new_id = id;
    return PA_OK;
  }
  if (pool->free_ids.empty()) return PA_ERR_NO_PAGES;
  int32_t fresh;
  pop_ids(pool, 1, &fresh);
  --pool->refs[id];
  page_table_row[logical_page] = fresh;
  *old_id = id;
  *new_id = fresh;
  return PA_OK;
}

}  // extern "C"
