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
// Free ids sit on a stack (the most recently freed page is reused first);
// a per-page flag catches double frees.  Every call is all-or-nothing: a
// request that cannot be met changes nothing.  One mutex per pool makes the
// calls thread-safe.  Device memory is never touched: the page-table rows
// the helpers edit are host arrays the caller copies to the device.
#include "pa.h"

#include <mutex>
#include <new>
#include <vector>

struct pa_page_pool {
  std::mutex mu;
  std::vector<int32_t> free_ids;
  std::vector<uint8_t> in_use;
};

namespace {

int32_t pages_for(int32_t len, int32_t page_size) {
  return len <= 0 ? 0 : (int32_t)(((int64_t)len + page_size - 1) / page_size);
}

// Pops n ids (caller holds the lock and has checked n <= free count).
void pop_ids(pa_page_pool* p, int32_t n, int32_t* ids) {
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = p->free_ids.back();
    p->free_ids.pop_back();
    p->in_use[id] = 1;
    ids[i] = id;
  }
}

// Checks that ids are distinct pages currently in use (caller holds the lock).
bool ids_releasable(const pa_page_pool* p, const int32_t* ids, int32_t n) {
  std::vector<uint8_t> seen(p->in_use.size(), 0);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (id < 0 || id >= (int32_t)p->in_use.size() || !p->in_use[id] || seen[id]) return false;
    seen[id] = 1;
  }
  return true;
}

void push_ids(pa_page_pool* p, const int32_t* ids, int32_t n) {
  for (int32_t i = 0; i < n; ++i) {
    p->in_use[ids[i]] = 0;
    p->free_ids.push_back(ids[i]);
  }
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
  p->in_use.assign(num_pages, 0);
  *out = p;
  return PA_OK;
}

void pa_pool_destroy(pa_page_pool* pool) { delete pool; }

int32_t pa_pool_num_free(pa_page_pool* pool) {
  if (pool == nullptr) return -1;
  std::lock_guard<std::mutex> lock(pool->mu);
  return (int32_t)pool->free_ids.size();
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
  push_ids(pool, ids, n);
  return PA_OK;
}

pa_status pa_pool_reserve(pa_page_pool* pool, int32_t* page_table_row, int32_t max_pages_per_seq,
                          int32_t old_len, int32_t new_len, int32_t page_size) {
  if (pool == nullptr || page_table_row == nullptr || max_pages_per_seq <= 0 || page_size <= 0 ||
      old_len < 0 || new_len < old_len)
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
  if (pool == nullptr || page_table_row == nullptr || max_pages_per_seq <= 0 || page_size <= 0 ||
      len < 0)
    return PA_ERR_ARG;
  const int32_t have = pages_for(len, page_size);
  if (have > max_pages_per_seq) return PA_ERR_ARG;
  std::lock_guard<std::mutex> lock(pool->mu);
  if (!ids_releasable(pool, page_table_row, have)) return PA_ERR_ARG;
  push_ids(pool, page_table_row, have);
  for (int32_t i = 0; i < have; ++i) page_table_row[i] = -1;
  return PA_OK;
}

}  // extern "C"
