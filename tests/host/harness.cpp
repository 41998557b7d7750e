// Host-only test harness for the library's host C++ (the dispatch guard,
// argument checks, workspace carving, metadata validation and the page
// allocator), built with g++ under AddressSanitizer + UndefinedBehavior-
// Sanitizer ("asan" mode) and under ThreadSanitizer ("tsan" mode, the
// allocator from several threads).  No GPU and no HIP runtime: the few
// runtime calls the host code makes and the kernel launchers are replaced
// below by stubs (launches are counted, hipMemcpyAsync copies host memory, so
// pa_validate_metadata runs on host arrays).  Exits non-zero on the first
// failed check.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <thread>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

#define CHECK(cond)                                                              \
  do {                                                                           \
    if (!(cond)) {                                                               \
      std::fprintf(stderr, "check failed at %s:%d: %s\n", __FILE__, __LINE__, #cond); \
      std::exit(1);                                                              \
    }                                                                            \
  } while (0)

// ---------------------------------------------------------------------------
// stubs for the HIP runtime calls the host code makes
// ---------------------------------------------------------------------------
extern "C" {
hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) {
  *v = 256;
  return hipSuccess;
}
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t) {
  std::memcpy(dst, src, n);
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
}

// ---------------------------------------------------------------------------
// stubs for the kernel launchers (the kernels live in the .hip sources):
// each counts its calls and checks the pointers it was handed are the ones
// the workspace carving promises (inside the caller's workspace)
// ---------------------------------------------------------------------------
static std::atomic<int> g_launches{0};
static const char* g_ws_lo = nullptr;
static const char* g_ws_hi = nullptr;
static bool in_ws(const void* p) {
  const char* c = static_cast<const char*>(p);
  return g_ws_lo == nullptr || (c >= g_ws_lo && c < g_ws_hi);
}
namespace pa {
hipError_t launch_decode(const DecodeArgs& a, int, int, int, hipStream_t) {
  if (a.write_partials) CHECK(in_ws(a.o_part) && in_ws(a.lse_part));
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_decode_dense(const DecodeArgs&, int, int, int, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_decode_balanced(const DecodeArgs& a, int, int, int, hipStream_t) {
  CHECK(in_ws(a.o_part) && in_ws(a.lse_part) && in_ws(a.range_meta));
  CHECK(a.num_splits % 4 == 0);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_decode_direct(const DirectArgs& a, int, int, int, hipStream_t) {
  CHECK(in_ws(a.scores));
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_merge(const MergeArgs& a, int, int, hipStream_t) {
  CHECK(in_ws(a.o_part) && in_ws(a.lse_part));
  ++g_launches;
  return hipSuccess;
}
int prefill_tile_rows(int) { return 128; }
int prefill_tile_keys() { return 64; }
hipError_t launch_prefill(const PrefillArgs& a, int, int, hipStream_t) {
  if (a.num_splits > 1) CHECK(in_ws(a.part_o) && in_ws(a.part_lse));
  ++g_launches;
  return hipSuccess;
}
long long mixed_items_bound(long long total_q, int num_seqs, int group) {
  return (total_q * group + 127) / 128 + num_seqs;
}
hipError_t launch_mixed(const PrefillArgs&, int, int, long long, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
int append_rows_per_wg() { return 4; }
hipError_t launch_append(const AppendArgs&, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_copy_pages(const CopyPagesArgs&, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_gather(const GatherArgs&, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_read_blocks(const ReadBlocksArgs&, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
}  // namespace pa

// ---------------------------------------------------------------------------
// asan mode: planner, argument checks, carving, validator, pool invariants
// ---------------------------------------------------------------------------
static pa_desc make(int B, int Hq, int Hkv, int d, int NP, int MP, int total_q, int max_seq, int max_q,
                    int dtype) {
  pa_desc x;
  x.num_seqs = B;
  x.num_q_heads = Hq;
  x.num_kv_heads = Hkv;
  x.head_dim = d;
  x.page_size = 16;
  x.num_pages = NP;
  x.max_pages_per_seq = MP;
  x.total_q = total_q;
  x.max_seq_len = max_seq;
  x.max_q_len = max_q;
  x.dtype = dtype;
  return x;
}

static void check_pool_invariants(pa_page_pool* p, int NP) {
  int held = 0;
  for (int id = 0; id < NP; ++id) {
    const int r = pa_pool_refcount(p, id);
    CHECK(r >= 0);
    held += r > 0;
  }
  CHECK(pa_pool_refcount(p, -1) == -1 && pa_pool_refcount(p, NP) == -1);
  CHECK(pa_pool_num_free(p) == NP - held);
}

static int count_bad_launches(bool expect_validation);

static int asan_mode() {
  std::mt19937 rng(1234);
  // ---- the dispatch guard on random descriptors: never a crash, plans
  // that fit their own workspace numbers
  const int Hkvs[] = {1, 2, 4, 8};
  for (int it = 0; it < 20000; ++it) {
    const int Hkv = Hkvs[rng() % 4];
    const int G = 1 + (int)(rng() % 20);
    const int B = (int)(rng() % 5000);
    const int d = (rng() % 3 == 0) ? 96 : (rng() % 2 ? 64 : 128);
    const int MP = 1 + (int)(rng() % 4096);
    const int max_seq = (int)(rng() % (MP * 16 + 1));
    const int max_q = rng() % 2 ? 1 : (int)(rng() % (max_seq + 1));
    pa_desc x = make(B, G * Hkv, Hkv, d, 1 + (int)(rng() % 100000), MP, max_q <= 1 ? B : B * max_q,
                     max_seq, max_q, (int)(rng() % 2));
    pa_plan_info plan;
    const pa_status st = pa_plan(&x, (int)(rng() % 512), &plan);
    CHECK(st == PA_OK || st == PA_ERR_ARG || st == PA_ERR_UNSUPPORTED);
    if (st == PA_OK) {
      CHECK(plan.num_splits >= 1);
      if (plan.path == PA_PATH_DECODE || plan.path == PA_PATH_PREFILL) CHECK(plan.grid_x >= 0);
      if (plan.path == PA_PATH_DECODE_SPLIT)
        CHECK(plan.workspace_bytes == pa_workspace_bytes(&x, plan.num_splits));
    }
    (void)pa_workspace_bytes(&x, (int)(rng() % 300) - 10);
  }
  CHECK(pa_plan(nullptr, 256, nullptr) == PA_ERR_ARG);

  // ---- pa_decode: argument checks, and the launches land in the workspace
  {
    pa_desc x = make(64, 32, 8, 128, 20000, 512, 64, 8192, 1, PA_BF16);
    pa_plan_info plan;
    CHECK(pa_plan(&x, 0, &plan) == PA_OK && plan.path == PA_PATH_DECODE_BALANCED);
    std::vector<char> ws(plan.workspace_bytes + 256);
    char* w = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(ws.data()) + 255) & ~uintptr_t(255));
    g_ws_lo = w;
    g_ws_hi = w + plan.workspace_bytes;
    alignas(16) static char buf[4096];
    const int launches = g_launches.load();
    CHECK(pa_decode(&x, buf, buf + 16, buf + 32, (int32_t*)(buf + 48), (int32_t*)(buf + 64), nullptr, 0.1f,
                    buf + 80, (float*)(buf + 96), w, plan.workspace_bytes, nullptr) == PA_OK);
    CHECK(g_launches.load() == launches + 2);   // decode + merge
    CHECK(pa_decode(&x, buf, buf + 16, buf + 32, (int32_t*)(buf + 48), (int32_t*)(buf + 64), nullptr, 0.1f,
                    buf + 80, nullptr, w, plan.workspace_bytes - 1, nullptr) == PA_ERR_WORKSPACE);
    CHECK(pa_decode(&x, buf + 1, buf + 16, buf + 32, (int32_t*)(buf + 48), (int32_t*)(buf + 64), nullptr,
                    0.1f, buf + 80, nullptr, w, plan.workspace_bytes, nullptr) == PA_ERR_ARG);
    CHECK(pa_decode(&x, buf, buf + 16, buf + 32, (int32_t*)(buf + 48), (int32_t*)(buf + 64), nullptr, -1.f,
                    buf + 80, nullptr, w, plan.workspace_bytes, nullptr) == PA_ERR_ARG);
    CHECK(pa_decode(&x, buf, buf + 16, buf + 32, (int32_t*)(buf + 48), (int32_t*)(buf + 64), nullptr, 0.1f,
                    buf, nullptr, w, plan.workspace_bytes, nullptr) == PA_ERR_ARG);   // out aliases q
    // split-K with a caller-chosen S
    const size_t need = pa_workspace_bytes(&x, 16);
    std::vector<char> ws2(need + 256);
    char* w2 = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(ws2.data()) + 255) & ~uintptr_t(255));
    g_ws_lo = w2;
    g_ws_hi = w2 + need;
    CHECK(pa_split_merge(&x, buf, buf + 16, buf + 32, (int32_t*)(buf + 48), (int32_t*)(buf + 64), nullptr,
                         0.1f, 16, w2, need, buf + 80, nullptr, nullptr) == PA_OK);
    CHECK(pa_split_merge(&x, buf, buf + 16, buf + 32, (int32_t*)(buf + 48), (int32_t*)(buf + 64), nullptr,
                         0.1f, 0, w2, need, buf + 80, nullptr, nullptr) == PA_ERR_ARG);
    g_ws_lo = g_ws_hi = nullptr;
  }

  // ---- pa_validate_metadata on host arrays (the stubbed copy is a memcpy)
  {
    const int B = 3, MP = 8;
    pa_desc x = make(B, 8, 2, 64, 32, MP, 10, 100, 5, PA_BF16);
    std::vector<int32_t> pt(B * MP, -1), sl = {20, 33, 5}, qo = {18, 30, 0};
    int next = 0;
    for (int r = 0; r < B; ++r)
      for (int p = 0; p < (sl[r] + 15) / 16; ++p) pt[r * MP + p] = next++;
    CHECK(pa_validate_metadata(&x, pt.data(), sl.data(), qo.data(), nullptr) == PA_OK);
    qo[1] = -1;
    CHECK(pa_validate_metadata(&x, pt.data(), sl.data(), qo.data(), nullptr) == PA_ERR_METADATA);
    qo[1] = 30;
    pt[1 * MP + 2] = 32;   // page id out of the pool
    CHECK(pa_validate_metadata(&x, pt.data(), sl.data(), qo.data(), nullptr) == PA_ERR_METADATA);
    pt[1 * MP + 2] = 4;
    sl[2] = 0;             // empty request
    CHECK(pa_validate_metadata(&x, pt.data(), sl.data(), qo.data(), nullptr) == PA_ERR_METADATA);
  }

  // ---- without PA_DEBUG_VALIDATE, bad device metadata is not looked at
  CHECK(count_bad_launches(false) > 0);

  // ---- the pool, single thread: random operations against invariants
  {
    const int NP = 300, MP = 40, ROWS = 12;
    pa_page_pool* p = nullptr;
    CHECK(pa_pool_create(NP, &p) == PA_OK);
    std::vector<int32_t> rows(ROWS * MP, -1);
    std::vector<int> len(ROWS, 0);
    for (int it = 0; it < 40000; ++it) {
      const int r = (int)(rng() % ROWS);
      int32_t* row = rows.data() + r * MP;
      switch (rng() % 5) {
        case 0: {   // grow
          const int nl = len[r] + (int)(rng() % 64);
          if (pa_pool_reserve(p, row, MP, len[r], nl, 16) == PA_OK) len[r] = nl;
          break;
        }
        case 1:     // finish
          CHECK(pa_pool_release(p, row, MP, len[r], 16) == PA_OK);
          len[r] = 0;
          break;
        case 2: {   // fork from another row into an empty one
          const int src = (int)(rng() % ROWS);
          if (len[r] == 0 && src != r && len[src] > 0 &&
              pa_pool_fork(p, rows.data() + src * MP, row, MP, len[src], 16) == PA_OK)
            len[r] = len[src];
          break;
        }
        case 3: {   // copy on write of a random held page
          if (len[r] == 0) break;
          const int lp = (int)(rng() % ((len[r] + 15) / 16));
          int32_t o = -2, n = -2;
          const pa_status st = pa_pool_cow(p, row, MP, lp, &o, &n);
          CHECK(st == PA_OK || st == PA_ERR_NO_PAGES);
          if (st == PA_OK) CHECK(row[lp] == n && pa_pool_refcount(p, n) >= 1);
          break;
        }
        default: {  // error paths change nothing
          const int before = pa_pool_num_free(p);
          int32_t bad[2] = {NP + 3, 0};
          CHECK(pa_pool_free(p, bad, 2) == PA_ERR_ARG);
          CHECK(pa_pool_share(p, bad, 1) == PA_ERR_ARG);
          std::vector<int32_t> big(NP + 1);
          CHECK(pa_pool_alloc(p, NP + 1, big.data()) == PA_ERR_NO_PAGES);
          CHECK(pa_pool_num_free(p) == before);
        }
      }
      if (it % 997 == 0) check_pool_invariants(p, NP);
    }
    for (int r = 0; r < ROWS; ++r) CHECK(pa_pool_release(p, rows.data() + r * MP, MP, len[r], 16) == PA_OK);
    CHECK(pa_pool_num_free(p) == NP);
    pa_pool_destroy(p);
  }
  // ---- pa_read_blocks: argument checks
  {
    alignas(16) static unsigned char blk[4096];
    int32_t order[2] = {0, 5};
    uint32_t sink = 0;
    const int before = g_launches.load();
    CHECK(pa_read_blocks(nullptr, 1, order, 2, 4096, &sink, nullptr) == PA_ERR_ARG);
    CHECK(pa_read_blocks(blk, 1, nullptr, 2, 4096, &sink, nullptr) == PA_ERR_ARG);
    CHECK(pa_read_blocks(blk, 1, order, 2, 4096, nullptr, nullptr) == PA_ERR_ARG);
    CHECK(pa_read_blocks(blk + 4, 1, order, 2, 4096, &sink, nullptr) == PA_ERR_ARG);   // misaligned
    CHECK(pa_read_blocks(blk, 1, order, 2, 2048, &sink, nullptr) == PA_ERR_ARG);       // size
    CHECK(pa_read_blocks(blk, -1, order, 2, 4096, &sink, nullptr) == PA_ERR_ARG);
    CHECK(pa_read_blocks(blk, 1, order, -1, 4096, &sink, nullptr) == PA_ERR_ARG);
    CHECK(g_launches.load() == before);
    CHECK(pa_read_blocks(blk, 1, order, 2, 4096, &sink, nullptr) == PA_OK);
    CHECK(g_launches.load() == before + 1);
  }
  std::printf("asan mode ok (%d launches stubbed)\n", g_launches.load());
  return 0;
}

// ---------------------------------------------------------------------------
// tsan mode: the allocator shared by threads, each owning its rows
// ---------------------------------------------------------------------------
static int tsan_mode() {
  const int NP = 4096, MP = 64, THREADS = 8, ROWS_PER = 6, ITERS = 4000;
  pa_page_pool* p = nullptr;
  CHECK(pa_pool_create(NP, &p) == PA_OK);
  // a shared prefix row all threads fork from (read-only after setup)
  std::vector<int32_t> prefix(MP, -1);
  CHECK(pa_pool_reserve(p, prefix.data(), MP, 0, 100, 16) == PA_OK);
  std::vector<std::thread> th;
  std::atomic<int> failures{0};
  for (int t = 0; t < THREADS; ++t) {
    th.emplace_back([&, t]() {
      std::mt19937 rng(77 + t);
      std::vector<int32_t> rows(ROWS_PER * MP, -1);
      std::vector<int> len(ROWS_PER, 0);
      for (int it = 0; it < ITERS; ++it) {
        const int r = (int)(rng() % ROWS_PER);
        int32_t* row = rows.data() + r * MP;
        const int op = (int)(rng() % 4);
        if (op == 0) {
          const int nl = len[r] + (int)(rng() % 48);
          const pa_status st = pa_pool_reserve(p, row, MP, len[r], nl, 16);
          if (st == PA_OK) len[r] = nl;
          else if (st != PA_ERR_NO_PAGES && st != PA_ERR_ARG) ++failures;
        } else if (op == 1) {
          if (pa_pool_release(p, row, MP, len[r], 16) != PA_OK) ++failures;
          len[r] = 0;
        } else if (op == 2) {
          if (len[r] == 0) {
            if (pa_pool_fork(p, prefix.data(), row, MP, 100, 16) == PA_OK) len[r] = 100;
            else ++failures;
          }
        } else if (len[r] > 0) {
          int32_t o, n;
          const pa_status st = pa_pool_cow(p, row, MP, (int)(rng() % ((len[r] + 15) / 16)), &o, &n);
          if (st != PA_OK && st != PA_ERR_NO_PAGES) ++failures;
        }
        if (pa_pool_num_free(p) < 0) ++failures;
      }
      for (int r = 0; r < ROWS_PER; ++r)
        if (pa_pool_release(p, rows.data() + r * MP, MP, len[r], 16) != PA_OK) ++failures;
    });
  }
  for (auto& x : th) x.join();
  CHECK(failures.load() == 0);
  CHECK(pa_pool_release(p, prefix.data(), MP, 100, 16) == PA_OK);
  CHECK(pa_pool_num_free(p) == NP);
  for (int id = 0; id < NP; ++id) CHECK(pa_pool_refcount(p, id) == 0);
  pa_pool_destroy(p);
  std::printf("tsan mode ok (%d threads x %d operations)\n", THREADS, ITERS);
  return 0;
}

// ---------------------------------------------------------------------------
// debug mode (run with PA_DEBUG_VALIDATE=1 in the environment): every call
// that reads a page table checks the metadata first, launches nothing and
// returns PA_ERR_METADATA when it is bad, and launches as usual when it is
// good; without the variable (asan mode) the same bad metadata launches
// ---------------------------------------------------------------------------
static int count_bad_launches(bool expect_validation) {
  const int B = 3, MP = 8, NP = 32;
  std::vector<int32_t> pt(B * MP, -1), sl = {20, 33, 5}, qo = {18, 30, 0};
  int next = 0;
  for (int r = 0; r < B; ++r)
    for (int p = 0; p < (sl[r] + 15) / 16; ++p) pt[r * MP + p] = next++;
  alignas(16) static char buf[1 << 16];
  char* q = buf;
  char* kp = buf + 8192;
  char* vp = buf + 16384;
  char* out = buf + 24576;
  float* lse = reinterpret_cast<float*>(buf + 32768);
  const pa_status bad = expect_validation ? PA_ERR_METADATA : PA_OK;
  // chunks: 2 + 3 + 5 query rows
  pa_desc x = make(B, 8, 2, 64, NP, MP, 10, 100, 5, PA_BF16);
  auto prefill = [&] {
    return pa_prefill_chunk(&x, q, kp, vp, pt.data(), sl.data(), qo.data(), nullptr, 0.1f, out, lse,
                            nullptr, 0, nullptr);
  };
  auto mixed = [&] {
    return pa_mixed_attention(&x, q, kp, vp, pt.data(), sl.data(), qo.data(), nullptr, 0.1f, out, lse,
                              nullptr);
  };
  auto append = [&] {
    return pa_append_kv(&x, q, out, pt.data(), sl.data(), qo.data(), nullptr, kp, vp, nullptr);
  };
  int n = g_launches.load();
  CHECK(prefill() == PA_OK && mixed() == PA_OK && append() == PA_OK);
  CHECK(g_launches.load() == n + 3);
  pt[1 * MP + 2] = NP;   // a page id past the pool
  n = g_launches.load();
  CHECK(prefill() == bad && mixed() == bad && append() == bad);
  const int prefill_launches = g_launches.load() - n;
  pt[1 * MP + 2] = 4;
  // decode rows: one per request at position seq_len - 1
  pa_desc y = make(B, 8, 2, 64, NP, MP, B, 100, 1, PA_BF16);
  pa_plan_info plan;
  CHECK(pa_plan(&y, 0, &plan) == PA_OK);
  std::vector<char> ws(plan.workspace_bytes + 256);
  char* w = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(ws.data()) + 255) & ~uintptr_t(255));
  auto decode = [&] {
    return pa_decode(&y, q, kp, vp, pt.data(), sl.data(), nullptr, 0.1f, out, lse, w, plan.workspace_bytes,
                     nullptr);
  };
  n = g_launches.load();
  CHECK(decode() == PA_OK);
  CHECK(g_launches.load() > n);
  sl[2] = 0;   // an empty request
  n = g_launches.load();
  CHECK(decode() == bad);
  return prefill_launches + (g_launches.load() - n);
}

static int debug_mode() {
  CHECK(count_bad_launches(true) == 0);
  std::printf("debug mode ok\n");
  return 0;
}

int main(int argc, char** argv) {
  if (argc > 1 && std::strcmp(argv[1], "tsan") == 0) return tsan_mode();
  if (argc > 1 && std::strcmp(argv[1], "debug") == 0) return debug_mode();
  return asan_mode();
}
