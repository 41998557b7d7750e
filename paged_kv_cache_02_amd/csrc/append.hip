// Append a step's new K and V rows into the paged KV cache, and copy whole
// pages for a copy on write (gfx950).
//
// Every request's new tokens (a prefill chunk, or the one token of a decode
// step) are written into the shared pool before attention reads them: token
// position p of request r goes to slot p % P of physical page
// page_table[r][p / P] (tiny-llm source reading, section "Paged KV Cache":
// pages come from a shared pool and a page table maps each request's logical
// sequence onto them).  The copy is bit-exact.
//
// Rows are packed by request then token, as the attention entry points pack
// their queries.  When the caller passes the requests' first rows
// (q_starts) and the batch has at most kThreads requests, one workgroup
// takes each kRowsPerWg consecutive packed rows: its threads read every
// request's first row, length and offset at once, mark in LDS which request
// owns each of its rows, then stride over the 16-byte chunks of the rows, K
// and V alike.  The grid then has one workgroup per kRowsPerWg rows of the
// step, however the rows split over requests.  Otherwise one workgroup per
// (request, group of kRowsPerWg of its new rows) does the same for one
// request.  A page id outside [0, num_pages) is a contract violation: the
// row is skipped, so a bad table can never make the kernel write outside the
// pool.
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerWg = 4;

// First packed row of request r: q_starts[r], or the sum of n over the earlier
// requests (whole workgroup; every thread gets the value).
__device__ int row_start_of(const AppendArgs& a, int r) {
  __shared__ int partial[kThreads / 64];
  if (a.q_starts != nullptr) return a.q_starts[r];
  int acc = 0;
  for (int i = threadIdx.x; i < r; i += kThreads) acc += a.seq_lens[i] - a.q_offsets[i];
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) acc += __shfl_xor(acc, s);
  if ((threadIdx.x & 63) == 0) partial[threadIdx.x >> 6] = acc;
  __syncthreads();
  int tot = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) tot += partial[w];
  return tot;
}

__global__ void __launch_bounds__(kThreads) append_kernel(AppendArgs a) {
  const int tiles = a.tiles_per_seq;
  const int r = blockIdx.x / tiles;
  const int t = blockIdx.x % tiles;
  const int L = a.seq_lens[r];
  const int o = a.q_offsets[r];
  const int n = L - o;
  const int i0 = t * kRowsPerWg;
  // a negative offset would put rows at negative positions, i.e. before the
  // request's first page: such a request is skipped, like a page id outside
  // the pool, so no metadata can make this kernel write outside the pool
  if (o < 0 || n <= 0 || i0 >= n) return;
  const int rows = n - i0 < kRowsPerWg ? n - i0 : kRowsPerWg;
  const int start = row_start_of(a, r);

  const int row_bytes = a.num_kv_heads * a.head_bytes;   // one packed new row
  const int row_chunks = row_bytes / 16;
  const int head_chunks = a.head_bytes / 16;
  const int32_t* __restrict__ ptab = a.page_table + (size_t)r * a.max_pages_per_seq;
  const unsigned char* __restrict__ kn = reinterpret_cast<const unsigned char*>(a.k_new);
  const unsigned char* __restrict__ vn = reinterpret_cast<const unsigned char*>(a.v_new);
  unsigned char* __restrict__ kp = reinterpret_cast<unsigned char*>(a.k_pool);
  unsigned char* __restrict__ vp = reinterpret_cast<unsigned char*>(a.v_pool);
  const size_t block_bytes = (size_t)kPageSize * a.head_bytes;   // one (page, KV head) block

  // unrolled so that several independent page-id -> load -> store chains
  // are in flight per thread
#pragma unroll 4
  for (int x = threadIdx.x; x < rows * row_chunks; x += kThreads) {
    const int i = x / row_chunks;            // row within the group
    const int w = x % row_chunks;
    const int h = w / head_chunks;           // KV head
    const int c = w % head_chunks;           // 16-byte chunk within the head's d values
    const int pos = o + i0 + i;
    const int pg = pos / kPageSize;
    if (pg >= a.max_pages_per_seq) continue;
    const int id = ptab[pg];
    if (id < 0 || id >= a.num_pages) continue;
    const size_t src = ((size_t)(start + i0 + i) * a.num_kv_heads + h) * a.head_bytes + (size_t)c * 16;
    const size_t dst = ((size_t)id * a.num_kv_heads + h) * block_bytes +
                       (size_t)(pos % kPageSize) * a.head_bytes + (size_t)c * 16;
    *reinterpret_cast<uint4*>(kp + dst) = *reinterpret_cast<const uint4*>(kn + src);
    *reinterpret_cast<uint4*>(vp + dst) = *reinterpret_cast<const uint4*>(vn + src);
  }
}

// Packed rows [x0, x0 + kRowsPerWg) of the step: every request r (one per
// thread) whose rows [q_starts[r], q_starts[r] + n_r) meet the range marks
// the rows it owns with (r + 1, position); the largest r wins where
// inconsistent metadata makes two requests claim a row.  Rows past total_q
// are never touched, so no metadata can make this kernel read past k_new.
// The new-row sources, row starts, lengths, offsets and sizes come before
// the argument struct as plain scalars and pointers (equal to the struct's
// fields of the same names; row_bytes = num_kv_heads * head_bytes), so that
// the library's build preloads them into SGPRs at launch: the owner scan's
// reads and the group's first source loads go out without waiting on a load
// of the kernel arguments.  The group's packed rows are contiguous in k_new
// and v_new (chunk x of the group sits at x0 * row_bytes + 16 x), so the
// first two chunks of each thread are requested before the metadata, on
// which only their destination depends: the source read and the metadata
// read share one memory round trip.  The two early chunks are loaded at a
// clamped index (always inside the group's rows) and used only if real.
__global__ void __launch_bounds__(kThreads)
append_flat_kernel(const unsigned char* __restrict__ kn, const unsigned char* __restrict__ vn,
                   const int32_t* q_starts, const int32_t* seq_lens, const int32_t* q_offsets,
                   int num_seqs, int row_bytes, long long total_rows, AppendArgs a) {
  __shared__ unsigned long long s_owner[kRowsPerWg];
  const int tid = threadIdx.x;
  const long long x0 = (long long)blockIdx.x * kRowsPerWg;
  const int rows = total_rows - x0 < kRowsPerWg ? (int)(total_rows - x0) : kRowsPerWg;
  const int row_chunks = row_bytes / 16;
  const int n_chunks = rows * row_chunks;
  const unsigned char* __restrict__ ksrc = kn + (size_t)x0 * row_bytes;
  const unsigned char* __restrict__ vsrc = vn + (size_t)x0 * row_bytes;
  const int xa = tid, xb = tid + kThreads;   // this thread's first two chunks
  const size_t oa = (size_t)(xa < n_chunks ? xa : n_chunks - 1) * 16;
  const size_t ob = (size_t)(xb < n_chunks ? xb : n_chunks - 1) * 16;
  const uint4 ka = *reinterpret_cast<const uint4*>(ksrc + oa);
  const uint4 va = *reinterpret_cast<const uint4*>(vsrc + oa);
  const uint4 kb = *reinterpret_cast<const uint4*>(ksrc + ob);
  const uint4 vb = *reinterpret_cast<const uint4*>(vsrc + ob);
  // this thread's request (if any), read before the barrier below
  long long st = 0;
  int L = 0, o = 0;
  if (tid < num_seqs) {
    st = q_starts[tid];
    L = seq_lens[tid];
    o = q_offsets[tid];
  }
  if (tid < kRowsPerWg) s_owner[tid] = 0ull;
  __syncthreads();
  if (tid < num_seqs) {
    const int n = L - o;
    if (o >= 0 && n > 0) {
      const long long lo = st > x0 ? st : x0;
      const long long hi = st + n < x0 + rows ? st + n : x0 + rows;
      for (long long x = lo; x < hi; ++x)
        atomicMax(&s_owner[x - x0], ((unsigned long long)(tid + 1) << 32) | (unsigned)(o + (int)(x - st)));
    }
  }
  __syncthreads();

  const int head_chunks = a.head_bytes / 16;
  unsigned char* __restrict__ kp = reinterpret_cast<unsigned char*>(a.k_pool);
  unsigned char* __restrict__ vp = reinterpret_cast<unsigned char*>(a.v_pool);
  const size_t block_bytes = (size_t)kPageSize * a.head_bytes;
  // chunk x of the group into its slot, if a request owns its row and the
  // page id is inside the pool
  auto put = [&](int x, const uint4& kv, const uint4& vv) __attribute__((always_inline)) {
    const int i = x / row_chunks;
    const int w = x % row_chunks;
    const unsigned long long own = s_owner[i];
    if (own == 0ull) return;   // no request owns the row
    const int r = (int)(own >> 32) - 1;
    const int pos = (int)(own & 0xFFFFFFFFull);
    const int pg = pos / kPageSize;
    if (pg >= a.max_pages_per_seq) return;
    const int id = a.page_table[(size_t)r * a.max_pages_per_seq + pg];
    if (id < 0 || id >= a.num_pages) return;
    const int h = w / head_chunks;
    const int c = w % head_chunks;
    const size_t dst = ((size_t)id * a.num_kv_heads + h) * block_bytes +
                       (size_t)(pos % kPageSize) * a.head_bytes + (size_t)c * 16;
    *reinterpret_cast<uint4*>(kp + dst) = kv;
    *reinterpret_cast<uint4*>(vp + dst) = vv;
  };
  if (xa < n_chunks) put(xa, ka, va);
  if (xb < n_chunks) put(xb, kb, vb);
  // wider rows: the rest, unrolled so that several independent page-id ->
  // load -> store chains are in flight per thread
#pragma unroll 4
  for (int x = tid + 2 * kThreads; x < n_chunks; x += kThreads)
    put(x, *reinterpret_cast<const uint4*>(ksrc + (size_t)x * 16),
        *reinterpret_cast<const uint4*>(vsrc + (size_t)x * 16));
}

// Copy whole pages (every KV head, K and V) from src[i] to dst[i]: the device
// half of a copy on write, when a request about to write into a shared page
// takes a private copy of it first.  One workgroup per (pair, slice of the
// page); pairs naming a page outside [0, num_pages) are skipped.
__global__ void __launch_bounds__(kThreads) copy_pages_kernel(CopyPagesArgs a) {
  const int i = blockIdx.x / a.slices;
  const int slice = blockIdx.x % a.slices;
  const int src = a.src[i];
  const int dst = a.dst[i];
  if (src < 0 || src >= a.num_pages || dst < 0 || dst >= a.num_pages || src == dst) return;
  const size_t chunks = a.page_bytes / 16;
  const size_t per_slice = (chunks + a.slices - 1) / a.slices;
  const size_t c0 = (size_t)slice * per_slice;
  const size_t c1 = c0 + per_slice < chunks ? c0 + per_slice : chunks;
  const uint4* __restrict__ ks = reinterpret_cast<const uint4*>(reinterpret_cast<const unsigned char*>(a.k_pool) + (size_t)src * a.page_bytes);
  const uint4* __restrict__ vs = reinterpret_cast<const uint4*>(reinterpret_cast<const unsigned char*>(a.v_pool) + (size_t)src * a.page_bytes);
  uint4* __restrict__ kd = reinterpret_cast<uint4*>(reinterpret_cast<unsigned char*>(a.k_pool) + (size_t)dst * a.page_bytes);
  uint4* __restrict__ vd = reinterpret_cast<uint4*>(reinterpret_cast<unsigned char*>(a.v_pool) + (size_t)dst * a.page_bytes);
#pragma unroll 4
  for (size_t c = c0 + threadIdx.x; c < c1; c += kThreads) {
    kd[c] = ks[c];
    vd[c] = vs[c];
  }
}

}  // namespace

int append_rows_per_wg() { return kRowsPerWg; }

hipError_t launch_copy_pages(const CopyPagesArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  if (a.page_bytes % 16 != 0 || a.slices < 1) return hipErrorInvalidValue;
  const long long grid = (long long)a.n * a.slices;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_pages_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  if (a.head_bytes % 16 != 0) return hipErrorInvalidValue;
  if (a.q_starts != nullptr && a.num_seqs <= kThreads) {
    const long long grid = (a.total_rows + kRowsPerWg - 1) / kRowsPerWg;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(append_flat_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s,
                       reinterpret_cast<const unsigned char*>(a.k_new),
                       reinterpret_cast<const unsigned char*>(a.v_new), a.q_starts, a.seq_lens,
                       a.q_offsets, a.num_seqs, a.num_kv_heads * a.head_bytes,
                       (long long)a.total_rows, a);
    return hipGetLastError();
  }
  const long long grid = (long long)a.num_seqs * a.tiles_per_seq;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
