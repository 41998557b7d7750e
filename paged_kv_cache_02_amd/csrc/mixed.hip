// Mixed prefill/decode attention in one launch (gfx950).
//
// One continuous-batching round carries requests in both phases at once: the
// model side sees a per-request slot map, so some requests run a prefill
// chunk while others decode (tiny-llm source reading, "Continuous Batching"
// and "Chunked Prefill"), and the attention dispatch guard picks the kernel
// by query length ("Prefill and decode need different kernels").  Here that
// choice is made per work item inside a single launch: request r, with
// n_r = seq_lens[r] - q_offsets[r] query rows, is a decode row when n_r = 1
// and a prefill chunk when n_r > 1.  Every workgroup (8 waves) takes one
// item of one KV head:
//   * a prefill row tile of 128 packed (token, head) rows: the tile body of
//     the chunked-prefill kernel, never split along its keys; or
//   * a whole decode (request, KV head): the request's pages dealt to the 8
//     waves and the wave states merged in LDS (the decode page walk), so no
//     partial leaves the workgroup and no merge pass follows.
//
// Item order.  The grid is laid out KV head fastest (with 8 KV heads, all of
// a head's items land on one XCD, whose L2 then holds that head's prefill
// K/V).  Per head, the prefill tiles and the decode items are interleaved
// in proportion to their counts, each list heaviest first (requests by
// context length, descending; a request's tiles from its last rows, which
// see the most keys, down), so MFMA-bound tiles and HBM-bound decode items
// share the chip from the start and the lightest items of both fill the
// tail.  Every workgroup derives the item lists from seq_lens and q_offsets
// itself (a count and an O(B) rank per request, in LDS), so the launch needs
// no host copy of the lengths and no device work list in memory.
#include "decode_core.h"
#include "prefill_core.h"

namespace pa {
namespace {

constexpr int kThreads = pf::kThreads;   // the prefill tile's 8 waves
constexpr int kWaves = kThreads / 64;
constexpr int kTileRows = pf::kTileRows;

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

template <int G>
__device__ __forceinline__ int tiles_of(int n) {
  return (n * G + kTileRows - 1) / kTileRows;
}

template <int D, int G>
__global__ void __launch_bounds__(kThreads, 1) mixed_kernel(PrefillArgs a) {
  __shared__ int s_len[kMaxMixedSeqs];
  __shared__ int s_rows[kMaxMixedSeqs];
  __shared__ int s_count[2];   // prefill tiles, decode requests (per KV head)
  __shared__ int s_pick[2];    // the item's request and row tile

  const int tid = threadIdx.x;
  const int B = a.num_seqs;
  const int Hkv = a.num_kv_heads;
  const int g = blockIdx.x % Hkv;
  const int k = blockIdx.x / Hkv;   // the item's place in this head's order

  if (tid < 2) s_count[tid] = 0;
  if (tid == 0) s_pick[0] = -1;
  __syncthreads();
  int np = 0, nd = 0;
  for (int r = tid; r < B; r += kThreads) {
    const int L = a.seq_lens[r];
    const int n = L - a.q_offsets[r];
    s_len[r] = L;
    s_rows[r] = n;
    if (n > 1) np += tiles_of<G>(n);
    else if (n == 1) ++nd;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    np += __shfl_xor(np, o);
    nd += __shfl_xor(nd, o);
  }
  if ((tid & 63) == 0) {
    atomicAdd(&s_count[0], np);
    atomicAdd(&s_count[1], nd);
  }
  __syncthreads();
  const int Np = s_count[0];
  const int N = Np + s_count[1];
  if (k >= N) return;

  // interleave: item k is a prefill tile when the count of prefill items
  // among the first k + 1 exceeds that among the first k
  const long long kp = (long long)k * Np;
  const int before = (int)(kp / N);   // prefill items ahead of item k
  const bool prefill = (int)((kp + Np) / N) > before;
  const int idx = prefill ? before : k - before;   // place within its own list

  // The lists order requests by (context length descending, index
  // ascending), a total order, so the requests' item ranges tile each list
  // exactly and one thread finds idx in its request's range.
  for (int r = tid; r < B; r += kThreads) {
    const int n = s_rows[r];
    if (prefill ? n <= 1 : n != 1) continue;
    const int L = s_len[r];
    int ahead = 0;
    for (int r2 = 0; r2 < B; ++r2) {
      const int n2 = s_rows[r2];
      const int L2 = s_len[r2];
      const bool same = prefill ? n2 > 1 : n2 == 1;
      if (same && (L2 > L || (L2 == L && r2 < r))) ahead += prefill ? tiles_of<G>(n2) : 1;
    }
    const int cnt = prefill ? tiles_of<G>(n) : 1;
    if (idx >= ahead && idx < ahead + cnt) {
      s_pick[0] = r;
      s_pick[1] = cnt - 1 - (idx - ahead);   // the heaviest tile first
    }
  }
  __syncthreads();
  const int r = uniform(s_pick[0]);
  if (r < 0) return;

  if (prefill) {
    pf::prefill_tile<D>(a, pf::prefill_hot(a), G, r, uniform(s_pick[1]), g, 0);
    return;
  }

  const int L = uniform(s_len[r]);
  const int qrow = uniform(pf::q_start_of(a, r, tid & 63));
  DecodeArgs d;
  d.q = a.q;
  d.k_pool = a.k_pool;
  d.v_pool = a.v_pool;
  d.page_table = a.page_table;
  d.seq_lens = a.seq_lens;
  d.out = a.out;
  d.lse = a.lse;
  d.o_part = nullptr;
  d.lse_part = nullptr;
  d.range_meta = nullptr;
  d.num_seqs = B;
  d.num_q_heads = a.num_q_heads;
  d.num_kv_heads = Hkv;
  d.max_pages_per_seq = a.max_pages_per_seq;
  d.num_pages = a.num_pages;
  d.num_splits = 1;
  d.write_partials = 0;
  d.scale_log2 = a.scale_log2;
  int npages = (L + kPageSize - 1) / kPageSize;
  npages = npages < a.max_pages_per_seq ? npages : a.max_pages_per_seq;
  dec::decode_range<__bf16, D, G, kWaves, false>(d, r, qrow, g, 0, 0, npages, L);
}

template <int D, int G>
hipError_t launch_dg(const PrefillArgs& a, long long items_per_head, hipStream_t s) {
  const long long grid = items_per_head * a.num_kv_heads;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((mixed_kernel<D, G>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, int group, long long items_per_head, hipStream_t s) {
  switch (group) {
    case 1: return launch_dg<D, 1>(a, items_per_head, s);
    case 2: return launch_dg<D, 2>(a, items_per_head, s);
    case 4: return launch_dg<D, 4>(a, items_per_head, s);
    case 8: return launch_dg<D, 8>(a, items_per_head, s);
  }
  return hipErrorNotSupported;
}

}  // namespace

long long mixed_items_bound(long long total_q, int num_seqs, int group) {
  // prefill tiles: sum over n_r > 1 of ceil(n_r G / 128) <= sum n_r G / 128 +
  // (prefill requests); decode items: one per remaining request
  return (total_q * group + kTileRows - 1) / kTileRows + num_seqs;
}

hipError_t launch_mixed(const PrefillArgs& a, int head_dim, int group, long long items_per_head,
                        hipStream_t s) {
  if (head_dim == 128) return launch_d<128>(a, group, items_per_head, s);
  if (head_dim == 64) return launch_d<64>(a, group, items_per_head, s);
  return hipErrorNotSupported;
}

}  // namespace pa
