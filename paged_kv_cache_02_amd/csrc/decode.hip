// Paged decode attention and its split-K partitions (gfx950).
//
// Kernels: decode_kernel / decode_split_mfma_kernel (one workgroup per
// (request, KV head, split): VALU for fp32, MFMA for bf16) and
// decode_balanced_kernel / decode_mfma_kernel (the page-balanced split: VALU
// for fp32, MFMA for bf16).
//
// One workgroup owns one (request, KV head, split) triple, so the G query
// heads of a GQA group share every K/V page load (GQA: week-1 material of the
// tiny-llm source reading; one kernel that walks the page table and runs
// online softmax: its "Paged KV Cache" section).  The page range of the
// split is dealt round-robin to the workgroup's 4 waves; each wave keeps its
// own online-softmax state and the states are merged at the end by the
// log-sum-exp rule (the same rule the split-K merge pass applies across
// workgroups; Flash-Decoding, adv04 of the mini-vllm-tutorial advanced
// series).
//
// The lane layout, the pipelined block loads and the per-page online-softmax
// update are in decode_core.h.
#include "decode_core.h"

#include <math.h>

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
using namespace dec;

// One workgroup per (request, KV head, split); the split's pages are dealt
// to the 4 waves.  kDense: over a dense cache [B, Hkv, MP * P, d] instead of
// the pool (a.max_pages_per_seq = capacity in pages).
template <typename T, int D, int G, bool kDense>
__global__ void __launch_bounds__(kThreads)
decode_kernel(DecodeArgs a) {
  const int nsplit = a.num_splits;
  const int bid = blockIdx.x;
  // the KV heads of one (request, split) are adjacent workgroups: they read
  // neighbouring blocks of the same pages at about the same time
  const int g = bid % a.num_kv_heads;
  const int rs = bid / a.num_kv_heads;
  const int split = rs % nsplit;
  const int r = rs / nsplit;
  const int L = a.seq_lens[r];
  int npages = (L + kPageSize - 1) / kPageSize;
  npages = npages < a.max_pages_per_seq ? npages : a.max_pages_per_seq;
  const int pps = (npages + nsplit - 1) / nsplit;
  const int pb = split * pps;
  const int pe = (pb + pps) < npages ? (pb + pps) : npages;
  decode_range<T, D, G, kWaves, kDense>(a, r, r, g, split, pb, pe, L);
}


// ---------------------------------------------------------------------------
// Page-balanced split-K decode.
//
// The pages of all requests, taken in (request, page) order, form one
// sequence per KV head; it is cut into V equal contiguous wave ranges and
// every wave of the grid owns one range of one KV head, so all waves carry
// the same load whatever the mix of context lengths, and the grid is a
// single round of resident workgroups.  A wave's range can end inside a
// request and can span several requests: at every request boundary (and at
// the range end) the wave writes its normalized partial output and lse for
// that request, and the merge pass combines the partials of each request by
// the log-sum-exp rule (the same combine as split-K; Flash-Decoding, adv04
// of the mini-vllm-tutorial advanced series).
//
// Partial slots: along a KV head's sequence both the request index r and the
// wave-range index v only grow, and one of them grows at every change of the
// pair (r, v), so slot r + v is unique per pair; B + V - 1 slots suffice.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int pages_of(int L, int max_pages) {
  if (L <= 0) return 0;
  const int p = (L + kPageSize - 1) / kPageSize;
  return p < max_pages ? p : max_pages;
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// pre[r] = pages of requests 0 .. r-1 for r in [0, B] (whole workgroup; ends
// with a barrier).
__device__ void page_prefix(int* pre, const int32_t* __restrict__ seq_lens, int B, int max_pages) {
  __shared__ int wave_tot[kWaves];
  const int t = threadIdx.x;
  const int per = (B + kThreads - 1) / kThreads;
  const int r0 = t * per;
  int local = 0;
  for (int k = 0; k < per; ++k)
    if (r0 + k < B) local += pages_of(seq_lens[r0 + k], max_pages);
  int x = local;  // inclusive scan over the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if ((t & 63) >= o) x += y;
  }
  if ((t & 63) == 63) wave_tot[t >> 6] = x;
  __syncthreads();
  int run = x - local;
  for (int w = 0; w < (t >> 6); ++w) run += wave_tot[w];
  if (t == 0) pre[0] = 0;
  for (int k = 0; k < per; ++k) {
    if (r0 + k < B) {
      run += pages_of(seq_lens[r0 + k], max_pages);
      pre[r0 + k + 1] = run;
    }
  }
  __syncthreads();
}

// Small batches (B <= kWaveSeqs): every wave computes the prefix on its own,
// one request per lane, into its own row of `pre` (kWaveSeqs + 1 ints per
// wave) and reads it back itself, so no workgroup barrier and no exchange
// between waves is needed.  The scan is the usual wave-64 one: inclusive
// within rows of 16 lanes by DPP row shifts, then carried across rows by the
// row-15 and row-31 broadcasts.  Returns the wave's row.
constexpr int kWaveSeqs = 64;
__device__ int* page_prefix_wave(int* pre, const int32_t* __restrict__ seq_lens, int B, int max_pages,
                                 int wave, int lane, int& excl) {
  int* row = pre + wave * (kWaveSeqs + 1);
  const int np = lane < B ? pages_of(seq_lens[lane], max_pages) : 0;
  int x = np;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
  if (lane == 0) row[0] = 0;
  if (lane < B) row[lane + 1] = x;
  __builtin_amdgcn_wave_barrier();
  excl = x - np;   // pre[lane]
  return row;
}

// The request holding page f0: the largest r < B with pre[r] <= f0 (pre is
// non-decreasing and pre[0] = 0).  Small batches count it from the lanes'
// exclusive prefixes with one ballot; others search the LDS prefix.
__device__ __forceinline__ int request_of_page(const int* pre, int B, int f0, bool small, int excl,
                                               int lane) {
  if (small) return __popcll(__ballot(lane >= 1 && lane < B && excl <= f0));
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (uniform(pre[mid]) <= f0) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// The metadata and the partial outputs come as separate restrict parameters:
// with them the compiler can prove that the kernel's own stores never touch
// the page table, and reads page ids with scalar loads (a vector load there
// would make each wait for a page id also wait for every K/V load in flight).
// They and the sizes the prologue needs first lead the argument list, ahead
// of the struct (whose fields of the same names they equal), so that the
// library's build (kernarg preloading) hands them to the wave in SGPRs at
// launch and the first length read waits on no load of the kernel arguments.
template <typename T, int D, int G>
__global__ void __launch_bounds__(kThreads)
decode_balanced_kernel(const int32_t* __restrict__ seq_lens, int B, int maxp, int Hkv, int V,
                       const int32_t* __restrict__ page_table, float* __restrict__ o_part,
                       float* __restrict__ lse_part, int32_t* __restrict__ range_meta, DecodeArgs a) {
  using S = Shape<T, D, G>;
  // the prefetched q of the next request costs one more q register set
  using P = Pipe<T, D, G, G * S::kChunksPerLane * 4>;
  constexpr int kDepth = P::kDepth;
  constexpr int kBufs = P::kBufs;
  __shared__ int pre_lds[kMaxBalancedSeqs + 1];

  const int32_t num_pages = a.num_pages;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int col = lane % S::kLpt;
  const int row0 = lane / S::kLpt;
  const int Hq = a.num_q_heads;
  const int g = blockIdx.x % Hkv;
  const int v = (blockIdx.x / Hkv) * kWaves + wave;

  // pre[r] = pages of requests 0 .. r-1, for r in [0, B]
  int* pre = pre_lds;
  int excl = 0;
  const bool small = B <= kWaveSeqs;
  if (small)
    pre = page_prefix_wave(pre_lds, seq_lens, B, maxp, wave, lane, excl);
  else
    page_prefix(pre_lds, seq_lens, B, maxp);
  const int N = uniform(pre[B]);
  const int per = N > 0 ? (N + V - 1) / V : 1;  // pages per wave range

  // one workgroup records which wave ranges each request spans
  if (blockIdx.x == 0) {
    for (int r = threadIdx.x; r < B; r += kThreads) {
      const int s0 = pre[r], s1 = pre[r + 1];
      range_meta[2 * r] = s0 < s1 ? s0 / per : 0;
      range_meta[2 * r + 1] = s0 < s1 ? (s1 - 1) / per : -1;
    }
  }

  const long long f0l = (long long)v * per;
  if (f0l >= N) return;
  const int f0 = (int)f0l;
  const int nw = (f0 + per < N ? f0 + per : N) - f0;  // pages of this wave, >= 1

  auto npages = [&](int r) -> int { return uniform(pre[r + 1]) - uniform(pre[r]); };
  // the first request after r that owns pages (B if none)
  auto next_req = [&](int r) -> int {
    ++r;
    while (r < B && npages(r) == 0) ++r;
    return r;
  };
  auto seq_len = [&](int r) -> int {
    const int L = seq_lens[r];
    return L < maxp * kPageSize ? L : maxp * kPageSize;
  };

  const int lo = uniform(request_of_page(pre, B, f0, small, excl, lane));

  const T* __restrict__ qp = reinterpret_cast<const T*>(a.q);
  const T* __restrict__ kpool = reinterpret_cast<const T*>(a.k_pool);
  const T* __restrict__ vpool = reinterpret_cast<const T*>(a.v_pool);
  const size_t blk = (size_t)kPageSize * D;
  auto block_ptr = [&](const T* pool, int phys) -> const T* {
    return pool + ((size_t)phys * Hkv + g) * blk;
  };

  // load cursor (request rl, page jl of it, its page count nl): the page
  // whose K/V loads are issued next
  int rl = lo, jl = f0 - uniform(pre[lo]), nl = npages(lo);
  auto advance_load = [&]() {
    ++jl;
    while (jl >= nl && rl + 1 < B) {
      ++rl;
      jl = 0;
      nl = npages(rl);
    }
  };
  auto load_id = [&]() -> int {
    int phys = page_table[(size_t)rl * maxp + jl];
    return phys < 0 ? 0 : (phys >= num_pages ? num_pages - 1 : phys);
  };

  // compute cursor
  int rc = lo, jc = f0 - uniform(pre[lo]), nc = npages(lo);
  int Lc = seq_len(rc);

  const int Gr = Hq / Hkv;   // real group size (G: the padded one the registers hold)
  uint4 qv[G][S::kChunksPerLane], qn[G][S::kChunksPerLane];
  load_q<T, D, G>(qv, qp, Hq, rc, g, Gr, true, col);
  int rq = next_req(rc);  // request whose q sits in qn
  load_q<T, D, G>(qn, qp, Hq, rq < B ? rq : B - 1, g, Gr, rq < B && uniform(pre[rq]) < f0 + nw, col);

  WaveState<T, D, G> st;
  reset_state<T, D, G>(st);

  Half<T, D, G> hk[kBufs], hv[kBufs];
#pragma unroll
  for (int u = 0; u < kDepth; ++u) {
    const int phys = load_id();
    load_half<T, D, G>(hk[u], block_ptr(kpool, phys), u < nw, row0, col);
    load_half<T, D, G>(hv[u], block_ptr(vpool, phys), u < nw, row0, col);
    if (u + 1 < nw) advance_load();
  }
  int next_phys = load_id();

  int i = 0;
#pragma unroll 1
  for (;;) {
#pragma unroll
    for (int u = 0; u < kBufs; ++u) {
      const int ahead = i + kDepth;
      const bool more = ahead < nw;
      const int nb = (u + kDepth) % kBufs;  // buffer of page i + kDepth
      const int phys = next_phys;
      load_half<T, D, G>(hk[nb], block_ptr(kpool, phys), more, row0, col);
      if (ahead + 1 < nw) advance_load();
      next_phys = load_id();
      const int live = Lc - jc * kPageSize;  // >= 16 except on a request's last page
      float pr[S::kKeysPerLane][G];
      page_scores<T, D, G>(hk[u], qv, st, live, row0, a.scale_log2, pr);
      load_half<T, D, G>(hv[nb], block_ptr(vpool, phys), more, row0, col);
      page_values<T, D, G>(hv[u], st, live, row0, pr);

      const bool range_end = i + 1 >= nw;
      if (jc + 1 >= nc || range_end) {
        // ---- the wave's share of request rc is complete: write its partial
        wave_combine<T, D, G>(st);
        if (row0 == 0) {
          const size_t slot = (size_t)rc + v;
#pragma unroll
          for (int h = 0; h < G; ++h) {
            if (h >= Gr) break;
            const int hq = g * Gr + h;
            const float l = st.l[h];
            const bool empty = !(l > 0.f);
            const float inv = empty ? 0.f : 1.f / l;
            float* o = o_part + (slot * Hq + hq) * D;
#pragma unroll
            for (int jj = 0; jj < S::kChunksPerLane; ++jj) {
#pragma unroll
              for (int e = 0; e < S::kVec; e += 4) {
                float4 w;
                w.x = st.acc[h][jj * S::kVec + e + 0] * inv;
                w.y = st.acc[h][jj * S::kVec + e + 1] * inv;
                w.z = st.acc[h][jj * S::kVec + e + 2] * inv;
                w.w = st.acc[h][jj * S::kVec + e + 3] * inv;
                *reinterpret_cast<float4*>(o + (col + S::kLpt * jj) * S::kVec + e) = w;
              }
            }
            if (col == 0) lse_part[slot * Hq + hq] = empty ? -INFINITY : (st.m[h] + __log2f(l)) * kLn2;
          }
        }
        if (range_end) return;
        reset_state<T, D, G>(st);
        // ---- move on to the next request of the range
        rc = rq;
        jc = 0;
        nc = npages(rc);
        Lc = seq_len(rc);
        // The copy must complete before the next q load is issued, so that the
        // load can land in the registers qn already occupies (a load into
        // temporaries followed by a copy would wait for every load in flight):
        // the empty asm reads the copied registers and orders memory.
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
          for (int jj = 0; jj < S::kChunksPerLane; ++jj) {
            qv[h][jj] = qn[h][jj];
            asm volatile("" : "+v"(qv[h][jj].x), "+v"(qv[h][jj].y), "+v"(qv[h][jj].z),
                         "+v"(qv[h][jj].w)::"memory");
          }
        }
        rq = next_req(rc);
        load_q<T, D, G>(qn, qp, Hq, rq < B ? rq : B - 1, g, Gr, rq < B && uniform(pre[rq]) < f0 + nw,
                        col);
      } else {
        ++jc;
      }
      ++i;
    }
  }
}

// ---------------------------------------------------------------------------
// Page-balanced decode with both contractions on MFMA (bf16).
//
// Same ranges, partial slots and merge as decode_balanced_kernel; only the
// work per (page, KV head) block differs.  With the VALU form above, the
// dot products, their DPP reductions and the p * V FMAs (about 350 VALU
// instructions per page and wave) hold the memory stream back; here one
// page costs D/32 + 2 D/16 MFMAs and a few dozen VALU instructions:
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: A = the page's 16 keys (lane
//     j holds key j%16, dims 32c + 8(j/16) .. +7 of k-step c: one 16-byte
//     load each), B = Q^T with the G query heads in columns 0..G-1 (the other
//     columns read zeros);
//   * the result holds, in lane j, keys 4(j/16) .. +3 of head j%16, which is
//     the A operand layout of O += P V with v_mfma_f32_16x16x16bf16_1k, so
//     the probabilities go from the softmax straight into the MFMA (as a
//     bf16 high part and a bf16 remainder, two MFMAs, so that the products
//     keep about 16 bits);
//   * V's B operand (4 consecutive keys of one dim per lane) comes from the
//     wave's own LDS slot through ds_read_b64_tr_b16: the wave writes its V
//     block there (16-byte chunks XOR-swizzled by key, so both the writes
//     and the transposing reads are free of bank conflicts) and reads it
//     back in the same order, so no barrier is needed;
//   * online softmax per head over the page's 16 keys: the running max is
//     kept per head (replicated in the head's four lanes), the running sum
//     per lane and folded at the request's end.
// Rows 0..G-1 of the 16-row MFMA tiles carry the G query heads; the others
// are padding whose results are never written.
// ---------------------------------------------------------------------------

// The arguments the prologue needs first (the lengths, the batch and pool
// sizes, the page table, the partial outputs) come before the argument
// struct as plain scalars and pointers, so that the library's build
// (kernarg preloading) hands them to the wave in SGPRs at launch: the first
// length read goes out without waiting on a load of the kernel arguments,
// whose other fields arrive while it is in flight.  They equal the struct's
// fields of the same names.
template <int D, int G>
__global__ void __launch_bounds__(kThreads, 2)
decode_mfma_kernel(const int32_t* __restrict__ seq_lens, int B, int maxp, int Hkv, int V,
                   const int32_t* __restrict__ page_table, float* __restrict__ o_part,
                   float* __restrict__ lse_part, int32_t* __restrict__ range_meta, DecodeArgs a) {
  using M = MShape<D>;
  static_assert(G <= 16, "at most 16 query heads per KV head");
  // pages whose K/V loads are in flight ahead of the one computed: with one
  // workgroup per CU at d = 128 (8 KB blocks) one measured as fast as two
  // or three, or 1-2% faster; d = 64 runs two workgroups per CU with three
  constexpr int kDepth = D >= 128 ? 1 : 3;
  constexpr int kBufs = kDepth + 1;
  __shared__ int pre_lds[kMaxBalancedSeqs + 1];
  __shared__ __align__(16) unsigned char vslots[kWaves][kPageSize * M::kRowBytes];

  const int32_t num_pages = a.num_pages;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int Hq = a.num_q_heads;
  const int g = blockIdx.x % Hkv;
  const int v = (blockIdx.x / Hkv) * kWaves + wave;
  unsigned char* vslot = vslots[wave];

  // pre[r] = pages of requests 0 .. r-1, for r in [0, B]
  int* pre = pre_lds;
  int excl = 0;
  const bool small = B <= kWaveSeqs;
  if (small)
    pre = page_prefix_wave(pre_lds, seq_lens, B, maxp, wave, lane, excl);
  else
    page_prefix(pre_lds, seq_lens, B, maxp);
  const int N = uniform(pre[B]);
  const int per = N > 0 ? (N + V - 1) / V : 1;  // pages per wave range

  if (blockIdx.x == 0) {
    for (int r = threadIdx.x; r < B; r += kThreads) {
      const int s0 = pre[r], s1 = pre[r + 1];
      range_meta[2 * r] = s0 < s1 ? s0 / per : 0;
      range_meta[2 * r + 1] = s0 < s1 ? (s1 - 1) / per : -1;
    }
  }

  const long long f0l = (long long)v * per;
  if (f0l >= N) return;
  const int f0 = (int)f0l;
  const int nw = (f0 + per < N ? f0 + per : N) - f0;

  auto npages = [&](int r) -> int { return uniform(pre[r + 1]) - uniform(pre[r]); };
  auto next_req = [&](int r) -> int {
    ++r;
    while (r < B && npages(r) == 0) ++r;
    return r;
  };
  auto seq_len = [&](int r) -> int {
    const int L = seq_lens[r];
    return L < maxp * kPageSize ? L : maxp * kPageSize;
  };
  // request holding page f0
  const int lo = uniform(request_of_page(pre, B, f0, small, excl, lane));

  const __bf16* __restrict__ qp = reinterpret_cast<const __bf16*>(a.q);
  const __bf16* __restrict__ kpool = reinterpret_cast<const __bf16*>(a.k_pool);
  const __bf16* __restrict__ vpool = reinterpret_cast<const __bf16*>(a.v_pool);
  const size_t blk = (size_t)kPageSize * D;
  auto block_ptr = [&](const __bf16* pool, int phys) -> const __bf16* {
    return pool + ((size_t)phys * Hkv + g) * blk;
  };

  int rl = lo, jl = f0 - uniform(pre[lo]), nl = npages(lo);
  auto advance_load = [&]() {
    ++jl;
    while (jl >= nl && rl + 1 < B) {
      ++rl;
      jl = 0;
      nl = npages(rl);
    }
  };
  auto load_id = [&]() -> int {
    int phys = page_table[(size_t)rl * maxp + jl];
    return phys < 0 ? 0 : (phys >= num_pages ? num_pages - 1 : phys);
  };

  int rc = lo, jc = f0 - uniform(pre[lo]), nc = npages(lo);
  int Lc = seq_len(rc);

  const int Gr = Hq / Hkv;   // real group size, at most the G the kernel is built for
  uint4 qv[M::kKSteps], qn[M::kKSteps];
  load_qt<D>(qv, qp, Hq, rc, g, Gr, true, lane);
  int rq = next_req(rc);
  load_qt<D>(qn, qp, Hq, rq < B ? rq : B - 1, g, Gr, rq < B && uniform(pre[rq]) < f0 + nw, lane);

  MState<D> st;
  mreset<D>(st);

  MBlock<D> bufs[kBufs];
#pragma unroll
  for (int u = 0; u < kDepth; ++u) {
    const int phys = load_id();
    load_mblock<D>(bufs[u], block_ptr(kpool, phys), block_ptr(vpool, phys), u < nw, lane);
    if (u + 1 < nw) advance_load();
  }
  int next_phys = load_id();

  int i = 0;
#pragma unroll 1
  for (;;) {
#pragma unroll
    for (int u = 0; u < kBufs; ++u) {
      const int ahead = i + kDepth;
      const bool more = ahead < nw;
      const int nb = (u + kDepth) % kBufs;
      const int phys = next_phys;
      load_mblock<D>(bufs[nb], block_ptr(kpool, phys), block_ptr(vpool, phys), more, lane);
      if (ahead + 1 < nw) advance_load();
      next_phys = load_id();
      const int live = Lc - jc * kPageSize;
      page_mfma<D, G>(bufs[u], qv, st, live, a.scale_log2, vslot, lane, Gr);

      const bool range_end = i + 1 >= nw;
      if (jc + 1 >= nc || range_end) {
        // ---- the wave's share of request rc is complete: write its partial
        const float lh = head_sum<D>(st);       // head lane&15's total
        const size_t slot = (size_t)rc + v;
        const int qg = lane >> 4;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int hh = 4 * qg + ii;            // this lane's output row
          const float l = __shfl(lh, hh);
          const bool empty = !(l > 0.f);
          const float inv = empty ? 0.f : 1.f / l;
          if (hh < Gr) {
            float* o = o_part + (slot * Hq + (size_t)g * Gr + hh) * D + (lane & 15);
#pragma unroll
            for (int bb = 0; bb < M::kDimBlocks; ++bb) o[16 * bb] = st.o[bb][ii] * inv;
          }
        }
        if (qg == 0 && (lane & 15) < Gr) {
          const bool empty = !(lh > 0.f);
          lse_part[slot * Hq + (size_t)g * Gr + (lane & 15)] = empty ? -INFINITY : (st.m + __log2f(lh)) * kLn2;
        }
        if (range_end) return;
        mreset<D>(st);
        rc = rq;
        jc = 0;
        nc = npages(rc);
        Lc = seq_len(rc);
#pragma unroll
        for (int c = 0; c < M::kKSteps; ++c) {
          qv[c] = qn[c];
          asm volatile("" : "+v"(qv[c].x), "+v"(qv[c].y), "+v"(qv[c].z), "+v"(qv[c].w)::"memory");
        }
        rq = next_req(rc);
        load_qt<D>(qn, qp, Hq, rq < B ? rq : B - 1, g, Gr, rq < B && uniform(pre[rq]) < f0 + nw, lane);
      } else {
        ++jc;
      }
      ++i;
    }
  }
}

template <int D, int G>
hipError_t launch_mfma_t(const DecodeArgs& a, hipStream_t s) {
  const long long grid = (long long)a.num_kv_heads * (a.num_splits / kWaves);
  if (grid <= 0 || a.num_seqs <= 0) return hipSuccess;
  if (grid > 0x7FFFFFFFLL || a.num_splits % kWaves != 0 || a.num_seqs > kMaxBalancedSeqs)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_mfma_kernel<D, G>), dim3((unsigned)grid), dim3(kThreads), 0, s, a.seq_lens,
                     a.num_seqs, a.max_pages_per_seq, a.num_kv_heads, a.num_splits, a.page_table,
                     a.o_part, a.lse_part, a.range_meta, a);
  return hipGetLastError();
}

// The kernels are built for padded group sizes 1, 2, 4, 8 (and 16 on the
// MFMA forms); a group size in between runs the next one up, with the heads
// past the real group masked.
int padded_group(int group) {
  int p = 1;
  while (p < group) p <<= 1;
  return p;
}

template <int D>
hipError_t launch_mfma_g(const DecodeArgs& a, int group, hipStream_t s) {
  switch (padded_group(group)) {
    case 1: return launch_mfma_t<D, 1>(a, s);
    case 2: return launch_mfma_t<D, 2>(a, s);
    case 4: return launch_mfma_t<D, 4>(a, s);
    case 8: return launch_mfma_t<D, 8>(a, s);
    case 16: return launch_mfma_t<D, 16>(a, s);
  }
  return hipErrorInvalidValue;
}

// decode_kernel with the page work on MFMA (bf16).
template <int D, int G, bool kDense>
__global__ void __launch_bounds__(kThreads, 2)
decode_split_mfma_kernel(DecodeArgs a) {
  const int nsplit = a.num_splits;
  const int bid = blockIdx.x;
  const int g = bid % a.num_kv_heads;
  const int rs = bid / a.num_kv_heads;
  const int split = rs % nsplit;
  const int r = rs / nsplit;
  const int L = a.seq_lens[r];
  int npages = (L + kPageSize - 1) / kPageSize;
  npages = npages < a.max_pages_per_seq ? npages : a.max_pages_per_seq;
  const int pps = (npages + nsplit - 1) / nsplit;
  const int pb = split * pps;
  const int pe = (pb + pps) < npages ? (pb + pps) : npages;
  decode_range_mfma<D, G, kDense>(a, r, r, g, split, pb, pe, L);
}

template <typename T, int D, int G, bool kDense>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s) {
  const long long grid = (long long)a.num_seqs * a.num_kv_heads * a.num_splits;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  if constexpr (sizeof(T) == 2)
    hipLaunchKernelGGL((decode_split_mfma_kernel<D, G, kDense>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((decode_kernel<T, D, G, kDense>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D, int G>
hipError_t launch_bal_t(const DecodeArgs& a, hipStream_t s) {
  const long long grid = (long long)a.num_kv_heads * (a.num_splits / kWaves);
  if (grid <= 0 || a.num_seqs <= 0) return hipSuccess;
  if (grid > 0x7FFFFFFFLL || a.num_splits % kWaves != 0 || a.num_seqs > kMaxBalancedSeqs)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_balanced_kernel<T, D, G>), dim3((unsigned)grid), dim3(kThreads), 0, s,
                     a.seq_lens, a.num_seqs, a.max_pages_per_seq, a.num_kv_heads, a.num_splits,
                     a.page_table, a.o_part, a.lse_part, a.range_meta, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_bal_g(const DecodeArgs& a, int group, hipStream_t s) {
  switch (padded_group(group)) {
    case 1: return launch_bal_t<T, D, 1>(a, s);
    case 2: return launch_bal_t<T, D, 2>(a, s);
    case 4: return launch_bal_t<T, D, 4>(a, s);
    case 8: return launch_bal_t<T, D, 8>(a, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D, bool kDense>
hipError_t launch_g(const DecodeArgs& a, int group, hipStream_t s) {
  switch (padded_group(group)) {
    case 1: return launch_t<T, D, 1, kDense>(a, s);
    case 2: return launch_t<T, D, 2, kDense>(a, s);
    case 4: return launch_t<T, D, 4, kDense>(a, s);
    case 8: return launch_t<T, D, 8, kDense>(a, s);
    case 16:
      if constexpr (sizeof(T) == 2) return launch_t<T, D, 16, kDense>(a, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_balanced(const DecodeArgs& a, int dtype, int head_dim, int group,
                                  hipStream_t s) {
  if (dtype == 0) {
    if (head_dim == 128) return launch_mfma_g<128>(a, group, s);
    if (head_dim == 64) return launch_mfma_g<64>(a, group, s);
  } else if (dtype == 1) {
    if (head_dim == 128) return launch_bal_g<float, 128>(a, group, s);
    if (head_dim == 64) return launch_bal_g<float, 64>(a, group, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, int head_dim, int group, hipStream_t s) {
  if (dtype == 0) {
    if (head_dim == 128) return launch_g<__bf16, 128, false>(a, group, s);
    if (head_dim == 64) return launch_g<__bf16, 64, false>(a, group, s);
  } else if (dtype == 1) {
    if (head_dim == 128) return launch_g<float, 128, false>(a, group, s);
    if (head_dim == 64) return launch_g<float, 64, false>(a, group, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_dense(const DecodeArgs& a, int dtype, int head_dim, int group, hipStream_t s) {
  if (a.num_splits != 1 || a.write_partials) return hipErrorInvalidValue;
  if (dtype == 0) {
    if (head_dim == 128) return launch_g<__bf16, 128, true>(a, group, s);
    if (head_dim == 64) return launch_g<__bf16, 64, true>(a, group, s);
  } else if (dtype == 1) {
    if (head_dim == 128) return launch_g<float, 128, true>(a, group, s);
    if (head_dim == 64) return launch_g<float, 64, true>(a, group, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
