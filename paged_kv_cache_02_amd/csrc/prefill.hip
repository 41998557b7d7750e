// Chunked-prefill attention over the paged KV cache with bf16 MFMA (gfx950).
//
// Request r contributes n_r query rows at absolute positions q_offsets[r] ..
// seq_lens[r]-1 (a bounded chunk of a prompt whose earlier part is already in
// the cache: the chunked-prefill item of the tiny-llm source reading); row i
// sees keys 0 .. q_offsets[r] + i (causal), read through the request's page
// table (its "Paged KV Cache" section), with online softmax so no score
// matrix is stored.  The G query heads of a KV head are packed token-major:
// packed row rho = token * G + h, so one K/V tile serves all of them (GQA).
//
// Workgroup = 4 waves = one tile of 128 packed rows of one (request, KV
// head); each wave owns 32 rows.  Keys stream in tiles of 64 (4 pages):
//   * K tile staged row-major in LDS, V tile staged transposed (V^T, dims x
//     keys), both double-buffered, loaded into registers one tile ahead;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: A = K rows from LDS, B = Q
//     held in registers, so every lane ends up owning one query row and 16 of
//     every 32 keys -- the row max/sum need one exchange with lane ^ 32;
//   * causal mask by select on the diagonal tiles only; lazy online-softmax
//     rescale (only when the max grows by more than 2^8);
//   * P is rounded to bf16 and O^T += V^T P^T with the same MFMA, so the
//     output accumulator also has one row per lane and the rescale stays
//     lane-local.
// The P^T operand comes straight out of the S^T accumulator registers; the
// key order that implies (within each 16 keys, quads 0 and 2 on the low lane
// half, 1 and 3 on the high half) is baked into the V^T tile when it is
// written to LDS, so every MFMA operand read from LDS is one 16-byte load.
//
// Keys at or past seq_len (page tails, possibly NaN) are zeroed while
// staging, and their scores are masked, so they cannot reach the output;
// page-table entries past the last needed page are never read.
#include "pa_internal.h"

#include <math.h>

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kTileRows = kWaves * kRowsPerWave;  // packed (token, head) rows per workgroup
constexpr int kTileKeys = 64;                     // keys per KV tile (4 pages)
constexpr int kPagesPerTile = kTileKeys / kPageSize;
constexpr float kRescaleLog2 = 8.0f;
constexpr float kLn2 = 0.693147180559945309f;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

template <int D>
struct Lds {
  static constexpr int kKStride = D + 8;           // bf16 per K row (16-byte pad)
  static constexpr int kVStride = kTileKeys + 8;   // bf16 per V^T row (16-byte pad)
  static constexpr int kKElems = kTileKeys * kKStride;
  static constexpr int kVElems = D * kVStride;
  static constexpr int kBufElems = kKElems + kVElems;
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8_t, u); }

// Quad permutation applied to V^T columns (see the file comment): within a
// group of 16 keys, quad q sits at position swap12(q).
__device__ __forceinline__ int swap12(int q) { return (q == 1) ? 2 : (q == 2 ? 1 : q); }

template <int D>
struct Staging {
  static_assert(D == 64 || D == 128, "staging layout is written for head_dim 64 or 128");
  static constexpr int kKChunks = kTileKeys * D / 8 / kThreads;  // 16-byte K chunks per thread
  // V: thread (kq = lane % 16, c8 = lane / 16 + 4 * wave) holds keys 4kq..4kq+3
  // of the tile at dims 8c8..8c8+7; threads with c8 >= D/8 stage nothing
  uint4 k[kKChunks];
  uint4 v[4];
};

// Page ids.  At kernel start the workgroup copies the page-table entries
// it needs (clamped into the pool) into LDS, so a tile's 4 page ids are LDS
// broadcast reads (short, lgkmcnt-tracked) instead of global round trips.
// A request whose needed pages exceed the LDS copy reads the page table
// directly (a slower path with the same results).
constexpr int kLdsPages = 2048;

struct PageIds {
  const int* lds;                  // LDS copy, or null
  const int32_t* __restrict__ ptab;
  int npages;                      // pages the workgroup needs
  int num_pages;                   // pool size
};

// Id of page m (uniform) of KV tile kt, or -1 past the needed pages.
__device__ __forceinline__ int tile_page(const PageIds& pi, int kt, int m) {
  const int lp = kt * kPagesPerTile + m;
  if (lp >= pi.npages) return -1;
  int id;
  if (pi.lds != nullptr) {
    id = pi.lds[lp];
  } else {
    id = pi.ptab[lp];
    id = id < 0 ? 0 : (id >= pi.num_pages ? pi.num_pages - 1 : id);
  }
  return __builtin_amdgcn_readfirstlane(id);
}

// Global -> registers for one KV tile kt (first key kb).  K: 16-byte chunk m
// of thread tid is key m * (256 / (D/8)) + tid / (D/8) of the tile, so the
// page of each load is uniform per wave; V: wave w stages page w (4 key
// quads x D/8 dim chunks).  When the whole tile is live the loads are plain;
// otherwise every load still comes from a valid address (page 0 stands in
// for a missing page) and dead keys (>= L, or on a missing page) are
// selected to zero.
template <int D>
__device__ __forceinline__ void stage_load(Staging<D>& st, const __bf16* __restrict__ kpool,
                                           const __bf16* __restrict__ vpool, const PageIds& pi,
                                           int kt, int L, int Hkv, int g, int tid, int wave) {
  const size_t blk = (size_t)kPageSize * D;
  const int kb = kt * kTileKeys;
  const int id0 = tile_page(pi, kt, 0);
  const int id1 = tile_page(pi, kt, 1);
  const int id2 = tile_page(pi, kt, 2);
  const int last_id = tile_page(pi, kt, kPagesPerTile - 1);
  const bool full = kb + kTileKeys <= L && last_id >= 0;
  constexpr int kRowChunks = D / 8;                        // 16-byte chunks per key row
  constexpr int kKeysPerPass = kThreads / kRowChunks;      // keys one pass of 256 threads covers
  constexpr int kWavesPerPage = kPageSize / (64 / kRowChunks);
#pragma unroll
  for (int m = 0; m < Staging<D>::kKChunks; ++m) {
    const int key = m * kKeysPerPass + tid / kRowChunks;   // key within the tile
    const int pm = (m * kKeysPerPass) / kPageSize + wave / kWavesPerPage;  // uniform per wave
    const int id = pm == 0 ? id0 : (pm == 1 ? id1 : (pm == 2 ? id2 : last_id));
    const int phys = id >= 0 ? id : 0;
    const __bf16* src = kpool + ((size_t)phys * Hkv + g) * blk + (key % kPageSize) * D +
                        (tid % kRowChunks) * 8;
    const uint4 val = *reinterpret_cast<const uint4*>(src);
    st.k[m] = (full || (id >= 0 && kb + key < L)) ? val : make_uint4(0, 0, 0, 0);
  }
  {
    const int lane = tid & 63;
    const int kq = lane % 16;
    const int c8raw = lane / 16 + 4 * wave;
    const bool active = c8raw < D / 8;
    const int c8 = active ? c8raw : 0;
    const int pm = kq / 4;  // page of this key quad within the tile
    const int id = pm == 0 ? id0 : (pm == 1 ? id1 : (pm == 2 ? id2 : last_id));
    const int phys = id >= 0 ? id : 0;
    const __bf16* base = vpool + ((size_t)phys * Hkv + g) * blk + ((4 * kq) % kPageSize) * D + c8 * 8;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 val = *reinterpret_cast<const uint4*>(base + j * D);
      const int key = kb + 4 * kq + j;
      st.v[j] = (full || (id >= 0 && key < L)) && active ? val : make_uint4(0, 0, 0, 0);
    }
  }
}

// Registers -> LDS buffer: K row-major, V transposed with the quad order of
// the P^T operand.
template <int D>
__device__ __forceinline__ void stage_store(const Staging<D>& st, __bf16* kbuf, __bf16* vbuf,
                                            int tid) {
  constexpr int kRowChunks = D / 8;
  constexpr int kKeysPerPass = kThreads / kRowChunks;
#pragma unroll
  for (int m = 0; m < Staging<D>::kKChunks; ++m) {
    const int key = m * kKeysPerPass + tid / kRowChunks;
    *reinterpret_cast<uint4*>(kbuf + key * Lds<D>::kKStride + (tid % kRowChunks) * 8) = st.k[m];
  }
  {
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int kq = lane % 16;             // key quad within the tile
    const int c8 = lane / 16 + 4 * wave;  // 8-dim chunk
    if (c8 < D / 8) {
      const int col = 16 * (kq / 4) + 4 * swap12(kq % 4);
      const uint32_t* k0 = reinterpret_cast<const uint32_t*>(&st.v[0]);
      const uint32_t* k1 = reinterpret_cast<const uint32_t*>(&st.v[1]);
      const uint32_t* k2 = reinterpret_cast<const uint32_t*>(&st.v[2]);
      const uint32_t* k3 = reinterpret_cast<const uint32_t*>(&st.v[3]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {   // dword w holds dims 2w (low half) and 2w+1 (high half)
        uint2 lo, hi;
        lo.x = (k0[w] & 0xFFFFu) | (k1[w] << 16);
        lo.y = (k2[w] & 0xFFFFu) | (k3[w] << 16);
        hi.x = (k0[w] >> 16) | (k1[w] & 0xFFFF0000u);
        hi.y = (k2[w] >> 16) | (k3[w] & 0xFFFF0000u);
        const int d0 = c8 * 8 + 2 * w;
        *reinterpret_cast<uint2*>(vbuf + d0 * Lds<D>::kVStride + col) = lo;
        *reinterpret_cast<uint2*>(vbuf + (d0 + 1) * Lds<D>::kVStride + col) = hi;
      }
    }
  }
}

template <int D>
__global__ void __launch_bounds__(kThreads, 2) prefill_kernel(PrefillArgs a, int group) {
  constexpr int kKSteps = D / 16;     // MFMA k-steps over the head dim
  constexpr int kDimBlocks = D / 32;  // 32-dim output blocks
  __shared__ __align__(16) __bf16 smem[2 * Lds<D>::kBufElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;     // which 8-element k slice this lane feeds
  const int lrow = lane & 31;     // the query row this lane owns

  const int Hkv = a.num_kv_heads;
  const int T = a.tiles_per_seq;
  // heavy work first: later tiles of a request see more keys; the KV head is
  // the fastest-varying index so a (request, head) pair's tiles share an XCD
  // when Hkv is a multiple of the XCD count
  const int bid = blockIdx.x;
  const int g = bid % Hkv;
  const int rt = bid / Hkv;
  const int t = T - 1 - (rt % T);
  const int r = a.num_seqs - 1 - rt / T;

  const int L = a.seq_lens[r];
  const int o = a.q_offsets[r];
  const int n = L - o;
  const int rows_total = n * group;
  const int row_base = t * kTileRows;
  if (n <= 0 || row_base >= rows_total) return;

  // first packed query row of this request
  int q_start;
  if (a.q_starts != nullptr) {
    q_start = a.q_starts[r];
  } else {
    int acc = 0;
    for (int i = lane; i < r; i += 64) acc += a.seq_lens[i] - a.q_offsets[i];
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) acc += __shfl_xor(acc, s);
    q_start = acc;
  }

  // keys the workgroup needs: up to the position of its last row
  const int last_row = min(row_base + kTileRows, rows_total) - 1;
  const int kmax = o + last_row / group + 1;
  const int npages = (kmax + kPageSize - 1) / kPageSize;
  const int ntiles = (kmax + kTileKeys - 1) / kTileKeys;

  // this lane's query row
  const int rho = row_base + wave * kRowsPerWave + lrow;
  const bool row_valid = rho < rows_total;
  const int rho_c = row_valid ? rho : rows_total - 1;
  const int tok = rho_c / group;
  const int hh = rho_c % group;
  const int pos = o + tok;
  // the wave's rows span positions [pos_lo, pos_hi]
  const int wrow0 = min(row_base + wave * kRowsPerWave, rows_total - 1);
  const int wrow1 = min(row_base + wave * kRowsPerWave + kRowsPerWave, rows_total) - 1;
  const int pos_lo = o + wrow0 / group;
  const int pos_hi = o + wrow1 / group;

  const int Hq = a.num_q_heads;
  const __bf16* __restrict__ qp = reinterpret_cast<const __bf16*>(a.q);
  const __bf16* qrow = qp + ((size_t)(q_start + tok) * Hq + (size_t)g * group + hh) * D;
  uint4 qv[kKSteps];
#pragma unroll
  for (int s = 0; s < kKSteps; ++s)
    qv[s] = *reinterpret_cast<const uint4*>(qrow + 16 * s + 8 * half);

  const __bf16* __restrict__ kpool = reinterpret_cast<const __bf16*>(a.k_pool);
  const __bf16* __restrict__ vpool = reinterpret_cast<const __bf16*>(a.v_pool);
  const int32_t* __restrict__ ptab = a.page_table + (size_t)r * a.max_pages_per_seq;
  const int npages_c = min(npages, a.max_pages_per_seq);

  floatx16_t oacc[kDimBlocks];
#pragma unroll
  for (int db = 0; db < kDimBlocks; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float sl2 = a.scale_log2;

  // one KV tile: S^T, mask, online softmax, O^T += V^T P^T (reads LDS only)
  auto compute_tile = [&](const __bf16* kbuf, int kb) {
    const __bf16* vbuf = kbuf + Lds<D>::kKElems;
    if (kb <= pos_hi) {  // some key of the tile is visible to some row of this wave
      // ---- S^T = K Q^T over two 32-key blocks ----
      floatx16_t sacc[2];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const __bf16* krow = kbuf + (kb2 * 32 + lrow) * Lds<D>::kKStride + 8 * half;
        const floatx16_t zero = {};
        sacc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            as_bf16x8(*reinterpret_cast<const uint4*>(krow)), as_bf16x8(qv[0]), zero, 0, 0, 0);
#pragma unroll
        for (int s = 1; s < kKSteps; ++s) {
          const uint4 kv = *reinterpret_cast<const uint4*>(krow + 16 * s);
          sacc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kv), as_bf16x8(qv[s]),
                                                              sacc[kb2], 0, 0, 0);
        }
      }
      // ---- causal mask (diagonal tiles only), tile max on raw scores ----
      if (kb + kTileKeys - 1 > pos_lo) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kb + kb2 * 32 + 8 * (i / 4) + 4 * half + (i % 4);
            sacc[kb2][i] = key <= pos ? sacc[kb2][i] : -INFINITY;
          }
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sacc[kb2][i]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32)) * sl2;   // scale > 0 commutes with max
      // ---- lazy online-softmax rescale (m_run is in scaled log2 units) ----
      const bool need = tmax > m_run + kRescaleLog2;
      if (__builtin_expect(__any(need), 0)) {
        const float mn = fmaxf(m_run, tmax);
        const float alpha = (mn == m_run) ? 1.f : fast_exp2(m_run - mn);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < kDimBlocks; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        m_run = mn;
      }
      // ---- probabilities p = exp2(s * scale_log2 - m), packed to bf16 as P^T ----
      // m_run is finite here: key 0 is visible to every row, so the first
      // tile sets it; masked scores are -inf and exp2(-inf) = 0.
      uint32_t pk[2][8];
      float lsum = 0.f;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float p0 = fast_exp2(fmaf(sacc[kb2][i], sl2, -m_run));
          const float p1 = fast_exp2(fmaf(sacc[kb2][i + 1], sl2, -m_run));
          lsum += p0 + p1;
          pk[kb2][i / 2] = pack_bf16x2(p0, p1);
        }
      }
      l_run += lsum;
      // ---- O^T += V^T P^T: 4 k-steps of 16 keys ----
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kb2 = ks / 2;
        const int th = ks % 2;
        uint4 pb;
        pb.x = pk[kb2][4 * th + 0];
        pb.y = pk[kb2][4 * th + 1];
        pb.z = pk[kb2][4 * th + 2];
        pb.w = pk[kb2][4 * th + 3];
        const __bf16* vcol = vbuf + 32 * kb2 + 16 * th + 8 * half;
#pragma unroll
        for (int db = 0; db < kDimBlocks; ++db) {
          const uint4 va = *reinterpret_cast<const uint4*>(vcol + (db * 32 + lrow) * Lds<D>::kVStride);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va), as_bf16x8(pb), oacc[db],
                                                             0, 0, 0);
        }
      }
    }
  };

  // Software pipeline over KV tiles, two tiles of loads in flight: while
  // tile kt is computed out of one LDS buffer, tile kt+1 sits in one set of
  // staging registers (loaded during the previous step) and tile kt+2 is
  // being loaded into the other.  Prefetch loads past the last tile read a
  // valid stand-in page and are never stored.  Unrolled by two so that the
  // staging register sets and LDS buffers are indexed statically.
  __shared__ int s_pages[kLdsPages];
  PageIds pi;
  pi.ptab = ptab;
  pi.npages = npages_c;
  pi.num_pages = a.num_pages;
  pi.lds = nullptr;
  if (npages_c <= kLdsPages) {
    for (int i = tid; i < npages_c; i += kThreads) {
      int id = ptab[i];
      s_pages[i] = id < 0 ? 0 : (id >= a.num_pages ? a.num_pages - 1 : id);
    }
    pi.lds = s_pages;
    __syncthreads();
  }
  Staging<D> sA, sB;
  stage_load<D>(sA, kpool, vpool, pi, 0, L, Hkv, g, tid, wave);
  stage_load<D>(sB, kpool, vpool, pi, 1, L, Hkv, g, tid, wave);
  __bf16* buf0 = smem;
  __bf16* buf1 = smem + Lds<D>::kBufElems;
  stage_store<D>(sA, buf0, buf0 + Lds<D>::kKElems, tid);
  __syncthreads();

  for (int kt = 0;;) {
    // even step: tile kt in buf0, tile kt+1 in sB, tile kt+2 -> sA
    stage_load<D>(sA, kpool, vpool, pi, kt + 2, L, Hkv, g, tid, wave);
    compute_tile(buf0, kt * kTileKeys);
    if (kt + 1 < ntiles) stage_store<D>(sB, buf1, buf1 + Lds<D>::kKElems, tid);
    __syncthreads();
    if (++kt >= ntiles) break;
    // odd step: tile kt in buf1, tile kt+1 in sA, tile kt+2 -> sB
    stage_load<D>(sB, kpool, vpool, pi, kt + 2, L, Hkv, g, tid, wave);
    compute_tile(buf1, kt * kTileKeys);
    if (kt + 1 < ntiles) stage_store<D>(sA, buf0, buf0 + Lds<D>::kKElems, tid);
    __syncthreads();
    if (++kt >= ntiles) break;
  }

  // ---- normalize and write ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (row_valid) {
    const float inv = 1.f / l_tot;
    __bf16* orow = reinterpret_cast<__bf16*>(a.out) + ((size_t)(q_start + tok) * Hq + (size_t)g * group + hh) * D;
#pragma unroll
    for (int db = 0; db < kDimBlocks; ++db) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        uint2 w;
        w.x = pack_bf16x2(oacc[db][4 * v + 0] * inv, oacc[db][4 * v + 1] * inv);
        w.y = pack_bf16x2(oacc[db][4 * v + 2] * inv, oacc[db][4 * v + 3] * inv);
        *reinterpret_cast<uint2*>(orow + db * 32 + 8 * v + 4 * half) = w;
      }
    }
    if (a.lse != nullptr && half == 0)
      a.lse[(size_t)(q_start + tok) * Hq + (size_t)g * group + hh] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, int group, hipStream_t s) {
  const long long grid = (long long)a.num_seqs * a.tiles_per_seq * a.num_kv_heads;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prefill_kernel<D>, dim3((unsigned)grid), dim3(kThreads), 0, s, a, group);
  return hipGetLastError();
}

}  // namespace

int prefill_tile_rows(int head_dim) {
  (void)head_dim;
  return kTileRows;
}

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int group, hipStream_t s) {
  if (group < 1 || group > 16) return hipErrorNotSupported;
  if (head_dim == 128) return launch_d<128>(a, group, s);
  if (head_dim == 64) return launch_d<64>(a, group, s);
  return hipErrorNotSupported;
}

}  // namespace pa
