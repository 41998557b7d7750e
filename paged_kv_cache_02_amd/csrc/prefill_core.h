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
// Work decomposition.  A workgroup of 8 waves owns a tile of 128 packed rows
// of one (request, KV head): two wave groups of 4 waves each cover the same
// 128 rows (32 per wave) and take the two halves of the tile's key range,
// and at the end group 1 hands its state to group 0 through LDS, which
// merges it lane by lane by the log-sum-exp rule.  When the grid holds fewer
// workgroups than the chip has CUs, a long key range is further cut into
// splits of `kv_tiles_per_split` KV tiles that run as separate workgroups
// and write partial results, combined by a merge pass.
//
// Keys stream in tiles of 64 (4 pages); per wave group and KV tile:
//   * K and V pages are copied straight from HBM into LDS with
//     global_load_lds (no staging registers), double-buffered one tile
//     ahead; K's 16-byte chunks are XOR-swizzled by key and V is stored as
//     [dim block][key] within each 1 KB piece, so the operand reads below
//     are bank-conflict free and every V read is one register plus an
//     immediate offset;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: A = K rows read from LDS,
//     B = Q held in registers, so a lane owns one query row and 16 of every
//     32 keys -- the row max and sum need one exchange with lane ^ 32;
//   * causal mask by select on diagonal tiles only; lazy online-softmax
//     rescale (only when the max grows by more than 2^8); the row max and
//     sum cross the two lane halves with permlane32_swap;
//   * P is rounded to bf16 and O^T += V^T P^T: the V^T operand comes from
//     V's natural [key][dim] layout through ds_read_b64_tr_b16 (gfx950's
//     transposing LDS read), in the key order the P^T registers carry, and
//     the output accumulator keeps one row per lane, so rescaling is local.
//
// Keys at or past a row's position are masked by select before the max.  K
// and V rows of keys at or past seq_len (page tails, possibly NaN) are never
// loaded: their LDS slots are zero-filled, so no NaN meets a zero weight.
// Page-table entries past the pages needed are never read.
#pragma once

#include "pa_internal.h"

#include <math.h>

namespace pa {
namespace pf {

constexpr int kGroups = 2;                        // wave groups splitting a tile's key range
constexpr int kWavesPerGroup = 4;
constexpr int kWaves = kGroups * kWavesPerGroup;
constexpr int kThreads = 64 * kWaves;
constexpr int kRB = 1;                            // 32-row MFMA blocks per wave
constexpr int kRowsPerWave = 32 * kRB;
constexpr int kTileRows = kWavesPerGroup * kRowsPerWave;  // packed (token, head) rows per workgroup
constexpr int kTileKeys = 64;                     // keys per KV tile (4 pages)
constexpr int kPagesPerTile = kTileKeys / kPageSize;
constexpr int kLdsPages = 2048;                   // page ids kept in LDS
constexpr float kRescaleLog2 = 8.0f;
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.4426950408889634f;
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x0008;
constexpr int kSchedDsRead = 0x0100;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short shortx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

template <int D>
struct Geo {
  static constexpr int kRowBytes = D * 2;             // one key row in LDS (no padding)
  static constexpr int kRowChunks = D / 8;            // 16-byte chunks per key row
  static constexpr int kKeysPerDma = 64 / kRowChunks; // key rows one 1 KB DMA instruction fills
  static constexpr int kTileBytes = kTileKeys * kRowBytes;
  static constexpr int kDmaPerTile = kTileBytes / 1024;  // per K (and per V) tile
  static constexpr int kKSteps = D / 16;              // MFMA k-steps over the head dim
  static constexpr int kDimBlocks = D / 32;           // 32-dim output blocks
  // byte offsets in a V stage ([1 KB piece of kKeysPerDma keys][dim block][key][4 chunks])
  static constexpr int kVDimBlockBytes = kKeysPerDma * 64;
  static constexpr int kVKeys8Bytes = (8 / kKeysPerDma) * 1024;   // 8 keys further on
  static constexpr int kVKStepBytes = (16 / kKeysPerDma) * 1024;  // 16 keys further on
};

// XOR swizzle of 16-byte chunk indices within a K row.  For d = 128 (16
// chunks per 256-byte row, LDS serving 256 bytes per cycle) it is a bijection
// on 16 consecutive keys, so the 16 rows of one K operand read land on 16
// different chunks.
template <int D>
__device__ __forceinline__ int swz(int key) {
  return D == 128 ? (((key & 3) << 2) | ((key >> 2) & 3)) : ((key >> 1) & 3);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8_t, u); }

// Max and sum of x over lanes l and l ^ 32, without an LDS round trip:
// permlane32_swap with both operands x returns x of this lane in one result
// and x of lane ^ 32 in the other, so combining the two results with a
// symmetric operation needs no knowledge of which is which.  The second
// operand passes through an empty asm statement: given the same value
// twice, the compiler would otherwise take the two results as equal and
// drop one of them.
__device__ __forceinline__ void lane_pair(float x, float& a, float& b) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  uint32_t w = u;
  asm volatile("" : "+v"(w));
  const auto pr = __builtin_amdgcn_permlane32_swap(u, w, false, false);
  const uint32_t r0 = pr[0], r1 = pr[1];   // copied out: a bit cast of a vector element reads element 0
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}

__device__ __forceinline__ float pair_max(float x) {
  float a, b;
  lane_pair(x, a, b);
  return fmaxf(a, b);
}

__device__ __forceinline__ float pair_sum(float x) {
  float a, b;
  lane_pair(x, a, b);
  return a + b;
}

// Geometry of one (request, row tile) shared by the attention kernel and the
// merge pass.
struct TileGeo {
  int L, o, n, rows_total, row_base, kmax, ntiles;
};

__device__ __forceinline__ TileGeo tile_geo(const PrefillArgs& a, int r, int t, int group) {
  TileGeo tg;
  tg.L = a.seq_lens[r];
  tg.o = a.q_offsets[r];
  tg.n = tg.L - tg.o;
  tg.rows_total = tg.n * group;
  tg.row_base = t * kTileRows;
  const int last_row = min(tg.row_base + kTileRows, tg.rows_total) - 1;
  tg.kmax = tg.o + last_row / group + 1;   // keys the tile's last row sees
  tg.ntiles = (tg.kmax + kTileKeys - 1) / kTileKeys;
  return tg;
}

__device__ __forceinline__ int num_splits_of(int ntiles, int kv_tiles_per_split) {
  return (ntiles + kv_tiles_per_split - 1) / kv_tiles_per_split;
}

// First packed query row of request r (from q_starts, or by summing n over
// the earlier requests).
__device__ __forceinline__ int q_start_of(const PrefillArgs& a, int r, int lane) {
  if (a.q_starts != nullptr) return a.q_starts[r];
  int acc = 0;
  for (int i = lane; i < r; i += 64) acc += a.seq_lens[i] - a.q_offsets[i];
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) acc += __shfl_xor(acc, s);
  return acc;
}

// Page id of page m of KV tile kt (uniform), or -1 past the needed pages.
struct PageIds {
  const int* lds;  // LDS copy of the needed page-table slice, clamped; or null
  const int32_t* __restrict__ ptab;
  int npages, num_pages;
};

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

// DMA one KV tile (K and V) from the pool into an LDS stage.  The 1 KB
// pieces of a tile split evenly over the 4 waves of a group so that wave w
// moves exactly page w of the tile; `id` is that page's physical id
// (uniform; -1 past the pages the request holds).  Lane l of a piece fills
// LDS slot (key, chunk) = (first key + l / kRowChunks, l % kRowChunks) with
// the key's chunk (l % kRowChunks) ^ swz(key).  A page whose keys are all
// below L goes by DMA; a page holding keys at or past L (or no page) is
// written with ordinary loads of the live keys and zeros for the rest, so a
// NaN in a page tail never reaches LDS.
template <int D>
__device__ __forceinline__ void dma_tile(unsigned char* kst, unsigned char* vst,
                                         const __bf16* __restrict__ kpool,
                                         const __bf16* __restrict__ vpool, int id, int kt, int L,
                                         int Hkv, int g, int wave, int lane) {
  using GE = Geo<D>;
  constexpr int kPerWave = GE::kDmaPerTile / kWavesPerGroup;
  static_assert(kPerWave * GE::kKeysPerDma == kPageSize, "each wave moves one page");
  const int key_base = kt * kTileKeys + wave * kPageSize;   // absolute key of the page's slot 0
  const size_t page_off = ((size_t)(id < 0 ? 0 : id) * Hkv + g) * ((size_t)kPageSize * D);
  const bool full = id >= 0 && key_base + kPageSize <= L;
  // lane offsets of piece i: K rows in order with their 16-byte chunks
  // XOR-swizzled by key; V as [dim block][key][4 chunks], so the transposing
  // reads of one dim block touch kKeysPerDma x 64 consecutive bytes
  auto kslot = [&](int i) { return i * GE::kKeysPerDma + lane / GE::kRowChunks; };
  auto vslot = [&](int i) { return i * GE::kKeysPerDma + (lane / 4) % GE::kKeysPerDma; };
  auto koff = [&](int i) {
    const int kchunk = (lane % GE::kRowChunks) ^ swz<D>(wave * kPageSize + kslot(i));
    return page_off + (size_t)kslot(i) * D + kchunk * 8;
  };
  auto voff = [&](int i) {
    const int vchunk = 4 * (lane / (4 * GE::kKeysPerDma)) + (lane & 3);
    return page_off + (size_t)vslot(i) * D + vchunk * 8;
  };
  if (full) {
    // the common case, decided once per page: kPerWave DMA instructions for
    // K and as many for V, back to back
#pragma unroll
    for (int i = 0; i < kPerWave; ++i)
      __builtin_amdgcn_global_load_lds(kpool + koff(i), (lds_void*)(kst + (wave * kPerWave + i) * 1024),
                                       16, 0, 0);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i)
      __builtin_amdgcn_global_load_lds(vpool + voff(i), (lds_void*)(vst + (wave * kPerWave + i) * 1024),
                                       16, 0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (id >= 0 && key_base + kslot(i) < L) kv = *reinterpret_cast<const uint4*>(kpool + koff(i));
      if (id >= 0 && key_base + vslot(i) < L) vv = *reinterpret_cast<const uint4*>(vpool + voff(i));
      *reinterpret_cast<uint4*>(kst + (wave * kPerWave + i) * 1024 + lane * 16) = kv;
      *reinterpret_cast<uint4*>(vst + (wave * kPerWave + i) * 1024 + lane * 16) = vv;
    }
  }
}

template <int N>
struct GroupTag {
  static constexpr int value = N;
};
// Row tile t of request r for KV head g, key-range split `split` (0 when
// unsplit): the whole workgroup of kThreads threads.  Writes the tile's rows
// of out and lse, or the split's partial rows.
template <int D>
__device__ __forceinline__ void prefill_tile(const PrefillArgs& a, int group, int r, int t, int g,
                                             int split) {
  using GE = Geo<D>;
  static_assert(kRB == 1, "the wave-group merge is written for one row block per wave");
  // two LDS stages per wave group, each K + V, named statically so the
  // compiler can tell the tile being copied in from the tile being read.
  // The V stages are laid out first (LDS variables are placed by decreasing
  // alignment), so every V operand address is one register plus an
  // immediate offset below 64 KB.
  __shared__ __align__(2048) unsigned char v_a0[GE::kTileBytes];
  __shared__ __align__(2048) unsigned char v_a1[GE::kTileBytes];
  __shared__ __align__(2048) unsigned char v_b0[GE::kTileBytes];
  __shared__ __align__(2048) unsigned char v_b1[GE::kTileBytes];
  __shared__ __align__(1024) unsigned char k_a0[GE::kTileBytes];
  __shared__ __align__(1024) unsigned char k_a1[GE::kTileBytes];
  __shared__ __align__(1024) unsigned char k_b0[GE::kTileBytes];
  __shared__ __align__(1024) unsigned char k_b1[GE::kTileBytes];
  __shared__ int s_pages[kLdsPages];
  __shared__ float s_ml[kWavesPerGroup][2][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave_id / kWavesPerGroup;      // which half of the key range
  const int wave = wave_id % kWavesPerGroup;     // wave within the group: its 32 rows
  const int half = lane >> 5;     // which 8-element k slice this lane feeds
  const int lrow = lane & 31;     // the query row (within a 32-row block) this lane owns

  const int Hkv = a.num_kv_heads;
  const int T = a.tiles_per_seq;
  const int S = a.num_splits;

  const TileGeo tg = tile_geo(a, r, t, group);
  if (tg.n <= 0 || tg.row_base >= tg.rows_total) return;
  const int nsp = num_splits_of(tg.ntiles, a.kv_tiles_per_split);
  if (split >= nsp) return;
  const int kt0 = split * a.kv_tiles_per_split;
  const int kt1 = min(kt0 + a.kv_tiles_per_split, tg.ntiles);
  const int q_start = q_start_of(a, r, lane);

  // this lane's query row (one 32-row block per wave)
  const int Hq = a.num_q_heads;
  const int o = tg.o;
  int pos[kRB], tok[kRB], hh[kRB];
  bool row_valid[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int rho = tg.row_base + wave * kRowsPerWave + rb * 32 + lrow;
    row_valid[rb] = rho < tg.rows_total;
    const int rc = row_valid[rb] ? rho : tg.rows_total - 1;
    tok[rb] = rc / group;
    hh[rb] = rc % group;
    pos[rb] = o + tok[rb];
  }
  const int wrow0 = min(tg.row_base + wave * kRowsPerWave, tg.rows_total - 1);
  const int wrow1 = min(tg.row_base + wave * kRowsPerWave + kRowsPerWave, tg.rows_total) - 1;
  const int pos_lo = o + wrow0 / group;   // the wave's rows span positions [pos_lo, pos_hi]
  const int pos_hi = o + wrow1 / group;

  const __bf16* __restrict__ qp = reinterpret_cast<const __bf16*>(a.q);
  uint4 qv[kRB][GE::kKSteps];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const __bf16* qrow = qp + ((size_t)(q_start + tok[rb]) * Hq + (size_t)g * group + hh[rb]) * D;
#pragma unroll
    for (int s = 0; s < GE::kKSteps; ++s)
      qv[rb][s] = *reinterpret_cast<const uint4*>(qrow + 16 * s + 8 * half);
  }

  const __bf16* __restrict__ kpool = reinterpret_cast<const __bf16*>(a.k_pool);
  const __bf16* __restrict__ vpool = reinterpret_cast<const __bf16*>(a.v_pool);
  const int32_t* __restrict__ ptab = a.page_table + (size_t)r * a.max_pages_per_seq;
  const int npages = min((tg.kmax + kPageSize - 1) / kPageSize, a.max_pages_per_seq);

  PageIds pi;
  pi.ptab = ptab;
  pi.npages = npages;
  pi.num_pages = a.num_pages;
  pi.lds = nullptr;
  const int p0 = kt0 * kPagesPerTile;
  const int p1 = min(kt1 * kPagesPerTile, npages);
  if (p1 - p0 <= kLdsPages) {
    for (int i = p0 + tid; i < p1; i += kThreads) {
      int id = ptab[i];
      s_pages[i - p0] = id < 0 ? 0 : (id >= a.num_pages ? a.num_pages - 1 : id);
    }
    pi.lds = s_pages - p0;   // indexed by logical page
    __syncthreads();
  }

  floatx16_t oacc[kRB][GE::kDimBlocks];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
    for (int db = 0; db < GE::kDimBlocks; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[rb][db][i] = 0.f;
  float m_run[kRB], l_run[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
  }
  const float sl2 = a.scale_log2;

  // lanes of a 16-lane group address 4 keys x 4 dim quads for the
  // transposing reads of the V^T operand: key 4 * half + vk (plus 16 per
  // k-step and 8 for the second read), dims vdim_off .. vdim_off + 3 of a
  // 32-dim block; vlane is that element's byte offset in a V stage
  const int vgrp = lane >> 4;
  const int vp = lane & 15;
  const int vk = vp >> 2;                                 // which of the 4 keys
  const int vdim_off = 16 * (vgrp & 1) + 4 * (vp & 3);   // dims within a 32-dim block
  const int vkey = 4 * half + vk;
  const uint32_t vlane = (uint32_t)((vkey / GE::kKeysPerDma) * 1024 + (vkey % GE::kKeysPerDma) * 64 +
                                    (vdim_off >> 3) * 16 + (vdim_off & 7) * 2);

  // one KV tile out of an LDS stage
  auto compute_tile = [&](const unsigned char* kst, const unsigned char* vst, int kb)
                          __attribute__((always_inline)) {
    if (kb > pos_hi) return;   // no key of the tile is visible to any row of this wave
    // ---- S^T = K Q^T: 2 key blocks x 2 row blocks ----
    // K operand address for k-step s: the swizzled chunk 2s + half of key
    // row kb2*32 + lrow sits at kbase ^ (32 s) (the swizzle is an XOR on
    // chunk bits 1..3, and the row base is a multiple of 256 bytes).
    // All 8 K operands of a key block are requested before its MFMAs, and
    // each register is refilled with the next block's operand as soon as its
    // MFMA has been issued, so the MFMAs never wait on one LDS round trip
    // each.
    static_assert(kRB == 1, "the operand pipeline below is written for one row block");
    floatx16_t sacc[kRB][2];
    uint32_t kbase[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      const int key = kb2 * 32 + lrow;
      const int sw = swz<D>(key);
      kbase[kb2] = (uint32_t)(key * GE::kRowBytes) + ((uint32_t)(half ^ (sw & 1)) << 4) +
                   ((uint32_t)(sw >> 1) << 5);
    }
    asm volatile("" : "+v"(kbase[0]), "+v"(kbase[1]));   // keep the addresses out of the loop preheader
    uint4 ka[GE::kKSteps];
#pragma unroll
    for (int s = 0; s < GE::kKSteps; ++s)
      ka[s] = *reinterpret_cast<const uint4*>(kst + (kbase[0] ^ (uint32_t)(s << 5)));
#pragma unroll
    for (int s = 0; s < GE::kKSteps; ++s) {
      const floatx16_t zero = {};
      sacc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[s]), as_bf16x8(qv[0][s]),
                                                           s == 0 ? zero : sacc[0][0], 0, 0, 0);
      ka[s] = *reinterpret_cast<const uint4*>(kst + (kbase[1] ^ (uint32_t)(s << 5)));
    }
#pragma unroll
    for (int s = 0; s < GE::kKSteps; ++s) {
      const floatx16_t zero = {};
      sacc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[s]), as_bf16x8(qv[0][s]),
                                                           s == 0 ? zero : sacc[0][1], 0, 0, 0);
    }
    // schedule: the first block's reads, then each MFMA followed by the read
    // that refills its operand register, then the second block's MFMAs
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, GE::kKSteps, 0);
#pragma unroll
    for (int s = 0; s < GE::kKSteps; ++s) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, GE::kKSteps, 0);
    // ---- mask, online softmax, P^T operand ----
    uint32_t pk[kRB][2][8];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      if (kb + kTileKeys - 1 > pos_lo) {
        // element i of key block kb2 holds key kb + kb2*32 + 8*(i/4) + 4*half + i%4
        const int lim = pos[rb] - kb - 4 * half;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            sacc[rb][kb2][i] = kb2 * 32 + 8 * (i / 4) + (i % 4) <= lim ? sacc[rb][kb2][i] : -INFINITY;
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sacc[rb][kb2][i]);
      tmax = pair_max(tmax) * sl2;   // scale > 0 commutes with max
      const bool need = tmax > m_run[rb] + kRescaleLog2;
      if (__builtin_expect(__any(need), 0)) {
        const float mn = fmaxf(m_run[rb], tmax);
        const float alpha = (mn == m_run[rb]) ? 1.f : fast_exp2(m_run[rb] - mn);
        l_run[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < GE::kDimBlocks; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[rb][db][i] *= alpha;
        m_run[rb] = mn;
      }
      // a row with no visible key so far keeps m = -inf: use 0 as the
      // reference so its (all -inf) scores give p = 0 rather than NaN
      const float mref = m_run[rb] == -INFINITY ? 0.f : m_run[rb];
      // the row sum adds the fp32 weights (a sum of their bf16 roundings
      // would be off by up to 2^-9 relative in a row with one dominant key,
      // about 2e-3 in the log-sum-exp)
      float lsum = 0.f;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float p0 = fast_exp2(fmaf(sacc[rb][kb2][i], sl2, -mref));
          const float p1 = fast_exp2(fmaf(sacc[rb][kb2][i + 1], sl2, -mref));
          lsum += p0 + p1;
          pk[rb][kb2][i / 2] = pack_bf16x2(p0, p1);
        }
      }
      l_run[rb] += lsum;
    }
    // ---- O^T += V^T P^T: 4 k-steps of 16 keys ----
    // V operand: two transposing 8-byte reads per (k-step, dim block), all
    // at fixed offsets from one per-lane address.  The reads of k-step ks+1
    // are issued before the MFMAs of k-step ks.
    auto v_operands = [&](int ks, uint4 (&av)[GE::kDimBlocks]) __attribute__((always_inline)) {
#pragma unroll
      for (int db = 0; db < GE::kDimBlocks; ++db) {
        const unsigned char* pa = vst + vlane + ks * GE::kVKStepBytes + db * GE::kVDimBlockBytes;
        const shortx4_t va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) shortx4_t*)(pa));
        const shortx4_t vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) shortx4_t*)(pa + GE::kVKeys8Bytes));
        av[db].x = __builtin_bit_cast(uint32_t, __builtin_shufflevector(va, va, 0, 1));
        av[db].y = __builtin_bit_cast(uint32_t, __builtin_shufflevector(va, va, 2, 3));
        av[db].z = __builtin_bit_cast(uint32_t, __builtin_shufflevector(vb, vb, 0, 1));
        av[db].w = __builtin_bit_cast(uint32_t, __builtin_shufflevector(vb, vb, 2, 3));
      }
    };
    uint4 avs[2][GE::kDimBlocks];
    v_operands(0, avs[0]);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks + 1 < 4) v_operands(ks + 1, avs[(ks + 1) & 1]);
      const int kb2 = ks >> 1;
      const int th = ks & 1;
      uint4 pb;
      pb.x = pk[0][kb2][4 * th + 0];
      pb.y = pk[0][kb2][4 * th + 1];
      pb.z = pk[0][kb2][4 * th + 2];
      pb.w = pk[0][kb2][4 * th + 3];
#pragma unroll
      for (int db = 0; db < GE::kDimBlocks; ++db)
        oacc[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(avs[ks & 1][db]),
                                                              as_bf16x8(pb), oacc[0][db], 0, 0, 0);
    }
    // schedule: k-step 0's reads, then each k-step's MFMAs interleaved with
    // the next k-step's reads (two per MFMA), then the last MFMAs
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * GE::kDimBlocks, 1);
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {
#pragma unroll
      for (int db = 0; db < GE::kDimBlocks; ++db) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 1);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 1);
      }
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, GE::kDimBlocks, 1);
  };

  // The two wave groups take the two halves of the key range, [kt0, mid)
  // and [mid, kt1), over the same rows.  Per group: tile i is computed out of
  // one LDS stage while tile i+1 is copied into the other by DMA; a barrier
  // per step (shared by both groups, which run the same number of steps)
  // hands stages over.  Unrolled by two so each step names its stages.
  const int L = tg.L;
  const int mid = kt0 + (kt1 - kt0 + 1) / 2;
  const int nloop = mid - kt0;
  auto run = [&](auto gtag) __attribute__((always_inline)) {
    constexpr int GRP = decltype(gtag)::value;
    unsigned char* ks0 = GRP == 0 ? k_a0 : k_b0;
    unsigned char* vs0 = GRP == 0 ? v_a0 : v_b0;
    unsigned char* ks1 = GRP == 0 ? k_a1 : k_b1;
    unsigned char* vs1 = GRP == 0 ? v_a1 : v_b1;
    const int my0 = GRP == 0 ? kt0 : mid;
    const int my1 = GRP == 0 ? mid : kt1;
    // The page this wave moves for the next tile is looked up one step
    // ahead (an LDS read whose latency the step's compute hides).
    auto wave_page = [&](int kt) { return tile_page(pi, min(kt, my1 - 1), wave); };
    if (my0 < my1) dma_tile<D>(ks0, vs0, kpool, vpool, wave_page(my0), my0, L, Hkv, g, wave, lane);
    int next_id = wave_page(my0 + 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int i = 0;;) {
      int kt = my0 + i;
      if (kt + 1 < my1) dma_tile<D>(ks1, vs1, kpool, vpool, next_id, kt + 1, L, Hkv, g, wave, lane);
      next_id = wave_page(kt + 2);
      if (kt < my1) compute_tile(ks0, vs0, kt * kTileKeys);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (++i >= nloop) break;
      kt = my0 + i;
      if (kt + 1 < my1) dma_tile<D>(ks0, vs0, kpool, vpool, next_id, kt + 1, L, Hkv, g, wave, lane);
      next_id = wave_page(kt + 2);
      if (kt < my1) compute_tile(ks1, vs1, kt * kTileKeys);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (++i >= nloop) break;
    }
  };
  if (grp == 0)
    run(GroupTag<0>{});
  else
    run(GroupTag<1>{});

  // ---- merge the groups: group 1 hands its per-lane state to group 0 ----
  // Every lane of both groups owns the same (row, dims), so the merge is the
  // log-sum-exp rule applied lane by lane.  Group 1's stage buffers are free
  // now (the last barrier above ended all reads); wave w of the group writes
  // its accumulator into one of them, float4 j of lane l at j*1024 + l*16.
  {
    unsigned char* xfer = wave == 0 ? k_b0 : (wave == 1 ? v_b0 : (wave == 2 ? k_b1 : v_b1));
    if (grp == 1) {
#pragma unroll
      for (int db = 0; db < GE::kDimBlocks; ++db)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float4 w;
          w.x = oacc[0][db][4 * v + 0];
          w.y = oacc[0][db][4 * v + 1];
          w.z = oacc[0][db][4 * v + 2];
          w.w = oacc[0][db][4 * v + 3];
          *reinterpret_cast<float4*>(xfer + (db * 4 + v) * 1024 + lane * 16) = w;
        }
      s_ml[wave][0][lane] = m_run[0];
      s_ml[wave][1][lane] = l_run[0];
    }
    __syncthreads();
    if (grp == 1) return;
    const float mB = s_ml[wave][0][lane];
    const float lB = s_ml[wave][1][lane];
    const float M = fmaxf(m_run[0], mB);
    const float fA = m_run[0] == -INFINITY ? 0.f : fast_exp2(m_run[0] - M);
    const float fB = mB == -INFINITY ? 0.f : fast_exp2(mB - M);
#pragma unroll
    for (int db = 0; db < GE::kDimBlocks; ++db)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float4 w = *reinterpret_cast<const float4*>(xfer + (db * 4 + v) * 1024 + lane * 16);
        oacc[0][db][4 * v + 0] = oacc[0][db][4 * v + 0] * fA + w.x * fB;
        oacc[0][db][4 * v + 1] = oacc[0][db][4 * v + 1] * fA + w.y * fB;
        oacc[0][db][4 * v + 2] = oacc[0][db][4 * v + 2] * fA + w.z * fB;
        oacc[0][db][4 * v + 3] = oacc[0][db][4 * v + 3] * fA + w.w * fB;
      }
    l_run[0] = l_run[0] * fA + lB * fB;
    m_run[0] = M;
  }

  // ---- normalize and write: final output, or this split's partial ----
  const bool partial = nsp > 1;
  const size_t unit = ((size_t)r * T + t) * Hkv + g;
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const float l_tot = pair_sum(l_run[rb]);
    if (!row_valid[rb]) continue;
    const bool empty = !(l_tot > 0.f);
    const float inv = empty ? 0.f : 1.f / l_tot;
    const float lse = empty ? -INFINITY : (m_run[rb] + __log2f(l_tot)) * kLn2;
    if (!partial) {
      __bf16* orow = reinterpret_cast<__bf16*>(a.out) +
                     ((size_t)(q_start + tok[rb]) * Hq + (size_t)g * group + hh[rb]) * D;
#pragma unroll
      for (int db = 0; db < GE::kDimBlocks; ++db)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          uint2 w;
          w.x = pack_bf16x2(oacc[rb][db][4 * v + 0] * inv, oacc[rb][db][4 * v + 1] * inv);
          w.y = pack_bf16x2(oacc[rb][db][4 * v + 2] * inv, oacc[rb][db][4 * v + 3] * inv);
          *reinterpret_cast<uint2*>(orow + db * 32 + 8 * v + 4 * half) = w;
        }
      if (a.lse != nullptr && half == 0)
        a.lse[(size_t)(q_start + tok[rb]) * Hq + (size_t)g * group + hh[rb]] = lse;
    } else {
      const int prow = wave * kRowsPerWave + rb * 32 + lrow;   // row within the tile
      const size_t pidx = (unit * S + split) * kTileRows + prow;
      float* po = a.part_o + pidx * D;
#pragma unroll
      for (int db = 0; db < GE::kDimBlocks; ++db)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float4 w;
          w.x = oacc[rb][db][4 * v + 0] * inv;
          w.y = oacc[rb][db][4 * v + 1] * inv;
          w.z = oacc[rb][db][4 * v + 2] * inv;
          w.w = oacc[rb][db][4 * v + 3] * inv;
          *reinterpret_cast<float4*>(po + db * 32 + 8 * v + 4 * half) = w;
        }
      if (half == 0) a.part_lse[pidx] = lse;
    }
  }
}

}  // namespace pf
}  // namespace pa
