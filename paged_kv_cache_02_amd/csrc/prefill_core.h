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
//   * K pages are copied straight from HBM into LDS by buffer loads with
//     the LDS flag (no staging registers), double-buffered one tile ahead,
//     K's 16-byte chunks XOR-swizzled by key; V pages are loaded into registers at the same
//     time and, once they have landed, converted from bf16 to fp16 and
//     written to the other LDS stage as [dim block][key] within each 1 KB
//     piece.  The operand reads below are bank-conflict free, and every
//     operand address is one register plus an immediate offset;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: A = K rows read from LDS,
//     B = Q held in registers, so a lane owns one query row and 16 of every
//     32 keys -- the row max and sum need one exchange with lane ^ 32;
//   * causal mask by select on diagonal tiles only; lazy online-softmax
//     rescale (only when the max grows by more than 2^8); the row max and
//     sum cross the two lane halves with permlane32_swap;
//   * O^T += V^T P^T runs on fp16 MFMA: V converted from bf16 to fp16 is
//     exact for |v| up to fp16's 65504 (smaller than 2^-14 it keeps an
//     absolute error under 2^-25), and P is rounded to fp16, whose 11-bit
//     significand keeps each weight within 2^-11 (relative) of its fp32
//     value (a bf16 P, 8 bits, moved outputs of rows dominated by a few
//     keys with |v| near 4 by up to 0.009, most of the 1e-2 bar).  The V^T
//     operand comes from V's natural [key][dim] layout through ds_read_b64_tr_b16
//     (gfx950's transposing LDS read), in the key order the P^T registers
//     carry, and the output accumulator keeps one row per lane, so
//     rescaling is local.
//
// Keys at or past a row's position are masked by select before the max.  K
// and V rows of keys at or past seq_len (page tails, possibly NaN) are never
// loaded: their LDS slots are zero-filled, so no NaN meets a zero weight.
// Page-table entries past the pages needed are never used: the prologue's
// read-ahead of the first tiles' entries stays inside the request's row and
// takes an entry only for a tile the request has.
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
constexpr int kSpecTiles = 64;                    // tiles whose page ids are read ahead (one per lane)
constexpr float kRescaleLog2 = 8.0f;
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.4426950408889634f;
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x0008;
constexpr int kSchedDsRead = 0x0100;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 halfx8_t __attribute__((ext_vector_type(8)));
typedef _Float16 halfx2_t __attribute__((ext_vector_type(2)));
typedef short shortx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

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

// Keys whose swizzle repeats: swz<D>(key) depends on key modulo this.
template <int D>
constexpr int swz_period() { return D == 128 ? 16 : 8; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8_t, u); }
__device__ __forceinline__ halfx8_t as_halfx8(const uint4& u) { return __builtin_bit_cast(halfx8_t, u); }

// Two fp32 values rounded to nearest-even fp16, packed (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  halfx2_t v;
  v[0] = (_Float16)lo;
  v[1] = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// A packed bf16 pair as a packed fp16 pair (exact within fp16's range).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t u) {
  return pack_f16x2(__uint_as_float(u << 16), __uint_as_float(u & 0xFFFF0000u));
}

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

__device__ __forceinline__ TileGeo tile_geo_of(int L, int o, int t, int group) {
  TileGeo tg;
  tg.L = L;
  tg.o = o;
  tg.n = tg.L - tg.o;
  tg.rows_total = tg.n * group;
  tg.row_base = t * kTileRows;
  const int last_row = min(tg.row_base + kTileRows, tg.rows_total) - 1;
  tg.kmax = tg.o + last_row / group + 1;   // keys the tile's last row sees
  tg.ntiles = (tg.kmax + kTileKeys - 1) / kTileKeys;
  return tg;
}

__device__ __forceinline__ TileGeo tile_geo(const PrefillArgs& a, int r, int t, int group) {
  return tile_geo_of(a.seq_lens[r], a.q_offsets[r], t, group);
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

// The same value in every lane, still in a vector register: a lookahead
// keeps it there until use, so the wait for its load falls where it is used.
__device__ __forceinline__ int tile_page_lanes(const PageIds& pi, int kt, int m) {
  const int lp = kt * kPagesPerTile + m;
  if (lp >= pi.npages) return -1;
  int id;
  if (pi.lds != nullptr) {
    id = pi.lds[lp];
  } else {
    id = pi.ptab[lp];
    id = id < 0 ? 0 : (id >= pi.num_pages ? pi.num_pages - 1 : id);
  }
  return id;
}

__device__ __forceinline__ int tile_page(const PageIds& pi, int kt, int m) {
  return __builtin_amdgcn_readfirstlane(tile_page_lanes(pi, kt, m));
}

// Copy one KV tile's K from the pool into an LDS stage, and load its V into
// registers.  The 1 KB pieces of a tile split evenly over the 4 waves of a
// group so that wave w moves exactly page w of the tile; `id` is that
// page's physical id (uniform; -1 past the pages the request holds).  Lane
// l of a piece fills LDS slot (key, chunk) = (first key + l / kRowChunks,
// l % kRowChunks) with the key's chunk (l % kRowChunks) ^ swz(key).  A page
// whose keys are all below L goes by DMA (K) and plain loads (V); a page
// holding keys at or past L (or no page) is loaded key by key with zeros
// for the rest, so a NaN in a page tail never reaches LDS.  V's registers
// are written to LDS, converted to fp16, by store_v once they have landed.
template <int D>
struct VRegs {
  uint4 c[Geo<D>::kDmaPerTile / kWavesPerGroup];
};

template <int D>
__device__ __forceinline__ void load_tile(unsigned char* kst, VRegs<D>& vr,
                                          const __bf16* __restrict__ kpool,
                                          const __bf16* __restrict__ vpool, int id, int kt, int L,
                                          int Hkv, int g, int wave, int lane) {
  using GE = Geo<D>;
  constexpr int kPerWave = GE::kDmaPerTile / kWavesPerGroup;
  static_assert(kPerWave * GE::kKeysPerDma == kPageSize, "each wave moves one page");
  const int key_base = kt * kTileKeys + wave * kPageSize;   // absolute key of the page's slot 0
  // the (page, KV head) block's first byte: uniform, so a page's loads take
  // a buffer resource in scalar registers and a 32-bit lane offset
  const size_t page_bytes = ((size_t)(id < 0 ? 0 : id) * Hkv + g) * ((size_t)kPageSize * GE::kRowBytes);
  const unsigned char* __restrict__ kpage = reinterpret_cast<const unsigned char*>(kpool) + page_bytes;
  const unsigned char* __restrict__ vpage = reinterpret_cast<const unsigned char*>(vpool) + page_bytes;
  const bool full = id >= 0 && key_base + kPageSize <= L;
  // lane offsets of piece i: K rows in order with their 16-byte chunks
  // XOR-swizzled by key; V as [dim block][key][4 chunks], so the transposing
  // reads of one dim block touch kKeysPerDma x 64 consecutive bytes
  auto kslot = [&](int i) { return i * GE::kKeysPerDma + lane / GE::kRowChunks; };
  auto vslot = [&](int i) { return i * GE::kKeysPerDma + (lane / 4) % GE::kKeysPerDma; };
  auto koff = [&](int i) {
    const int kchunk = (lane % GE::kRowChunks) ^ swz<D>(wave * kPageSize + kslot(i));
    return (uint32_t)(kslot(i) * GE::kRowBytes + kchunk * 16);
  };
  auto voff = [&](int i) {
    const int vchunk = 4 * (lane / (4 * GE::kKeysPerDma)) + (lane & 3);
    return (uint32_t)(vslot(i) * GE::kRowBytes + vchunk * 16);
  };
  if (full) {
    // the common case, decided once per page: kPerWave DMA instructions for
    // K and as many register loads for V, back to back, through buffer
    // resources spanning the page's block (the lane offsets are the same for
    // every page, and piece i's part of them is an immediate offset)
    constexpr int kBlockBytes = kPageSize * GE::kRowBytes;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(kpage), (short)0, kBlockBytes, kBufferWord3);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(vpage), (short)0, kBlockBytes, kBufferWord3);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(kst + (wave * kPerWave + i) * 1024), 16,
                                               (int)koff(i), 0, 0, 0);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(vrs, (int)voff(i), 0, 0);
      vr.c[i] = make_uint4(x[0], x[1], x[2], x[3]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (id >= 0 && key_base + kslot(i) < L) kv = *reinterpret_cast<const uint4*>(kpage + koff(i));
      if (id >= 0 && key_base + vslot(i) < L) vv = *reinterpret_cast<const uint4*>(vpage + voff(i));
      *reinterpret_cast<uint4*>(kst + (wave * kPerWave + i) * 1024 + lane * 16) = kv;
      vr.c[i] = vv;
    }
  }
}

// Write this wave's V page (loaded by load_tile) into stage `vst`, each
// value converted from bf16 to fp16.
template <int D>
__device__ __forceinline__ void store_v(unsigned char* vst, const VRegs<D>& vr, int wave, int lane) {
  using GE = Geo<D>;
  constexpr int kPerWave = GE::kDmaPerTile / kWavesPerGroup;
#pragma unroll
  for (int i = 0; i < kPerWave; ++i) {
    uint4 x = vr.c[i];
    x.x = bf16x2_to_f16x2(x.x);
    x.y = bf16x2_to_f16x2(x.y);
    x.z = bf16x2_to_f16x2(x.z);
    x.w = bf16x2_to_f16x2(x.w);
    *reinterpret_cast<uint4*>(vst + (wave * kPerWave + i) * 1024 + lane * 16) = x;
  }
}

template <int N>
struct GroupTag {
  static constexpr int value = N;
};
// The fields of PrefillArgs that a row tile reads first (the request's
// length, offset and first row, and its page-table row).  The prefill
// kernel takes them as leading scalar arguments, which the library's build
// preloads into SGPRs, so the first reads need no load of the kernel
// arguments; the single launch copies them out of its argument struct.
struct PrefillHot {
  const int32_t* seq_lens;
  const int32_t* q_offsets;
  const int32_t* q_starts;
  const int32_t* page_table;
  int max_pages_per_seq;
};

__device__ __forceinline__ PrefillHot prefill_hot(const PrefillArgs& a) {
  return PrefillHot{a.seq_lens, a.q_offsets, a.q_starts, a.page_table, a.max_pages_per_seq};
}

// Row tile t of request r for KV head g, key-range split `split` (0 when
// unsplit): the whole workgroup of kThreads threads.  Writes the tile's rows
// of out and lse, or the split's partial rows.  `h` holds the same values as
// the corresponding fields of `a`.
template <int D>
__device__ __forceinline__ void prefill_tile(const PrefillArgs& a, const PrefillHot& h, int group,
                                             int r, int t, int g, int split) {
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
  __shared__ int s_spec[kWaves][kSpecTiles];

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

  // The request's length, offset and first row are requested first (scalar
  // loads, so waiting for them never waits for the copies below).  Beside
  // them, lane j of each wave copies entry 4j + wave of the request's table
  // row (the page this wave moves for KV tile j) into the wave's row of
  // s_spec by DMA: once the tile geometry says which tile the wave's group
  // starts at, its page id is one LDS read away, and the first tile's copy
  // waits for one memory round trip after the lengths instead of two.
  // Groups starting past kSpecTiles read the entry itself.
  const int maxp = h.max_pages_per_seq;
  const int req_L = h.seq_lens[r];
  const int req_o = h.q_offsets[r];
  const int req_q0 = h.q_starts != nullptr ? h.q_starts[r] : 0;
  const int32_t* __restrict__ ptab = h.page_table + (size_t)r * maxp;
  {
    const int lp = kPagesPerTile * lane + wave;
    __builtin_amdgcn_global_load_lds(ptab + (lp < maxp ? lp : maxp - 1),
                                     (lds_void*)&s_spec[wave_id][0], 4, 0, 0);
  }

  // a workgroup that leaves early first waits for its read-ahead copy, so
  // no copy lands in LDS that the next workgroup on the CU already owns
  auto leave = [&]() { __builtin_amdgcn_s_waitcnt(0); };
  const TileGeo tg = tile_geo_of(req_L, req_o, t, group);
  if (tg.n <= 0 || tg.row_base >= tg.rows_total) return leave();
  const int nsp = num_splits_of(tg.ntiles, a.kv_tiles_per_split);
  if (split >= nsp) return leave();
  const int kt0 = split * a.kv_tiles_per_split;
  const int kt1 = min(kt0 + a.kv_tiles_per_split, tg.ntiles);
  const int q_start = h.q_starts != nullptr ? req_q0 : q_start_of(a, r, lane);

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
  // this lane's query operand registers, filled from LDS in run()
  uint4 qv[kRB][GE::kKSteps];

  const __bf16* __restrict__ kpool = reinterpret_cast<const __bf16*>(a.k_pool);
  const __bf16* __restrict__ vpool = reinterpret_cast<const __bf16*>(a.v_pool);
  const int npages = min((tg.kmax + kPageSize - 1) / kPageSize, maxp);

  PageIds pi;
  pi.ptab = ptab;
  pi.npages = npages;
  pi.num_pages = a.num_pages;
  pi.lds = nullptr;
  const int mid = kt0 + (kt1 - kt0 + 1) / 2;
  const int first_kt = grp == 0 ? kt0 : mid;
  const int first_lp = first_kt * kPagesPerTile + wave;
  const bool first_valid = first_kt < (grp == 0 ? mid : kt1) && first_lp < npages;
  const int L = tg.L;
  // the group's first tile into stage 0 (K by DMA, V into registers)
  VRegs<D> vr;
  if (first_kt < (grp == 0 ? mid : kt1)) {
    int id = -1;
    if (first_valid) {
      id = first_kt < kSpecTiles ? s_spec[wave_id][first_kt] : ptab[first_lp];
      id = __builtin_amdgcn_readfirstlane(id);
      id = id < 0 ? 0 : (id >= a.num_pages ? a.num_pages - 1 : id);
    }
    load_tile<D>(grp == 0 ? k_a0 : k_b0, vr, kpool, vpool, id, first_kt, L, Hkv, g, wave, lane);
  }
  // The wave's 32 query rows come in by DMA, whole rows per instruction,
  // into the slices of its group's stage-1 K and V buffers that this wave's
  // own copies overwrite first (rows 0-15 in the K slice, 16-31 in the V
  // slice), laid out like K rows (16-byte chunks XOR-swizzled by row).  They
  // are read into registers after the first barrier and waited for before
  // this wave's first copy into stage 1, so no other wave is involved.  They
  // are requested after the group's first tile (whose page id comes from
  // s_spec), and the page-id copy below after both, so all three are in
  // flight together.
  constexpr int kSlice = (GE::kDmaPerTile / kWavesPerGroup) * 1024;   // a wave's part of a stage
  static_assert(16 * GE::kRowBytes == kSlice, "16 query rows fill a wave's slice");
  unsigned char* const qk = (grp == 0 ? k_a1 : k_b1) + wave * kSlice;
  unsigned char* const qvs = (grp == 0 ? v_a1 : v_b1) + wave * kSlice;
  // packed row -> (token, head): rho / group by a multiply with the rounded-up
  // reciprocal, exact while rho * group < 2^32 (else a plain division)
  auto load_q_rows = [&](auto div) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 32 / GE::kKeysPerDma; ++i) {
      const int row = i * GE::kKeysPerDma + lane / GE::kRowChunks;   // of the wave's 32
      const int rho0 = tg.row_base + wave * kRowsPerWave + row;
      const int rho = rho0 < tg.rows_total ? rho0 : tg.rows_total - 1;
      const int tk = div(rho);
      const int hd = rho - tk * group;
      const int chunk = (lane % GE::kRowChunks) ^ swz<D>(row);
      const __bf16* src = qp + ((size_t)(q_start + tk) * Hq + (size_t)g * group + hd) * D + chunk * 8;
      unsigned char* dst = (row < 16 ? qk : qvs) + (i % (16 / GE::kKeysPerDma)) * 1024;
      __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 0);
    }
  };
  if (group == 1) {
    load_q_rows([&](int rho) { return rho; });
  } else if ((unsigned long long)tg.rows_total * (unsigned)group < 0x100000000ull) {
    // ceil(2^32 / group) fits 32 bits for group >= 2
    const uint32_t gmul = (uint32_t)((0x100000000ull + (uint32_t)group - 1) / (uint32_t)group);
    load_q_rows([&](int rho) { return (int)__umulhi((uint32_t)rho, gmul); });
  } else {
    load_q_rows([&](int rho) { return rho / group; });
  }

  const int p0 = kt0 * kPagesPerTile;
  const int p1 = min(kt1 * kPagesPerTile, npages);
  if (p1 - p0 <= kLdsPages) {
    // published by the barrier after the first tile's copy, which reads its
    // page straight from the table
    for (int i = p0 + tid; i < p1; i += kThreads) {
      int id = ptab[i];
      s_pages[i - p0] = id < 0 ? 0 : (id >= a.num_pages ? a.num_pages - 1 : id);
    }
    pi.lds = s_pages - p0;   // indexed by logical page
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

  // K operand addresses within a stage, the same for every tile: for k-step
  // s the swizzled chunk 2s + half of key row lrow sits at kbase ^ (32 s)
  // (the swizzle is an XOR on chunk bits 1..3, and the row base is a
  // multiple of the row size).  The swizzle depends on the key modulo 16
  // only, so the second key block's rows sit kKeyBlockBytes further on.
  // The registers hold the offsets plus kKBias, the 64 KB that the V stages
  // take before the K stages at d = 128, hidden from the compiler: a read
  // then is one register plus an immediate offset (the stage's address
  // minus the bias, plus the key block), instead of a register plus an
  // address past the 16-bit offset field that needs an add per read.
  constexpr uint32_t kKeyBlockBytes = 32 * GE::kRowBytes;
  constexpr uint32_t kKBias = (4u * GE::kTileBytes) & ~0xFFFFu;
  static_assert(swz_period<D>() <= 32, "key block 1 has key block 0's swizzle");
  uint32_t kaddr[GE::kKSteps];
  {
    const int sw = swz<D>(lrow);
    const uint32_t kbase = (uint32_t)(lrow * GE::kRowBytes) + ((uint32_t)(half ^ (sw & 1)) << 4) +
                           ((uint32_t)(sw >> 1) << 5);
#pragma unroll
    for (int s = 0; s < GE::kKSteps; ++s) {
      kaddr[s] = (kbase ^ (uint32_t)(s << 5)) + kKBias;
      asm volatile("" : "+v"(kaddr[s]));
    }
  }

  // one KV tile out of an LDS stage
  auto compute_tile = [&](const unsigned char* kst, const unsigned char* vst, int kb)
                          __attribute__((always_inline)) {
    if (kb > pos_hi) return;   // no key of the tile is visible to any row of this wave
    // ---- S^T = K Q^T: 2 key blocks x 2 row blocks ----
    // All 8 K operands of a key block are requested before its MFMAs, and
    // each register is refilled with the next block's operand as soon as its
    // MFMA has been issued, so the MFMAs never wait on one LDS round trip
    // each.
    static_assert(kRB == 1, "the operand pipeline below is written for one row block");
    floatx16_t sacc[kRB][2];
    uint4 ka[GE::kKSteps];
#pragma unroll
    for (int s = 0; s < GE::kKSteps; ++s)
      ka[s] = *reinterpret_cast<const uint4*>(kst + (kaddr[s] - kKBias));
#pragma unroll
    for (int s = 0; s < GE::kKSteps; ++s) {
      const floatx16_t zero = {};
      sacc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[s]), as_bf16x8(qv[0][s]),
                                                           s == 0 ? zero : sacc[0][0], 0, 0, 0);
      ka[s] = *reinterpret_cast<const uint4*>(kst + (kaddr[s] - kKBias + kKeyBlockBytes));
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
      // the row max and the row sum below reduce in four independent
      // chains, so their dependent-issue latency is a quarter of one chain's
      float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx[i & 3] = fmaxf(mx[i & 3], sacc[rb][kb2][i]);
      float tmax = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
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
      // the row sum adds the fp32 weights (a sum of their fp16 roundings
      // would be off by up to 2^-11 relative in a row with one dominant
      // key)
      float ls[4];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float p0 = fast_exp2(fmaf(sacc[rb][kb2][i], sl2, -mref));
          const float p1 = fast_exp2(fmaf(sacc[rb][kb2][i + 1], sl2, -mref));
          const int c = (i / 2) & 3;
          // each chain starts from its first pair (no add of zero)
          ls[c] = kb2 == 0 && i < 8 ? p0 + p1 : ls[c] + (p0 + p1);
          pk[rb][kb2][i / 2] = pack_f16x2(p0, p1);
        }
      }
      l_run[rb] += (ls[0] + ls[1]) + (ls[2] + ls[3]);
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
        oacc[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_halfx8(avs[ks & 1][db]),
                                                             as_halfx8(pb), oacc[0][db], 0, 0, 0);
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
    auto wave_page = [&](int kt) { return tile_page_lanes(pi, min(kt, my1 - 1), wave); };
    __builtin_amdgcn_s_waitcnt(0);   // the first tile (requested above), the query rows, the page ids
    if (my0 < my1) store_v<D>(vs0, vr, wave, lane);
    __syncthreads();   // stage 0, the query rows and the page ids in LDS
    {
      const int sw = swz<D>(lrow);
      const uint32_t qbase = (uint32_t)((lrow & 15) * GE::kRowBytes) + ((uint32_t)(half ^ (sw & 1)) << 4) +
                             ((uint32_t)(sw >> 1) << 5);
      const unsigned char* qsrc = lrow < 16 ? qk : qvs;
#pragma unroll
      for (int s = 0; s < GE::kKSteps; ++s)
        qv[0][s] = *reinterpret_cast<const uint4*>(qsrc + (qbase ^ (uint32_t)(s << 5)));
      __builtin_amdgcn_s_waitcnt(0);   // read before this wave's first copy into stage 1
    }
    int next_id = wave_page(my0 + 1);
    for (int i = 0;;) {
      int kt = my0 + i;
      if (kt + 1 < my1)
        load_tile<D>(ks1, vr, kpool, vpool, __builtin_amdgcn_readfirstlane(next_id), kt + 1, L, Hkv, g, wave, lane);
      next_id = wave_page(kt + 2);
      if (kt < my1) compute_tile(ks0, vs0, kt * kTileKeys);
      __builtin_amdgcn_s_waitcnt(0);
      if (kt + 1 < my1) store_v<D>(vs1, vr, wave, lane);
      __syncthreads();
      if (++i >= nloop) break;
      kt = my0 + i;
      if (kt + 1 < my1)
        load_tile<D>(ks0, vr, kpool, vpool, __builtin_amdgcn_readfirstlane(next_id), kt + 1, L, Hkv, g, wave, lane);
      next_id = wave_page(kt + 2);
      if (kt < my1) compute_tile(ks1, vs1, kt * kTileKeys);
      __builtin_amdgcn_s_waitcnt(0);
      if (kt + 1 < my1) store_v<D>(vs0, vr, wave, lane);
      __syncthreads();
      if (++i >= nloop) break;
    }
  };
  if (grp == 0)
    run(GroupTag<0>{});
  else
    run(GroupTag<1>{});

  // ---- merge the groups ----
  // Every lane of both groups owns the same (row, dims), so the merge is the
  // log-sum-exp rule applied lane by lane.  Each group keeps half of the dim
  // blocks (group 0 the first, group 1 the second) and hands the other half
  // to the other group through its own stage buffers, which are free now
  // (the last barrier above ended all reads): wave w of a group writes into
  // one buffer, float4 j of lane l at j*1024 + l*16.  Both groups then
  // finalize and store their half, so the exchange and the output stores
  // are shared by all eight waves.  The merged values are formed by the
  // same expression in both groups (group 0's state first), so the row sums
  // the two halves are normalized by are bit-identical.
  constexpr int kHalf = GE::kDimBlocks / 2;
  static_assert(GE::kDimBlocks % 2 == 0, "two halves of the dim blocks");
  // the running max and sum follow the float4s in the same buffer
  constexpr int kMlOff = kHalf * 4 * 1024;
  static_assert(kMlOff + 2 * 64 * 4 <= GE::kTileBytes, "exchange fits a stage buffer");
  // the final rows go out through a wave-private region after the exchange
  // data: 32 rows x kHalf * 64 bytes of bf16, 16-byte chunks XOR-swizzled
  // by row
  constexpr int kRowB = kHalf * 64;          // bytes of a row's half
  constexpr int kChunks = kRowB / 16;        // 16-byte chunks per row half
  constexpr int kRowsPerStore = 64 / kChunks;
  constexpr int kTransOff = kMlOff + 2 * 64 * 4;
  static_assert(kTransOff + 32 * kRowB <= GE::kTileBytes, "transpose region fits a stage buffer");
  auto finish = [&](auto gtag) __attribute__((always_inline)) {
    constexpr int GRP = decltype(gtag)::value;
    constexpr int kKeep = GRP == 0 ? 0 : kHalf;   // first dim block this group keeps
    constexpr int kGive = GRP == 0 ? kHalf : 0;   // first dim block it hands over
    unsigned char* mine = GRP == 0 ? (wave == 0 ? k_a0 : (wave == 1 ? v_a0 : (wave == 2 ? k_a1 : v_a1)))
                                   : (wave == 0 ? k_b0 : (wave == 1 ? v_b0 : (wave == 2 ? k_b1 : v_b1)));
    const unsigned char* theirs =
        GRP == 1 ? (wave == 0 ? k_a0 : (wave == 1 ? v_a0 : (wave == 2 ? k_a1 : v_a1)))
                 : (wave == 0 ? k_b0 : (wave == 1 ? v_b0 : (wave == 2 ? k_b1 : v_b1)));
#pragma unroll
    for (int j = 0; j < kHalf; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float4 w;
        w.x = oacc[0][kGive + j][4 * v + 0];
        w.y = oacc[0][kGive + j][4 * v + 1];
        w.z = oacc[0][kGive + j][4 * v + 2];
        w.w = oacc[0][kGive + j][4 * v + 3];
        *reinterpret_cast<float4*>(mine + (j * 4 + v) * 1024 + lane * 16) = w;
      }
    reinterpret_cast<float*>(mine + kMlOff)[lane] = m_run[0];
    reinterpret_cast<float*>(mine + kMlOff)[64 + lane] = l_run[0];
    __syncthreads();
    const float mO = reinterpret_cast<const float*>(theirs + kMlOff)[lane];
    const float lO = reinterpret_cast<const float*>(theirs + kMlOff)[64 + lane];
    const float mA = GRP == 0 ? m_run[0] : mO;   // group 0's state
    const float mB = GRP == 0 ? mO : m_run[0];
    const float lA = GRP == 0 ? l_run[0] : lO;
    const float lB = GRP == 0 ? lO : l_run[0];
    const float M = fmaxf(mA, mB);
    const float fA = mA == -INFINITY ? 0.f : fast_exp2(mA - M);
    const float fB = mB == -INFINITY ? 0.f : fast_exp2(mB - M);
#pragma unroll
    for (int j = 0; j < kHalf; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float4 w = *reinterpret_cast<const float4*>(theirs + (j * 4 + v) * 1024 + lane * 16);
        const float o4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float own = oacc[0][kKeep + j][4 * v + e];
          const float xa = GRP == 0 ? own : o4[e];
          const float xb = GRP == 0 ? o4[e] : own;
          oacc[0][kKeep + j][4 * v + e] = xa * fA + xb * fB;
        }
      }
    l_run[0] = lA * fA + lB * fB;
    m_run[0] = M;

    // ---- normalize and write this group's half: final output, or the split's partial
    const bool partial = nsp > 1;
    const size_t unit = ((size_t)r * T + t) * Hkv + g;
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      const float l_tot = pair_sum(l_run[rb]);
      const bool empty = !(l_tot > 0.f);
      const float inv = empty ? 0.f : 1.f / l_tot;
      const float lse = empty ? -INFINITY : (m_run[rb] + __log2f(l_tot)) * kLn2;
      if (!partial) {
        // Each lane writes its pieces of its row into the wave's region,
        // then reads 16 contiguous bytes of one row: a store instruction
        // then writes whole row halves (kRowsPerStore rows of kRowB bytes)
        // instead of 16 bytes in each of 32 rows.  Only this wave touches
        // the region, and its LDS operations complete in order.
        unsigned char* tp = mine + kTransOff;
#pragma unroll
        for (int j = 0; j < kHalf; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int db = kKeep + j;
            const int c = 4 * j + v;   // 16-byte chunk of the row half (8 dims)
            uint2 w;
            w.x = pack_bf16x2(oacc[rb][db][4 * v + 0] * inv, oacc[rb][db][4 * v + 1] * inv);
            w.y = pack_bf16x2(oacc[rb][db][4 * v + 2] * inv, oacc[rb][db][4 * v + 3] * inv);
            *reinterpret_cast<uint2*>(tp + lrow * kRowB + ((c ^ (lrow & (kChunks - 1))) * 16) + 8 * half) = w;
          }
        // output row of this lane's row (lanes 0-31 hold rows 0-31), or -1
        const int out_row =
            row_valid[rb] ? (q_start + tok[rb]) * Hq + g * group + hh[rb] : -1;
        __builtin_amdgcn_wave_barrier();
        constexpr int kStores = 32 / kRowsPerStore;
        const int cc = lane % kChunks;
        uint4 x[kStores];
        int orr[kStores];
#pragma unroll
        for (int i = 0; i < kStores; ++i) {   // all reads first, then the stores
          const int rr = lane / kChunks + i * kRowsPerStore;
          x[i] = *reinterpret_cast<const uint4*>(tp + rr * kRowB + ((cc ^ (rr & (kChunks - 1))) * 16));
          orr[i] = __shfl(out_row, rr);
        }
        // keep the reads ahead of the conditional stores (left alone, the
        // compiler sinks each read into its store's branch, one LDS round
        // trip after another)
#pragma unroll
        for (int i = 0; i < kStores; ++i) asm volatile("" : "+v"(x[i].x), "+v"(x[i].y), "+v"(x[i].z), "+v"(x[i].w));
#pragma unroll
        for (int i = 0; i < kStores; ++i)
          if (orr[i] >= 0)
            __builtin_nontemporal_store(
                u32x4_t{x[i].x, x[i].y, x[i].z, x[i].w},
                reinterpret_cast<u32x4_t*>(reinterpret_cast<__bf16*>(a.out) + (size_t)orr[i] * D + kKeep * 32 + cc * 8));
        if (GRP == 0 && a.lse != nullptr && half == 0 && row_valid[rb])
          a.lse[(size_t)(q_start + tok[rb]) * Hq + (size_t)g * group + hh[rb]] = lse;
      } else {
        if (!row_valid[rb]) continue;
        const int prow = wave * kRowsPerWave + rb * 32 + lrow;   // row within the tile
        const size_t pidx = (unit * S + split) * kTileRows + prow;
        float* po = a.part_o + pidx * D;
#pragma unroll
        for (int j = 0; j < kHalf; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int db = kKeep + j;
            float4 w;
            w.x = oacc[rb][db][4 * v + 0] * inv;
            w.y = oacc[rb][db][4 * v + 1] * inv;
            w.z = oacc[rb][db][4 * v + 2] * inv;
            w.w = oacc[rb][db][4 * v + 3] * inv;
            *reinterpret_cast<float4*>(po + db * 32 + 8 * v + 4 * half) = w;
          }
        if (GRP == 0 && half == 0) a.part_lse[pidx] = lse;
      }
    }
  };
  if (grp == 0)
    finish(GroupTag<0>{});
  else
    finish(GroupTag<1>{});
}

}  // namespace pf
}  // namespace pa
