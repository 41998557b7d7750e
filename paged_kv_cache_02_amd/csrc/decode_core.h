// Device building blocks of the paged decode kernels (gfx950): the lane
// layout of a (page, KV head) block, pipelined K/V block loads, the
// per-page online-softmax update, and the body that walks one (request, KV
// head) page range with a workgroup of 4 or 8 waves.  Shared by the decode
// kernels and the mixed prefill/decode kernel.
//
// Lane layout inside a wave, for one (page, KV head) block of 16 keys x d:
// the block is read as 16-byte chunks; LPT consecutive lanes cover one key
// row (LPT in {4, 8, 16}, chosen so that the G x d accumulator costs at most
// 64 floats per lane), so one wave load instruction reads 64/LPT full key
// rows and every row segment it touches is LPT*16 contiguous bytes.  A
// lane's score partial for its key is reduced over the LPT lanes of the row
// with DPP butterflies (quad_perm, row_half_mirror, row_mirror); the softmax
// state (running max m, running sum l) is per lane and per head, and the
// lane accumulates p * v for its own dims only.  The running max is updated
// lazily: the accumulator is rescaled only when a score exceeds the current
// reference max by more than 2^8, which keeps exp2 bounded and leaves the
// result exact up to rounding.
//
// Scores use v_dot2_f32_bf16 on the stored bf16 pairs (exact products,
// float32 sums); everything after the dot product is float32.  Scores are
// kept in base-2 units (scale * log2 e folded in), and lse is converted back
// to natural log on output.
//
// Keys past seq_len in the last page are masked with selects (never a
// multiply by zero), so NaN in page tails cannot leak; page-table entries
// past the request's last page are never read.
#pragma once

#include "pa_internal.h"

#include <math.h>

namespace pa {
namespace dec {

constexpr float kRescaleLog2 = 8.0f;
constexpr float kLn2 = 0.693147180559945309f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <typename T, int D, int G>
struct Shape {
  static constexpr int kVec = 16 / (int)sizeof(T);   // elements per 16-byte chunk
  static constexpr int kChunks = D / kVec;            // chunks per key row
  static constexpr int kAccMax = 32;                  // accumulator floats per lane
  static constexpr int kLptMin = (G * D + kAccMax - 1) / kAccMax;
  static constexpr int kLpt0 = kLptMin <= 4 ? 4 : (kLptMin <= 8 ? 8 : 16);
  static constexpr int kLpt = kLpt0 > kChunks ? kChunks : kLpt0;  // lanes per key row
  static constexpr int kRowsPerLoad = 64 / kLpt;      // key rows per wave load
  static constexpr int kKeysPerLane = kPageSize / kRowsPerLoad;
  static constexpr int kChunksPerLane = kChunks / kLpt;
  static constexpr int kDimsPerLane = kChunksPerLane * kVec;
  static_assert(kPageSize % kRowsPerLoad == 0, "page must split into whole wave loads");
  static_assert(kChunks % kLpt == 0, "row must split into whole lane groups");
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the LPT consecutive lanes that share a key row; every lane of the
// group receives the total.
template <int LPT>
__device__ __forceinline__ float row_group_sum(float x) {
  x += dpp<0xB1>(x);                              // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);                              // quad_perm [2,3,0,1]
  if constexpr (LPT >= 8) x += dpp<0x141>(x);     // row_half_mirror
  if constexpr (LPT >= 16) x += dpp<0x140>(x);    // row_mirror
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u) {
  return __builtin_bit_cast(bf16x2_t, u);
}

// Dot product of one 16-byte chunk of q with one 16-byte chunk of k.
template <typename T>
__device__ __forceinline__ float chunk_dot(const uint4& q, const uint4& k, float acc);

template <>
__device__ __forceinline__ float chunk_dot<__bf16>(const uint4& q, const uint4& k, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.x), as_bf16x2(k.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.y), as_bf16x2(k.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.z), as_bf16x2(k.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.w), as_bf16x2(k.w), acc, false);
  return acc;
}

template <>
__device__ __forceinline__ float chunk_dot<float>(const uint4& q, const uint4& k, float acc) {
  acc = fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
  acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
  acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
  acc = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
  return acc;
}

// Unpack one 16-byte chunk of V to float32.
template <typename T>
__device__ __forceinline__ void chunk_unpack(const uint4& v, float* f);

template <>
__device__ __forceinline__ void chunk_unpack<__bf16>(const uint4& v, float* f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

template <>
__device__ __forceinline__ void chunk_unpack<float>(const uint4& v, float* f) {
  f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}

template <typename T>
__device__ __forceinline__ T from_float(float x);
template <>
__device__ __forceinline__ __bf16 from_float<__bf16>(float x) { return (__bf16)x; }
template <>
__device__ __forceinline__ float from_float<float>(float x) { return x; }

template <typename T, int D, int G>
struct Half {  // the K (or V) registers of one (page, KV head) block
  using S = Shape<T, D, G>;
  uint4 c[S::kKeysPerLane][S::kChunksPerLane];
};

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// Cache-policy bits of a buffer load: nontemporal (streamed past the caches).
constexpr int kLoadNontemporal = 2;

// Issue the loads of one K or V block (16 keys x d, contiguous) through a
// raw buffer resource that covers exactly that block.  Every K/V byte is read
// once, so the loads are nontemporal.  A resource with zero records makes
// every load of the block return zeros without touching memory, which lets
// the software pipeline issue its lookahead loads unconditionally (the
// wait counts the compiler inserts then stay exact across iterations).
template <typename T, int D, int G>
__device__ __forceinline__ void load_half(Half<T, D, G>& hr, const T* blk, bool live, int row0,
                                          int col) {
  using S = Shape<T, D, G>;
  const int bytes = live ? kPageSize * D * (int)sizeof(T) : 0;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(blk), (short)0, bytes, kBufferWord3);
#pragma unroll
  for (int kk = 0; kk < S::kKeysPerLane; ++kk) {
#pragma unroll
    for (int jj = 0; jj < S::kChunksPerLane; ++jj) {
      const int off = (row0 + S::kRowsPerLoad * kk) * D + (col + S::kLpt * jj) * S::kVec;
      const u32x4_t v =
          __builtin_amdgcn_raw_buffer_load_b128(rs, off * (int)sizeof(T), 0, kLoadNontemporal);
      hr.c[kk][jj] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  }
}

template <typename T, int D, int G>
struct WaveState {
  using S = Shape<T, D, G>;
  float m[G];
  float l[G];
  float acc[G][S::kDimsPerLane];
};

// Scores of the lane's keys of one page -> probabilities p[kk][h], with the
// online-softmax reference max and running sum updated.  All scores of the
// page are formed first and the reference max is moved at most once per
// page, before any probability is taken, so every p of the page shares the
// reference the accumulator is kept at.  Keys at index >= live_keys inside
// the page get p = 0 through selects.
template <typename T, int D, int G>
__device__ __forceinline__ void page_scores(const Half<T, D, G>& kr,
                                            const uint4 (&qv)[G][Shape<T, D, G>::kChunksPerLane],
                                            WaveState<T, D, G>& st, int live_keys, int row0,
                                            float scale_log2,
                                            float (&p)[Shape<T, D, G>::kKeysPerLane][G]) {
  using S = Shape<T, D, G>;
  float x[S::kKeysPerLane][G];
  float xmax[G];
#pragma unroll
  for (int h = 0; h < G; ++h) xmax[h] = -INFINITY;
#pragma unroll
  for (int kk = 0; kk < S::kKeysPerLane; ++kk) {
    const bool valid = row0 + S::kRowsPerLoad * kk < live_keys;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float s = 0.f;
#pragma unroll
      for (int jj = 0; jj < S::kChunksPerLane; ++jj) s = chunk_dot<T>(qv[h][jj], kr.c[kk][jj], s);
      s = row_group_sum<S::kLpt>(s);
      x[kk][h] = valid ? s * scale_log2 : -INFINITY;
      xmax[h] = fmaxf(xmax[h], x[kk][h]);
    }
  }
  bool need = false;
#pragma unroll
  for (int h = 0; h < G; ++h) need |= xmax[h] > st.m[h] + kRescaleLog2;
  if (__builtin_expect(__any(need), 0)) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mn = fmaxf(st.m[h], xmax[h]);
      const float alpha = (mn == st.m[h]) ? 1.f : fast_exp2(st.m[h] - mn);
      st.l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < S::kDimsPerLane; ++e) st.acc[h][e] *= alpha;
      st.m[h] = mn;
    }
  }
#pragma unroll
  for (int kk = 0; kk < S::kKeysPerLane; ++kk) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      // x = -inf (dead key) gives exp2(-inf) = 0; m = -inf only while every
      // key seen so far is dead, and then x is -inf as well
      p[kk][h] = x[kk][h] == -INFINITY ? 0.f : fast_exp2(x[kk][h] - st.m[h]);
      st.l[h] += p[kk][h];
    }
  }
}

// acc += p * V for the lane's keys and dims of one page.
template <typename T, int D, int G>
__device__ __forceinline__ void page_values(const Half<T, D, G>& vr, WaveState<T, D, G>& st,
                                            int live_keys, int row0,
                                            const float (&p)[Shape<T, D, G>::kKeysPerLane][G]) {
  using S = Shape<T, D, G>;
#pragma unroll
  for (int kk = 0; kk < S::kKeysPerLane; ++kk) {
    const bool valid = row0 + S::kRowsPerLoad * kk < live_keys;
#pragma unroll
    for (int jj = 0; jj < S::kChunksPerLane; ++jj) {
      uint4 raw = vr.c[kk][jj];
      // a dead key's V may hold NaN: select it to zero (0 * NaN would leak)
      raw.x = valid ? raw.x : 0u;
      raw.y = valid ? raw.y : 0u;
      raw.z = valid ? raw.z : 0u;
      raw.w = valid ? raw.w : 0u;
      float vf[S::kVec];
      chunk_unpack<T>(raw, vf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 0; e < S::kVec; ++e)
          st.acc[h][jj * S::kVec + e] = fmaf(p[kk][h], vf[e], st.acc[h][jj * S::kVec + e]);
      }
    }
  }
}

template <typename T, int D, int G>
__device__ __forceinline__ void reset_state(WaveState<T, D, G>& st) {
  using S = Shape<T, D, G>;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.m[h] = -INFINITY;
    st.l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < S::kDimsPerLane; ++e) st.acc[h][e] = 0.f;
  }
}

// Combine the wave's lanes that hold different keys of the same dims (the
// lanes that differ in row0): afterwards every lane holds the wave's total
// m, l and acc for its dims, by the log-sum-exp rule.
template <typename T, int D, int G>
__device__ __forceinline__ void wave_combine(WaveState<T, D, G>& st) {
  using S = Shape<T, D, G>;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float M = st.m[h];
#pragma unroll
    for (int o = S::kLpt; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float f = (st.m[h] == -INFINITY) ? 0.f : fast_exp2(st.m[h] - M);
    float lsum = st.l[h] * f;
#pragma unroll
    for (int o = S::kLpt; o < 64; o <<= 1) lsum += __shfl_xor(lsum, o);
    st.l[h] = lsum;
    st.m[h] = M;
#pragma unroll
    for (int e = 0; e < S::kDimsPerLane; ++e) {
      float v = st.acc[h][e] * f;
#pragma unroll
      for (int o = S::kLpt; o < 64; o <<= 1) v += __shfl_xor(v, o);
      st.acc[h][e] = v;
    }
  }
}

// q chunks of the lane's dims for the G query heads of KV head g of request
// r, through a buffer resource; valid = false gives zeros and reads nothing.
template <typename T, int D, int G>
using QRegs = uint4[G][Shape<T, D, G>::kChunksPerLane];

// G is the padded head count the registers hold; Gr <= G is the real group
// size: heads Gr .. G-1 read zeros (the resource covers Gr heads).
template <typename T, int D, int G>
__device__ __forceinline__ void load_q(QRegs<T, D, G>& qv, const T* q, int Hq, int r, int g, int Gr,
                                       bool valid, int col) {
  using S = Shape<T, D, G>;
  const T* base = q + ((size_t)r * Hq + (size_t)g * Gr) * D;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(base), (short)0, valid ? Gr * D * (int)sizeof(T) : 0, kBufferWord3);
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int jj = 0; jj < S::kChunksPerLane; ++jj) {
      const int off = h * D + (col + S::kLpt * jj) * S::kVec;
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, off * (int)sizeof(T), 0, 0);
      qv[h][jj] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  }
}

// Depth of the K/V software pipeline: while page i is scored and accumulated,
// the K and V blocks of pages i+1 .. i+kDepth are in flight.  The depth is
// the largest (up to 4) whose buffers still leave room for two waves per
// SIMD: accumulator + q (+ kExtraRegs) + scores/probabilities + 2 (depth + 1)
// K/V buffers within 224 VGPRs.
template <typename T, int D, int G, int kExtraRegs>
struct Pipe {
  using S = Shape<T, D, G>;
  static constexpr int kHalfRegs = (int)(sizeof(Half<T, D, G>) / 4);
  static constexpr int kFixedRegs = G * S::kDimsPerLane + G * S::kChunksPerLane * 4 +
                                    2 * G * S::kKeysPerLane + kExtraRegs;
  static constexpr int kDepth = kFixedRegs + 10 * kHalfRegs <= 224  ? 4
                                : kFixedRegs + 8 * kHalfRegs <= 224 ? 3
                                : kFixedRegs + 6 * kHalfRegs <= 224 ? 2
                                                                    : 1;
  static constexpr int kBufs = kDepth + 1;
};

// ---------------------------------------------------------------------------
// The (page, KV head) block on MFMA (bf16): S^T = K Q^T with
// v_mfma_f32_16x16x32_bf16 (lane j holds key j%16, dims 32c + 8(j/16) .. +7
// of k-step c; the G query heads sit in the 16 columns of Q^T, the others
// load zeros), whose result (lane j: keys 4(j/16) .. +3 of head j%16) is
// the A operand of O += P V with v_mfma_f32_16x16x16bf16_1k; V's B operand
// comes from the wave's own LDS slot through ds_read_b64_tr_b16.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short shortx4_t __attribute__((ext_vector_type(4)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

template <int D>
struct MShape {
  static constexpr int kKSteps = D / 32;                // 16x16x32 steps of S^T
  static constexpr int kDimBlocks = D / 16;             // 16-dim output blocks of O
  static constexpr int kRowBytes = D * 2;               // one key row (bf16)
  static constexpr int kChunks = D / 8;                 // 16-byte chunks per key row
  static constexpr int kVLoads = kPageSize * D * 2 / 1024;   // 1 KB wave loads per V block
  static constexpr int kKeysPerVLoad = 1024 / kRowBytes;
};

// XOR swizzle of a key row's 16-byte chunks in the LDS slot (bit 0 left
// alone: the two chunks of one 16-dim block differ in it).
template <int D>
__device__ __forceinline__ int vswz(int key) {
  return D == 128 ? ((key & 7) << 1) : (((key >> 1) & 3) << 1);
}

template <int D>
struct MBlock {  // one (page, KV head) block in registers: K as the S^T A operand, V as loaded
  uint4 k[MShape<D>::kKSteps];
  uint4 v[MShape<D>::kVLoads];
};

template <int D>
__device__ __forceinline__ void load_mblock(MBlock<D>& b, const __bf16* kblk, const __bf16* vblk, bool live,
                                            int lane) {
  using M = MShape<D>;
  const int bytes = live ? kPageSize * M::kRowBytes : 0;
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(kblk), (short)0, bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(vblk), (short)0, bytes, kBufferWord3);
#pragma unroll
  for (int c = 0; c < M::kKSteps; ++c) {
    const int off = (lane & 15) * M::kRowBytes + (32 * c + 8 * (lane >> 4)) * 2;
    const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, kLoadNontemporal);
    b.k[c] = make_uint4(x[0], x[1], x[2], x[3]);
  }
#pragma unroll
  for (int t = 0; t < M::kVLoads; ++t) {
    const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(rv, t * 1024 + lane * 16, 0, kLoadNontemporal);
    b.v[t] = make_uint4(x[0], x[1], x[2], x[3]);
  }
}

template <int D>
struct MState {
  floatx4_t o[MShape<D>::kDimBlocks];   // lane j, reg i: head 4(j/16)+i, dim 16b + j%16
  float m;                              // running max of head j%16 (log2 units)
  float l;                              // this lane's part of head j%16's running sum
};

template <int D>
__device__ __forceinline__ void mreset(MState<D>& st) {
#pragma unroll
  for (int b = 0; b < MShape<D>::kDimBlocks; ++b) st.o[b] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;
}

// Q^T for one (row, KV head): lane j holds head j%16's dims 32c + 8(j/16)
// .. +7; heads at or past the group size Gr read zeros (the resource covers
// Gr heads).
template <int D>
__device__ __forceinline__ void load_qt(uint4 (&qt)[MShape<D>::kKSteps], const __bf16* q, int Hq, int row,
                                        int g, int Gr, bool valid, int lane) {
  using M = MShape<D>;
  const __bf16* base = q + ((size_t)row * Hq + (size_t)g * Gr) * D;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__bf16*>(base), (short)0, valid ? Gr * M::kRowBytes : 0, kBufferWord3);
#pragma unroll
  for (int c = 0; c < M::kKSteps; ++c) {
    const int off = (lane & 15) * M::kRowBytes + (32 * c + 8 * (lane >> 4)) * 2;
    const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    qt[c] = make_uint4(x[0], x[1], x[2], x[3]);
  }
}

// G: the padded group size the kernel is built for (it sets how many V
// operands are read ahead); Gr <= G: the real one (heads Gr.. are masked).
template <int D, int G>
__device__ __forceinline__ void page_mfma(const MBlock<D>& b, const uint4 (&qt)[MShape<D>::kKSteps],
                                          MState<D>& st, int live, float scale_log2,
                                          unsigned char* vslot, int lane, int Gr) {
  using M = MShape<D>;
  const int qg = lane >> 4;
  const int h = lane & 15;
  // ---- S^T = K Q^T
  floatx4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < M::kKSteps; ++c)
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, b.k[c]),
                                                __builtin_bit_cast(bf16x8_t, qt[c]), s, 0, 0, 0);
  // ---- V into the wave's LDS slot; keys at or past `live` (possibly NaN)
  // become zeros
#pragma unroll
  for (int t = 0; t < M::kVLoads; ++t) {
    const int key = t * M::kKeysPerVLoad + lane / M::kChunks;
    const int chunk = lane % M::kChunks;
    uint4 x = b.v[t];
    const bool ok = key < live;
    x.x = ok ? x.x : 0u;
    x.y = ok ? x.y : 0u;
    x.z = ok ? x.z : 0u;
    x.w = ok ? x.w : 0u;
    *reinterpret_cast<uint4*>(vslot + key * M::kRowBytes + ((chunk ^ vswz<D>(key)) << 4)) = x;
  }
  // ---- online softmax of head h over keys 4qg .. 4qg + 3 of the page
  float x[4];
  float xm = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = (4 * qg + i < live && h < Gr) ? s[i] * scale_log2 : -INFINITY;
    xm = fmaxf(xm, x[i]);
  }
  xm = fmaxf(xm, __shfl_xor(xm, 16));
  xm = fmaxf(xm, __shfl_xor(xm, 32));
  if (__builtin_expect(__any(xm > st.m + kRescaleLog2), 0)) {
    const float mn = fmaxf(st.m, xm);
    const float alpha = (mn == st.m) ? 1.f : fast_exp2(st.m - mn);
    st.l *= alpha;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ai = __shfl(alpha, 4 * qg + i);   // output row 4qg + i is head 4qg + i
#pragma unroll
      for (int bb = 0; bb < M::kDimBlocks; ++bb) st.o[bb][i] *= ai;
    }
    st.m = mn;
  }
  const float mref = st.m == -INFINITY ? 0.f : st.m;
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[i] = x[i] == -INFINITY ? 0.f : fast_exp2(x[i] - mref);
    st.l += p[i];
  }
  // p as the sum of two bf16 parts: a single bf16 rounding (up to 2^-8
  // relative) would move outputs of a few keys by up to |v| * 2^-8, which
  // with |v| ~ 4 is a bf16 output step; with hi + lo the products keep
  // about 16 bits, and V itself is exact
  bf16x4_t pa, pb;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pa[i] = (__bf16)p[i];
    pb[i] = (__bf16)(p[i] - (float)pa[i]);
  }
  // ---- O += P V: V's B operand through the transposing LDS read (key
  // 4qg + h/4, dims 16bb + 4(h%4) .. +3 in this lane's address)
  // the V operands are requested in batches of kBatch dim blocks ahead of
  // their MFMAs, so a page waits for a few LDS round trips rather than one
  // per dim block
  constexpr int kBatch = G >= 8 ? 2 : (M::kDimBlocks >= 4 ? 4 : M::kDimBlocks);   // G = 8 has no registers to spare
  const int vkey = 4 * qg + (h >> 2);
#pragma unroll
  for (int b0 = 0; b0 < M::kDimBlocks; b0 += kBatch) {
    shortx4_t vr[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int dim = 16 * (b0 + k) + 4 * (h & 3);
      const unsigned char* pa_addr =
          vslot + vkey * M::kRowBytes + (((dim >> 3) ^ vswz<D>(vkey)) << 4) + (dim & 7) * 2;
      vr[k] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) shortx4_t*)(pa_addr));
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const bf16x4_t vb = __builtin_bit_cast(bf16x4_t, vr[k]);
      st.o[b0 + k] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, st.o[b0 + k], 0, 0, 0);
      st.o[b0 + k] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pb, vb, st.o[b0 + k], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x0100, kBatch, 0);      // the batch's transposing reads
    __builtin_amdgcn_sched_group_barrier(0x0008, 2 * kBatch, 0);  // then its MFMAs
  }
}

// Head totals at a request's end: l summed over the head's four lanes.
template <int D>
__device__ __forceinline__ float head_sum(const MState<D>& st) {
  float l = st.l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  return l;
}


// One (request r, KV head g) over the request's logical pages [pb, pe), the
// pages dealt round-robin to the workgroup's kW waves (64 * kW threads).
// Each wave keeps its own online-softmax state; the states are merged
// through LDS by the log-sum-exp rule (with 8 waves, waves 4..7 first fold
// into waves 0..3, so the LDS holds four states).  qrow is the request's row
// of q, out and lse: r itself in a decode batch, the request's packed row in
// a mixed batch.  Writes out and lse, or the split's normalized partial when
// a.write_partials.
//
// kDense: the same walk over a dense cache [B, Hkv, MP * P, d] (request r's
// keys of KV head g contiguous, no page table), for measuring what the
// paging costs; a.max_pages_per_seq is then the cache capacity in pages.
template <typename T, int D, int G, int kW, bool kDense>
__device__ __forceinline__ void decode_range(const DecodeArgs& a, int r, int qrow, int g, int split,
                                             int pb, int pe, int L) {
  static_assert(kW == 4 || kW == 8, "4 or 8 waves per workgroup");
  constexpr int kSlots = 4;   // wave states LDS holds at once
  using S = Shape<T, D, G>;
  const int32_t num_pages = a.num_pages;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane % S::kLpt;
  const int row0 = lane / S::kLpt;
  const int nsplit = a.num_splits;
  const int Hq = a.num_q_heads;
  const int Hkv = a.num_kv_heads;

  const T* __restrict__ qp = reinterpret_cast<const T*>(a.q);
  const T* __restrict__ kpool = reinterpret_cast<const T*>(a.k_pool);
  const T* __restrict__ vpool = reinterpret_cast<const T*>(a.v_pool);
  const int32_t* __restrict__ ptab = kDense ? nullptr : a.page_table + (size_t)r * a.max_pages_per_seq;

  // q chunks of the lane's dims for every head of the group (G registers
  // sets, the real group size Gr of them loaded)
  const int Gr = Hq / Hkv;
  uint4 qv[G][S::kChunksPerLane];
  load_q<T, D, G>(qv, qp, Hq, qrow, g, Gr, true, col);

  WaveState<T, D, G> st;
  reset_state<T, D, G>(st);

  const size_t blk = (size_t)kPageSize * D;  // elements of one (page, head) block

  // The wave's pages are pb + wave + kW * i for i in [0, nw).  The physical
  // id of the page whose loads are issued next is fetched one step earlier
  // (a uniform, scalar load), so its latency is hidden behind a page of
  // work.
  const int first = pb + wave;
  const int nw = first < pe ? (pe - first + kW - 1) / kW : 0;
  auto page_id = [&](int i) -> int {  // clamped index: always a valid entry
    const int ic = i < nw ? i : nw - 1;
    if (kDense) return first + kW * ic;
    int phys = ptab[first + kW * ic];
    return phys < 0 ? 0 : (phys >= num_pages ? num_pages - 1 : phys);
  };
  auto block_ptr = [&](const T* pool, int phys) -> const T* {
    if (kDense) return pool + (((size_t)r * Hkv + g) * a.max_pages_per_seq + phys) * blk;
    return pool + ((size_t)phys * Hkv + g) * blk;
  };

  // Software pipeline Pipe::kDepth pages deep.  K of page i+kDepth is
  // requested before page i's scores and its V before page i's value update.
  // The kDepth+1 register buffers rotate through a fully unrolled inner loop,
  // so no buffer is ever copied.  Lookahead pages past the wave's last one
  // are loaded with zero-record resources.
  constexpr int kDepth = Pipe<T, D, G, 0>::kDepth;
  constexpr int kBufs = Pipe<T, D, G, 0>::kBufs;
  if (nw > 0) {
    Half<T, D, G> hk[kBufs], hv[kBufs];
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      const int phys = page_id(u);
      load_half<T, D, G>(hk[u], block_ptr(kpool, phys), u < nw, row0, col);
      load_half<T, D, G>(hv[u], block_ptr(vpool, phys), u < nw, row0, col);
    }
    int next_phys = page_id(kDepth);
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
        next_phys = page_id(ahead + 1);
        const int live = L - (first + kW * i) * kPageSize;  // >= 16 except on the last page
        float pr[S::kKeysPerLane][G];
        page_scores<T, D, G>(hk[u], qv, st, live, row0, a.scale_log2, pr);
        load_half<T, D, G>(hv[nb], block_ptr(vpool, phys), more, row0, col);
        page_values<T, D, G>(hv[u], st, live, row0, pr);
        if (++i >= nw) goto pages_done;
      }
    }
  }
pages_done:

  wave_combine<T, D, G>(st);

  // ---- merge the waves through LDS ----
  __shared__ float sm_m[kSlots][G];
  __shared__ float sm_l[kSlots][G];
  __shared__ float sm_acc[kSlots][G][D];
  auto put = [&](int slot) {
    if (row0 == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        if (col == 0) {
          sm_m[slot][h] = st.m[h];
          sm_l[slot][h] = st.l[h];
        }
#pragma unroll
        for (int jj = 0; jj < S::kChunksPerLane; ++jj)
#pragma unroll
          for (int e = 0; e < S::kVec; ++e)
            sm_acc[slot][h][(col + S::kLpt * jj) * S::kVec + e] = st.acc[h][jj * S::kVec + e];
      }
    }
  };
  if constexpr (kW > kSlots) {
    // waves kSlots.. hand their states to waves 0..kSlots-1, lane by lane
    if (wave >= kSlots) put(wave - kSlots);
    __syncthreads();
    if (wave < kSlots && row0 == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mb = sm_m[wave][h];
        const float lb = sm_l[wave][h];
        const float M = fmaxf(st.m[h], mb);
        const float fa = (st.m[h] == -INFINITY) ? 0.f : fast_exp2(st.m[h] - M);
        const float fb = (mb == -INFINITY) ? 0.f : fast_exp2(mb - M);
#pragma unroll
        for (int jj = 0; jj < S::kChunksPerLane; ++jj)
#pragma unroll
          for (int e = 0; e < S::kVec; ++e) {
            const float vb = sm_acc[wave][h][(col + S::kLpt * jj) * S::kVec + e];
            st.acc[h][jj * S::kVec + e] = st.acc[h][jj * S::kVec + e] * fa + vb * fb;
          }
        st.l[h] = st.l[h] * fa + lb * fb;
        st.m[h] = M;
      }
    }
    __syncthreads();
  }
  if (wave < kSlots) put(wave);
  __syncthreads();

  for (int idx = threadIdx.x; idx < Gr * D; idx += 64 * kW) {
    const int h = idx / D;
    const int dim = idx % D;
    float Mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < kSlots; ++w) Mt = fmaxf(Mt, sm_m[w][h]);
    float lt = 0.f, ot = 0.f;
#pragma unroll
    for (int w = 0; w < kSlots; ++w) {
      const float mw = sm_m[w][h];
      const float f = (mw == -INFINITY) ? 0.f : fast_exp2(mw - Mt);
      lt += f * sm_l[w][h];
      ot += f * sm_acc[w][h][dim];
    }
    const int hq = g * Gr + h;
    const bool empty = !(lt > 0.f);
    const float o = empty ? 0.f : ot / lt;
    const float lse2 = empty ? -INFINITY : (Mt + __log2f(lt)) * kLn2;
    if (!a.write_partials) {
      T* out = reinterpret_cast<T*>(a.out);
      out[((size_t)qrow * Hq + hq) * D + dim] = from_float<T>(o);
      if (a.lse != nullptr && dim == 0) a.lse[(size_t)qrow * Hq + hq] = lse2;
    } else {
      const size_t row = ((size_t)qrow * Hq + hq) * nsplit + split;
      a.o_part[row * D + dim] = o;
      if (dim == 0) a.lse_part[row] = lse2;
    }
  }
}

// decode_range with the page work on MFMA (bf16, 4 waves): the same page
// walk and LDS merge, with each wave's state in the MFMA layout (output
// rows = query heads) and a 4 KB LDS slot per wave for V's transposing
// reads.
template <int D, int G, bool kDense>
__device__ __forceinline__ void decode_range_mfma(const DecodeArgs& a, int r, int qrow, int g, int split,
                                                  int pb, int pe, int L) {
  using M = MShape<D>;
  constexpr int kW = 4;
  constexpr int kDepth = 3;
  constexpr int kBufs = kDepth + 1;
  __shared__ __align__(16) unsigned char vslots[kW][kPageSize * M::kRowBytes];
  const int32_t num_pages = a.num_pages;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nsplit = a.num_splits;
  const int Hq = a.num_q_heads;
  const int Hkv = a.num_kv_heads;
  const __bf16* __restrict__ qp = reinterpret_cast<const __bf16*>(a.q);
  const __bf16* __restrict__ kpool = reinterpret_cast<const __bf16*>(a.k_pool);
  const __bf16* __restrict__ vpool = reinterpret_cast<const __bf16*>(a.v_pool);
  const int32_t* __restrict__ ptab = kDense ? nullptr : a.page_table + (size_t)r * a.max_pages_per_seq;

  const int Gr = Hq / Hkv;
  uint4 qt[M::kKSteps];
  load_qt<D>(qt, qp, Hq, qrow, g, Gr, true, lane);
  MState<D> st;
  mreset<D>(st);

  const size_t blk = (size_t)kPageSize * D;
  const int first = pb + wave;
  const int nw = first < pe ? (pe - first + kW - 1) / kW : 0;
  auto page_id = [&](int i) -> int {
    const int ic = i < nw ? i : nw - 1;
    if (kDense) return first + kW * ic;
    int phys = ptab[first + kW * ic];
    return phys < 0 ? 0 : (phys >= num_pages ? num_pages - 1 : phys);
  };
  auto block_ptr = [&](const __bf16* pool, int phys) -> const __bf16* {
    if (kDense) return pool + (((size_t)r * Hkv + g) * a.max_pages_per_seq + phys) * blk;
    return pool + ((size_t)phys * Hkv + g) * blk;
  };
  if (nw > 0) {
    MBlock<D> bufs[kBufs];
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      const int phys = page_id(u);
      load_mblock<D>(bufs[u], block_ptr(kpool, phys), block_ptr(vpool, phys), u < nw, lane);
    }
    int next_phys = page_id(kDepth);
    int i = 0;
#pragma unroll 1
    for (;;) {
#pragma unroll
      for (int u = 0; u < kBufs; ++u) {
        const int ahead = i + kDepth;
        const int nb = (u + kDepth) % kBufs;
        const int phys = next_phys;
        load_mblock<D>(bufs[nb], block_ptr(kpool, phys), block_ptr(vpool, phys), ahead < nw, lane);
        next_phys = page_id(ahead + 1);
        const int live = L - (first + kW * i) * kPageSize;
        page_mfma<D, G>(bufs[u], qt, st, live, a.scale_log2, vslots[wave], lane, Gr);
        if (++i >= nw) goto pages_done;
      }
    }
  }
pages_done:

  // ---- merge the waves through LDS (heads' totals, rows in [head][dim])
  const float lh = head_sum<D>(st);
  __shared__ float sm_m[kW][G];
  __shared__ float sm_l[kW][G];
  __shared__ float sm_acc[kW][G][D];
  if (lane < Gr) {
    sm_m[wave][lane] = st.m;
    sm_l[wave][lane] = lh;
  }
  const int qg = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hh = 4 * qg + i;
    if (hh < Gr) {
#pragma unroll
      for (int bb = 0; bb < M::kDimBlocks; ++bb) sm_acc[wave][hh][16 * bb + (lane & 15)] = st.o[bb][i];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < Gr * D; idx += 64 * kW) {
    const int h = idx / D;
    const int dim = idx % D;
    float Mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < kW; ++w) Mt = fmaxf(Mt, sm_m[w][h]);
    float lt = 0.f, ot = 0.f;
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      const float mw = sm_m[w][h];
      const float f = (mw == -INFINITY) ? 0.f : fast_exp2(mw - Mt);
      lt += f * sm_l[w][h];
      ot += f * sm_acc[w][h][dim];
    }
    const int hq = g * Gr + h;
    const bool empty = !(lt > 0.f);
    const float o = empty ? 0.f : ot / lt;
    const float lse2 = empty ? -INFINITY : (Mt + __log2f(lt)) * kLn2;
    if (!a.write_partials) {
      __bf16* out = reinterpret_cast<__bf16*>(a.out);
      out[((size_t)qrow * Hq + hq) * D + dim] = (__bf16)o;
      if (a.lse != nullptr && dim == 0) a.lse[(size_t)qrow * Hq + hq] = lse2;
    } else {
      const size_t row = ((size_t)qrow * Hq + hq) * nsplit + split;
      a.o_part[row * D + dim] = o;
      if (dim == 0) a.lse_part[row] = lse2;
    }
  }
}

}  // namespace dec
}  // namespace pa
