// Paged decode attention and its split-K partitions (gfx950).
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
#include "pa_internal.h"

#include <math.h>

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kRescaleLog2 = 8.0f;
constexpr float kLn2 = 0.693147180559945309f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <typename T, int D, int G>
struct Shape {
  static constexpr int kVec = 16 / (int)sizeof(T);   // elements per 16-byte chunk
  static constexpr int kChunks = D / kVec;            // chunks per key row
  static constexpr int kLptMin = (G * D + 63) / 64;   // accumulator <= 64 floats
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

// Issue the loads of one K or V block (16 keys x d, contiguous).  Every K/V
// byte is read exactly once, so the loads are marked nontemporal (streamed
// past the caches), which sustains a higher HBM read rate.
template <typename T, int D, int G>
__device__ __forceinline__ void load_half(Half<T, D, G>& hr, const T* __restrict__ blk, int row0,
                                          int col) {
  using S = Shape<T, D, G>;
#pragma unroll
  for (int kk = 0; kk < S::kKeysPerLane; ++kk) {
#pragma unroll
    for (int jj = 0; jj < S::kChunksPerLane; ++jj) {
      const int off = (row0 + S::kRowsPerLoad * kk) * D + (col + S::kLpt * jj) * S::kVec;
      const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(blk + off));
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
__global__ void __launch_bounds__(kThreads)
decode_kernel(DecodeArgs a) {
  using S = Shape<T, D, G>;
  const int32_t num_pages = a.num_pages;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane % S::kLpt;
  const int row0 = lane / S::kLpt;

  const int nsplit = a.num_splits;
  const int bid = blockIdx.x;
  const int split = bid % nsplit;
  const int rg = bid / nsplit;
  const int g = rg % a.num_kv_heads;
  const int r = rg / a.num_kv_heads;
  const int Hq = a.num_q_heads;
  const int Hkv = a.num_kv_heads;

  const int L = a.seq_lens[r];
  int npages = (L + kPageSize - 1) / kPageSize;
  npages = npages < a.max_pages_per_seq ? npages : a.max_pages_per_seq;
  const int pps = (npages + nsplit - 1) / nsplit;
  const int pb = split * pps;
  const int pe = (pb + pps) < npages ? (pb + pps) : npages;

  const T* __restrict__ qp = reinterpret_cast<const T*>(a.q);
  const T* __restrict__ kpool = reinterpret_cast<const T*>(a.k_pool);
  const T* __restrict__ vpool = reinterpret_cast<const T*>(a.v_pool);
  const int32_t* __restrict__ ptab = a.page_table + (size_t)r * a.max_pages_per_seq;

  // q chunks of the lane's dims for every head of the group
  uint4 qv[G][S::kChunksPerLane];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const T* qrow = qp + ((size_t)r * Hq + (size_t)g * G + h) * D;
#pragma unroll
    for (int jj = 0; jj < S::kChunksPerLane; ++jj)
      qv[h][jj] = *reinterpret_cast<const uint4*>(qrow + (col + S::kLpt * jj) * S::kVec);
  }

  WaveState<T, D, G> st;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.m[h] = -INFINITY;
    st.l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < S::kDimsPerLane; ++e) st.acc[h][e] = 0.f;
  }

  const size_t blk = (size_t)kPageSize * D;  // elements of one (page, head) block
  auto block_of = [&](int pg) -> size_t {
    int phys = ptab[pg];
    phys = phys < 0 ? 0 : (phys >= num_pages ? num_pages - 1 : phys);
    return ((size_t)phys * Hkv + g) * blk;
  };

  // Staggered software pipeline over the wave's pages p, p+4, p+8, ...:
  // K of the next page is requested before the current page's scores, V of
  // the next page before the current page's value update, so each load has a
  // full half-iteration of work in front of it while at most one extra block
  // of K and one of V are held in registers.
  int p = pb + wave;
  if (p < pe) {
    Half<T, D, G> kc, kn, vc, vn;
    size_t off = block_of(p);
    load_half<T, D, G>(kc, kpool + off, row0, col);
    load_half<T, D, G>(vc, vpool + off, row0, col);
#pragma unroll 1
    for (;;) {
      const int pn = p + kWaves;
      const bool more = pn < pe;
      size_t offn = 0;
      if (more) {
        offn = block_of(pn);
        load_half<T, D, G>(kn, kpool + offn, row0, col);
      }
      const int live = L - p * kPageSize;  // >= 16 except on the last page
      float pr[S::kKeysPerLane][G];
      page_scores<T, D, G>(kc, qv, st, live, row0, a.scale_log2, pr);
      if (more) load_half<T, D, G>(vn, vpool + offn, row0, col);
      page_values<T, D, G>(vc, st, live, row0, pr);
      if (!more) break;
      kc = kn;
      vc = vn;
      p = pn;
    }
  }

  // ---- merge the wave's lanes that hold different keys of the same dims ----
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

  // ---- merge the waves through LDS ----
  __shared__ float sm_m[kWaves][G];
  __shared__ float sm_l[kWaves][G];
  __shared__ float sm_acc[kWaves][G][D];
  if (row0 == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (col == 0) {
        sm_m[wave][h] = st.m[h];
        sm_l[wave][h] = st.l[h];
      }
#pragma unroll
      for (int jj = 0; jj < S::kChunksPerLane; ++jj)
#pragma unroll
        for (int e = 0; e < S::kVec; ++e)
          sm_acc[wave][h][(col + S::kLpt * jj) * S::kVec + e] = st.acc[h][jj * S::kVec + e];
    }
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D;
    const int dim = idx % D;
    float Mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) Mt = fmaxf(Mt, sm_m[w][h]);
    float lt = 0.f, ot = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm_m[w][h];
      const float f = (mw == -INFINITY) ? 0.f : fast_exp2(mw - Mt);
      lt += f * sm_l[w][h];
      ot += f * sm_acc[w][h][dim];
    }
    const int hq = g * G + h;
    const bool empty = !(lt > 0.f);
    const float o = empty ? 0.f : ot / lt;
    const float lse2 = empty ? -INFINITY : (Mt + __log2f(lt)) * kLn2;
    if (!a.write_partials) {
      T* out = reinterpret_cast<T*>(a.out);
      out[((size_t)r * Hq + hq) * D + dim] = from_float<T>(o);
      if (a.lse != nullptr && dim == 0) a.lse[(size_t)r * Hq + hq] = lse2;
    } else {
      const size_t row = ((size_t)r * Hq + hq) * nsplit + split;
      a.o_part[row * D + dim] = o;
      if (dim == 0) a.lse_part[row] = lse2;
    }
  }
}

template <typename T, int D, int G>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s) {
  const long long grid = (long long)a.num_seqs * a.num_kv_heads * a.num_splits;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_kernel<T, D, G>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_g(const DecodeArgs& a, int group, hipStream_t s) {
  switch (group) {
    case 1: return launch_t<T, D, 1>(a, s);
    case 2: return launch_t<T, D, 2>(a, s);
    case 4: return launch_t<T, D, 4>(a, s);
    case 8: return launch_t<T, D, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool decode_group_supported(int group) {
  return group == 1 || group == 2 || group == 4 || group == 8;
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, int head_dim, int group, hipStream_t s) {
  if (dtype == 0) {
    if (head_dim == 128) return launch_g<__bf16, 128>(a, group, s);
    if (head_dim == 64) return launch_g<__bf16, 64>(a, group, s);
  } else if (dtype == 1) {
    if (head_dim == 128) return launch_g<float, 128>(a, group, s);
    if (head_dim == 64) return launch_g<float, 64>(a, group, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
