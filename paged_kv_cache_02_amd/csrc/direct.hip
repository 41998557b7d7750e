// Direct (non-flash) paged decode attention (gfx950): a baseline for
// measuring what the online softmax saves.
//
// The pages name two forms of attention over the paged cache ("Build a vLLM
// from Scratch", Week 3): direct paged attention, which reads K and V
// through the page table instead of first concatenating them, and Paged
// FlashAttention, which also keeps no score matrix ("tiny-llm source
// reading", section "Paged KV Cache").  This kernel is the first without the
// second: one workgroup per (request, KV
// head) computes every score of its G query heads and stores them (fp32, in
// log2 units) in a scratch row, turns each head's row into softmax weights
// in place (max, then p = exp2(s - max) and their sum), and then sums the
// values weighted by p.  K and V are each read once, as in the fused kernel;
// the score rows add two writes and three reads of B * Hq * L floats.
//
// Page ids outside [0, num_pages) are clamped, as in the fused kernels; keys
// at or past seq_len are never read.
#include "pa_internal.h"

#include <math.h>

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr float kLn2 = 0.693147180559945309f;

template <typename T>
__device__ __forceinline__ float to_f(T x);
template <>
__device__ __forceinline__ float to_f<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f<__bf16>(__bf16 x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f(float x);
template <>
__device__ __forceinline__ float from_f<float>(float x) { return x; }
template <>
__device__ __forceinline__ __bf16 from_f<__bf16>(float x) { return (__bf16)x; }

// Workgroup max (op 0) or sum (op 1) of x; every thread gets the result.
__device__ __forceinline__ float block_reduce(float x, float* red, int op) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    const float y = __shfl_xor(x, s);
    x = op == 0 ? fmaxf(x, y) : x + y;
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float t = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) t = op == 0 ? fmaxf(t, red[w]) : t + red[w];
  return t;
}

template <typename T, int D, int G>
__global__ void __launch_bounds__(kThreads) direct_kernel(DirectArgs a) {
  __shared__ float q_s[G][D];
  __shared__ float red[kWaves];
  __shared__ float stat[2][G];           // per head: max, sum (log2 units)
  __shared__ float acc_s[kWaves][G][D];

  const int tid = threadIdx.x;
  const int Hkv = a.num_kv_heads;
  const int Hq = a.num_q_heads;
  const int g = blockIdx.x % Hkv;
  const int r = blockIdx.x / Hkv;
  const int L = a.seq_lens[r];
  const int Lcap = a.max_pages_per_seq * kPageSize;
  const int Lc = L < Lcap ? L : Lcap;
  const int32_t* __restrict__ ptab = a.page_table + (size_t)r * a.max_pages_per_seq;
  const T* __restrict__ kpool = reinterpret_cast<const T*>(a.k_pool);
  const T* __restrict__ vpool = reinterpret_cast<const T*>(a.v_pool);
  float* __restrict__ srow = a.scores + ((size_t)r * Hq + (size_t)g * G) * Lcap;   // [G][Lcap]

  for (int i = tid; i < G * D; i += kThreads) {
    const int h = i / D, c = i % D;
    q_s[h][c] = to_f(reinterpret_cast<const T*>(a.q)[((size_t)r * Hq + (size_t)g * G + h) * D + c]);
  }
  // the request's page ids, clamped, in LDS (read once, used for every key)
  extern __shared__ int ids_s[];
  const int npages = (Lc + kPageSize - 1) / kPageSize;
  for (int i = tid; i < npages; i += kThreads) {
    const int id = ptab[i];
    ids_s[i] = id < 0 ? 0 : (id >= a.num_pages ? a.num_pages - 1 : id);
  }
  __syncthreads();

  auto key_ptr = [&](const T* pool, int t) -> const T* {
    return pool + (((size_t)ids_s[t / kPageSize] * Hkv + g) * kPageSize + (t % kPageSize)) * D;
  };

  // ---- pass 1: every score, stored ----
  // A key's row is kLanes 16-byte chunks read by kLanes lanes together (a
  // wave covers kKeys keys per step); each lane holds its chunk of every
  // group head's query and the partial dots meet by a butterfly over the
  // key's lanes.
  constexpr int kPer = 16 / (int)sizeof(T);            // elements per 16-byte chunk
  constexpr int kLanes = D / kPer;                     // lanes per key
  constexpr int kKeys = 64 / kLanes;                   // keys per wave step
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int sub = lane / kLanes;
  const int ch = lane % kLanes;
  float qr[G][kPer];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < kPer; ++e) qr[h][e] = q_s[h][ch * kPer + e];
  for (int t0 = wave * kKeys; t0 < Lc; t0 += kWaves * kKeys) {
    const int t = t0 + sub;
    float s[G];
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = 0.f;
    if (t < Lc) {
      const uint4 raw = *reinterpret_cast<const uint4*>(key_ptr(kpool, t) + ch * kPer);
      const T* kv = reinterpret_cast<const T*>(&raw);
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        const float x = to_f(kv[e]);
#pragma unroll
        for (int h = 0; h < G; ++h) s[h] = fmaf(qr[h][e], x, s[h]);
      }
    }
#pragma unroll
    for (int o = 1; o < kLanes; o <<= 1)
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] += __shfl_xor(s[h], o);
    if (ch == 0 && t < Lc) {
#pragma unroll
      for (int h = 0; h < G; ++h) srow[(size_t)h * Lcap + t] = s[h] * a.scale_log2;
    }
  }
  __syncthreads();

  // ---- pass 2: softmax over the stored scores, each head's row replaced
  // by its weights p = exp2(s - max), and their sum ----
  for (int h = 0; h < G; ++h) {
    float m = -INFINITY;
    for (int t = tid; t < Lc; t += kThreads) m = fmaxf(m, srow[(size_t)h * Lcap + t]);
    m = block_reduce(m, red, 0);
    float l = 0.f;
    for (int t = tid; t < Lc; t += kThreads) {
      const float p = exp2f(srow[(size_t)h * Lcap + t] - m);
      srow[(size_t)h * Lcap + t] = p;
      l += p;
    }
    l = block_reduce(l, red, 1);
    if (tid == 0) {
      stat[0][h] = m;
      stat[1][h] = l;
    }
  }
  __syncthreads();

  // ---- pass 3: the weighted sum of the values ----
  // As in pass 1, a value row is read by kLanes lanes together, a wave
  // covering kKeys keys per step; each lane sums its chunk of dims over its
  // keys for every group head, then the key groups of a wave meet by a
  // butterfly and the waves through LDS.
  float acc[G][kPer];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < kPer; ++e) acc[h][e] = 0.f;
  for (int t0 = wave * kKeys; t0 < Lc; t0 += kWaves * kKeys) {
    const int t = t0 + sub;
    if (t < Lc) {
      const uint4 raw = *reinterpret_cast<const uint4*>(key_ptr(vpool, t) + ch * kPer);
      const T* vv = reinterpret_cast<const T*>(&raw);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = srow[(size_t)h * Lcap + t];
#pragma unroll
        for (int e = 0; e < kPer; ++e) acc[h][e] = fmaf(p, to_f(vv[e]), acc[h][e]);
      }
    }
  }
#pragma unroll
  for (int o = kLanes; o < 64; o <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < kPer; ++e) acc[h][e] += __shfl_xor(acc[h][e], o);
  if (sub == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < kPer; ++e) acc_s[wave][h][ch * kPer + e] = acc[h][e];
  }
  __syncthreads();
  for (int i = tid; i < G * D; i += kThreads) {
    const int h = i / D, c = i % D;
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) o += acc_s[w][h][c];
    const float l = stat[1][h];
    const bool empty = !(l > 0.f);
    const size_t row = (size_t)r * Hq + (size_t)g * G + h;
    reinterpret_cast<T*>(a.out)[row * D + c] = from_f<T>(empty ? 0.f : o / l);
    if (a.lse != nullptr && c == 0) a.lse[row] = empty ? -INFINITY : (stat[0][h] + __log2f(l)) * kLn2;
  }
}

template <typename T, int D>
hipError_t launch_g(const DirectArgs& a, int group, hipStream_t s) {
  const long long grid = (long long)a.num_seqs * a.num_kv_heads;
  if (grid <= 0) return hipSuccess;
  const size_t lds = (size_t)a.max_pages_per_seq * sizeof(int);   // the page ids of one request
  if (grid > 0x7FFFFFFFLL || lds > 48 * 1024) return hipErrorInvalidValue;
  switch (group) {
    case 1: hipLaunchKernelGGL((direct_kernel<T, D, 1>), dim3((unsigned)grid), dim3(kThreads), lds, s, a); break;
    case 2: hipLaunchKernelGGL((direct_kernel<T, D, 2>), dim3((unsigned)grid), dim3(kThreads), lds, s, a); break;
    case 4: hipLaunchKernelGGL((direct_kernel<T, D, 4>), dim3((unsigned)grid), dim3(kThreads), lds, s, a); break;
    case 8: hipLaunchKernelGGL((direct_kernel<T, D, 8>), dim3((unsigned)grid), dim3(kThreads), lds, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_direct(const DirectArgs& a, int dtype, int head_dim, int group, hipStream_t s) {
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
