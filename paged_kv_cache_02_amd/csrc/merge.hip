// Log-sum-exp merge of split-K partials (gfx950).
//
// Split s of a (row, head) carries a partial output O_s normalized by its own
// softmax sum and lse_s = ln(sum of exp(score) over the split's keys).  The
// full result is LSE = M + ln(sum_s exp(lse_s - M)) with M = max_s lse_s and
// out = sum_s exp(lse_s - LSE) * O_s; an empty split (lse_s = -inf) has zero
// weight.  This is the combine step of split-K long-context decode
// (Flash-Decoding, adv04 in the mini-vllm-tutorial advanced-series design).
//
// One wave per (row, head): lanes read the S partial lse values (strided by
// 64), reduce max and sum with wave shuffles, then each lane produces d/64 of
// the output dims, reading the S partial rows coalesced, eight partials per
// batch of loads; the first batch is requested together with the lse values.  Partials come
// either S per (row, head) (equal splits) or as a variable run of slots per
// row given by a range table (page-balanced splits).
#include "pa_internal.h"

#include <math.h>

namespace pa {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <typename T>
__device__ __forceinline__ T cast_out(float x);
template <>
__device__ __forceinline__ __bf16 cast_out<__bf16>(float x) { return (__bf16)x; }
template <>
__device__ __forceinline__ float cast_out<float>(float x) { return x; }

// The range table, the sizes and the partial arrays come before the
// argument struct as plain scalars and pointers (equal to the struct's fields
// of the same names), so that the library's build (kernarg preloading) hands
// them to the wave in SGPRs at launch and the first read of the range table
// does not wait on a load of the kernel arguments.
template <typename T, int D>
__global__ void __launch_bounds__(64 * kWavesPerBlock)
merge_kernel(const int32_t* __restrict__ range_meta, int rows, int heads, int num_splits,
             const float* __restrict__ o_part, const float* __restrict__ lse_part, MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const long long rh = (long long)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const long long nrh = (long long)rows * heads;
  if (rh >= nrh) return;
  // partial s of this (row, head) is row  base + s * step  of the partial arrays
  long long base, step;
  int S;
  if (range_meta == nullptr) {
    S = num_splits;
    base = rh * S;
    step = 1;
  } else {
    const long long r = rh / heads;
    const int first = range_meta[2 * r];
    const int last = range_meta[2 * r + 1];
    S = last >= first ? last - first + 1 : 0;
    base = (r + first) * heads + rh % heads;
    step = heads;
  }
  const float* lp = lse_part;
  const float* op = o_part;
  constexpr int kPer = D / 64;
  constexpr int kBatch = 8;   // partial rows requested together

  // The first batch of partial rows is requested together with the lse
  // values (it does not depend on them), so a (row, head) with at most
  // kBatch partials waits for one memory round trip after the range table.
  float o0[kBatch][kPer];
#pragma unroll
  for (int j = 0; j < kBatch; ++j) {
    const long long row = base + (long long)(j < S ? j : 0) * step;
#pragma unroll
    for (int i = 0; i < kPer; ++i) o0[j][i] = j < S ? op[row * D + lane + 64 * i] : 0.f;
  }
  const float v_lane = lane < S ? lp[base + (long long)lane * step] : -INFINITY;   // slot `lane`'s lse

  float M = v_lane;
  for (int s = lane + 64; s < S; s += 64) M = fmaxf(M, lp[base + s * step]);
  M = wave_max(M);
  const float Mb = (M == -INFINITY) ? 0.f : M;   // all splits empty: weights stay 0
  float tot = (v_lane == -INFINITY) ? 0.f : exp2f((v_lane - Mb) * kLog2e);
  for (int s = lane + 64; s < S; s += 64) {
    const float v = lp[base + s * step];
    tot += (v == -INFINITY) ? 0.f : exp2f((v - Mb) * kLog2e);
  }
  tot = wave_sum(tot);
  const bool empty = !(tot > 0.f);
  const float LSE = empty ? -INFINITY : Mb + logf(tot);

  float acc[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) acc[i] = 0.f;
  if (!empty) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const float v = __shfl(v_lane, j);
      const float w = (v == -INFINITY) ? 0.f : exp2f((v - LSE) * kLog2e);
#pragma unroll
      for (int i = 0; i < kPer; ++i) acc[i] = fmaf(w, o0[j][i], acc[i]);
    }
    // the rows of the later batches (and their lse) are requested a batch
    // at a time, before any is used
    for (int s0 = kBatch; s0 < S; s0 += kBatch) {
      float v[kBatch];
      float o[kBatch][kPer];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const bool live = s0 + j < S;
        const long long row = base + (long long)(live ? s0 + j : s0) * step;
        v[j] = live ? lp[row] : -INFINITY;
#pragma unroll
        for (int i = 0; i < kPer; ++i) o[j][i] = live ? op[row * D + lane + 64 * i] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const float w = (v[j] == -INFINITY) ? 0.f : exp2f((v[j] - LSE) * kLog2e);
#pragma unroll
        for (int i = 0; i < kPer; ++i) acc[i] = fmaf(w, o[j][i], acc[i]);
      }
    }
  }
  T* out = reinterpret_cast<T*>(a.out) + rh * D;
#pragma unroll
  for (int i = 0; i < kPer; ++i) out[lane + 64 * i] = cast_out<T>(acc[i]);
  if (a.lse != nullptr && lane == 0) a.lse[rh] = LSE;
}

template <typename T, int D>
hipError_t launch_t(const MergeArgs& a, hipStream_t s) {
  const long long nrh = (long long)a.rows * a.heads;
  if (nrh <= 0) return hipSuccess;
  const long long grid = (nrh + kWavesPerBlock - 1) / kWavesPerBlock;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((merge_kernel<T, D>), dim3((unsigned)grid), dim3(64 * kWavesPerBlock), 0, s,
                     a.range_meta, a.rows, a.heads, a.num_splits, a.o_part, a.lse_part, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int out_dtype, int head_dim, hipStream_t s) {
  if (out_dtype == 0) {
    if (head_dim == 128) return launch_t<__bf16, 128>(a, s);
    if (head_dim == 64) return launch_t<__bf16, 64>(a, s);
  } else if (out_dtype == 1) {
    if (head_dim == 128) return launch_t<float, 128>(a, s);
    if (head_dim == 64) return launch_t<float, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
