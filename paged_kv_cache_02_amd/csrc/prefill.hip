// Chunked-prefill attention over the paged KV cache with bf16 MFMA (gfx950):
// the grid of row tiles and the merge pass for split tiles.  The tile body
// (work decomposition, LDS staging, MFMA layout, masking) is in
// prefill_core.h.
#include "prefill_core.h"

namespace pa {
namespace {

using namespace pf;

// The grid decomposition and the values the tile reads first come before
// the argument struct as plain scalars and pointers (equal to the struct's
// fields of the same names), so that the library's build preloads them into
// SGPRs at launch.
template <int D>
__global__ void __launch_bounds__(kThreads, 1)
prefill_kernel(const int32_t* seq_lens, const int32_t* q_offsets, const int32_t* q_starts,
               const int32_t* page_table, int Hkv, int T, int S, int num_seqs, int maxp, int group,
               PrefillArgs a) {
  // grid: KV head fastest (a (request, head) pair's tiles share an XCD when
  // Hkv is a multiple of 8), then split, then row tiles and requests in
  // reverse so the heavier tiles start first
  int bid = blockIdx.x;
  const int g = bid % Hkv;
  bid /= Hkv;
  const int split = bid % S;
  bid /= S;
  const int t = T - 1 - (bid % T);
  const int r = num_seqs - 1 - bid / T;
  const PrefillHot h{seq_lens, q_offsets, q_starts, page_table, maxp};
  prefill_tile<D>(a, h, group, r, t, g, split);
}

// Merge pass for split row tiles: one workgroup per (request, row tile, KV
// head); each wave takes rows, each lane D/64 dims.  LSE = M + ln sum_s
// exp(lse_s - M), out = sum_s exp(lse_s - LSE) * O_s.
template <int D>
__global__ void __launch_bounds__(256) prefill_merge_kernel(PrefillArgs a, int group) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int Hkv = a.num_kv_heads;
  const int T = a.tiles_per_seq;
  const int S = a.num_splits;
  int bid = blockIdx.x;
  const int g = bid % Hkv;
  bid /= Hkv;
  const int t = bid % T;
  const int r = bid / T;
  const TileGeo tg = tile_geo(a, r, t, group);
  if (tg.n <= 0 || tg.row_base >= tg.rows_total) return;
  const int nsp = num_splits_of(tg.ntiles, a.kv_tiles_per_split);
  if (nsp <= 1) return;
  const int q_start = q_start_of(a, r, lane);
  const int Hq = a.num_q_heads;
  const size_t unit = ((size_t)r * T + t) * Hkv + g;
  constexpr int kPer = D / 64;
  for (int prow = wave; prow < kTileRows; prow += 4) {
    const int rho = tg.row_base + prow;
    if (rho >= tg.rows_total) break;
    float M = -INFINITY;
    for (int s = 0; s < nsp; ++s) M = fmaxf(M, a.part_lse[(unit * S + s) * kTileRows + prow]);
    const float Mb = M == -INFINITY ? 0.f : M;
    float tot = 0.f;
    for (int s = 0; s < nsp; ++s) {
      const float v = a.part_lse[(unit * S + s) * kTileRows + prow];
      tot += v == -INFINITY ? 0.f : exp2f((v - Mb) * kLog2e);
    }
    const float LSE = Mb + logf(tot);
    float acc[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) acc[i] = 0.f;
    for (int s = 0; s < nsp; ++s) {
      const size_t pidx = (unit * S + s) * kTileRows + prow;
      const float v = a.part_lse[pidx];
      const float w = v == -INFINITY ? 0.f : exp2f((v - LSE) * kLog2e);
#pragma unroll
      for (int i = 0; i < kPer; ++i) acc[i] = fmaf(w, a.part_o[pidx * D + lane + 64 * i], acc[i]);
    }
    const int tok = rho / group;
    const int hh = rho % group;
    const size_t orow = (size_t)(q_start + tok) * Hq + (size_t)g * group + hh;
    __bf16* out = reinterpret_cast<__bf16*>(a.out) + orow * D;
#pragma unroll
    for (int i = 0; i < kPer; ++i) out[lane + 64 * i] = (__bf16)acc[i];
    if (a.lse != nullptr && lane == 0) a.lse[orow] = LSE;
  }
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, int group, hipStream_t s) {
  const long long units = (long long)a.num_seqs * a.tiles_per_seq * a.num_kv_heads;
  const long long grid = units * a.num_splits;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prefill_kernel<D>, dim3((unsigned)grid), dim3(kThreads), 0, s, a.seq_lens,
                     a.q_offsets, a.q_starts, a.page_table, a.num_kv_heads, a.tiles_per_seq,
                     a.num_splits, a.num_seqs, a.max_pages_per_seq, group, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_splits <= 1) return e;
  hipLaunchKernelGGL(prefill_merge_kernel<D>, dim3((unsigned)units), dim3(256), 0, s, a, group);
  return hipGetLastError();
}

}  // namespace

int prefill_tile_rows(int head_dim) {
  (void)head_dim;
  return kTileRows;
}

int prefill_tile_keys() { return kTileKeys; }

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int group, hipStream_t s) {
  if (group < 1) return hipErrorNotSupported;
  if (head_dim == 128) return launch_d<128>(a, group, s);
  if (head_dim == 64) return launch_d<64>(a, group, s);
  return hipErrorNotSupported;
}

}  // namespace pa
