// Page gather (test hook): copies one request's keys out of the paged pools
// into contiguous [seq_len, Hkv, d] tensors.  It is the page-table
// translation of the paged KV cache on its own -- logical key j of the
// request is slot j % P of physical page page_row[j / P] (tiny-llm source
// reading, "Paged KV Cache") -- and a pure copy, so its result is compared
// bit for bit.  The attention kernels never materialize this copy.
#include "pa_internal.h"

namespace pa {
namespace {

// One thread moves 16 bytes.  Element (j, g, c) of the output comes from
// pool element ((page_row[j / P] * Hkv + g) * P + j % P) * d + c.
__global__ void __launch_bounds__(256) gather_kernel(GatherArgs a) {
  const int row_bytes = a.head_dim * a.elem_bytes;        // one (key, head) row
  const int chunks_per_row = row_bytes / 16;
  const long long total = (long long)a.seq_len * a.num_kv_heads * chunks_per_row;
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int chunk = (int)(i % chunks_per_row);
  const long long jg = i / chunks_per_row;
  const int g = (int)(jg % a.num_kv_heads);
  const int j = (int)(jg / a.num_kv_heads);
  int page = a.page_row[j / kPageSize];
  page = page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page);
  const int slot = j % kPageSize;
  const long long src_row = ((long long)page * a.num_kv_heads + g) * kPageSize + slot;
  const char* ks = reinterpret_cast<const char*>(a.k_pool) + src_row * row_bytes + chunk * 16;
  const char* vs = reinterpret_cast<const char*>(a.v_pool) + src_row * row_bytes + chunk * 16;
  char* kd = reinterpret_cast<char*>(a.k_out) + jg * row_bytes + chunk * 16;
  char* vd = reinterpret_cast<char*>(a.v_out) + jg * row_bytes + chunk * 16;
  *reinterpret_cast<uint4*>(kd) = *reinterpret_cast<const uint4*>(ks);
  *reinterpret_cast<uint4*>(vd) = *reinterpret_cast<const uint4*>(vs);
}

}  // namespace

hipError_t launch_gather(const GatherArgs& a, hipStream_t s) {
  const long long total = (long long)a.seq_len * a.num_kv_heads * (a.head_dim * a.elem_bytes / 16);
  if (total <= 0) return hipSuccess;
  const long long grid = (total + 255) / 256;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
