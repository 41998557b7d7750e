// Read-bandwidth reference for the attention kernels' access pattern
// (measurement hook, not part of the attention path).  Whole blocks are read
// in a caller-given order with the loads the decode kernels use for K and V
// (16 bytes per lane through a buffer resource over the block, nontemporal),
// so timing it over one (page, KV head) block size in a random order gives
// the rate such reads reach on the device: the practical side of the decode
// kernels' HBM roofline.
#include "pa_internal.h"

namespace pa {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kNontemporal = 2;   // cache-policy bits of the K/V loads

// Workgroup j takes blocks j, j + grid, ...; kPer 4 KB pieces per block, one
// 16-byte load per lane each, all in flight before any is used.
template <int kPer>
__global__ void __launch_bounds__(256) read_blocks_kernel(ReadBlocksArgs a) {
  unsigned acc = 0;
  for (int j = blockIdx.x; j < a.nblocks; j += gridDim.x) {
    const int id = a.order[j];
    if (id < 0 || (long long)id >= a.buf_blocks) continue;
    const unsigned char* blk = reinterpret_cast<const unsigned char*>(a.buf) + (size_t)id * (kPer * 4096);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(blk), (short)0, kPer * 4096, kBufferWord3);
    u32x4 v[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, u * 4096 + (int)threadIdx.x * 16, 0, kNontemporal);
#pragma unroll
    for (int u = 0; u < kPer; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  // every word read is folded into the sink, so no load can be dropped
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0 && acc != 0) atomicXor(a.sink, acc);
}

}  // namespace

hipError_t launch_read_blocks(const ReadBlocksArgs& a, hipStream_t s) {
  if (a.nblocks <= 0) return hipSuccess;
  const unsigned grid = (unsigned)(a.nblocks < kReadBlocksGrid ? a.nblocks : kReadBlocksGrid);
  switch (a.block_bytes) {
    case 4096: hipLaunchKernelGGL(read_blocks_kernel<1>, dim3(grid), dim3(256), 0, s, a); break;
    case 8192: hipLaunchKernelGGL(read_blocks_kernel<2>, dim3(grid), dim3(256), 0, s, a); break;
    case 16384: hipLaunchKernelGGL(read_blocks_kernel<4>, dim3(grid), dim3(256), 0, s, a); break;
    case 32768: hipLaunchKernelGGL(read_blocks_kernel<8>, dim3(grid), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
