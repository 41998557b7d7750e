// pa_decode_noalloc: pa_decode for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation).  The decode routes that need scratch (the page-balanced
// partials and range table, or the equal-split partials) run on a fixed
// array of device memory that this file defines; nothing is allocated and
// no workspace is passed in.
//
// The array is a file-scope __device__ variable.  In host code its name is
// only a stand-in for the symbol, not a device address: the address is
// looked up once per device with hipGetSymbolAddress (with that device
// current) and cached, and only that address is ever handed to a kernel.
// Each device holds its own copy of the array for the life of the process.
#include <mutex>

#include "pa.h"
#include "pa_internal.h"

namespace {

constexpr size_t kScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size keeps 256-byte alignment");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];   // device address of `scratch` per device, once looked up

// Device address of this device's scratch array (looked up on the first
// call on the device).
pa_status scratch_address(void** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return PA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return PA_ERR_HIP;
    }
    g_scratch[dev] = p;
  }
  *addr = g_scratch[dev];
  return PA_OK;
}

}  // namespace

extern "C" pa_status pa_decode_noalloc(const pa_desc* d, const void* q, const void* k_pool,
                                       const void* v_pool, const int32_t* page_table,
                                       const int32_t* seq_lens, const int32_t* q_offsets,
                                       float scale, void* out, float* lse, void* stream) {
  pa_status st = pa::check_decode_call(d, q, k_pool, v_pool, page_table, seq_lens, scale, out, lse);
  if (st != PA_OK || d->num_seqs == 0) return st;
  pa_plan_info plan;
  st = pa_plan(d, 0, &plan);
  if (st != PA_OK) return st;
  if (plan.workspace_bytes > kScratchBytes) return PA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (plan.workspace_bytes > 0) {
    st = scratch_address(&ws);
    if (st != PA_OK) return st;
  }
  // the same routes and kernels as pa_decode, with the scratch array as the
  // workspace (no route reads scratch it has not written in the same call)
  return pa_decode(d, q, k_pool, v_pool, page_table, seq_lens, q_offsets, scale, out, lse, ws,
                   plan.workspace_bytes, stream);
}
