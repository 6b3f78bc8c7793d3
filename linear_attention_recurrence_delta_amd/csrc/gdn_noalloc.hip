// gdn_chunk_fwd_noalloc: gdn_chunk_fwd with its workspace in a file-scope
// device array of this library, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc). It runs the same three kernels on the same workspace
// layout; nothing here allocates or frees.
//
// The array's name is a host-side stand-in in host code, not a device
// address: its address on each device comes from hipGetSymbolAddress, taken
// once per device (with that device current) on the first call there and
// kept; only that address is handed to the kernels. Every call on one GPU
// shares that GPU's array, so calls that overlap on one GPU (other streams,
// other threads) race. Nothing needs clearing between calls: no kernel reads
// a workspace byte that an earlier kernel of the same call did not write.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn.h"
#include "gdn_internal.h"

namespace {

constexpr size_t kScratchBytes = GDN_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte blocks");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

extern "C" gdn_status_t gdn_chunk_fwd_noalloc(const gdn_dims_t* dims, const void* q, const void* k,
                                              const void* v, const float* log_alpha, const float* beta,
                                              const float* init_state, const int32_t* cu_seqlens, void* o,
                                              float* final_state, hipStream_t stream) {
  gdn_workspace_layout_t lay;
  const gdn_status_t st = gdn_chunk_fwd_workspace_layout(dims, &lay);
  if (st != GDN_SUCCESS) return st;
  if (lay.total > kScratchBytes)
    return gdn::api_fail(GDN_ERROR_WORKSPACE,
                         "gdn_chunk_fwd_noalloc: these dims need %zu workspace bytes; its scratch array holds %zu "
                         "(GDN_NOALLOC_SCRATCH_BYTES); use gdn_chunk_fwd with a caller-owned workspace",
                         lay.total, kScratchBytes);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return gdn::api_fail(GDN_ERROR_HIP, "gdn_chunk_fwd_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return gdn::api_fail(GDN_ERROR_NOT_SUPPORTED, "gdn_chunk_fwd_noalloc: device %d (at most %d devices)", dev,
                         kMaxDevices);
  void* ptr;
  {
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch_ptr[dev]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return gdn::api_fail(GDN_ERROR_HIP, "gdn_chunk_fwd_noalloc: hipGetSymbolAddress of its scratch array: %s",
                             hipGetErrorString(e));
      g_scratch_ptr[dev] = p;
    }
    ptr = g_scratch_ptr[dev];
  }
  // the stages one after the other on `stream`: gdn_chunk_fwd's two-stream
  // form would create the library's second stream on first use
  gdn_status_t r = gdn_chunk_fwd_stages(dims, q, k, v, log_alpha, beta, init_state, cu_seqlens, o, final_state, ptr,
                                        kScratchBytes, stream, 1, 1);
  if (r == GDN_SUCCESS)
    r = gdn_chunk_fwd_stages(dims, q, k, v, log_alpha, beta, init_state, cu_seqlens, o, final_state, ptr,
                             kScratchBytes, stream, 2, 2);
  return r;
}
