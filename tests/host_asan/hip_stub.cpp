// Host-only stand-ins for the HIP runtime calls and kernel launchers that
// gdn_api.cpp uses, so that the C ABI's host code (validation, workspace
// carving, the GDN_DEBUG and GDN_DEBUG_SYNC paths) can be built with g++ and
// run under AddressSanitizer and UndefinedBehaviorSanitizer on a machine
// without a GPU. "Device" pointers are host memory here: the copy stand-in
// is memcpy. The launchers record the argument block they were given.
#include <string.h>

#include "gdn_internal.h"
#include "stub_state.h"

StubState g_stub;

extern "C" {

const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "hipSuccess" : "stub HIP error"; }

hipError_t hipGetLastError(void) { return hipSuccess; }

hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind, hipStream_t) {
  ++g_stub.copies;
  memcpy(dst, src, bytes);
  return hipSuccess;
}

hipError_t hipStreamSynchronize(hipStream_t) {
  ++g_stub.syncs;
  return g_stub.fail_sync ? hipErrorLaunchFailure : hipSuccess;
}

}  // extern "C"

namespace gdn {

hipError_t launch_prefill(const PrefillArgs& a, int, int, int, hipStream_t, int first, int last) {
  ++g_stub.launches;
  g_stub.prefill = a;
  g_stub.first = first;
  g_stub.last = last;
  return g_stub.fail_launch ? hipErrorInvalidValue : hipSuccess;
}

hipError_t launch_backward(const PrefillArgs& a, int, int, int, hipStream_t, int first, int last) {
  ++g_stub.launches;
  g_stub.prefill = a;
  g_stub.first = first;
  g_stub.last = last;
  return g_stub.fail_launch ? hipErrorInvalidValue : hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, int, int, hipStream_t) {
  ++g_stub.launches;
  g_stub.decode = a;
  return g_stub.fail_launch ? hipErrorInvalidValue : hipSuccess;
}

hipError_t launch_decode_multi(const DecodeArgs& a, int, int, hipStream_t) {
  ++g_stub.launches;
  g_stub.decode = a;
  return g_stub.fail_launch ? hipErrorInvalidValue : hipSuccess;
}

}  // namespace gdn
