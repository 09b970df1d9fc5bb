// r2l_layer_fwd_noalloc: the layer forward for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  The workspace r2l_layer_fwd takes from its caller
// comes instead from a static device array of this library, one copy per
// GPU, resolved once per device and then reused by every call on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/r2l.h"

namespace {

constexpr size_t kScratchBytes = (size_t)R2L_NOALLOC_SCRATCH_BYTES;
// The device array.  In host code `scratch` names a host-side shadow, not a
// device address: only the address resolved below is ever handed to kernels.
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// The array's address on the current device (resolved on the first call on
// that device, with that device current).
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return R2L_ERR_HIP;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = p;
  });
  if (g_err[dev] != hipSuccess || g_ptr[dev] == nullptr) return R2L_ERR_HIP;
  *out = g_ptr[dev];
  return R2L_OK;
}

}  // namespace

extern "C" int r2l_layer_fwd_noalloc(const r2l_dims* dims, r2l_dtype act, uint32_t flags, const r2l_weights* w,
                                     const void* h_in, void* h_out, const int32_t* cu_seqlens, int32_t nseq,
                                     int64_t n_tokens, int32_t max_seqlen, float* branch_out, void* stream) {
  // the training mode keeps activations for a later backward in the
  // workspace; a shared array would be overwritten by the next call
  if (flags & R2L_FLAG_TRAIN) return R2L_ERR_UNSUPPORTED;
  const size_t need = r2l_layer_workspace_bytes(dims, act, n_tokens, nseq, max_seqlen);
  if (need == 0) return R2L_ERR_INVALID_ARG;   // the query rejects invalid shapes
  if (need > kScratchBytes) return R2L_ERR_WORKSPACE;
  void* ws = nullptr;
  const int rc = scratch_on_current_device(&ws);
  if (rc != R2L_OK) return rc;
  // r2l_layer_fwd ignores its workspace's contents on entry: nothing has to
  // be cleared between calls
  return r2l_layer_fwd(dims, act, flags, w, h_in, h_out, cu_seqlens, nseq, n_tokens, max_seqlen, ws, kScratchBytes,
                       branch_out, stream);
}
