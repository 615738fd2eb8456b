// csa_decode_noalloc: csa_decode with its workspace in a static device array, for callers that
// cannot allocate (graph capture, serving loops, harnesses that forbid hipMalloc).  The array is
// part of this file's code object, so every device the library is loaded on holds its own copy for
// the life of the process; its device address is looked up once per device (hipGetSymbolAddress
// with that device current) and only that address is ever handed to kernels or copies.
#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/csa.h"
#include "csa_internal.h"

namespace {

static __device__ __align__(256) uint8_t scratch[CSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

extern "C" csa_status csa_decode_noalloc(int32_t B, int32_t H, int32_t HI, int32_t k, const void* q, int32_t q_dt,
                                         const float* sink, const void* qI, const uint8_t* qI_scale, int32_t qI_dt,
                                         const float* w, const csa_paged_idx* keys, const csa_paged_kv* comp,
                                         const void* win_ring, int32_t win_fmt, const int32_t* ctx_len,
                                         int64_t max_ctx, float softmax_scale, void* out, int32_t out_dt,
                                         int32_t* idx_out, hipStream_t stream) {
  const size_t need = csa_decode_workspace_bytes(B, H, HI, max_ctx, k);
  if (need > CSA_NOALLOC_SCRATCH_BYTES) return CSA_ERR_SCRATCH;   // (0: invalid sizes, refused below)
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (csa_status)csa::record_hip_error(e);
  if (dev < 0 || dev >= kMaxDevices) return CSA_ERR_UNSUPPORTED;
  void* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr) return (csa_status)csa::record_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol);
      g_scratch_ptr[dev] = p;
    }
    ptr = g_scratch_ptr[dev];
  }
  return csa_decode(B, H, HI, k, q, q_dt, sink, qI, qI_scale, qI_dt, w, keys, comp, win_ring, win_fmt, ctx_len,
                    max_ctx, softmax_scale, out, out_dt, idx_out, ptr, CSA_NOALLOC_SCRATCH_BYTES, stream);
}
