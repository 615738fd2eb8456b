// Host-only stand-ins for the kernel launchers, linked instead of the HIP kernels into the
// sanitizer build of the C ABI layer (api.cpp and plan.cpp built by a host compiler with address
// and undefined-behaviour sanitizers).  That build exercises argument validation, workspace
// carving and status reporting on a machine without a GPU; any call that passes validation and
// would launch a kernel fails loudly with CSA_ERR_HIP (hipErrorNotSupported) instead.
#include "../../include/csa.h"
#include "csa_internal.h"

namespace csa {

hipError_t launch_indexer(const IndexerArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_topk_hist(const TopkArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_topk_select(const TopkArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_topk_single(const TopkArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_topk_sketch(const TopkArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_prep(const PrepArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attention(const AttnArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_compress(const CompressArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace csa

// the no-allocation entry point has no device array here: its size check runs, then the call is
// refused as a launch would be
extern "C" csa_status csa_decode_noalloc(int32_t B, int32_t H, int32_t HI, int32_t k, const void*, int32_t,
                                         const float*, const void*, const uint8_t*, int32_t, const float*,
                                         const csa_paged_idx*, const csa_paged_kv*, const void*, int32_t,
                                         const int32_t*, int64_t max_ctx, float, void*, int32_t, int32_t*,
                                         hipStream_t) {
  if (csa_decode_workspace_bytes(B, H, HI, max_ctx, k) > CSA_NOALLOC_SCRATCH_BYTES) return CSA_ERR_SCRATCH;
  return (csa_status)csa::record_hip_error(hipErrorNotSupported);
}
