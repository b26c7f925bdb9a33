// Stand-ins for the device-side launchers of libpa (pa_kernels.hip,
// pa_cache_kernels.hip, pa_noalloc.hip), so the host library (pa_api.cpp) can
// be built alone with the host compiler's sanitizers.  Every launcher fails
// with hipErrorInvalidValue: the sanitizer driver exercises validation and
// planning only.
#include "pa_internal.h"

namespace pa {

#define PA_STUB_HEAD_DIM(DV)                                                                   \
  hipError_t launch_fwd_d##DV(const FwdParams&, int, int, bool, bool, int64_t, hipStream_t) {  \
    return hipErrorInvalidValue;                                                               \
  }                                                                                            \
  hipError_t launch_decode_d##DV(const FwdParams&, int, bool, bool, int64_t, hipStream_t) {    \
    return hipErrorInvalidValue;                                                               \
  }                                                                                            \
  hipError_t launch_fwd8_d##DV(const FwdParams&, int, bool, int64_t, hipStream_t) {            \
    return hipErrorInvalidValue;                                                               \
  }                                                                                            \
  int decode_blocks_per_cu_d##DV(int, bool, bool) { return 2; }                                \
  hipError_t launch_merge_d##DV(const MergeParams&, bool, hipStream_t) {                       \
    return hipErrorInvalidValue;                                                               \
  }                                                                                            \
  hipError_t launch_merge2_d##DV(const Merge2Params&, bool, hipStream_t) {                     \
    return hipErrorInvalidValue;                                                               \
  }
PA_STUB_HEAD_DIM(64)
PA_STUB_HEAD_DIM(96)
PA_STUB_HEAD_DIM(128)
PA_STUB_HEAD_DIM(256)
#undef PA_STUB_HEAD_DIM

hipError_t launch_rank(const FwdParams&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_cache_write(const CacheWriteParams&, bool, bool, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t noalloc_scratch(void**) { return hipErrorInvalidValue; }

}  // namespace pa
