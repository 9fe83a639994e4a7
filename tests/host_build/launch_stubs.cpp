// Host-only stand-ins for the kernel launchers of libpagedattn.so, so that the
// C-ABI layer (pa_api.cpp) and the block pool (pa_pool.cpp) can be built with a
// host compiler under the address and undefined-behaviour sanitizers and run
// on a machine without a GPU.  Every launcher reports "no device"; the tests
// that use this build exercise validation, sizing and the pool only.
#include "pa_internal.h"

namespace pa {

hipError_t launch_decode(int, int, int, int, int, const AttnArgs&, hipStream_t,
                         const KernelEvents&) {
  return hipErrorNoDevice;
}
int split_workgroups_per_cu(int, int, int, int) { return 1; }
int multiq_split_workgroups_per_cu(int, int) { return 1; }
hipError_t launch_split_decode(int, int, int, const AttnArgs&, hipStream_t, const KernelEvents&) {
  return hipErrorNoDevice;
}
hipError_t launch_multiq(int, int, int, int, int, const AttnArgs&, hipStream_t,
                         const KernelEvents&) {
  return hipErrorNoDevice;
}
hipError_t launch_gather(void*, void*, const void*, const void*, const int32_t*, const int32_t*,
                         const int32_t*, int, int, int, int, int, int, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_append(void*, void*, const void*, const void*, const int32_t*, const int32_t*,
                         const int32_t*, int, int, int, int, int, int, int, int, int, hipStream_t,
                         const KernelEvents&) {
  return hipErrorNoDevice;
}
hipError_t launch_copy_blocks(void*, void*, const int32_t*, int, int, int, int, int, int,
                              hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_cascade_fold(const CascadeFold&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_stream_read(const void*, size_t, unsigned*, int, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t scratch_buffer(void**) { return hipErrorNoDevice; }
hipError_t launch_check(const int32_t*, const int32_t*, int, int, int, int, int, int32_t*,
                        hipStream_t) {
  return hipErrorNoDevice;
}

}  // namespace pa
