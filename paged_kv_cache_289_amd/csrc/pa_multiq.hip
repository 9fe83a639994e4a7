// Multi-query paged attention (speculative verification, prefill chunks).
#include "pa_common.h"

namespace pa {

hipError_t launch_multiq(int, int, int, int, int, const AttnArgs&, hipStream_t,
                         const KernelEvents&) {
  return hipErrorNotSupported;
}

}  // namespace pa
