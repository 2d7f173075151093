// Kernel launchers for the sanitizer build of the library's host code (argument
// validation and launch planning, compiled with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_sanitizers.py).  That build runs on
// machines without a GPU, where no operation can be created, so no execution
// reaches these: they report that no device is present.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace mpa {

hipError_t launch_prefill(const PrefillParams&, int, int, int, int, hipStream_t, const LaunchEvents&) {
  return hipErrorNoDevice;
}
hipError_t launch_mla(const MlaParams&, int, hipStream_t, const LaunchEvents&) { return hipErrorNoDevice; }
hipError_t launch_lse_merge(const LseMergeParams&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t static_scratch(void**, size_t*) { return hipErrorNoDevice; }

}  // namespace mpa
