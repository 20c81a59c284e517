// Stand-ins for libfattn's kernel launchers and device scratch lookup, for the host-only
// sanitizer build of api.cpp (tests/test_sanitized_abi.py). Every one reports that no device is
// present; the ABI checks that run against this library never get that far.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace fattn {

hipError_t launch_prefill_bf16(const Problem&, int, int, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_prefill_varlen_bf16(const Problem&, const Packed&, int, int, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_prefill_f32(const Problem&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_bf16(const Problem&, int, int, int, float*, float*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_decode_paged_bf16(const Problem&, const PagedKV&, int, int, float*, float*,
                                    hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_backward_bf16(const BwdProblem&, float*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_backward_varlen_bf16(const BwdProblem&, const Packed&, float*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t static_scratch(int, float**) { return hipErrorNoDevice; }

}  // namespace fattn
