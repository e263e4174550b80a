// Stub launchers for the host-only sanitizer build of the C ABI (test
// infrastructure): instead of enqueuing kernels they record the problem they
// were handed and return a status chosen by the driver, so every argument
// check of the C ABI runs under AddressSanitizer and UndefinedBehaviorSanitizer
// on a machine without a GPU.
#include "stub_launch.h"

#include <cstdint>

namespace stub {
int calls = 0;
Kind last_kind = Kind::none;
attnjvp::Problem last_problem{};
attnjvp::MergeProblem last_merge{};
attnjvp::ProjProblem last_proj{};
attnjvp::NormRopeProblem last_norm_rope{};
hipError_t next_status = hipSuccess;
}  // namespace stub

namespace attnjvp {

static hipError_t record(stub::Kind k) {
  ++stub::calls;
  stub::last_kind = k;
  return stub::next_status;
}

hipError_t launch_bf16(const Problem& p, hipStream_t) {
  stub::last_problem = p;
  return record(stub::Kind::bf16);
}

hipError_t launch_fp32(const Problem& p, hipStream_t) {
  stub::last_problem = p;
  return record(stub::Kind::fp32);
}

hipError_t launch_merge(const MergeProblem& p, hipStream_t) {
  stub::last_merge = p;
  return record(stub::Kind::merge);
}

hipError_t launch_proj(const ProjProblem& p, hipStream_t) {
  stub::last_proj = p;
  return record(stub::Kind::proj);
}

hipError_t launch_norm_rope(const NormRopeProblem& p, hipStream_t) {
  stub::last_norm_rope = p;
  return record(stub::Kind::norm_rope);
}

}  // namespace attnjvp

// The one HIP runtime function the C ABI calls on the host (on a failed launch).
const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "hipSuccess" : "stub HIP error"; }
