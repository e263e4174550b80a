// Shared state of the stub launchers (sanitizer build of the C ABI).
#pragma once
#include "launch.h"

namespace stub {
enum class Kind { none, bf16, fp32, merge, proj, norm_rope };
extern int calls;
extern Kind last_kind;
extern attnjvp::Problem last_problem;
extern attnjvp::MergeProblem last_merge;
extern attnjvp::ProjProblem last_proj;
extern attnjvp::NormRopeProblem last_norm_rope;
extern hipError_t next_status;
}  // namespace stub
