// Internal launcher interface between the C ABI and the kernels.
#pragma once
#include <hip/hip_runtime.h>

namespace attnjvp {

struct Problem {
  const void* q;
  const void* k;
  const void* v;
  const void* tq;
  const void* tk;
  const void* tv;
  void* o;
  void* to;
  float* lse;
  int B, H, Lq, Lk, d;
  float scale;
};

// Both assume validated arguments (see the C ABI) and B*H*Lq > 0, Lk > 0.
hipError_t launch_bf16(const Problem& p, hipStream_t stream);
hipError_t launch_fp32(const Problem& p, hipStream_t stream);

}  // namespace attnjvp
