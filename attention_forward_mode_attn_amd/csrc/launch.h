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
  float* tlse;  // may be null (not written)
  int B, H, Lq, Lk, d;
  int kv_rows;  // rows between consecutive K/V heads in memory (>= Lk)
  float scale;
};

// Both assume validated arguments (see the C ABI) and B*H*Lq > 0, Lk > 0.
hipError_t launch_bf16(const Problem& p, hipStream_t stream);
hipError_t launch_fp32(const Problem& p, hipStream_t stream);

constexpr int kMaxMergeParts = 16;

struct MergeProblem {
  int n;  // 1 .. kMaxMergeParts
  const void* o[kMaxMergeParts];
  const void* to[kMaxMergeParts];
  const float* lse[kMaxMergeParts];
  const float* tlse[kMaxMergeParts];
  void* out_o;
  void* out_to;
  float* out_lse;
  float* out_tlse;  // may be null
  int64_t rows;     // > 0
  int d;            // 64 or 128
  bool bf16;
};

hipError_t launch_merge(const MergeProblem& p, hipStream_t stream);

struct ProjProblem {
  const void* x;
  const void* tx;    // null: no tangent (ty null too)
  const void* w;
  const void* bias;  // may be null
  void* y;
  void* ty;
  int B, L, D, n_out, H, d;  // validated: d in {64, 128}, D % 64 == 0, B*L > 0, n_out*H > 0
};

hipError_t launch_proj(const ProjProblem& p, hipStream_t stream);

}  // namespace attnjvp
