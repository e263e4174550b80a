// Internal launcher interface between the C ABI and the kernels.
#pragma once
#include <hip/hip_runtime.h>

namespace attnjvp {

// Enqueue `kernel`, whose one parameter is the by-value struct `a`, on a 1-D
// grid, and return the status of this launch itself.  (Reading
// hipGetLastError() after a launch would also return, and clear, an error
// that an unrelated earlier call left pending on the calling thread.)
template <typename Args>
inline hipError_t launch_1d(const void* kernel, unsigned blocks, unsigned threads, const Args& a,
                            hipStream_t stream) {
  void* args[] = {const_cast<Args*>(&a)};
  return hipLaunchKernel(kernel, dim3(blocks), dim3(threads), args, 0, stream);
}

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
  bool out_f32;  // bf16 inputs: O and tO written as float32 instead of bf16
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
  bool in_bf16;     // partial O, tO in bf16 (else float32)
  bool out_bf16;    // merged O, tO in bf16 (else float32)
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

struct NormRopeProblem {
  const void* x;
  const void* tx;     // null: no tangent (ty null too)
  void* y;            // may equal x
  void* ty;           // may equal tx
  const void* gamma;  // [d] in the element type, or null (gain 1)
  const float* cos;   // [L, d/2], or null together with sin (no rotation)
  const float* sin;
  int BH, L, d;       // validated: d in {64, 128}, BH * L > 0
  int n_blocks;       // set by the launcher
  float eps;
  bool bf16;
};

hipError_t launch_norm_rope(const NormRopeProblem& p, hipStream_t stream);

}  // namespace attnjvp
