// Exact merge of attention-JVP results computed over disjoint key ranges.
//
// A pass over key shard s returns, per query row, the normalised output O_s,
// its tangent tO_s, the log-sum-exp lse_s of its logits and the tangent of that
// log-sum-exp mu_s = sum_j P_sj tS_sj (P_s the softmax over the shard).  With
// w_s = exp(lse_s - lse), lse = log sum_s exp(lse_s), the softmax over all keys
// is w_s P_s on shard s, so
//   O   = sum_s w_s O_s
//   mu  = sum_s w_s mu_s
//   tO  = sum_s w_s (tO_s + (mu_s - mu) O_s)
// (tO_s + mu_s O_s is shard s's P_s tV + (P_s * tS) V; subtracting mu O over
// the union re-centres the tangent logits on the full softmax).  This is the
// partial-state exchange that the context-parallel reading of the rCM pages
// needs: ai.info summary of "Large Scale Diffusion Distillation via
// Score-Regularized Continuous-Time Consistency", "Methodology in Plain
// English" (tangents distributed with Q, K, V under context parallelism).
//
// The merge is bound by memory traffic: each thread merges 8 consecutive
// elements of one row (16-byte bf16 / 32-byte fp32 accesses), the row's
// weights recomputed per thread from the n scalars in one pass with a running
// maximum.  The first part's data are requested before that pass and each
// next part's during the current part's arithmetic, so every thread keeps a
// part in flight (66-68 VGPRs: 7 waves per SIMD).  Partials are bf16 or
// float32 (a bf16 pass can write float32 partials, so that the result is
// rounded to bf16 once, here); the result is bf16 or float32.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "device_common.h"
#include "launch.h"

namespace attnjvp {
namespace {

struct MergeArgs {
  MergeProblem p;
};

__device__ inline float bf16_lo(unsigned x) { return __uint_as_float(x << 16); }
__device__ inline float bf16_hi(unsigned x) { return __uint_as_float(x & 0xFFFF0000u); }

template <bool BF16>
__device__ inline void load8(const void* base, size_t elem, float (&x)[8]) {
  if constexpr (BF16) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const char*>(base) + elem * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_lo(v[i]);
      x[2 * i + 1] = bf16_hi(v[i]);
    }
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const char*>(base) + elem * 4);
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = a[i];
      x[4 + i] = b[i];
    }
  }
}

template <bool BF16>
__device__ inline void store8(void* base, size_t elem, const float (&x)[8]) {
  if constexpr (BF16) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = pack_bf16(x[2 * i], x[2 * i + 1]);
    *reinterpret_cast<u32x4*>(static_cast<char*>(base) + elem * 2) = v;
  } else {
    f32x4* p = reinterpret_cast<f32x4*>(static_cast<char*>(base) + elem * 4);
    p[0] = f32x4{x[0], x[1], x[2], x[3]};
    p[1] = f32x4{x[4], x[5], x[6], x[7]};
  }
}

template <bool kInBF16, bool kOutBF16, int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs args) {
  const MergeProblem& p = args.p;
  constexpr int kThreadsPerRow = D / 8;
  constexpr int kRowsPerBlock = 256 / kThreadsPerRow;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kThreadsPerRow;
  if (row >= p.rows) return;
  const int col = (threadIdx.x % kThreadsPerRow) * 8;
  const int n = p.n;
  const size_t elem = (size_t)row * D + col;

  // part 0's data in flight while the row's weights are computed
  float os[8], ts[8];
  load8<kInBF16>(p.o[0], elem, os);
  load8<kInBF16>(p.to[0], elem, ts);

  // one pass over the n (lse, tlse) pairs with a running maximum
  float lmax = -INFINITY, wsum = 0.0f, mun = 0.0f;
  for (int s = 0; s < n; ++s) {
    const float l = p.lse[s][row], t = p.tlse[s][row];
    const float m = fmaxf(lmax, l);
    const float r = expf(lmax - m), e = expf(l - m);
    wsum = wsum * r + e;
    mun = mun * r + e * t;
    lmax = m;
  }
  const float inv = 1.0f / wsum, mu = mun * inv;

  float o[8] = {}, to[8] = {};
  for (int s = 0; s < n; ++s) {
    float on[8], tn[8];
    if (s + 1 < n) {  // the next part's data in flight under this part's arithmetic
      load8<kInBF16>(p.o[s + 1], elem, on);
      load8<kInBF16>(p.to[s + 1], elem, tn);
    }
    const float w = expf(p.lse[s][row] - lmax) * inv;
    const float shift = p.tlse[s][row] - mu;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      o[i] += w * os[i];
      to[i] += w * (ts[i] + shift * os[i]);
    }
    if (s + 1 < n) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        os[i] = on[i];
        ts[i] = tn[i];
      }
    }
  }
  store8<kOutBF16>(p.out_o, elem, o);
  store8<kOutBF16>(p.out_to, elem, to);
  if (col == 0) {
    p.out_lse[row] = lmax + logf(wsum);
    if (p.out_tlse) p.out_tlse[row] = mu;
  }
}

template <bool kInBF16, bool kOutBF16, int D>
hipError_t launch(const MergeProblem& p, hipStream_t stream) {
  constexpr int kRowsPerBlock = 256 / (D / 8);
  const int64_t blocks = (p.rows + kRowsPerBlock - 1) / kRowsPerBlock;
  MergeArgs a{p};
  return launch_1d(reinterpret_cast<const void*>(&merge_kernel<kInBF16, kOutBF16, D>), (unsigned)blocks, 256, a,
                   stream);
}

}  // namespace

hipError_t launch_merge(const MergeProblem& p, hipStream_t stream) {
  if (p.in_bf16) return p.d == 128 ? launch<true, true, 128>(p, stream) : launch<true, true, 64>(p, stream);
  if (p.out_bf16) return p.d == 128 ? launch<false, true, 128>(p, stream) : launch<false, true, 64>(p, stream);
  return p.d == 128 ? launch<false, false, 128>(p, stream) : launch<false, false, 64>(p, stream);
}

}  // namespace attnjvp
