// RMS normalisation and rotary embedding of queries or keys, with the JVP, on
// gfx950.
//
// The rCM pages refactor every layer of the distilled networks to take and
// return tangents and hand the tangents of Q and K to the attention kernel
// laid out like Q and K (ai.info summary of "Large Scale Diffusion
// Distillation via Score-Regularized Continuous-Time Consistency",
// "Methodology in Plain English" and "Key Contributions" item 1).  The layer
// between the projection and attention is read as: each row x (one token of
// one head) is RMS-normalised over the head dimension with a gain g, then its
// adjacent pairs (2i, 2i+1) are rotated by the angles of the token's position,
// given as cos/sin tables; gain, eps and angles carry no tangent:
//   r  = (mean(x^2) + eps)^(-1/2),   n = g x r,
//   tn = g (tx r - x r^3 mean(x tx)),
//   y  = R(t) n,   ty = R(t) tn,   R(t) rotating pair i by the angle (cos[t,i], sin[t,i]).
//
// Bound by memory traffic (4 d elements per row with the tangent, the tables
// read once per XCD): one row is spread over kLanes lanes of 16 bytes each,
// so a wave reads 1 KB of consecutive rows per tensor and instruction; the row
// sums are xor-shuffles within those lanes; each lane holds whole pairs, so the
// rotation needs no exchange.  A lane reads all of its elements before it
// writes any, so y may alias x and ty may alias tx.  Workgroups walk the
// heads of one block of positions together, XCD by XCD, so each XCD fetches a
// block of table rows once for all heads.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "device_common.h"
#include "launch.h"

namespace attnjvp {
namespace {

template <bool BF16, int D>
struct NrCfg {
  static constexpr int kElemBytes = BF16 ? 2 : 4;
  static constexpr int kPerLane = 16 / kElemBytes;       // elements per lane (8 bf16, 4 fp32)
  static constexpr int kLanes = D / kPerLane;             // lanes per row
  static constexpr int kRowsPerBlock = 256 / kLanes;      // rows of one workgroup
  static_assert(kLanes >= 8 && kLanes <= 32 && (kLanes & (kLanes - 1)) == 0, "row lanes");
};

__device__ inline float bf16_lo(unsigned x) { return __uint_as_float(x << 16); }
__device__ inline float bf16_hi(unsigned x) { return __uint_as_float(x & 0xFFFF0000u); }

template <bool BF16, int N>
__device__ inline void load_row(const void* base, size_t byte_off, float (&v)[N]) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const char*>(base) + byte_off);
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_lo(w[i]);
      v[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(w[i]);
  }
}

template <bool BF16, int N>
__device__ inline void store_row(void* base, size_t byte_off, const float (&v)[N]) {
  u32x4 w;
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16(v[2 * i], v[2 * i + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(v[i]);
  }
  *reinterpret_cast<u32x4*>(static_cast<char*>(base) + byte_off) = w;
}

// Sum over the kLanes lanes of one row (aligned groups of consecutive lanes).
template <int kLanes>
__device__ inline float row_sum(float x) {
#pragma unroll
  for (int m = 1; m < kLanes; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

template <bool BF16, int D>
__global__ __launch_bounds__(256) void norm_rope_kernel(NormRopeProblem p) {
  using C = NrCfg<BF16, D>;
  constexpr int N = C::kPerLane;
  const int n_tb = (p.L + C::kRowsPerBlock - 1) / C::kRowsPerBlock;
  const int blk = xcd_logical_block(blockIdx.x, p.n_blocks);
  const int tb = blk / p.BH, bh = blk % p.BH;  // position block major, head minor
  const int lane_in_row = threadIdx.x % C::kLanes;
  const int t = tb * C::kRowsPerBlock + threadIdx.x / C::kLanes;
  (void)n_tb;
  if (t >= p.L) return;  // whole row groups leave together: the shuffles stay within live lanes
  const int col = lane_in_row * N;  // first element of this lane
  const size_t off = (((size_t)bh * p.L + t) * D + col) * C::kElemBytes;

  float x[N], tx[N] = {}, g[N];
  load_row<BF16>(p.x, off, x);
  const bool tangent = p.tx != nullptr;
  if (tangent) load_row<BF16>(p.tx, off, tx);
  if (p.gamma) {
    load_row<BF16>(p.gamma, (size_t)col * C::kElemBytes, g);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) g[i] = 1.0f;
  }
  float c[N / 2], s[N / 2];
  if (p.cos) {
    const float* cr = p.cos + (size_t)t * (D / 2) + col / 2;
    const float* sr = p.sin + (size_t)t * (D / 2) + col / 2;
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      c[i] = cr[i];
      s[i] = sr[i];
    }
  }

  float ss = 0.0f, xt = 0.0f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    ss = __builtin_fmaf(x[i], x[i], ss);
    xt = __builtin_fmaf(x[i], tx[i], xt);
  }
  ss = row_sum<C::kLanes>(ss);
  const float r = 1.0f / sqrtf(ss * (1.0f / D) + p.eps);
  float y[N], ty[N];
#pragma unroll
  for (int i = 0; i < N; ++i) y[i] = g[i] * x[i] * r;
  if (tangent) {
    xt = row_sum<C::kLanes>(xt);
    const float k = r * r * r * (xt * (1.0f / D));
#pragma unroll
    for (int i = 0; i < N; ++i) ty[i] = g[i] * (tx[i] * r - x[i] * k);
  }
  if (p.cos) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const float a = y[2 * i], b = y[2 * i + 1];
      y[2 * i] = c[i] * a - s[i] * b;
      y[2 * i + 1] = s[i] * a + c[i] * b;
      if (tangent) {
        const float ta = ty[2 * i], tb2 = ty[2 * i + 1];
        ty[2 * i] = c[i] * ta - s[i] * tb2;
        ty[2 * i + 1] = s[i] * ta + c[i] * tb2;
      }
    }
  }
  store_row<BF16>(p.y, off, y);
  if (tangent) store_row<BF16>(p.ty, off, ty);
}

template <bool BF16, int D>
hipError_t launch(NormRopeProblem p, hipStream_t stream) {
  using C = NrCfg<BF16, D>;
  const int n_tb = (p.L + C::kRowsPerBlock - 1) / C::kRowsPerBlock;
  p.n_blocks = n_tb * p.BH;
  return launch_1d(reinterpret_cast<const void*>(&norm_rope_kernel<BF16, D>), p.n_blocks, 256, p, stream);
}

}  // namespace

hipError_t launch_norm_rope(const NormRopeProblem& p, hipStream_t stream) {
  if (p.bf16) return p.d == 128 ? launch<true, 128>(p, stream) : launch<true, 64>(p, stream);
  return p.d == 128 ? launch<false, 128>(p, stream) : launch<false, 64>(p, stream);
}

}  // namespace attnjvp
