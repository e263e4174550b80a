// Device-side helpers shared by the bf16 and fp32 attention-JVP kernels (gfx950).
//
// Conventions used throughout:
//  * A wave (64 lanes) owns 32 query rows.  Lane l serves query n = l % 32 and
//    "half" hh = l / 32.  All products are computed transposed (keys or head
//    dimension in the MFMA M slot, queries in the N slot), so the 32x32 MFMA
//    accumulator layout puts one query per lane:
//        accumulator register r of lane l  ->  row 8*(r/4) + 4*hh + r%4, column n.
//    Per-query statistics are therefore per-lane values; the two halves of a
//    query (lanes l and l^32) hold disjoint key subsets and are combined with
//    v_permlane32_swap.
//  * Online softmax runs in the log2 domain: x = S * scale * log2(e).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace attnjvp {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaveRows = 32;              // query rows per wave
constexpr int kWaves = 4;                  // waves per workgroup
constexpr int kThreads = kWaves * 64;      // 256
constexpr int kBlockRows = kWaves * kWaveRows;  // 128 query rows per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Rescale threshold (log2 units): the running max used for exponentiation is
// only moved when a row's max grows by more than this, so exp2 arguments stay
// <= kRescaleSlack and p <= 2^32.  Softmax is shift invariant, so the result is
// the same up to rounding (relative rounding does not depend on magnitude).
// Headroom: with Lk < 2^23 the sums stay below 2^55 * max|v|, far from fp32
// overflow for any input below 2^73 in magnitude; weights more than 2^-94 below
// the row max flush to zero.  A large slack keeps peaky softmaxes (logit std
// ~8) from leaving the hot loop to rescale on most tiles.
constexpr float kRescaleSlack = 32.0f;

__device__ inline bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// Two floats to a packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ inline unsigned pack_bf16(float a, float b) {
  f32x2 f = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}

// Scheduling fence: the compiler may not move instructions across it.  The
// pipelined loops are written as sequences of small units (one MFMA plus a
// slice of independent work) separated by fences, so that the vector ALU and
// the memory pipes work while the matrix core runs instead of the two
// alternating in long runs.
__device__ inline void fence() { __builtin_amdgcn_sched_barrier(0); }

template <int I>
using IC = std::integral_constant<int, I>;

// Compile-time loop: f(std::integral_constant<int, i>) for i in [B, E).  Every
// register-array index in a pipelined loop is a constant, so the arrays stay
// in registers (a runtime index would send them to memory).
template <int B, int E, typename F>
__device__ inline void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Buffer resource over [base, base + bytes): loads past the end return 0 and
// stores past the end are dropped by the hardware range check.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ inline u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ inline void buf_store4(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}

// Direct global -> LDS copy of 16 bytes per lane (buffer_load_dwordx4 ... lds):
// lane l of the wave writes LDS bytes lds_addr + 16 l .. + 15.
// It is issued with inline asm rather than the builtin on purpose: the
// compiler treats a builtin LDS DMA as a store that may alias every LDS read
// that follows, and waits for it (vmcnt(0)) before the next read even though
// the two stages never overlap.  Here the pipeline orders the copies itself:
// each stage is refilled only after a barrier that follows its last read, and
// read only after an explicit vmcnt(0) and a barrier.  The instruction has no
// register outputs; its LDS destination (a wave-uniform LDS byte address) is
// passed in M0.
__device__ inline void lds_dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds_addr, uint32_t voff) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(r), "{m0}"(lds_addr) : "memory");
}
// The same with a wave-uniform byte offset in the scalar offset field.  The
// buffer range check covers the sum of the vector and scalar offsets, so
// bytes past the resource still read as zero.
__device__ inline void lds_dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" : : "v"(voff), "s"(r), "s"(soff), "{m0}"(lds_addr) : "memory");
}

// LDS byte address of a __shared__ object.
__device__ inline uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2).
// Renumber them so that XCD x owns one contiguous range of logical ids: the
// query tiles of one head then run on the same XCD and share K/V in its L2.
__device__ inline int xcd_logical_block(int hw_id, int n_blocks) {
  const int per = n_blocks / 8, rem = n_blocks % 8;
  const int x = hw_id % 8, slot = hw_id / 8;
  return (x < rem) ? x * (per + 1) + slot : rem * (per + 1) + (x - rem) * per + slot;
}

// Reductions across the two 32-lane halves (lane l with lane l ^ 32).
__device__ inline float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Pair accumulator groups g (in x) and g + 1 (in y) of one lane across the two
// half-waves with v_permlane32_swap: a lane of half 0 ends up with the 8
// consecutive rows of group g (its own 4 and its partner's 4), a lane of half
// 1 with those of group g + 1, as one 16-byte store of packed bf16 pairs.
__device__ inline u32x4 pair_halves(u32x2 x, u32x2 y) {
  const auto s0 = __builtin_amdgcn_permlane32_swap(x[0], y[0], false, false);
  const auto s1 = __builtin_amdgcn_permlane32_swap(x[1], y[1], false, false);
  return u32x4{s0[0], s1[0], s0[1], s1[1]};
}

// Key offset (within a 32-key block) held by accumulator register r of half hh.
__device__ inline int acc_row(int r, int hh) { return 8 * (r >> 2) + 4 * hh + (r & 3); }

// Running per-query state.  m: max (log2 domain) used for exponentiation;
// l, a: this lane's partial sums of p and p*tS over its half of the keys;
// lb: of bf16(p), the weights the products consume; c: the value the tangent
// logits are centred on (bf16 kernel only: a holds the sum of p*(tS - c)).
struct RowState {
  float m;
  float l;
  float a;
  float lb;
  float c;
};

// Mask keys >= valid (tile-relative) of a tile made of NB 32-key blocks.
template <int NB>
__device__ inline void mask_tail(f32x16 (&s)[NB], int valid, int hh) {
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (32 * b + acc_row(r, hh) >= valid) s[b][r] = -INFINITY;
}

// Tile max of the raw logits, combined over both halves, in the log2 domain.
template <int NB>
__device__ inline float tile_max_log2(const f32x16 (&s)[NB], float c) {
  float mx = -INFINITY;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[b][r]);
  return xhalf_max(mx) * c;
}

// Does this tile move the exponent base of any row of the wave?  (wave-uniform)
__device__ inline bool needs_rescale(const RowState& st, float mt) {
  return __builtin_amdgcn_ballot_w64(mt > st.m + kRescaleSlack) != 0;
}

// Move the exponent base of the rows that need it; returns each row's factor
// (1 for the others) and rescales st.l, st.a and st.lb.  The caller rescales its matrix
// accumulators by the returned factor.
__device__ inline float apply_rescale(RowState& st, float mt) {
  const bool need = mt > st.m + kRescaleSlack;
  const float m_new = need ? mt : st.m;
  const float alpha = need ? fast_exp2(st.m - m_new) : 1.0f;
  st.m = m_new;
  st.l *= alpha;
  st.a *= alpha;
  st.lb *= alpha;
  return alpha;
}

}  // namespace attnjvp
