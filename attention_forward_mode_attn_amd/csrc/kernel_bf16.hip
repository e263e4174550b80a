// bf16 attention forward + JVP on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// The kernel follows the fused design the rCM pages describe — the JVP is
// carried through the same block-wise tiling as the FlashAttention-2 forward
// (ai.info summary of "Large Scale Diffusion Distillation via Score-Regularized
// Continuous-Time Consistency", "Methodology in Plain English"; papernotes.org
// notes on the same paper, "Key designs" item 1) — laid out for CDNA4:
//
//  * one workgroup = 4 waves = 128 query rows of one (batch, head); each wave
//    owns 32 rows and keeps their Q and tQ bf16 fragments in registers;
//  * the keys stream in tiles of 64 through double-buffered LDS; per tile and
//    wave the six dense products run on MFMA with fp32 accumulation:
//      S^T  = K Q^T                (16 MFMAs at d = 128)
//      tS^T = K tQ^T + tK Q^T      (32)
//      O^T += V^T P^T              (16)
//      tO^T += tV^T P^T + V^T (P*tS)^T   (32)
//    Everything is transposed so that a lane owns one query: the softmax
//    statistics are per-lane registers, and the S accumulator already has the
//    layout of the P operand of the next products, so P never leaves registers;
//  * all four K/V tiles go global -> LDS by buffer_load ... lds (no staging
//    registers; rows past Lk read as zero), row-major with XOR-swizzled
//    16-byte units; K fragments are one ds_read_b128, V fragments are built by
//    two ds_read_b64_tr_b16 transposing reads, whose 4-key runs match the
//    accumulator layout of P, so V never needs an explicit transpose;
//  * online softmax in the log2 domain with a lazily moved exponent base, per
//    row running sums l = sum p and a = sum p*tS, and the epilogue
//      O = acc_o / l,  tO = (acc_t - (a / l) acc_o) / l,  lse = (m + log2 l) ln 2.
#include "device_common.h"
#include "launch.h"

namespace attnjvp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kBc = 64;  // keys per tile

struct Params {
  const void* q;
  const void* k;
  const void* v;
  const void* tq;
  const void* tk;
  const void* tv;
  void* o;
  void* to;
  float* lse;
  int Lq, Lk, n_qtiles, n_blocks;
  float scale;
};

template <int D>
struct Cfg {
  static constexpr int kRow = D * 2;               // bytes of one tile row (one key)
  static constexpr int kTile = kBc * kRow;          // bytes of one K/tK/V/tV tile
  static constexpr int kStage = 4 * kTile;          // K | tK | V | tV
  static constexpr int kUnitsPerRow = kRow / 16;    // 16-byte units per row
  static constexpr int kRowsPerLoad = 1024 / kRow;  // rows one 64-lane x 16-byte load fills
  static constexpr int kLoadsPerWave = kTile / 1024 / kWaves;  // per tensor per tile
  static constexpr int kChunksD = D / 16;           // 16-wide head-dim chunks (S products)
  static constexpr int kBlocksD = D / 32;           // 32-row head-dim blocks (O products)
  static_assert(kTile % (1024 * kWaves) == 0, "tile split");
};

// LDS tile layout: row-major [key][dim], 16-byte units XOR-swizzled per row.
//  * K, tK: unit u of key r sits at u ^ (r & 7).  The S products read one unit
//    from each of 32 consecutive keys, so 8 consecutive lanes hit 8 distinct
//    bank groups.
//  * V, tV: unit u of key r sits at u ^ (2 * (r & 3)).  The O products read them
//    with ds_read_b64_tr_b16: a 16-lane group reads 32 bytes from each of 4
//    consecutive keys, which then land in 4 disjoint bank groups.
__device__ inline int k_swz(int r) { return r & 7; }
__device__ inline int v_swz(int r) { return 2 * (r & 3); }

// Direct global->LDS copy of one tile: every wave-instruction fills 1 KB of LDS
// in lane order (lane l -> bytes 16l..16l+15), so the swizzle is applied on the
// global side by choosing which 16 bytes each lane fetches.  Rows past the end
// of the tensor read as zero (buffer range check), so the last tile is padded
// with zero keys.
template <int D>
__device__ inline uint32_t tile_load_voff(int blk, int lane, bool vswz) {
  using C = Cfg<D>;
  const int r = blk * C::kRowsPerLoad + lane / C::kUnitsPerRow;
  const int pu = lane % C::kUnitsPerRow;
  const int u = pu ^ (vswz ? v_swz(r) : k_swz(r));
  return (uint32_t)(r * C::kRow + u * 16);
}

__device__ inline void lds_dma16(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// LDS read helpers.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ inline i16x4 lds_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(__attribute__((address_space(3))) const char*)p);
}

__device__ inline bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ inline unsigned pack_bf16(float a, float b) {
  f32x2 f = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}

__device__ inline f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_jvp_bf16_kernel(Params p) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(1024))) char smem[2 * C::kStage];

  const int t = threadIdx.x;
  const int lane = t & 63, n = lane & 31, hh = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const int blk = xcd_logical_block(blockIdx.x, p.n_blocks);
  const int bh = blk / p.n_qtiles, qt = blk % p.n_qtiles;
  const int Lq = p.Lq, Lk = p.Lk;

  const size_t qhead = (size_t)bh * Lq * D * 2, khead = (size_t)bh * Lk * D * 2;
  const uint32_t qbytes = (uint32_t)Lq * D * 2;
  const auto rq = make_rsrc((const char*)p.q + qhead, qbytes);
  const auto rtq = make_rsrc((const char*)p.tq + qhead, qbytes);
  const char* kbase[4] = {(const char*)p.k + khead, (const char*)p.tk + khead,
                          (const char*)p.v + khead, (const char*)p.tv + khead};

  // Q and tQ fragments (B operand of S^T = K Q^T): lane (n, hh) holds dims
  // 16c + 8hh .. +7 of its query row.  Rows past Lq read as zero.
  const int qrow = qt * kBlockRows + wv * kWaveRows + n;
  bf16x8 qf[C::kChunksD], tqf[C::kChunksD];
#pragma unroll
  for (int c = 0; c < C::kChunksD; ++c) {
    const uint32_t off = ((uint32_t)qrow * D + 16 * c + 8 * hh) * 2;
    qf[c] = as_bf16x8(buf_load16(rq, off));
    tqf[c] = as_bf16x8(buf_load16(rtq, off));
  }

  f32x16 acc_o[C::kBlocksD], acc_t[C::kBlocksD];
#pragma unroll
  for (int b = 0; b < C::kBlocksD; ++b) {
    acc_o[b] = f32x16{};
    acc_t[b] = f32x16{};
  }
  RowState st = {-INFINITY, 0.0f, 0.0f};
  const float scale = p.scale;
  const float c2 = scale * kLog2e;

  // Per-lane global offsets of this wave's share of a tile copy (loop invariant).
  uint32_t voff_k[C::kLoadsPerWave], voff_v[C::kLoadsPerWave];
#pragma unroll
  for (int i = 0; i < C::kLoadsPerWave; ++i) {
    voff_k[i] = tile_load_voff<D>(wv * C::kLoadsPerWave + i, lane, false);
    voff_v[i] = tile_load_voff<D>(wv * C::kLoadsPerWave + i, lane, true);
  }
  auto issue_tile = [&](int j) {
    const int key0 = j * kBc;
    const uint32_t left = (uint32_t)(Lk - key0) * D * 2;
    char* stage = smem + (j & 1) * C::kStage;
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
      const auto r = make_rsrc(kbase[tn] + (size_t)key0 * D * 2, left);
#pragma unroll
      for (int i = 0; i < C::kLoadsPerWave; ++i)
        lds_dma16(r, stage + tn * C::kTile + (wv * C::kLoadsPerWave + i) * 1024, tn < 2 ? voff_k[i] : voff_v[i]);
    }
  };

  // Per-lane LDS read offsets.
  // K fragment (key block kb, dim chunk c): key 32kb + n, unit (2c + hh) ^ (n & 7).
  const uint32_t krow = n * C::kRow;
  const int ksw = n & 7;
  // V fragment via ds_read_b64_tr_b16: in 16-lane group G = lane / 16 (half
  // hh = G / 2, dims 16(G & 1) .. +15 of the 32-dim block), source lane s reads
  // 4 dims starting at 4(s & 3) of key 4hh + (s >> 2) (+ 16cc + 8rho).
  const int G = lane >> 4, sl = lane & 15;
  const int vkey = 4 * (G >> 1) + (sl >> 2);
  uint32_t voff_tr[C::kBlocksD];
#pragma unroll
  for (int b = 0; b < C::kBlocksD; ++b) {
    const int d0 = 32 * b + 16 * (G & 1) + 4 * (sl & 3);
    voff_tr[b] = vkey * C::kRow + ((((d0 >> 3) ^ v_swz(vkey)) << 4) | ((d0 & 7) * 2));
  }

  // P and P*tS of one tile as bf16 B operands, accumulated into l and a:
  // chunk cc (keys 16cc..16cc+15) is registers 8*(cc%2) .. +7 of key block cc/2.
  auto probabilities = [&](const f32x16 (&s)[2], const f32x16 (&ts)[2], bf16x8 (&pf)[4], bf16x8 (&ptf)[4]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(s[kb][r], c2, -st.m));
        const float p1 = fast_exp2(__builtin_fmaf(s[kb][r + 1], c2, -st.m));
        const float q0 = p0 * (ts[kb][r] * scale);
        const float q1 = p1 * (ts[kb][r + 1] * scale);
        st.l += p0 + p1;
        st.a += q0 + q1;
        const int cc = 2 * kb + (r >> 3), i = r & 7;
        const unsigned pp = pack_bf16(p0, p1), qq = pack_bf16(q0, q1);
        pf[cc][i] = __builtin_bit_cast(bf16x2, pp)[0];
        pf[cc][i + 1] = __builtin_bit_cast(bf16x2, pp)[1];
        ptf[cc][i] = __builtin_bit_cast(bf16x2, qq)[0];
        ptf[cc][i + 1] = __builtin_bit_cast(bf16x2, qq)[1];
      }
    }
  };
  // O^T += V^T P^T and tO^T += tV^T P^T + V^T (P*tS)^T for one tile.  The V^T
  // fragment (dim block b, key chunk cc) has keys 16cc + 4hh + 0..3 in elements
  // 0..3 and 16cc + 8 + 4hh + 0..3 in elements 4..7, matching the P registers.
  auto accumulate = [&](const char* cur, const bf16x8 (&pf)[4], const bf16x8 (&ptf)[4]) {
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      bf16x8 vv[C::kBlocksD];
#pragma unroll
      for (int b = 0; b < C::kBlocksD; ++b) {
        const char* vb = cur + 2 * C::kTile + 16 * cc * C::kRow + voff_tr[b];
        const i16x4 lo = lds_tr16(vb), hi = lds_tr16(vb + 8 * C::kRow);
        const char* tb = vb + C::kTile;
        const i16x4 tlo = lds_tr16(tb), thi = lds_tr16(tb + 8 * C::kRow);
        vv[b] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        const bf16x8 tvv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(tlo, thi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc_o[b] = mfma(vv[b], pf[cc], acc_o[b]);
        acc_t[b] = mfma(tvv, pf[cc], acc_t[b]);
      }
#pragma unroll
      for (int b = 0; b < C::kBlocksD; ++b) acc_t[b] = mfma(vv[b], ptf[cc], acc_t[b]);
    }
  };

  const int nt = (Lk + kBc - 1) / kBc;
  issue_tile(0);
  int j = 0;
  f32x16 s[2], ts[2];
  float mt = 0.0f;
  // The hot loop only feeds the accumulators to MFMAs.  A tile whose row max
  // moves the exponent base (always the first, rarely a later one) leaves the
  // loop, rescales the accumulators outside it and re-enters.
  while (true) {
    bool rescale = false;
    for (; j < nt; ++j) {
      // the tile j copy must have landed for every wave before it is read
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
      const char* cur = smem + (j & 1) * C::kStage;
      if (j + 1 < nt) issue_tile(j + 1);

      // ---- logits and tangent logits ------------------------------------
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        ts[kb] = f32x16{};
      }
#pragma unroll
      for (int c = 0; c < C::kChunksD; ++c) {
        const uint32_t u = krow + (((2 * c + hh) ^ ksw) << 4);
        const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(cur + u);
        const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(cur + 32 * C::kRow + u);
        const bf16x8 tk0 = *reinterpret_cast<const bf16x8*>(cur + C::kTile + u);
        const bf16x8 tk1 = *reinterpret_cast<const bf16x8*>(cur + C::kTile + 32 * C::kRow + u);
        s[0] = mfma(k0, qf[c], s[0]);
        s[1] = mfma(k1, qf[c], s[1]);
        ts[0] = mfma(k0, tqf[c], ts[0]);
        ts[1] = mfma(k1, tqf[c], ts[1]);
        ts[0] = mfma(tk0, qf[c], ts[0]);
        ts[1] = mfma(tk1, qf[c], ts[1]);
      }

      // ---- online softmax ------------------------------------------------
      if (j == nt - 1 && (Lk % kBc) != 0) mask_tail<2>(s, Lk - j * kBc, hh);
      mt = tile_max_log2<2>(s, c2);
      if (needs_rescale(st, mt)) {
        rescale = true;
        break;
      }
      bf16x8 pf[4], ptf[4];
      probabilities(s, ts, pf, ptf);
      accumulate(cur, pf, ptf);
    }
    if (!rescale) break;
    // ---- tile j with a new exponent base ----------------------------------
    const float alpha = apply_rescale(st, mt);
#pragma unroll
    for (int b = 0; b < C::kBlocksD; ++b) {
      acc_o[b] *= alpha;
      acc_t[b] *= alpha;
    }
    bf16x8 pf[4], ptf[4];
    probabilities(s, ts, pf, ptf);
    accumulate(smem + (j & 1) * C::kStage, pf, ptf);
    ++j;
  }

  // ---- epilogue ------------------------------------------------------------
  const float l = xhalf_sum(st.l), a = xhalf_sum(st.a);
  const float inv = 1.0f / l, mu = a * inv;
  const auto ro = make_rsrc((const char*)p.o + qhead, qbytes);
  const auto rto = make_rsrc((const char*)p.to + qhead, qbytes);
#pragma unroll
  for (int b = 0; b < C::kBlocksD; ++b) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float ov[4], tv4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = acc_o[b][4 * g + i];
        ov[i] = x * inv;
        tv4[i] = (acc_t[b][4 * g + i] - mu * x) * inv;
      }
      const uint32_t off = ((uint32_t)qrow * D + 32 * b + 8 * g + 4 * hh) * 2;
      buf_store8(ro, off, u32x2{pack_bf16(ov[0], ov[1]), pack_bf16(ov[2], ov[3])});
      buf_store8(rto, off, u32x2{pack_bf16(tv4[0], tv4[1]), pack_bf16(tv4[2], tv4[3])});
    }
  }
  if (hh == 0) {
    const auto rl = make_rsrc((const char*)p.lse + (size_t)bh * Lq * 4, (uint32_t)Lq * 4);
    buf_store4(rl, (uint32_t)qrow * 4, (st.m + __builtin_amdgcn_logf(l)) * kLn2);
  }
}

template <int D>
hipError_t launch(const Problem& pr, hipStream_t stream) {
  Params p;
  p.q = pr.q; p.k = pr.k; p.v = pr.v; p.tq = pr.tq; p.tk = pr.tk; p.tv = pr.tv;
  p.o = pr.o; p.to = pr.to; p.lse = pr.lse;
  p.Lq = pr.Lq; p.Lk = pr.Lk; p.scale = pr.scale;
  p.n_qtiles = (pr.Lq + kBlockRows - 1) / kBlockRows;
  p.n_blocks = pr.B * pr.H * p.n_qtiles;
  hipLaunchKernelGGL(attn_jvp_bf16_kernel<D>, dim3(p.n_blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bf16(const Problem& p, hipStream_t stream) {
  return p.d == 128 ? launch<128>(p, stream) : launch<64>(p, stream);
}

}  // namespace attnjvp
