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
// gfx950 LDS has 64 banks (256 bytes per cycle); a 16-byte read is served 16
// lanes at a time, a ds_read_b64_tr_b16 32 lanes at a time.
//  * K, tK: the S products read unit u of 32 consecutive keys; the swizzle
//    spreads any 16 consecutive keys over all 16 bank groups (d = 128: rows are
//    256 bytes, unit ^ (key & 15); d = 64: rows are 128 bytes, two per bank
//    window, unit ^ ((key >> 1) & 7)).
//  * V, tV: a 32-lane half of a transposing read takes 64 bytes from each of 4
//    consecutive keys; the swizzle moves each key's 4-unit group to its own
//    quarter of the bank window (d = 128: unit ^ 4(key & 3); d = 64: two keys
//    per window, unit ^ 4((key >> 1) & 1)).
// Both layouts were checked conflict-free with the SQ_LDS_BANK_CONFLICT counter.
template <int D>
__device__ inline int k_swz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ inline int v_swz(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

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
  const int u = pu ^ (vswz ? v_swz<D>(r) : k_swz<D>(r));
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
  // LDS stage s holds K | tK | V | tV.  K/tK of tile j and V/tV of tile j live in
  // stage j & 1; the K half is fetched two tiles ahead, the V half one tile
  // ahead.  Tiles at or past the end are fetched as zeros (empty range).
  auto issue = [&](int j, int tn0) {
    const int key0 = j * kBc;
    const uint32_t left = key0 < Lk ? (uint32_t)(Lk - key0) * D * 2 : 0u;
    char* stage = smem + (j & 1) * C::kStage;
#pragma unroll
    for (int tn = tn0; tn < tn0 + 2; ++tn) {
      const auto r = make_rsrc(kbase[tn] + (size_t)key0 * D * 2, left);
#pragma unroll
      for (int i = 0; i < C::kLoadsPerWave; ++i)
        lds_dma16(r, stage + tn * C::kTile + (wv * C::kLoadsPerWave + i) * 1024, tn < 2 ? voff_k[i] : voff_v[i]);
    }
  };

  // Per-lane LDS read offsets.
  // K fragment (key block kb, dim chunk c): key 32kb + n, unit (2c + hh) ^ k_swz(n).
  const uint32_t krow = n * C::kRow;
  const int ksw = k_swz<D>(n);
  // V fragment via ds_read_b64_tr_b16: in 16-lane group G = lane / 16 (half
  // hh = G / 2, dims 16(G & 1) .. +15 of the 32-dim block), source lane s reads
  // 4 dims starting at 4(s & 3) of key 4hh + (s >> 2) (+ 16cc + 8rho).
  const int G = lane >> 4, sl = lane & 15;
  const int vkey = 4 * (G >> 1) + (sl >> 2);
  uint32_t voff_tr[C::kBlocksD];
#pragma unroll
  for (int b = 0; b < C::kBlocksD; ++b) {
    const int d0 = 32 * b + 16 * (G & 1) + 4 * (sl & 3);
    voff_tr[b] = vkey * C::kRow + ((((d0 >> 3) ^ v_swz<D>(vkey)) << 4) | ((d0 & 7) * 2));
  }

  // S^T = K Q^T and tS^T = K tQ^T + tK Q^T of tile j (K half of stage j & 1).
  auto logits = [&](int j, f32x16 (&s)[2], f32x16 (&ts)[2]) {
    const char* cur = smem + (j & 1) * C::kStage;
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
  };

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
  // O^T += V^T P^T and tO^T += tV^T P^T + V^T (P*tS)^T for tile j.  The V^T
  // fragment (dim block b, key chunk cc) has keys 16cc + 4hh + 0..3 in elements
  // 0..3 and 16cc + 8 + 4hh + 0..3 in elements 4..7, matching the P registers.
  auto accumulate = [&](int j, const bf16x8 (&pf)[4], const bf16x8 (&ptf)[4]) {
    const char* cur = smem + (j & 1) * C::kStage;
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
  const bool ragged = (Lk % kBc) != 0;
  f32x16 s[2], ts[2];    // logits of the tile whose probabilities come next
  f32x16 sn[2], tsn[2];  // logits of the following tile, being accumulated

  // Prologue: tile 0 logits; its max sets the exponent base.
  issue(0, 0);
  issue(0, 2);
  issue(1, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): all DMA of this wave landed
  __syncthreads();
  logits(0, s, ts);
  if (nt == 1 && ragged) mask_tail<2>(s, Lk, hh);
  float mt = tile_max_log2<2>(s, c2);
  apply_rescale(st, mt);  // accumulators are still zero
  __syncthreads();        // every wave is done with K of tile 0 before it is refilled

  // Iteration j: probabilities of tile j while the logits of tile j + 1 are
  // computed, then the O / tO products of tile j while the max of tile j + 1 is
  // reduced.  In flight meanwhile: K of tile j + 2 and V of tile j + 1.
  auto iteration = [&](int j, bool mask_next) {
    issue(j + 2, 0);
    issue(j + 1, 2);
    bf16x8 pf[4], ptf[4];
    probabilities(s, ts, pf, ptf);
    logits(j + 1, sn, tsn);
    accumulate(j, pf, ptf);
    if (mask_next) mask_tail<2>(sn, Lk - (j + 1) * kBc, hh);
    mt = tile_max_log2<2>(sn, c2);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = sn[kb];
      ts[kb] = tsn[kb];
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
  };

  int j = 0;
  // The hot loop only feeds the accumulators to MFMAs: a tile that moves the
  // exponent base (rare after the first) leaves it, and the accumulators are
  // rescaled outside before it re-enters.
  while (true) {
    bool rescale = false;
    while (j < nt - 2) {
      iteration(j, false);
      ++j;
      if (needs_rescale(st, mt)) {
        rescale = true;
        break;
      }
    }
    if (!rescale) break;
    const float alpha = apply_rescale(st, mt);
#pragma unroll
    for (int b = 0; b < C::kBlocksD; ++b) {
      acc_o[b] *= alpha;
      acc_t[b] *= alpha;
    }
  }
  if (j == nt - 2) {  // the last tile's logits (masked if ragged)
    iteration(j, ragged);
    ++j;
    if (needs_rescale(st, mt)) {
      const float alpha = apply_rescale(st, mt);
#pragma unroll
      for (int b = 0; b < C::kBlocksD; ++b) {
        acc_o[b] *= alpha;
        acc_t[b] *= alpha;
      }
    }
  }
  {  // drain: the last tile's probabilities and products
    bf16x8 pf[4], ptf[4];
    probabilities(s, ts, pf, ptf);
    accumulate(j, pf, ptf);
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
