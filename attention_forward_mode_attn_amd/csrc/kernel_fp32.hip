// fp32 attention forward + JVP on gfx950 matrix cores (v_mfma_f32_32x32x2_f32).
//
// Same tiling, transposed products and online softmax as the bf16 kernel, in
// IEEE fp32 throughout (fp32 MFMA has no reduced-precision inputs).  Each MFMA
// contracts two elements, one per half-wave, so:
//  * S^T = K Q^T pairs head dims c and c + d/2 (half hh supplies dim
//    hh*d/2 + c): each lane keeps d/2 of its query's Q and tQ values;
//  * O^T += V^T P^T pairs the two keys that accumulator register r holds in the
//    two halves, so P comes straight from the S accumulator as an fp32 operand
//    and V is read row-major from LDS (32 consecutive dims per half-wave).
// Tiles hold 32 keys (one accumulator block) to bound register use.
#include "device_common.h"
#include "launch.h"

namespace attnjvp {
namespace {

constexpr int kBcF = 32;  // keys per tile

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
  float* tlse;
  int Lq, Lk, kv_rows, n_qtiles, n_blocks;
  float scale;
};

template <int D>
struct Cfg {
  static constexpr int kTile = kBcF * D * 4;           // bytes of one tile, [key][dim]
  static constexpr int kStage = 4 * kTile;             // K, tK, V, tV
  static constexpr int kLoadsPerWave = kTile / 1024 / kWaves;  // 1 KB copies per tensor per tile
  static constexpr int kBlocksD = D / 32;
  static_assert(kTile % (1024 * kWaves) == 0, "tile split");
};

// K/tK rows are XOR-swizzled by 16-byte unit so that the 16 lanes that a
// 16-byte LDS read serves together (16 consecutive keys, same column) hit all
// 16 bank groups of gfx950's 64-bank LDS.  V/tV rows are not swizzled: their
// readers take 32 consecutive floats of one row.
template <int D>
__device__ inline uint32_t k_off(int r, int u) {
  return r * (D * 4) + ((u ^ (r & 15)) << 4);
}

__device__ inline f32x16 mfma(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Tiles go global -> LDS by buffer_load ... lds: the lane that fills LDS slot
// 16 s of a tile (row r = s / (D/4), physical unit pu) fetches the 16 bytes of
// logical unit pu ^ (r & 15) for K/tK (the swizzle of k_off), pu for V/tV.
// Rows past Lk read as zero (buffer range check).
template <int D>
__device__ inline uint32_t tile_voff(int slice, int lane, bool kswz) {
  const int slot = slice * 64 + lane, r = slot / (D / 4), pu = slot % (D / 4);
  return (uint32_t)(r * D + 4 * (kswz ? (pu ^ (r & 15)) : pu)) * 4;
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_jvp_fp32_kernel(Params p) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(1024))) char smem[2 * C::kStage];

  const int t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6, n = lane & 31, hh = lane >> 5;
  const int blk = xcd_logical_block(blockIdx.x, p.n_blocks);
  const int bh = blk / p.n_qtiles, qt = blk % p.n_qtiles;
  const int Lq = p.Lq, Lk = p.Lk;

  const size_t qhead = (size_t)bh * Lq * D * 4, khead = (size_t)bh * p.kv_rows * D * 4;
  const uint32_t qbytes = (uint32_t)Lq * D * 4, kbytes = (uint32_t)Lk * D * 4;
  const auto rq = make_rsrc((const char*)p.q + qhead, qbytes);
  const auto rtq = make_rsrc((const char*)p.tq + qhead, qbytes);
  const __amdgpu_buffer_rsrc_t rkv[4] = {
      make_rsrc((const char*)p.k + khead, kbytes),
      p.tk ? make_rsrc((const char*)p.tk + khead, kbytes) : make_rsrc(p.k, 0),  // NULL: an empty range reads zeros
      make_rsrc((const char*)p.v + khead, kbytes),
      p.tv ? make_rsrc((const char*)p.tv + khead, kbytes) : make_rsrc(p.v, 0)};

  // Lane (n, hh) keeps dims hh*D/2 .. hh*D/2 + D/2 - 1 of its query's Q and tQ.
  const int qrow = qt * kBlockRows + wv * kWaveRows + n;
  float qf[D / 2], tqf[D / 2];
#pragma unroll
  for (int i = 0; i < D / 8; ++i) {
    const uint32_t off = ((uint32_t)qrow * D + hh * (D / 2) + 4 * i) * 4;
    const u32x4 a = buf_load16(rq, off), b = buf_load16(rtq, off);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qf[4 * i + e] = __uint_as_float(a[e]);
      tqf[4 * i + e] = __uint_as_float(b[e]);
    }
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
  const int sw = n & 15;

  // P and P*tS of one tile (fp32, straight from the S accumulator), and the
  // O / tO products: MFMA r pairs the keys that register r holds in the two halves.
  //
  // Two-level sums: every tile's contributions to l, a and the accumulators are
  // summed on their own (16 terms per lane, 32 keys per MFMA chain) and then
  // added to the running totals once.  One fp32 chain over all Lk keys would
  // carry a rounding error that grows with Lk: on 6082 keys with peaky logits it
  // reached 2e-5 of max|tO|, while per-tile partial sums keep it near 1e-6.
  auto probabilities = [&](const f32x16& s, const f32x16& ts, float (&pv)[16], float (&ptv)[16]) {
    float lt = 0.0f, at = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pv[r] = fast_exp2(__builtin_fmaf(s[r], c2, -st.m));
      ptv[r] = pv[r] * (ts[r] * scale);
      lt += pv[r];
      at += ptv[r];
    }
    st.l += lt;
    st.a += at;
  };
  auto accumulate = [&](const char* cur, const float (&pv)[16], const float (&ptv)[16]) {
    const char* vbase = cur + 2 * C::kTile;
    const char* tvbase = cur + 3 * C::kTile;
    // Block b's partial sums are added to the totals under block b + 1's first
    // MFMAs, not right behind their own last one.
    f32x16 to_[2], tt_[2];
#pragma unroll
    for (int b = 0; b < C::kBlocksD; ++b) {
      const int k = b & 1;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t off = (acc_row(r, hh) * D + 32 * b + n) * 4;
        const float vv = *reinterpret_cast<const float*>(vbase + off);
        const float tvv = *reinterpret_cast<const float*>(tvbase + off);
        to_[k] = mfma(vv, pv[r], r == 0 ? f32x16{} : to_[k]);
        tt_[k] = mfma(tvv, pv[r], r == 0 ? f32x16{} : tt_[k]);
        tt_[k] = mfma(vv, ptv[r], tt_[k]);
        if (b > 0 && r == 1) {
          acc_o[b - 1] += to_[k ^ 1];
          acc_t[b - 1] += tt_[k ^ 1];
        }
      }
    }
    acc_o[C::kBlocksD - 1] += to_[(C::kBlocksD - 1) & 1];
    acc_t[C::kBlocksD - 1] += tt_[(C::kBlocksD - 1) & 1];
  };

  // Tile j lives in LDS stage j & 1; tile j + 1 is copied while tile j is used
  // (its stage was last read before the previous barrier).
  uint32_t voff_k[C::kLoadsPerWave], voff_v[C::kLoadsPerWave];
#pragma unroll
  for (int i = 0; i < C::kLoadsPerWave; ++i) {
    voff_k[i] = tile_voff<D>(wv * C::kLoadsPerWave + i, lane, true);
    voff_v[i] = tile_voff<D>(wv * C::kLoadsPerWave + i, lane, false);
  }
  const uint32_t smem_lds = __builtin_amdgcn_readfirstlane(lds_address(smem));
  auto issue = [&](int j) {
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
#pragma unroll
      for (int i = 0; i < C::kLoadsPerWave; ++i)
        lds_dma16(rkv[tn], smem_lds + (j & 1) * C::kStage + tn * C::kTile + (wv * C::kLoadsPerWave + i) * 1024,
                  (tn < 2 ? voff_k[i] : voff_v[i]) + (uint32_t)j * C::kTile);
  };
  const int nt = (Lk + kBcF - 1) / kBcF;
  issue(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  int j = 0;
  f32x16 s, ts;
  float mt = 0.0f;
  // Same structure as the bf16 kernel: tiles that move the exponent base leave
  // the hot loop so that the accumulators are rescaled outside it.
  while (true) {
    bool rescale = false;
    for (; j < nt; ++j) {
      const char* cur = smem + (j & 1) * C::kStage;
      if (j + 1 < nt) issue(j + 1);

      s = f32x16{};
      ts = f32x16{};
#pragma unroll
      for (int i = 0; i < D / 8; ++i) {
        // logical unit hh*D/8 + i of row n holds dims hh*D/2 + 4i .. +3
        const uint32_t off = n * (D * 4) + (((hh * (D / 8) + i) ^ sw) << 4);
        const f32x4 kk = *reinterpret_cast<const f32x4*>(cur + off);
        const f32x4 tkk = *reinterpret_cast<const f32x4*>(cur + C::kTile + off);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s = mfma(kk[e], qf[4 * i + e], s);
          ts = mfma(kk[e], tqf[4 * i + e], ts);
          ts = mfma(tkk[e], qf[4 * i + e], ts);
        }
      }
      if (j == nt - 1 && (Lk % kBcF) != 0) {
        f32x16 sm[1] = {s};
        mask_tail<1>(sm, Lk - j * kBcF, hh);
        s = sm[0];
      }
      {
        const f32x16 sm[1] = {s};
        mt = tile_max_log2<1>(sm, c2);
      }
      if (needs_rescale(st, mt)) {
        rescale = true;
        break;
      }
      float pv[16], ptv[16];
      probabilities(s, ts, pv, ptv);
      accumulate(cur, pv, ptv);
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile j + 1 of this wave landed
      __syncthreads();
    }
    if (!rescale) break;
    const float alpha = apply_rescale(st, mt);
#pragma unroll
    for (int b = 0; b < C::kBlocksD; ++b) {
      acc_o[b] *= alpha;
      acc_t[b] *= alpha;
    }
    float pv[16], ptv[16];
    probabilities(s, ts, pv, ptv);
    accumulate(smem + (j & 1) * C::kStage, pv, ptv);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    ++j;
  }

  const float l = xhalf_sum(st.l), a = xhalf_sum(st.a);
  const float inv = 1.0f / l, mu = a * inv;
  const auto ro = make_rsrc((const char*)p.o + qhead, qbytes);
  const auto rto = make_rsrc((const char*)p.to + qhead, qbytes);
  // All values first (each in its own registers), then the stores from one
  // address register: reusing a store's registers right after issuing it makes
  // the next write wait until the queued store has read them.  Group g of a
  // lane holds dims 8g + 4hh .. +3 of its query (16 bytes).
  u32x4 ov[C::kBlocksD][4], tv4[C::kBlocksD][4];
#pragma unroll
  for (int b = 0; b < C::kBlocksD; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = acc_o[b][4 * g + i];
        ov[b][g][i] = __float_as_uint(x * inv);
        tv4[b][g][i] = __float_as_uint((acc_t[b][4 * g + i] - mu * x) * inv);
      }
  __builtin_amdgcn_sched_barrier(0);
  const uint32_t obase = ((uint32_t)qrow * D + 4 * hh) * 4;  // rows past Lq: out of range, dropped
#pragma unroll
  for (int b = 0; b < C::kBlocksD; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      __builtin_amdgcn_raw_buffer_store_b128(ov[b][g], ro, obase, (32 * b + 8 * g) * 4, 0);
      __builtin_amdgcn_raw_buffer_store_b128(tv4[b][g], rto, obase, (32 * b + 8 * g) * 4, 0);
    }
  if (hh == 0) {
    const auto rl = make_rsrc((const char*)p.lse + (size_t)bh * Lq * 4, (uint32_t)Lq * 4);
    buf_store4(rl, (uint32_t)qrow * 4, (st.m + __builtin_amdgcn_logf(l)) * kLn2);
    if (p.tlse) {
      const auto rtl = make_rsrc((const char*)p.tlse + (size_t)bh * Lq * 4, (uint32_t)Lq * 4);
      buf_store4(rtl, (uint32_t)qrow * 4, mu);
    }
  }
}

template <int D>
hipError_t launch(const Problem& pr, hipStream_t stream) {
  Params p;
  p.q = pr.q; p.k = pr.k; p.v = pr.v; p.tq = pr.tq; p.tk = pr.tk; p.tv = pr.tv;
  p.o = pr.o; p.to = pr.to; p.lse = pr.lse; p.tlse = pr.tlse;
  p.Lq = pr.Lq; p.Lk = pr.Lk; p.kv_rows = pr.kv_rows; p.scale = pr.scale;
  p.n_qtiles = (pr.Lq + kBlockRows - 1) / kBlockRows;
  p.n_blocks = pr.B * pr.H * p.n_qtiles;
  return launch_1d(reinterpret_cast<const void*>(&attn_jvp_fp32_kernel<D>), p.n_blocks, kThreads, p, stream);
}

}  // namespace

hipError_t launch_fp32(const Problem& p, hipStream_t stream) {
  return p.d == 128 ? launch<128>(p, stream) : launch<64>(p, stream);
}

}  // namespace attnjvp
