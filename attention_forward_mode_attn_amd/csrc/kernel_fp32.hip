// fp32 attention forward + JVP on gfx950 matrix cores.
//
// The logits S = q.k are accumulated in fp64 (v_mfma_f64_16x16x4_f64 on the
// exact fp64 images of the fp32 operands); the tangent logits and the output
// products run in fp32 (v_mfma_f32_16x16x4_f32).  An fp32 sum of the d
// products of S rounds at 2^-24 of |S| at every step, and every probability
// inherits that absolute error through exp(scale * S), so an fp32 S bounds
// the accuracy of P, O and tO by the magnitude of the logits.  In fp64 the
// error of S is negligible, and exp2 is evaluated on (S * scale * log2 e - m)
// formed in fp64 and rounded once to fp32: the weights then carry a relative
// error of about 2^-24 * (slack + 1), whatever the logits' size.  tS enters
// the result only through P * tS, where an fp32 relative error suffices.
//
// Layout (transposed products, 16 x 16 blocks): a wave owns 32 queries (two
// blocks qb of 16) and a tile 32 keys (two blocks kb of 16).  Lane l = n + 16 g
// (n = l % 16, g = l / 16) serves queries 16 qb + n.  Both instructions take
// A[m][k] from lane m + 16 k and B[k][j] from lane j + 16 k; accumulator
// register i of lane l holds row 4 g + i of column n for the fp32 one, row
// g + 4 i for the fp64 one.  Hence:
//  * S^T = K Q^T and tS^T = K tQ^T + tK Q^T: the contraction step takes one
//    head dim per lane group, dims 16 G + 4 g + e at step (G, e), so a lane
//    reads 16 bytes of a K row per G and keeps 4 D/16 values of Q and of tQ;
//  * for S^T lane (n, g) reads key row 16 kb + n, and register i of block
//    (kb, qb) holds key 16 kb + g + 4 i of query 16 qb + n.  The tS^T products
//    read rows 16 kb + sigma(n), sigma(m) = 4 (m % 4) + m / 4, so that their
//    register i (row 4 g + i) holds that same key;
//  * that is the P^T operand of O^T += V^T P^T at step (kb, i), with V^T
//    read from key row 16 kb + g + 4 i;
//  * O^T rows of block (G4, r) are dims 64 G4 + 4 m + r (m = 0..15), so a lane
//    reads the 16 bytes of V at dims 64 G4 + 4 n .. + 3 once for the four
//    blocks r, and holds 4 consecutive dims of its query for each (G4, i).
// Each query's keys are spread over the four lane groups; its statistics are
// combined across them with shuffles.
#include "device_common.h"
#include "launch.h"

namespace attnjvp {
namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int kBcF = 32;  // keys per tile
constexpr double kLog2eD = 1.4426950408889634;  // log2(e), for the fp64 exponents

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
  static constexpr int kG = D / 16;                    // contraction groups of 16 dims (4 steps each)
  static constexpr int kG4 = D / 64;                   // output groups of 64 dims
  static_assert(kTile % (1024 * kWaves) == 0, "tile split");
  static_assert(D % 64 == 0, "head dim");
};

__device__ inline f64x4 mfma64(double a, double b, f64x4 c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}
__device__ inline f32x4 mfma32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// A value the compiler must treat as new at this point: keeps the fp64
// conversions of the loop-invariant query operands inside the loop (hoisted,
// they would need 2 * D more registers than the kernel has).
__device__ inline float opaque(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Max / sum over the four lane groups that share a query (lanes n, n + 16,
// n + 32, n + 48).
__device__ inline float group_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ inline float group_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

// K/tK rows are XOR-swizzled by 16-byte unit so that the 16 lanes of one
// group, which read 16 consecutive keys at the same logical unit, hit all 16
// bank groups of gfx950's 64-bank LDS.  V/tV rows are not swizzled: the 16
// lanes of a group read 256 consecutive bytes of one row.
template <int D>
__device__ inline uint32_t k_off(int r, int u) {
  return r * (D * 4) + ((u ^ (r & 15)) << 4);
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
  const int lane = t & 63, wv = t >> 6, n = lane & 15, g = lane >> 4;
  const int sig = 4 * (n & 3) + (n >> 2);  // sigma(n)
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

  // Lane (n, g) keeps dims 16 G + 4 g .. + 3 (G = 0 .. D/16 - 1) of queries
  // 16 qb + n: element 4 G + e of qf[qb] is dim 16 G + 4 g + e.
  const int qrow0 = qt * kBlockRows + wv * kWaveRows + n;
  float qf[2][D / 4], tqf[2][D / 4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int G = 0; G < C::kG; ++G) {
      const uint32_t off = ((uint32_t)(qrow0 + 16 * qb) * D + 16 * G + 4 * g) * 4;
      const u32x4 a = buf_load16(rq, off), b = buf_load16(rtq, off);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[qb][4 * G + e] = __uint_as_float(a[e]);
        tqf[qb][4 * G + e] = __uint_as_float(b[e]);
      }
    }

  // acc[G4][r][qb]: O^T rows 64 G4 + 4 m + r of queries 16 qb + n (m = 4 g + i).
  f32x4 acc_o[C::kG4][4][2], acc_t[C::kG4][4][2];
#pragma unroll
  for (int G4 = 0; G4 < C::kG4; ++G4)
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        acc_o[G4][r][qb] = f32x4{};
        acc_t[G4][r][qb] = f32x4{};
      }
  // Per query block: m (log2 domain), and this lane's partial l and a.
  float st_m[2] = {-INFINITY, -INFINITY}, st_l[2] = {0.0f, 0.0f}, st_a[2] = {0.0f, 0.0f};
  const float scale = p.scale;
  const float c2f = scale * kLog2e;
  const double c2d = (double)scale * kLog2eD;

  // P and P*tS of one tile: pv[kb][qb][i] is the weight of key 16 kb + g + 4 i
  // for query 16 qb + n.  Two-level sums: the tile's contributions to l, a and
  // the accumulators are summed on their own and then added to the totals once.
  auto probabilities = [&](const f64x4 (&s)[2][2], const f32x4 (&ts)[2][2], float (&pv)[2][2][4],
                           float (&ptv)[2][2][4]) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const double md = (double)st_m[qb];
      float lt = 0.0f, at = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = (float)__builtin_fma(s[kb][qb][i], c2d, -md);
          pv[kb][qb][i] = fast_exp2(x);
          ptv[kb][qb][i] = pv[kb][qb][i] * (ts[kb][qb][i] * scale);
          lt += pv[kb][qb][i];
          at += ptv[kb][qb][i];
        }
      st_l[qb] += lt;
      st_a[qb] += at;
    }
  };
  auto accumulate = [&](const char* cur, const float (&pv)[2][2][4], const float (&ptv)[2][2][4]) {
    const char* vbase = cur + 2 * C::kTile;
    const char* tvbase = cur + 3 * C::kTile;
    // Step u = 8 G4 + 4 kb + i; the V and tV fragments of step u + 1 are read
    // while step u's products run.
    f32x4 vr[2], tvr[2];
    auto read_v = [&](int u, f32x4& vx, f32x4& tvx) {
      const int G4 = u >> 3, kb = (u >> 2) & 1, i = u & 3;
      const uint32_t off = (16 * kb + g + 4 * i) * (D * 4) + (16 * G4 + n) * 16;
      vx = *reinterpret_cast<const f32x4*>(vbase + off);
      tvx = *reinterpret_cast<const f32x4*>(tvbase + off);
    };
    read_v(0, vr[0], tvr[0]);
#pragma unroll
    for (int G4 = 0; G4 < C::kG4; ++G4) {
      f32x4 po[4][2], pt[4][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int u = 8 * G4 + 4 * kb + i;
          fence();
          if (u + 1 < 8 * C::kG4) read_v(u + 1, vr[(u + 1) & 1], tvr[(u + 1) & 1]);
          const f32x4 vv = vr[u & 1], tvv = tvr[u & 1];
          const bool first = kb == 0 && i == 0;
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
              po[r][qb] = mfma32(vv[r], pv[kb][qb][i], first ? f32x4{} : po[r][qb]);
              pt[r][qb] = mfma32(tvv[r], pv[kb][qb][i], first ? f32x4{} : pt[r][qb]);
              pt[r][qb] = mfma32(vv[r], ptv[kb][qb][i], pt[r][qb]);
            }
        }
      fence();
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          acc_o[G4][r][qb] += po[r][qb];
          acc_t[G4][r][qb] += pt[r][qb];
        }
    }
    fence();
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
  f64x4 s[2][2];
  f32x4 ts[2][2];
  for (int j = 0; j < nt; ++j) {
    const char* cur = smem + (j & 1) * C::kStage;
    if (j + 1 < nt) issue(j + 1);

#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        s[kb][qb] = f64x4{};
        ts[kb][qb] = f32x4{};
      }
    // K (rows n and sigma(n)) and tK (rows sigma(n)) fragments of group G + 1
    // are read while group G's products run.
    f32x4 kk[2][2], ks[2][2], tks[2][2];
    auto read_k = [&](int G, f32x4 (&kx)[2], f32x4 (&ksx)[2], f32x4 (&tksx)[2]) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint32_t off = k_off<D>(16 * kb + n, 4 * G + g);
        const uint32_t offs = k_off<D>(16 * kb + sig, 4 * G + g);
        kx[kb] = *reinterpret_cast<const f32x4*>(cur + off);
        ksx[kb] = *reinterpret_cast<const f32x4*>(cur + offs);
        tksx[kb] = *reinterpret_cast<const f32x4*>(cur + C::kTile + offs);
      }
    };
    read_k(0, kk[0], ks[0], tks[0]);
#pragma unroll
    for (int G = 0; G < C::kG; ++G) {
      fence();
      if (G + 1 < C::kG) read_k(G + 1, kk[(G + 1) & 1], ks[(G + 1) & 1], tks[(G + 1) & 1]);
      const f32x4(&kx)[2] = kk[G & 1];
      const f32x4(&ksx)[2] = ks[G & 1];
      const f32x4(&tksx)[2] = tks[G & 1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double qd[2] = {(double)opaque(qf[0][4 * G + e]), (double)opaque(qf[1][4 * G + e])};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const double kd = (double)kx[kb][e];
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            s[kb][qb] = mfma64(kd, qd[qb], s[kb][qb]);
            ts[kb][qb] = mfma32(ksx[kb][e], tqf[qb][4 * G + e], ts[kb][qb]);
            ts[kb][qb] = mfma32(tksx[kb][e], qf[qb][4 * G + e], ts[kb][qb]);
          }
        }
      }
    }
    fence();
    if (j == nt - 1 && (Lk % kBcF) != 0) {
      const int valid = Lk - j * kBcF;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (16 * kb + g + 4 * i >= valid) s[kb][qb][i] = -INFINITY;
    }
    // Tile max per query (log2 domain); the exponent base of a query moves
    // only when it grows by more than the slack (a wave-uniform branch).
    float mt[2];
    bool need = false;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      double mx = s[0][qb][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = __builtin_fmax(mx, s[kb][qb][i]);
      mt[qb] = group_max((float)mx) * c2f;
      need = need || mt[qb] > st_m[qb] + kRescaleSlack;
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const bool mv = mt[qb] > st_m[qb] + kRescaleSlack;
        const float m_new = mv ? mt[qb] : st_m[qb];
        const float alpha = mv ? fast_exp2(st_m[qb] - m_new) : 1.0f;
        st_m[qb] = m_new;
        st_l[qb] *= alpha;
        st_a[qb] *= alpha;
#pragma unroll
        for (int G4 = 0; G4 < C::kG4; ++G4)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            acc_o[G4][r][qb] *= alpha;
            acc_t[G4][r][qb] *= alpha;
          }
      }
    }
    float pv[2][2][4], ptv[2][2][4];
    probabilities(s, ts, pv, ptv);
    accumulate(cur, pv, ptv);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile j + 1 of this wave landed
    __syncthreads();
  }

  const auto ro = make_rsrc((const char*)p.o + qhead, qbytes);
  const auto rto = make_rsrc((const char*)p.to + qhead, qbytes);
  float inv[2], mu[2], l[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    l[qb] = group_sum(st_l[qb]);
    inv[qb] = 1.0f / l[qb];
    mu[qb] = group_sum(st_a[qb]) * inv[qb];
  }
  // All values first (each in its own registers), then the stores: reusing a
  // store's registers right after issuing it makes the next write wait until
  // the queued store has read them.  Value (qb, G4, i) of a lane holds dims
  // 64 G4 + 16 g + 4 i .. + 3 of query 16 qb + n (16 bytes).
  u32x4 ov[2][C::kG4][4], tv4[2][C::kG4][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int G4 = 0; G4 < C::kG4; ++G4)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = acc_o[G4][r][qb][i];
          ov[qb][G4][i][r] = __float_as_uint(x * inv[qb]);
          tv4[qb][G4][i][r] = __float_as_uint((acc_t[G4][r][qb][i] - mu[qb] * x) * inv[qb]);
        }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    // rows past Lq: out of range, dropped
    const uint32_t obase = ((uint32_t)(qrow0 + 16 * qb) * D + 16 * g) * 4;
#pragma unroll
    for (int G4 = 0; G4 < C::kG4; ++G4)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_raw_buffer_store_b128(ov[qb][G4][i], ro, obase, (64 * G4 + 4 * i) * 4, 0);
        __builtin_amdgcn_raw_buffer_store_b128(tv4[qb][G4][i], rto, obase, (64 * G4 + 4 * i) * 4, 0);
      }
  }
  if (g == 0) {
    const auto rl = make_rsrc((const char*)p.lse + (size_t)bh * Lq * 4, (uint32_t)Lq * 4);
    const auto rtl = make_rsrc(p.tlse ? (const char*)p.tlse + (size_t)bh * Lq * 4 : (const char*)p.lse,
                               p.tlse ? (uint32_t)Lq * 4 : 0u);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const uint32_t qoff = (uint32_t)(qrow0 + 16 * qb) * 4;
      buf_store4(rl, qoff, (st_m[qb] + __builtin_amdgcn_logf(l[qb])) * kLn2);
      if (p.tlse) buf_store4(rtl, qoff, mu[qb]);
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
