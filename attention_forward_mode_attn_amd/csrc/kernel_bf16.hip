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
//  * K and tK tiles are copied to LDS row-major; V and tV are transposed on the
//    way (4 keys x 8 dims per thread, v_perm_b32) into [dim][key] rows whose keys
//    are permuted to match the accumulator layout, so every MFMA operand read is
//    one 16-byte ds_read; 16-byte units are XOR-swizzled to avoid bank conflicts;
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
  static constexpr int kTileK = kBc * D * 2;        // bytes of one K (or tK) tile, [key][dim]
  static constexpr int kTileV = D * kBc * 2;        // bytes of one V^T (or tV^T) tile, [dim][key]
  static constexpr int kOffTK = kTileK;
  static constexpr int kOffV = 2 * kTileK;
  static constexpr int kOffTV = 2 * kTileK + kTileV;
  static constexpr int kStage = 2 * kTileK + 2 * kTileV;
  static constexpr int kKUnits = kBc * D / 8;       // 16-byte units in a K tile
  static constexpr int kKPerThread = kKUnits / kThreads;
  static constexpr int kVUnits = (kBc / 4) * (D / 8);  // (4 keys x 8 dims) units in a V tile
  static constexpr int kVPerThread = 2 * kVUnits / kThreads;  // V and tV together
  static constexpr int kChunksD = D / 16;           // 16-wide head-dim chunks (S products)
  static constexpr int kBlocksD = D / 32;           // 32-row head-dim blocks (O products)
  static_assert(kKUnits % kThreads == 0 && (2 * kVUnits) % kThreads == 0, "tile split");
};

// Byte offset of 16-byte unit u of K-tile row r (row = one key).
template <int D>
__device__ inline uint32_t k_off(int r, int u) {
  return r * (D * 2) + ((u ^ (r & 7)) << 4);
}
// Byte offset, in a V^T tile, of the 4-key group starting at permuted position
// pos (a multiple of 4) in row d (row = one head-dim index, 64 keys = 128 bytes).
__device__ inline uint32_t vt_off(int d, int pos) {
  return d * (kBc * 2) + ((((pos >> 3) ^ (d & 7))) << 4) + (((pos >> 2) & 1) << 3);
}
// Keys 4g..4g+3 of a 16-key chunk are stored at these positions, so that
// positions 8*hh .. 8*hh+7 hold the keys that accumulator registers 8*c'..8*c'+7
// of half hh carry (see acc_row).
__device__ inline int vt_pos(int g) {
  const int gg = g & 3;
  return 16 * (g >> 2) + (gg == 0 ? 0 : gg == 1 ? 8 : gg == 2 ? 4 : 12);
}

template <int D>
struct Staging {
  u32x4 k[Cfg<D>::kKPerThread];
  u32x4 tk[Cfg<D>::kKPerThread];
  u32x4 v[Cfg<D>::kVPerThread][4];
};

// V-unit z (over V then tV) -> (tensor, key group g, dim octet o).
template <int D>
__device__ inline void v_unit(int z, int& tensor, int& g, int& o) {
  tensor = z / Cfg<D>::kVUnits;
  const int zz = z % Cfg<D>::kVUnits;
  g = zz % (kBc / 4);
  o = zz / (kBc / 4);
}

template <int D>
__device__ inline void issue_tile_loads(Staging<D>& sg, __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rtk,
                                        __amdgpu_buffer_rsrc_t rv, __amdgpu_buffer_rsrc_t rtv, int key0, int t) {
#pragma unroll
  for (int i = 0; i < Cfg<D>::kKPerThread; ++i) {
    const int e = t + kThreads * i;
    const int r = e / (D / 8), u = e % (D / 8);
    const uint32_t off = ((key0 + r) * D + u * 8) * 2;
    sg.k[i] = buf_load16(rk, off);
    sg.tk[i] = buf_load16(rtk, off);
  }
#pragma unroll
  for (int i = 0; i < Cfg<D>::kVPerThread; ++i) {
    int tensor, g, o;
    v_unit<D>(t + kThreads * i, tensor, g, o);
    // tensor is uniform over each wave (it depends on i and on the wave index only)
    tensor = __builtin_amdgcn_readfirstlane(tensor);
    const __amdgpu_buffer_rsrc_t r = tensor ? rtv : rv;
#pragma unroll
    for (int j = 0; j < 4; ++j) sg.v[i][j] = buf_load16(r, ((key0 + 4 * g + j) * D + 8 * o) * 2);
  }
}

template <int D>
__device__ inline void store_tile(const Staging<D>& sg, char* stage, int t) {
#pragma unroll
  for (int i = 0; i < Cfg<D>::kKPerThread; ++i) {
    const int e = t + kThreads * i;
    const int r = e / (D / 8), u = e % (D / 8);
    *reinterpret_cast<u32x4*>(stage + k_off<D>(r, u)) = sg.k[i];
    *reinterpret_cast<u32x4*>(stage + Cfg<D>::kOffTK + k_off<D>(r, u)) = sg.tk[i];
  }
#pragma unroll
  for (int i = 0; i < Cfg<D>::kVPerThread; ++i) {
    int tensor, g, o;
    v_unit<D>(t + kThreads * i, tensor, g, o);
    char* base = stage + Cfg<D>::kOffV + tensor * Cfg<D>::kTileV;
    const int pos = vt_pos(g);
    const u32x4 &r0 = sg.v[i][0], &r1 = sg.v[i][1], &r2 = sg.v[i][2], &r3 = sg.v[i][3];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // dword w of a row holds dims 8o+2w (low half) and 8o+2w+1 (high half)
      u32x2 lo, hi;
      lo[0] = __builtin_amdgcn_perm(r1[w], r0[w], 0x05040100u);
      lo[1] = __builtin_amdgcn_perm(r3[w], r2[w], 0x05040100u);
      hi[0] = __builtin_amdgcn_perm(r1[w], r0[w], 0x07060302u);
      hi[1] = __builtin_amdgcn_perm(r3[w], r2[w], 0x07060302u);
      *reinterpret_cast<u32x2*>(base + vt_off(8 * o + 2 * w, pos)) = lo;
      *reinterpret_cast<u32x2*>(base + vt_off(8 * o + 2 * w + 1, pos)) = hi;
    }
  }
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
  __shared__ __attribute__((aligned(16))) char smem[2 * C::kStage];

  const int t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6, n = lane & 31, hh = lane >> 5;
  const int blk = xcd_logical_block(blockIdx.x, p.n_blocks);
  const int bh = blk / p.n_qtiles, qt = blk % p.n_qtiles;
  const int Lq = p.Lq, Lk = p.Lk;

  const size_t qhead = (size_t)bh * Lq * D * 2, khead = (size_t)bh * Lk * D * 2;
  const uint32_t qbytes = (uint32_t)Lq * D * 2, kbytes = (uint32_t)Lk * D * 2;
  const auto rq = make_rsrc((const char*)p.q + qhead, qbytes);
  const auto rtq = make_rsrc((const char*)p.tq + qhead, qbytes);
  const auto rk = make_rsrc((const char*)p.k + khead, kbytes);
  const auto rtk = make_rsrc((const char*)p.tk + khead, kbytes);
  const auto rv = make_rsrc((const char*)p.v + khead, kbytes);
  const auto rtv = make_rsrc((const char*)p.tv + khead, kbytes);

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

  // Per-lane LDS read offsets (the swizzle term is n & 7 for every read).
  const int sw = n & 7;
  const uint32_t krow_off = n * (D * 2);   // + 32*kb*(D*2)
  const uint32_t vrow_off = n * (kBc * 2); // + 32*b*(kBc*2)

  const int nt = (Lk + kBc - 1) / kBc;
  Staging<D> sg;
  issue_tile_loads<D>(sg, rk, rtk, rv, rtv, 0, t);
  store_tile<D>(sg, smem, t);
  __syncthreads();

  for (int j = 0; j < nt; ++j) {
    const char* cur = smem + (j & 1) * C::kStage;
    if (j + 1 < nt) issue_tile_loads<D>(sg, rk, rtk, rv, rtv, (j + 1) * kBc, t);

    // ---- logits and tangent logits --------------------------------------
    f32x16 s[2] = {f32x16{}, f32x16{}}, ts[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int c = 0; c < C::kChunksD; ++c) {
      const uint32_t u = ((2 * c + hh) ^ sw) << 4;
      const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(cur + krow_off + u);
      const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(cur + krow_off + 32 * D * 2 + u);
      const bf16x8 tk0 = *reinterpret_cast<const bf16x8*>(cur + C::kOffTK + krow_off + u);
      const bf16x8 tk1 = *reinterpret_cast<const bf16x8*>(cur + C::kOffTK + krow_off + 32 * D * 2 + u);
      s[0] = mfma(k0, qf[c], s[0]);
      s[1] = mfma(k1, qf[c], s[1]);
      ts[0] = mfma(k0, tqf[c], ts[0]);
      ts[1] = mfma(k1, tqf[c], ts[1]);
      ts[0] = mfma(tk0, qf[c], ts[0]);
      ts[1] = mfma(tk1, qf[c], ts[1]);
    }

    // ---- online softmax --------------------------------------------------
    if (j == nt - 1 && (Lk % kBc) != 0) mask_tail<2>(s, Lk - j * kBc, hh);
    float alpha;
    if (update_max(st, tile_max_log2<2>(s, c2), alpha)) {
#pragma unroll
      for (int b = 0; b < C::kBlocksD; ++b) {
        acc_o[b] *= alpha;
        acc_t[b] *= alpha;
      }
    }
    // P and P*tS as bf16 B operands: chunk cc (keys 16cc..16cc+15) is
    // registers 8*(cc%2) .. +7 of key block cc/2.
    bf16x8 pf[4], ptf[4];
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

    // ---- O and tO products ---------------------------------------------
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const uint32_t u = ((2 * cc + hh) ^ sw) << 4;
#pragma unroll
      for (int b = 0; b < C::kBlocksD; ++b) {
        const uint32_t off = vrow_off + 32 * b * (kBc * 2) + u;
        const bf16x8 vv = *reinterpret_cast<const bf16x8*>(cur + C::kOffV + off);
        const bf16x8 tvv = *reinterpret_cast<const bf16x8*>(cur + C::kOffTV + off);
        acc_o[b] = mfma(vv, pf[cc], acc_o[b]);
        acc_t[b] = mfma(tvv, pf[cc], acc_t[b]);
        acc_t[b] = mfma(vv, ptf[cc], acc_t[b]);
      }
    }

    if (j + 1 < nt) store_tile<D>(sg, smem + ((j + 1) & 1) * C::kStage, t);
    __syncthreads();
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
