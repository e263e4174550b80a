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
//    row running sums l = sum p (fp32), lb = sum bf16(p) and a = sum bf16(p*tS)
//    (the weights and products the MFMAs consume), and the epilogue
//      O = acc_o / lb,  tO = (acc_t - (a / lb) acc_o) / lb,  lse = (m + log2 l) ln 2;
//  * software pipeline: iteration j computes the softmax of tile j under the
//    logit MFMAs of tile j + 1 (phase A), then the product MFMAs of tile j
//    while the logits of tile j + 1 leave their accumulators, already scaled
//    and shifted for the exponentials (phase B); written as fenced units of
//    one MFMA plus a slice of VALU work, the VALU steps of each item staged
//    one unit apart so that no unit waits on its own results;
//  * variants: a frozen context (tK = tV = 0) skips the tK and tV products
//    and copies; a key shard (kv_rows > Lk) is the same pass on part of the
//    keys, with the tangent of lse as an extra output for an exact merge;
//  * d = 64: a tile holds half the MFMAs for the same softmax work, and the
//    registers allow two waves per SIMD (two workgroups per CU, 64 KB of LDS
//    each): the tiles then run one at a time (logits, softmax, products, no
//    logits carried across tiles), and the other wave's MFMAs hide each
//    wave's softmax.
#include "device_common.h"
#include "launch.h"

namespace attnjvp {
namespace {

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
  float* tlse;
  int Lq, Lk, kv_rows, n_qtiles, n_blocks;
  float scale;
  int out_f32;  // O and tO written as float32 (else bf16)
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

// LDS read helpers.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ inline i16x4 lds_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(__attribute__((address_space(3))) const char*)p);
}

// c + x.lo + x.hi for a packed bf16 pair x (fp32 arithmetic).
__device__ inline float sum_bf16x2(unsigned x, float c) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), one, c, false);
}

__device__ inline f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Keep a value computed here.  Values that are only used in the next
// iteration (the running sums, the logits waiting for their softmax) would
// otherwise be sunk by the optimizer past the fences to the loop latch, where
// they run as one long VALU block with the matrix core idle.
__device__ inline void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ inline void pin(unsigned& x) { asm volatile("" : "+v"(x)); }


// kFrozen: the key-side tangents are zero (tK = tV = 0, a frozen context):
// the tK Q^T and tV P^T products and the tK/tV tile copies are skipped.
template <int D, bool kFrozen>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1, D == 64 ? 2 : 1)))
void attn_jvp_bf16_kernel(Params p) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(1024))) char smem[2 * C::kStage];

  const int t = threadIdx.x;
  const int lane = t & 63, n = lane & 31, hh = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  // All kernel arguments in scalar registers before the first is used: one
  // round trip to the argument buffer instead of one per use site.
  asm volatile("" : : "s"(p.q), "s"(p.k), "s"(p.v), "s"(p.tq), "s"(p.tk), "s"(p.tv), "s"(p.n_blocks));
  const int blk = xcd_logical_block(blockIdx.x, p.n_blocks);
  const int bh = blk / p.n_qtiles, qt = blk % p.n_qtiles;
  const int Lq = p.Lq, Lk = p.Lk;

  const size_t qhead = (size_t)bh * Lq * D * 2, khead = (size_t)bh * p.kv_rows * D * 2;
  const uint32_t qbytes = (uint32_t)Lq * D * 2;
  const auto rq = make_rsrc((const char*)p.q + qhead, qbytes);
  const auto rtq = make_rsrc((const char*)p.tq + qhead, qbytes);
  // One resource per tensor over this head's Lk rows: tiles are addressed by
  // the per-lane offset, and rows at or past Lk read as zero.
  const uint32_t kbytes = (uint32_t)Lk * D * 2;
  const __amdgpu_buffer_rsrc_t rkv[4] = {
      make_rsrc((const char*)p.k + khead, kbytes), make_rsrc(kFrozen ? (const char*)p.k : (const char*)p.tk + khead, kFrozen ? 0 : kbytes),
      make_rsrc((const char*)p.v + khead, kbytes), make_rsrc(kFrozen ? (const char*)p.v : (const char*)p.tv + khead, kFrozen ? 0 : kbytes)};

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
  RowState st = {-INFINITY, 0.0f, 0.0f, 0.0f, 0.0f};
  const float scale = p.scale;
  const float c2 = scale * kLog2e;

  // ---- tile copies -----------------------------------------------------------
  // Per-lane global offsets of this wave's share of a tile copy (loop invariant).
  uint32_t voff_k[C::kLoadsPerWave], voff_v[C::kLoadsPerWave];
#pragma unroll
  for (int i = 0; i < C::kLoadsPerWave; ++i) {
    voff_k[i] = tile_load_voff<D>(wv * C::kLoadsPerWave + i, lane, false);
    voff_v[i] = tile_load_voff<D>(wv * C::kLoadsPerWave + i, lane, true);
  }
  // LDS stage s holds K | tK | V | tV.  K/tK of tile j and V/tV of tile j live in
  // stage j & 1; the K half is fetched two tiles ahead, the V half one tile
  // ahead.  Tiles at or past the end are fetched as zeros (out of range).
  // One 1 KB slice (i) of tensor tn's tile j.
  const uint32_t smem_lds = __builtin_amdgcn_readfirstlane(lds_address(smem));
  auto issue_one = [&](int j, int tn, int i) {
    const uint32_t toff = (uint32_t)j * C::kTile;
    const uint32_t dst = smem_lds + (j & 1) * C::kStage + tn * C::kTile + (wv * C::kLoadsPerWave + i) * 1024;
    lds_dma16(rkv[tn], dst, (tn < 2 ? voff_k[i] : voff_v[i]) + toff);
  };
  // tensors copied: K, tK, V, tV (tn = 0..3); K and V only when frozen
  constexpr int kTensors = kFrozen ? 2 : 4;
  auto tensor = [](int x) { return kFrozen ? 2 * x : x; };
  auto issue = [&](int j, int tn0) {
#pragma unroll
    for (int tn = tn0; tn < tn0 + 2; tn += kFrozen ? 2 : 1)
#pragma unroll
      for (int i = 0; i < C::kLoadsPerWave; ++i) issue_one(j, tn, i);
  };
  // The copies of one pipelined iteration (K|tK of tile j + 2, V|tV of tile
  // j + 1), numbered q = 0 .. kDmaPerIter - 1.
  constexpr int kDmaPerIter = kTensors * C::kLoadsPerWave;
  auto issue_q = [&](int j, auto iq) {
    constexpr int q = decltype(iq)::value;
    const int tn = tensor(q / C::kLoadsPerWave), i = q % C::kLoadsPerWave;
    issue_one(tn < 2 ? j + 2 : j + 1, tn, i);
  };

  // ---- fragment reads ------------------------------------------------------
  // K fragment (key block kb, dim chunk c): key 32kb + n, unit (2c + hh) ^ k_swz(n).
  const uint32_t krow = n * C::kRow;
  const int ksw = k_swz<D>(n);
  auto load_k = [&](const char* stage, int c, bf16x8 (&kf)[4]) {
    const uint32_t u = krow + (((2 * c + hh) ^ ksw) << 4);
    kf[0] = *reinterpret_cast<const bf16x8*>(stage + u);
    kf[1] = *reinterpret_cast<const bf16x8*>(stage + 32 * C::kRow + u);
    if constexpr (!kFrozen) {
      kf[2] = *reinterpret_cast<const bf16x8*>(stage + C::kTile + u);
      kf[3] = *reinterpret_cast<const bf16x8*>(stage + C::kTile + 32 * C::kRow + u);
    }
  };
  // One of those four fragments: x = 2 * (tK ? 1 : 0) + key block.
  auto load_k1 = [&](const char* stage, int c, int x, bf16x8 (&kf)[4]) {
    const uint32_t u = krow + (((2 * c + hh) ^ ksw) << 4);
    kf[x] = *reinterpret_cast<const bf16x8*>(stage + (x & 2 ? C::kTile : 0) + (x & 1 ? 32 * C::kRow : 0) + u);
  };
  // V fragment via ds_read_b64_tr_b16: in 16-lane group G = lane / 16 (half
  // hh = G / 2, dims 16(G & 1) .. +15 of the 32-dim block), source lane s reads
  // 4 dims starting at 4(s & 3) of key 4hh + (s >> 2) (+ 16cc, + 8 for the
  // second read).  The result has keys 16cc + 4hh + 0..3 in elements 0..3 and
  // 16cc + 8 + 4hh + 0..3 in elements 4..7, which are exactly the keys the P
  // operand registers of half hh hold.
  const int G = lane >> 4, sl = lane & 15;
  const int vkey = 4 * (G >> 1) + (sl >> 2);
  uint32_t voff_tr[C::kBlocksD];
#pragma unroll
  for (int b = 0; b < C::kBlocksD; ++b) {
    const int d0 = 32 * b + 16 * (G & 1) + 4 * (sl & 3);
    voff_tr[b] = vkey * C::kRow + ((((d0 >> 3) ^ v_swz<D>(vkey)) << 4) | ((d0 & 7) * 2));
  }
  // V^T (tn = 0) or tV^T (tn = 1) fragment of dim block b, key chunk cc
  auto load_v = [&](const char* stage, int cc, int b, int tn) {
    const char* vb = stage + (2 + tn) * C::kTile + 16 * cc * C::kRow + voff_tr[b];
    const i16x4 lo = lds_tr16(vb), hi = lds_tr16(vb + 8 * C::kRow);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // ---- the six products and the softmax, as building blocks -----------------
  // Logit element e (0..31) of a tile is register e % 16 of key block e / 16:
  // key 32 (e / 16) + acc_row(e % 16, hh).
  //
  // S^T = K Q^T and tS^T = K tQ^T + tK Q^T of one 64-key tile, chunk c of the
  // head dimension: kUPC MFMAs (unit u = 0 .. kUPC - 1; 6, or 4 when frozen).
  constexpr int kUPC = kFrozen ? 4 : 6;
  auto logit_mfma = [&](auto iu, auto ic, const bf16x8 (&k)[4], f32x16 (&sn)[2], f32x16 (&tsn)[2]) {
    constexpr int u = decltype(iu)::value, c = decltype(ic)::value;
    if constexpr (u == 0) sn[0] = mfma(k[0], qf[c], c == 0 ? f32x16{} : sn[0]);
    if constexpr (u == 1) sn[1] = mfma(k[1], qf[c], c == 0 ? f32x16{} : sn[1]);
    if constexpr (u == 2) tsn[0] = mfma(k[0], tqf[c], c == 0 ? f32x16{} : tsn[0]);
    if constexpr (u == 3) tsn[1] = mfma(k[1], tqf[c], c == 0 ? f32x16{} : tsn[1]);
    if constexpr (u == 4) tsn[0] = mfma(k[2], qf[c], tsn[0]);
    if constexpr (u == 5) tsn[1] = mfma(k[3], qf[c], tsn[1]);
  };
  // The logits of a tile wait for their softmax in VGPRs, already in the form
  // the exponentials need: y = S * scale * log2(e) - m (so p = 2^y) and
  // ts = tS * scale.  Element e (0..31) is register e % 16 of key block e / 16.
  float yv[32], tsv[32];
  // Moving the 64 logits of the tile just computed (accumulators sn, tsn; S
  // then tS, x = 0..63) into (yv, tsv) takes three steps per value: read it
  // out of the accumulator, transform it, fold y into the row max.
  struct Take {
    float raw[64];
    float mx;
  };
  auto take_step = [&](auto is, auto ix, Take& tk, const f32x16 (&sn)[2], const f32x16 (&tsn)[2]) {
    constexpr int step = decltype(is)::value, x = decltype(ix)::value;
    if constexpr (step == 0) {
      if constexpr (x < 32)
        tk.raw[x] = sn[x >> 4][x & 15];
      else
        tk.raw[x] = tsn[(x - 32) >> 4][x & 15];
      pin(tk.raw[x]);
    } else if constexpr (step == 1) {
      if constexpr (x < 32) {
        yv[x] = __builtin_fmaf(tk.raw[x], c2, -st.m);
        pin(yv[x]);
      } else {
        tsv[x - 32] = __builtin_fmaf(tk.raw[x], scale, -st.c);
        pin(tsv[x - 32]);
      }
    } else if constexpr (x < 32) {
      tk.mx = fmaxf(tk.mx, yv[x]);
    }
  };
  // Softmax element e: p = 2^y, q = p * ts.  P and P*tS become bf16 B
  // operands, packed in pairs: chunk cc (keys 16cc..16cc+15) is elements
  // 8cc .. 8cc + 7.  l += p is summed in fp32 (it sets the log-sum-exp); lb
  // and a are taken over the packed bf16 pairs (sum_a), the same rounded
  // weights and products that the O and tO products consume, so that O and tO
  // are normalised by the weights they were built from.
  // Four steps per element: exp; q and l; pack (odd e); the operands.
  struct Probs {
    bf16x8 pf[4], ptf[4];
    float p[32], q[32];
    unsigned pp[16], qq[16];
  };
  auto elem_step = [&](auto is, auto ie, Probs& pr) {
    constexpr int step = decltype(is)::value, e = decltype(ie)::value;
    if constexpr (step == 0) {
      pr.p[e] = fast_exp2(yv[e]);
      pin(pr.p[e]);
    } else if constexpr (step == 1) {
      pr.q[e] = pr.p[e] * tsv[e];
      pin(pr.q[e]);
      st.l += pr.p[e];
      pin(st.l);
    } else if constexpr (step == 2) {
      if constexpr (e & 1) {
        pr.pp[e >> 1] = pack_bf16(pr.p[e - 1], pr.p[e]);
        pr.qq[e >> 1] = pack_bf16(pr.q[e - 1], pr.q[e]);
        pin(pr.pp[e >> 1]);
        pin(pr.qq[e >> 1]);
      }
    } else if constexpr (e & 1) {
      constexpr int cc = e >> 3, i = (e & 7) - 1;
      pr.pf[cc][i] = __builtin_bit_cast(bf16x2, pr.pp[e >> 1])[0];
      pr.pf[cc][i + 1] = __builtin_bit_cast(bf16x2, pr.pp[e >> 1])[1];
      pr.ptf[cc][i] = __builtin_bit_cast(bf16x2, pr.qq[e >> 1])[0];
      pr.ptf[cc][i + 1] = __builtin_bit_cast(bf16x2, pr.qq[e >> 1])[1];
    }
  };
  // a += the 32 rounded products and lb += the 32 rounded weights of the
  // tile: one v_dot2 with (1, 1) per packed pair, all 32 in one unit as
  // independent chains.  On gfx950 the first v_dot2 after an MFMA waits ~17
  // cycles and each further one issues in 4, so one batch per tile costs
  // little where a v_dot2 in every other unit cost ~270 cycles per tile.
  auto sum_a = [&](const Probs& pr) {
    float s4[4], b4[4];
    static_for<0, 16>([&](auto ix) {
      constexpr int x = decltype(ix)::value;
      s4[x & 3] = sum_bf16x2(pr.qq[x], x == 0 ? st.a : (x < 4 ? 0.0f : s4[x & 3]));
      b4[x & 3] = sum_bf16x2(pr.pp[x], x == 0 ? st.lb : (x < 4 ? 0.0f : b4[x & 3]));
    });
    st.a = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    st.lb = (b4[0] + b4[1]) + (b4[2] + b4[3]);
    pin(st.a);
    pin(st.lb);
  };
  // Software pipeline over a sequence of N units that handle n items (N
  // units, items [g n / N, (g + 1) n / N) start in unit g): unit g runs step s
  // of the items that started in unit g - s, so that no instruction of a unit
  // waits for another of the same unit (one wave issues in order; a dependent
  // VALU op would hold back the next MFMA).  Slot g runs for g in [0, N + S - 1).
  auto pipeline_slot = [&](auto ig, auto in_units, auto in_items, auto in_steps, auto&& step) {
    constexpr int g = decltype(ig)::value, N = decltype(in_units)::value;
    constexpr int n = decltype(in_items)::value, S = decltype(in_steps)::value;
    static_for<0, S>([&](auto is) {
      constexpr int s = S - 1 - decltype(is)::value;  // oldest items first
      constexpr int u = g - s;
      if constexpr (u >= 0 && u < N)
        static_for<(u * n) / N, ((u + 1) * n) / N>([&](auto ix) { step(std::integral_constant<int, s>{}, ix); });
    });
  };
  // All steps of items [X0, X1) at once (prologue and drain, no MFMA to hide under).
  auto all_steps = [&](auto ix0, auto ix1, auto in_steps, auto&& step) {
    static_for<decltype(ix0)::value, decltype(ix1)::value>([&](auto ix) {
      static_for<0, decltype(in_steps)::value>([&](auto is) { step(is, ix); });
    });
  };
  // V and tV fragments of key chunk 0, read ahead of the products.
  auto load_v0 = [&](const char* stage, bf16x8 (&vf)[C::kBlocksD], bf16x8 (&tvf)[C::kBlocksD]) {
    static_for<0, C::kBlocksD>([&](auto ib) {
      constexpr int b = decltype(ib)::value;
      vf[b] = load_v(stage, 0, b, 0);
      if constexpr (!kFrozen) tvf[b] = load_v(stage, 0, b, 1);
    });
  };
  // O^T += V^T P^T and tO^T += tV^T P^T + V^T (P*tS)^T over one tile: 12 MFMAs
  // per key chunk, starting from the chunk-0 fragments in (vf, tvf).
  // `work(unit)` runs after each MFMA; fragments are reloaded for the next
  // chunk right after their last use.
  auto products = [&](const char* stage, const Probs& pr, bf16x8 (&vf)[C::kBlocksD], bf16x8 (&tvf)[C::kBlocksD],
                      auto&& work) {
    if constexpr (kFrozen) {
      // no tV: O^T += V^T P^T and tO^T += V^T (P*tS)^T, 8 MFMAs per key chunk
      static_for<0, 4>([&](auto icc) {
        constexpr int cc = decltype(icc)::value;
        static_for<0, C::kBlocksD>([&](auto ib) {
          constexpr int b = decltype(ib)::value;
          acc_o[b] = mfma(vf[b], pr.pf[cc], acc_o[b]);
          work(std::integral_constant<int, 2 * C::kBlocksD * cc + 2 * b>{});
          fence();
          acc_t[b] = mfma(vf[b], pr.ptf[cc], acc_t[b]);
          if constexpr (cc + 1 < 4) vf[b] = load_v(stage, cc + 1, b, 0);
          work(std::integral_constant<int, 2 * C::kBlocksD * cc + 2 * b + 1>{});
          fence();
        });
      });
      return;
    }
    static_for<0, 4>([&](auto icc) {
      constexpr int cc = decltype(icc)::value;
      static_for<0, C::kBlocksD>([&](auto ib) {
        constexpr int b = decltype(ib)::value;
        acc_o[b] = mfma(vf[b], pr.pf[cc], acc_o[b]);
        work(std::integral_constant<int, 3 * C::kBlocksD * cc + 2 * b>{});
        fence();
        acc_t[b] = mfma(tvf[b], pr.pf[cc], acc_t[b]);
        if constexpr (cc + 1 < 4) tvf[b] = load_v(stage, cc + 1, b, 1);
        work(std::integral_constant<int, 3 * C::kBlocksD * cc + 2 * b + 1>{});
        fence();
      });
      static_for<0, C::kBlocksD>([&](auto ib) {
        constexpr int b = decltype(ib)::value;
        acc_t[b] = mfma(vf[b], pr.ptf[cc], acc_t[b]);
        if constexpr (cc + 1 < 4) vf[b] = load_v(stage, cc + 1, b, 0);
        work(std::integral_constant<int, 3 * C::kBlocksD * cc + 2 * C::kBlocksD + b>{});
        fence();
      });
    });
  };
  constexpr int kUnitsA = kUPC * C::kChunksD;  // logit MFMAs of one tile
  constexpr int kPreSlots = 2;               // softmax slots run before the first logit MFMA
  constexpr int kUnitsB = (kFrozen ? 8 : 12) * C::kBlocksD;  // MFMAs of products(), 0 .. kUnitsB - 1
  constexpr int kSumAUnit = 3 - kPreSlots;  // first phase-B unit after the tile's last softmax step

  // Tangent-logit centring (d = 128).  q = p (tS - c) is what gets rounded to
  // bf16, so its rounding scales with |tS - c| rather than |tS|: when a tile
  // moves a row's exponent base, c moves to that tile's weighted mean of tS (at
  // the new base), and what was accumulated around the old c is re-expressed
  // around the new one (acc_t -= dc acc_o, a -= dc lb: exact in the algebra).
  // The tile's waiting logits (yv, tsv) are taken relative to the current base
  // and c; rows with moved == false keep their c.  Outside the hot loop.  The
  // one-tile-at-a-time loop of d = 64 keeps c = 0: there the step would sit in
  // the tile loop, which it costs 59 registers and 4% of the time.
  auto recentre = [&](bool moved) {
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int x = 0; x < 32; ++x) {
      const float pw = fast_exp2(yv[x]);
      num = __builtin_fmaf(pw, tsv[x], num);
      den += pw;
    }
    num = xhalf_sum(num);
    den = xhalf_sum(den);
    const float dc = moved ? num / den : 0.0f;
    st.c += dc;
    st.a -= dc * st.lb;
#pragma unroll
    for (int x = 0; x < 32; ++x) tsv[x] -= dc;
#pragma unroll
    for (int b = 0; b < C::kBlocksD; ++b) acc_t[b] -= dc * acc_o[b];
  };

  const int nt = (Lk + kBc - 1) / kBc;
  const bool ragged = (Lk % kBc) != 0;
  float my;  // row max of y over the tile waiting in (yv, tsv)

  if constexpr (D == 64) {
    // Two waves per SIMD: one tile at a time, no logits carried across tiles
    // (195 registers).  Tile j + 1 is copied into the other stage, released by
    // the barrier that opens tile j, while tile j is used.
    issue(0, 0);
    issue(0, 2);
    for (int j = 0; j < nt; ++j) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile j landed
      __syncthreads();                     // ... for every wave; tile j - 1 is no longer read
      if (j + 1 < nt) {
        issue(j + 1, 0);
        issue(j + 1, 2);
      }
      const char* stage = smem + (j & 1) * C::kStage;
      f32x16 sn[2], tsn[2];
      static_for<0, C::kChunksD>([&](auto ic) {
        bf16x8 k[4];
        load_k(stage, decltype(ic)::value, k);
        static_for<0, kUPC>([&](auto iu) { logit_mfma(iu, ic, k, sn, tsn); });
      });
      if (j == nt - 1 && ragged) mask_tail<2>(sn, Lk - j * kBc, hh);
      const float mt = tile_max_log2<2>(sn, c2);
      if (needs_rescale(st, mt)) {
        const float alpha = apply_rescale(st, mt);
#pragma unroll
        for (int b = 0; b < C::kBlocksD; ++b) {
          acc_o[b] *= alpha;
          acc_t[b] *= alpha;
        }
      }
      Take tk;
      tk.mx = -INFINITY;
      all_steps(IC<0>{}, IC<64>{}, IC<2>{}, [&](auto is, auto ix) { take_step(is, ix, tk, sn, tsn); });
      Probs pr;
      all_steps(IC<0>{}, IC<32>{}, IC<4>{}, [&](auto is, auto ie) { elem_step(is, ie, pr); });
      sum_a(pr);
      bf16x8 vf[C::kBlocksD], tvf[C::kBlocksD];
      load_v0(stage, vf, tvf);
      products(stage, pr, vf, tvf, [](auto) {});
    }
  } else {
  // ---- prologue: tile 0 logits; its max sets the exponent base --------------
  // The tile-0 logits need Q and K|tK of tile 0 only: the later copies (V|tV
  // of tile 0, K|tK of tile 1) keep landing under them.  Vector memory
  // operations complete in order, so vmcnt(kLater) leaves exactly those in
  // flight.
  issue(0, 0);
  issue(0, 2);
  issue(1, 0);
  constexpr int kLater = 2 * (kFrozen ? 1 : 2) * C::kLoadsPerWave;
  static_assert(kLater < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (kLater & 15) | ((kLater >> 4) << 14));  // vmcnt(kLater)
  __syncthreads();
  {
    f32x16 sn[2], tsn[2];
    static_for<0, C::kChunksD>([&](auto ic) {
      bf16x8 k[4];
      load_k(smem, decltype(ic)::value, k);
      static_for<0, kUPC>([&](auto iu) { logit_mfma(iu, ic, k, sn, tsn); });
    });
    fence();
    if (nt == 1 && ragged) mask_tail<2>(sn, Lk, hh);
    st.m = tile_max_log2<2>(sn, c2);
    Take tk;
    all_steps(IC<0>{}, IC<64>{}, IC<2>{}, [&](auto is, auto ix) { take_step(is, ix, tk, sn, tsn); });
    recentre(true);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): V|tV of tile 0 and K|tK of tile 1 landed
  __syncthreads();  // ... for every wave, and every wave is done with K of tile 0 before it is refilled

  // ---- one pipelined iteration ------------------------------------------------
  // Phase A: the 48 logit MFMAs of tile j + 1, each paired with softmax
  // elements of tile j.  Phase B: the 48 product MFMAs of tile j, each paired
  // with moving logits of tile j + 1 out of the accumulators into (yv, tsv)
  // and the row max.  In flight meanwhile: K of tile j + 2 and V of tile j + 1.
  auto iteration = [&](int j, bool mask_next) {
    const char* kstage = smem + ((j + 1) & 1) * C::kStage;
    const char* vstage = smem + (j & 1) * C::kStage;

    f32x16 sn[2], tsn[2];
    Probs pr;
    auto elem = [&](auto is, auto ie) { elem_step(is, ie, pr); };
    bf16x8 kf[2][4];
    bf16x8 vf[C::kBlocksD], tvf[C::kBlocksD];
    load_k(kstage, 0, kf[0]);
    // while the first K fragments are in flight: the first softmax slots
    static_for<0, kPreSlots>([&](auto ig) { pipeline_slot(ig, IC<kUnitsA>{}, IC<32>{}, IC<4>{}, elem); });
    fence();
    constexpr int kKFrags = kFrozen ? 2 : 4;  // K fragments per chunk
    static_for<0, C::kChunksD>([&](auto ic) {
      constexpr int c = decltype(ic)::value;
      static_for<0, kUPC>([&](auto iu) {
        constexpr int u = decltype(iu)::value;
        logit_mfma(iu, ic, kf[c & 1], sn, tsn);
        constexpr int g = kUPC * c + u;
        // Each unit: the MFMA, then the tile copies of this iteration (K|tK of
        // tile j + 2, V|tV of tile j + 1) spread over the phase-A units, then
        // one K fragment of the next chunk (or, in the last chunk, the
        // chunk-0 V fragments of one dim block for the products), then its
        // softmax slot.  Issuing the copies first and reading the fragments
        // one per unit measured faster than bursts at the chunk start.
        static_for<(g * kDmaPerIter + kUnitsA - 1) / kUnitsA, ((g + 1) * kDmaPerIter + kUnitsA - 1) / kUnitsA>(
            [&](auto iq) { issue_q(j, iq); });
        if constexpr (c + 1 < C::kChunksD && u < kKFrags) load_k1(kstage, c + 1, u, kf[(c + 1) & 1]);
        if constexpr (c + 1 == C::kChunksD && u < C::kBlocksD) {
          vf[u] = load_v(vstage, 0, u, 0);
          if constexpr (!kFrozen) tvf[u] = load_v(vstage, 0, u, 1);
        }
        pipeline_slot(IC<g + kPreSlots>{}, IC<kUnitsA>{}, IC<32>{}, IC<4>{}, elem);
        fence();
      });
    });

    if (mask_next) mask_tail<2>(sn, Lk - (j + 1) * kBc, hh);
    Take tk;
    tk.mx = -INFINITY;
    auto take = [&](auto is, auto ix) { take_step(is, ix, tk, sn, tsn); };
    products(vstage, pr, vf, tvf, [&](auto iunit) {
      constexpr int unit = decltype(iunit)::value;
      // the last softmax steps of tile j run under its first product MFMAs
      // (they complete chunk 3, which the products reach last)
      if constexpr (unit + kPreSlots < 3)
        pipeline_slot(IC<kUnitsA + kPreSlots + unit>{}, IC<kUnitsA>{}, IC<32>{}, IC<4>{}, elem);
      if constexpr (unit == kSumAUnit) sum_a(pr);  // every pair of the tile is packed by now
      pipeline_slot(iunit, IC<kUnitsB>{}, IC<64>{}, IC<3>{}, take);
    });
    pipeline_slot(IC<kUnitsB>{}, IC<kUnitsB>{}, IC<64>{}, IC<3>{}, take);
    pipeline_slot(IC<kUnitsB + 1>{}, IC<kUnitsB>{}, IC<64>{}, IC<3>{}, take);
    my = xhalf_max(tk.mx);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
  };

  // A tile whose max exceeds the exponent base by more than kRescaleSlack moves
  // the base of its rows up to that max: the sums and accumulators are scaled
  // by 2^-delta and the waiting logits shifted by -delta.
  auto rescale = [&]() {
    const float delta = my > kRescaleSlack ? my : 0.0f;
    const float alpha = fast_exp2(-delta);
    st.m += delta;
    st.l *= alpha;
    st.a *= alpha;
    st.lb *= alpha;
#pragma unroll
    for (int x = 0; x < 32; ++x) yv[x] -= delta;
#pragma unroll
    for (int b = 0; b < C::kBlocksD; ++b) {
      acc_o[b] *= alpha;
      acc_t[b] *= alpha;
    }
    recentre(delta > 0.0f);
  };
  auto needs_rescale = [&]() { return __builtin_amdgcn_ballot_w64(my > kRescaleSlack) != 0; };

  // ---- main loop --------------------------------------------------------------
  // The hot loop only feeds the accumulators to MFMAs: a tile that moves the
  // exponent base (rare after the first) leaves it, and the accumulators are
  // rescaled outside before it re-enters.  The logits of the last tile (masked
  // when ragged) are computed by a peeled iteration.
  int j = 0;
  while (true) {
    bool moved = false;
    while (j < nt - 2) {
      iteration(j, false);
      ++j;
      if (needs_rescale()) {
        moved = true;
        break;
      }
    }
    if (!moved) break;
    rescale();
  }
  if (j == nt - 2) {
    iteration(j, ragged);
    ++j;
    if (needs_rescale()) rescale();
  }
  {  // drain: the last tile's probabilities and products
    Probs pr;
    all_steps(IC<0>{}, IC<32>{}, IC<4>{}, [&](auto is, auto ie) { elem_step(is, ie, pr); });
    sum_a(pr);
    bf16x8 vf[C::kBlocksD], tvf[C::kBlocksD];
    load_v0(smem + (j & 1) * C::kStage, vf, tvf);
    products(smem + (j & 1) * C::kStage, pr, vf, tvf, [](auto) {});
  }

  }  // D != 64
  // ---- epilogue ------------------------------------------------------------
  // O and tO are normalised by the sum of the bf16 weights they were built
  // from (so the centring cancels exactly where one key carries the row), the
  // log-sum-exp by the fp32 sum.
  const float l = xhalf_sum(st.l), lb = xhalf_sum(st.lb), a = xhalf_sum(st.a);
  const float inv = 1.0f / lb, mu = a * inv;
  if (p.out_f32) {
    // float32 O and tO (the partial results of a key shard, rounded to bf16
    // only once, after the merge): group g of a lane is 4 consecutive dims,
    // one 16-byte store each.
    const auto ro32 = make_rsrc((const char*)p.o + 2 * qhead, 2 * qbytes);
    const auto rto32 = make_rsrc((const char*)p.to + 2 * qhead, 2 * qbytes);
    u32x4 o32[C::kBlocksD][4], t32[C::kBlocksD][4];
#pragma unroll
    for (int b = 0; b < C::kBlocksD; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = acc_o[b][4 * g + i];
          o32[b][g][i] = __float_as_uint(x * inv);
          t32[b][g][i] = __float_as_uint((acc_t[b][4 * g + i] - mu * x) * inv);
        }
    fence();
    const uint32_t obase32 = ((uint32_t)qrow * D + 4 * hh) * 4;
#pragma unroll
    for (int b = 0; b < C::kBlocksD; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        __builtin_amdgcn_raw_buffer_store_b128(o32[b][g], ro32, obase32, (32 * b + 8 * g) * 4, 0);
        __builtin_amdgcn_raw_buffer_store_b128(t32[b][g], rto32, obase32, (32 * b + 8 * g) * 4, 0);
      }
  } else {
  const auto ro = make_rsrc((const char*)p.o + qhead, qbytes);
  const auto rto = make_rsrc((const char*)p.to + qhead, qbytes);
  // Accumulator group g (registers 4g..4g+3) of a lane holds head dims
  // 8g + 4hh .. +3 of its query.  Groups g, g + 1 (g even) are paired across the
  // half-waves with v_permlane32_swap so that each lane holds 8 consecutive
  // dims: half 0 dims 8g .. 8g + 7, half 1 dims 8(g + 1) .. +7, one 16-byte
  // store each.  Every value is packed into its own registers before the
  // first store: reusing a store's data registers right after it makes the
  // next write wait until the queued store has read them.
  u32x4 ost[C::kBlocksD][2], tst[C::kBlocksD][2];
#pragma unroll
  for (int b = 0; b < C::kBlocksD; ++b) {
#pragma unroll
    for (int gp = 0; gp < 2; ++gp) {
      u32x2 op[2], tp[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int g = 2 * gp + h;
        float ov[4], tv4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = acc_o[b][4 * g + i];
          ov[i] = x * inv;
          tv4[i] = (acc_t[b][4 * g + i] - mu * x) * inv;
        }
        op[h] = u32x2{pack_bf16(ov[0], ov[1]), pack_bf16(ov[2], ov[3])};
        tp[h] = u32x2{pack_bf16(tv4[0], tv4[1]), pack_bf16(tv4[2], tv4[3])};
      }
      ost[b][gp] = pair_halves(op[0], op[1]);
      tst[b][gp] = pair_halves(tp[0], tp[1]);
    }
  }
  fence();
  // one address register for all stores; the (b, gp) part rides in the scalar
  // offset (read at issue, so reusing it does not wait on earlier stores).
  // Rows past Lq have obase past the end of the range: their stores drop.
  const uint32_t obase = ((uint32_t)qrow * D + 8 * hh) * 2;
#pragma unroll
  for (int b = 0; b < C::kBlocksD; ++b)
#pragma unroll
    for (int gp = 0; gp < 2; ++gp) {
      __builtin_amdgcn_raw_buffer_store_b128(ost[b][gp], ro, obase, (32 * b + 16 * gp) * 2, 0);
      __builtin_amdgcn_raw_buffer_store_b128(tst[b][gp], rto, obase, (32 * b + 16 * gp) * 2, 0);
    }
  }
  if (hh == 0) {
    const auto rl = make_rsrc((const char*)p.lse + (size_t)bh * Lq * 4, (uint32_t)Lq * 4);
    buf_store4(rl, (uint32_t)qrow * 4, (st.m + __builtin_amdgcn_logf(l)) * kLn2);
    if (p.tlse) {
      const auto rtl = make_rsrc((const char*)p.tlse + (size_t)bh * Lq * 4, (uint32_t)Lq * 4);
      buf_store4(rtl, (uint32_t)qrow * 4, mu + st.c);
    }
  }
}

template <int D, bool kFrozen>
hipError_t launch(const Problem& pr, hipStream_t stream) {
  Params p;
  p.q = pr.q; p.k = pr.k; p.v = pr.v; p.tq = pr.tq; p.tk = pr.tk; p.tv = pr.tv;
  p.o = pr.o; p.to = pr.to; p.lse = pr.lse; p.tlse = pr.tlse;
  p.Lq = pr.Lq; p.Lk = pr.Lk; p.kv_rows = pr.kv_rows; p.scale = pr.scale;
  p.out_f32 = pr.out_f32 ? 1 : 0;
  p.n_qtiles = (pr.Lq + kBlockRows - 1) / kBlockRows;
  p.n_blocks = pr.B * pr.H * p.n_qtiles;
  return launch_1d(reinterpret_cast<const void*>(&attn_jvp_bf16_kernel<D, kFrozen>), p.n_blocks, kThreads, p, stream);
}

}  // namespace

hipError_t launch_bf16(const Problem& p, hipStream_t stream) {
  if (p.tk == nullptr)  // frozen context: tK = tV = 0
    return p.d == 128 ? launch<128, true>(p, stream) : launch<64, true>(p, stream);
  return p.d == 128 ? launch<128, false>(p, stream) : launch<64, false>(p, stream);
}

}  // namespace attnjvp
