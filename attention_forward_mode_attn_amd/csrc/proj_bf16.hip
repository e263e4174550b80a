// Projection of hidden states into attention heads, with its tangent, on gfx950
// matrix cores (v_mfma_f32_32x32x16_bf16):
//
//   Y = X W^T + b,   TY = TX W^T,   feature f = (n*H + h)*d + j of token t of
//   batch b written to [n, b, h, t, j] (the layout the attention kernel reads).
//
// The rCM pages make every layer take and return tangents and hand the Q, K, V
// tangents to attention laid out like Q, K, V (ai.info summary of "Large Scale
// Diffusion Distillation via Score-Regularized Continuous-Time Consistency",
// "Methodology in Plain English").  The layer in front of attention is read as
// a linear map; its JVP is the same weight applied to the tangent, so one pass
// computes both products from every weight tile it stages:
//
//  * one workgroup = 4 waves = 256 output features x 128 tokens of one batch;
//    wave w owns tokens 32w .. 32w + 31 and all 256 features, for X and TX:
//    16 accumulators of 32 x 32 (all 256 accumulation registers);
//  * the products are transposed, Y^T = W X^T (features in the MFMA M slot,
//    tokens in N), so a lane owns one token and the epilogue stores runs of 8
//    consecutive features of one head;
//  * the hidden dimension streams in steps of 64 through double-buffered LDS
//    (W | X | TX tiles, 64 KB per stage) by buffer_load ... lds, rows of 128
//    bytes with XOR-swizzled 16-byte units; each W fragment read from LDS
//    feeds two MFMAs (X and TX);
//  * software pipeline per step: fenced units of one MFMA each, fragment reads
//    16 units ahead of their use.  The barrier that publishes the next step's
//    tiles sits three quarters into the step, after the last read of the
//    current stage, so the next step's first fragments are read before the
//    step ends (no step starts by waiting on LDS), and most copies of the step
//    after next are issued right behind it, into the stage just released, a
//    whole step ahead of the barrier that waits for them;
//  * the bias initialises the X accumulators; the epilogue rounds to bf16 and
//    stores 16 bytes per lane after pairing the half-waves with v_permlane32_swap.
//  * kT = false (a frozen input, no TX): X tiles and accumulators only.
//  * grids that would leave half the CUs or more idle (at most 128 workgroups
//    of 256 features) use tiles of 128 features instead, twice as many
//    workgroups, each wave 32 tokens x 128 features; without a tangent the
//    hidden step is then 128 wide, so that a step still holds 32 MFMAs per
//    wave.  Each tile shape has its own step schedule (Sched below).
#include "device_common.h"
#include "launch.h"

namespace attnjvp {
namespace {

constexpr int kTT = kWaves * kWaveRows;        // tokens per workgroup (128)
// Feature tiles per dispatch group: 16 on large grids (each X/TX tile, which does
// not fit the last-level cache as a whole, is read by 16 workgroups at once);
// 4 on grids of fewer than 2048 workgroups, where the grid is a few generations
// deep and the narrower groups measured faster (the text-context projection:
// 9%).
constexpr int kGroupFLarge = 16, kGroupFSmall = 4, kSmallGrid = 2048;
constexpr int kRing = 16;                      // W fragment registers in flight
// Grids of at most this many 256-feature workgroups use 128-feature tiles.
constexpr int kNarrowGrid = 128;

// Tile geometry: kTF output features x kTT tokens per workgroup, kTK hidden
// elements per step; rows of kTK bf16 in LDS.
template <bool kT, int kTF_, int kTK_>
struct Geom {
  static constexpr int kTF = kTF_, kTK = kTK_;
  static constexpr int kFB = kTF / 32;                 // 32-feature blocks (per wave)
  static constexpr int kC = kTK / 16;                  // 16-wide hidden chunks per step
  static constexpr int kQ = kFB * kC;                  // W fragments per step
  static constexpr int kRowB = kTK * 2;                // bytes of one tile row
  static constexpr int kUPR = kRowB / 16;              // 16-byte units per row
  static constexpr int kRowsPerSlice = 1024 / kRowB;   // rows of one 1 KB copy slice
  static constexpr int kWTile = kTF * kRowB;
  static constexpr int kXTile = kTT * kRowB;
  static constexpr int kNX = kT ? 2 : 1;               // X fragments per chunk (X, TX)
  // W | X | TX; the 256-feature tiles keep the TX slot in every stage also
  // without a tangent (the stage layout their schedules were measured with)
  static constexpr int kStageB = kWTile + (kTF == 256 ? 2 : kNX) * kXTile;
  static constexpr int kWDma = kWTile / 1024 / kWaves;   // W slices per wave and step
  static constexpr int kXDma = kXTile / 1024 / kWaves;   // X (and TX) slices per wave and step
  static constexpr int kDma = kWDma + kNX * kXDma;
  static_assert(kRowB == 128 || kRowB == 256, "row swizzle");
  static_assert(kWTile % (1024 * kWaves) == 0 && kXTile % (1024 * kWaves) == 0, "copy slices");
  static_assert(kC % 2 == 0, "X chunks alternate between two register slots");
  // Unit u of tile row r sits at slot u ^ swz(r): the 16 lanes that a
  // ds_read_b128 serves together read one unit column of 16 consecutive rows,
  // and the swizzle spreads them over all 16 bank groups of the 64-bank LDS
  // (128-byte rows: two rows per bank sweep; 256-byte rows: one).
  static __device__ inline int swz(int r) { return kRowB == 128 ? (r >> 1) & 7 : r & 15; }
};

struct ProjParams {
  const void* x;
  const void* tx;
  const void* w;
  const void* bias;
  void* y;
  void* ty;
  int B, L, D, F, H, d;
  int n_ft, n_tt, n_blocks, group_f;
};

__device__ inline f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Per-lane global offset of one 1 KB slice (kRowsPerSlice rows) of a tile whose
// rows are D elements apart: lane l fills LDS bytes 16l of the slice, i.e. row
// kRowsPerSlice s + l / kUPR, slot l % kUPR, which holds unit (l % kUPR) ^
// swz(row) of that row.
template <class G>
__device__ inline uint32_t slice_voff(int s, int lane, int D) {
  const int r = G::kRowsPerSlice * s + lane / G::kUPR;
  const int u = (lane % G::kUPR) ^ G::swz(r);
  return (uint32_t)r * (uint32_t)D * 2u + (uint32_t)u * 16u;
}

// Schedule of one step (see the file comment).  W fragment q = kFB c + fb
// (hidden chunk c of 16, feature block fb) is used by units q*kPer .. q*kPer +
// kPer - 1 and lives in register slot q % kRing; X fragment c in slot c % 2.
// Step k computes on stage k & 1.  Its copies are issued in two parts: kTail
// slices of step k + 2 right after step k's barrier (from then on no wave reads
// stage k & 1), and the other slices of step k + 1 in the first units of step
// k, one every kHeadStride units.  The barrier at unit kBar waits for all of
// them.  Per tile shape: kLead (W read this many units before its use), kXLead
// (X read this many units before its chunk starts), kBar, kTail, kHeadStride,
// and kJoin (how many next-stage reads share the barrier's unit besides X).
template <bool kT, int kTF, int kTK>
struct Tune;
template <>
struct Tune<true, 256, 64> {
  static constexpr int kLead = 16, kXLead = 16, kBar = 48, kTail = 12, kHeadStride = 2, kJoin = 0;
};
template <>
struct Tune<false, 256, 64> {
  static constexpr int kLead = 5, kXLead = 7, kBar = 27, kTail = 4, kHeadStride = 1, kJoin = 0;
};
template <>
struct Tune<true, 128, 64> {
  static constexpr int kLead = 8, kXLead = 8, kBar = 24, kTail = 6, kHeadStride = 2, kJoin = 0;
};
template <>
struct Tune<false, 128, 128> {
  static constexpr int kLead = 5, kXLead = 4, kBar = 28, kTail = 4, kHeadStride = 1, kJoin = 1;
};

template <bool kT, int kTF, int kTK>
struct Sched : Geom<kT, kTF, kTK>, Tune<kT, kTF, kTK> {
  using G = Geom<kT, kTF, kTK>;
  using T = Tune<kT, kTF, kTK>;
  static constexpr int kPer = kT ? 2 : 1;                   // MFMAs per W fragment
  static constexpr int kUnits = G::kQ * kPer;               // MFMAs per step and wave
  static constexpr int kChunkU = G::kFB * kPer;             // units per hidden chunk
  static constexpr int kPre = (T::kLead + kPer - 1) / kPer; // W fragments read in the previous step
  // unit of the i-th next-stage read (X fragments first, then W 0 .. kPre - 1;
  // the first kJoin W reads share the unit of the last X read); reads that do
  // not fit go to the last unit
  static constexpr int next_unit(int i) {
    const int u = T::kBar + (i < G::kNX ? i : (i - T::kJoin < G::kNX - 1 ? G::kNX - 1 : i - T::kJoin));
    return u < kUnits ? u : kUnits - 1;
  }
  // a next-stage W fragment goes into a slot whose current fragment is done
  static constexpr bool next_w_slots_free() {
    for (int q2 = 0; q2 < kPre; ++q2)
      for (int q = q2 % kRing; q < G::kQ; q += kRing)
        if ((q + 1) * kPer - 1 >= next_unit(G::kNX + q2)) return false;
    return true;
  }
  static_assert((G::kQ - 1) * kPer - T::kLead < T::kBar, "current-stage W reads end before the barrier");
  static_assert((G::kC - 1) * kChunkU - T::kXLead + G::kNX - 1 < T::kBar,
                "current-stage X reads end before the barrier");
  static_assert(T::kLead <= (kRing - 1) * kPer, "a W read does not overwrite a fragment still in use");
  static_assert(T::kXLead <= kChunkU, "an X read does not overwrite a chunk still in use");
  static_assert(next_unit(0) >= (G::kC - 1) * kChunkU,
                "next-stage X chunk 0 (slot 0) is read after the last use of chunk kC - 2");
  static_assert(next_w_slots_free(), "next-stage W reads do not overwrite fragments still in use");
  static_assert((G::kDma - T::kTail - 1) * T::kHeadStride < T::kBar, "head copies issued before the barrier");
  static_assert(T::kBar + T::kTail <= kUnits, "tail copies fit after the barrier");
  // every next-stage fragment is read at least 4 units before its first use
  static_assert(kUnits - next_unit(G::kNX + kPre - 1) + (kPre - 1) * kPer >= 4, "next-stage lead");
  static_assert(kUnits - next_unit(G::kNX) >= 4, "next-stage lead of W fragment 0");
  static_assert(kUnits - next_unit(G::kNX - 1) >= 4, "next-stage lead of the X fragments");
};
template <bool kT, int kTF, int kTK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void proj_bf16_kernel(ProjParams p) {
  using S = Sched<kT, kTF, kTK>;
  constexpr int kRowB = S::kRowB, kWTile = S::kWTile, kXTile = S::kXTile, kStageB = S::kStageB, kFB = S::kFB;
  __shared__ __attribute__((aligned(1024))) char smem[2 * kStageB];

  const int t = threadIdx.x;
  const int lane = t & 63, n = lane & 31, hh = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);

  // Dispatch order: the logical blocks of one XCD are contiguous, and within
  // them groups of group_f feature tiles sweep the token tiles together, so the
  // workgroups running at once on an XCD share W and X tiles in its L2.
  const int l = xcd_logical_block(blockIdx.x, p.n_blocks);
  const int n_t = p.n_tt * p.B;
  const int gf = p.group_f;
  const int group = l / (gf * n_t);
  const int first_ft = group * gf;
  const int gsz = min(p.n_ft - first_ft, gf);
  const int r_in = l - group * gf * n_t;
  const int ft = first_ft + r_in % gsz;
  const int tg = r_in / gsz;
  const int b = tg / p.n_tt, tt = tg % p.n_tt;
  const int f0 = ft * kTF, t0 = tt * kTT;
  const int D = p.D, L = p.L, F = p.F;

  // Resources: rows past F (features) or past L (tokens) read as zero.
  const size_t xoff = ((size_t)b * L + t0) * D * 2;
  const auto rw = make_rsrc((const char*)p.w + (size_t)f0 * D * 2, (uint32_t)(F - f0) * (uint32_t)D * 2u);
  const auto rx = make_rsrc((const char*)p.x + xoff, (uint32_t)(L - t0) * (uint32_t)D * 2u);
  const auto rtx = make_rsrc(kT ? (const char*)p.tx + xoff : (const char*)p.x, kT ? (uint32_t)(L - t0) * (uint32_t)D * 2u : 0u);

  // This wave's copy slices: W slices kWDma wv .. kWDma wv + kWDma - 1, X (and
  // TX) slices kXDma wv .. kXDma wv + kXDma - 1.
  uint32_t voff[S::kDma];
#pragma unroll
  for (int i = 0; i < S::kDma; ++i) {
    const int wi = i < S::kWDma ? i : (i - S::kWDma) % S::kXDma;
    voff[i] = slice_voff<S>(i < S::kWDma ? S::kWDma * wv + wi : S::kXDma * wv + wi, lane, D);
  }
  const uint32_t smem_lds = __builtin_amdgcn_readfirstlane(lds_address(smem));
  // copy slice i of this wave for step k into stage k & 1
  auto issue = [&](int k, auto ii) {
    constexpr int i = decltype(ii)::value;
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)k * kRowB);
    const uint32_t st = smem_lds + (k & 1) * kStageB;
    if constexpr (i < S::kWDma) {
      lds_dma16(rw, st + (S::kWDma * wv + i) * 1024, voff[i], soff);
    } else if constexpr (i < S::kWDma + S::kXDma) {
      lds_dma16(rx, st + kWTile + (S::kXDma * wv + i - S::kWDma) * 1024, voff[i], soff);
    } else {
      lds_dma16(rtx, st + kWTile + kXTile + (S::kXDma * wv + i - S::kWDma - S::kXDma) * 1024, voff[i], soff);
    }
  };

  // Fragment offsets in a stage: W fragment (chunk c, block fb) of lane (n, hh)
  // is row 32fb + n, unit 2c + hh; X fragment c is row 32wv + n of the X tile.
  // Both rows have the swizzle of row n.
  uint32_t lo[S::kC];
#pragma unroll
  for (int c = 0; c < S::kC; ++c) lo[c] = n * kRowB + (((2 * c + hh) ^ S::swz(n)) << 4);
  const int xrow = kWTile + wv * 32 * kRowB;

  // Accumulators: X products start from the bias (register r of block fb holds
  // feature f0 + 32fb + 8(r/4) + 4hh + r%4), TX products from zero.
  f32x16 acc[2][kFB];
  {
    const auto rb = make_rsrc(p.bias ? (const char*)p.bias + (size_t)f0 * 2 : (const char*)p.x,
                              p.bias ? (uint32_t)(F - f0) * 2u : 0u);
#pragma unroll
    for (int fb = 0; fb < kFB; ++fb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rb, (32 * fb + 8 * g + 4 * hh) * 2, 0, 0);
        acc[0][fb][4 * g + 0] = __uint_as_float(v[0] << 16);
        acc[0][fb][4 * g + 1] = __uint_as_float(v[0] & 0xFFFF0000u);
        acc[0][fb][4 * g + 2] = __uint_as_float(v[1] << 16);
        acc[0][fb][4 * g + 3] = __uint_as_float(v[1] & 0xFFFF0000u);
      }
      acc[1][fb] = f32x16{};
    }
  }

  bf16x8 wf[kRing], xf[2][2];
  auto read_w = [&](const char* st, auto iq) {
    constexpr int q = decltype(iq)::value;
    wf[q % kRing] = *reinterpret_cast<const bf16x8*>(st + (q % kFB) * 32 * kRowB + lo[q / kFB]);
  };
  auto read_x = [&](const char* st, auto ic, auto iw) {
    constexpr int c = decltype(ic)::value, which = decltype(iw)::value;
    xf[c & 1][which] = *reinterpret_cast<const bf16x8*>(st + xrow + which * kXTile + lo[c]);
  };

  // One step: MFMAs on stage k & 1; with kMore, the copies of step k + 1, the
  // barrier that publishes them and the first reads of step k + 1; with kMore2,
  // the tail copies of step k + 2.
  auto step = [&](int k, auto more, auto more2) {
    constexpr bool kMore = decltype(more)::value;
    constexpr bool kMore2 = decltype(more2)::value;
    const char* cur = smem + (k & 1) * kStageB;
    const char* nxt = smem + ((k + 1) & 1) * kStageB;
    static_for<0, S::kUnits>([&](auto iu) {
      constexpr int u = decltype(iu)::value;
      constexpr int q = u / S::kPer, c = q / kFB, fb = q % kFB, which = u % S::kPer;
      acc[which][fb] = mfma(wf[q % kRing], xf[c & 1][which], acc[which][fb]);
      if constexpr (kMore && u % S::kHeadStride == 0 && u / S::kHeadStride < S::kDma - S::kTail)
        issue(k + 1, IC<S::kTail + u / S::kHeadStride>{});
      // current stage: W fragment q2 read kLead units before its first use
      static_for<S::kPre, S::kQ>([&](auto iq) {
        constexpr int q2 = decltype(iq)::value;
        if constexpr (q2 * S::kPer - S::kLead == u) read_w(cur, iq);
      });
      static_for<1, S::kC>([&](auto ic) {
        constexpr int c2 = decltype(ic)::value;
        static_for<0, S::kNX>([&](auto iw) {
          constexpr int w2 = decltype(iw)::value;
          if constexpr (c2 * S::kChunkU - S::kXLead + w2 == u) read_x(cur, ic, iw);
        });
      });
      if constexpr (kMore) {
        if constexpr (u == S::kBar) {
          __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0): copies landed, reads done
          __syncthreads();
        }
        static_for<0, S::kNX>([&](auto iw) {
          constexpr int w2 = decltype(iw)::value;
          if constexpr (S::next_unit(w2) == u) read_x(nxt, IC<0>{}, iw);
        });
        static_for<0, S::kPre>([&](auto iq) {
          constexpr int q2 = decltype(iq)::value;
          if constexpr (S::next_unit(S::kNX + q2) == u) read_w(nxt, iq);
        });
        if constexpr (kMore2 && u >= S::kBar && u < S::kBar + S::kTail) issue(k + 2, IC<u - S::kBar>{});
      }
      fence();
    });
  };

  const int nk = D / kTK;  // the host checks that kTK divides D
  // prologue: step 0's tiles, then its first fragments
  static_for<0, S::kDma>([&](auto ii) { issue(0, ii); });
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  static_for<0, S::kNX>([&](auto iw) { read_x(smem, IC<0>{}, iw); });
  if (nk > 1) static_for<0, S::kTail>([&](auto ii) { issue(1, ii); });  // step 1's tail slices: stage 1 is free
  static_for<0, S::kPre>([&](auto iq) { read_w(smem, iq); });
  for (int k = 0; k < nk - 2; ++k) step(k, std::true_type{}, std::true_type{});
  if (nk > 1) step(nk - 2, std::true_type{}, std::false_type{});
  step(nk - 1, std::false_type{}, std::false_type{});

  // ---- epilogue ----------------------------------------------------------------
  // Accumulator group g (registers 4g .. 4g + 3) of a lane holds features
  // 8g + 4hh .. +3 of its block; groups 2gp and 2gp + 1 are paired across the
  // half-waves so that each lane holds 8 consecutive features (half 0:
  // 16gp .. +7, half 1: 16gp + 8 .. +15), one 16-byte store each.  Everything is
  // packed before the first store.
  u32x4 pk[S::kNX][kFB][2];
#pragma unroll
  for (int w2 = 0; w2 < S::kNX; ++w2)
#pragma unroll
    for (int fb = 0; fb < kFB; ++fb)
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        u32x2 h2[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int g = 2 * gp + h;
          h2[h] = u32x2{pack_bf16(acc[w2][fb][4 * g], acc[w2][fb][4 * g + 1]),
                        pack_bf16(acc[w2][fb][4 * g + 2], acc[w2][fb][4 * g + 3])};
        }
        pk[w2][fb][gp] = pair_halves(h2[0], h2[1]);
      }
  fence();
  const int token = t0 + wv * 32 + n;  // rows at or past L fall outside the output range: dropped
  const uint32_t obase = ((uint32_t)token * p.d + 8 * hh) * 2;
  const int HD = p.H * p.d;
#pragma unroll
  for (int fb = 0; fb < kFB; ++fb) {
    const int f = f0 + 32 * fb;
    if (f >= F) break;  // wave-uniform: the partial last feature tile
    const int np = f / HD, h = (f % HD) / p.d, j0 = f % p.d;
    const size_t head = (((size_t)np * p.B + b) * p.H + h) * (size_t)L * p.d * 2;
    const uint32_t hbytes = (uint32_t)L * p.d * 2u;
#pragma unroll
    for (int w2 = 0; w2 < S::kNX; ++w2) {
      const auto ro = make_rsrc((const char*)(w2 ? p.ty : p.y) + head, hbytes);
#pragma unroll
      for (int gp = 0; gp < 2; ++gp)
        __builtin_amdgcn_raw_buffer_store_b128(pk[w2][fb][gp], ro, obase, (j0 + 16 * gp) * 2, 0);
    }
  }
}

template <bool kT, int kTF, int kTK>
hipError_t launch(const ProjProblem& pr, hipStream_t stream) {
  ProjParams p;
  p.x = pr.x; p.tx = pr.tx; p.w = pr.w; p.bias = pr.bias; p.y = pr.y; p.ty = pr.ty;
  p.B = pr.B; p.L = pr.L; p.D = pr.D; p.H = pr.H; p.d = pr.d;
  p.F = pr.n_out * pr.H * pr.d;
  p.n_ft = (p.F + kTF - 1) / kTF;
  p.n_tt = (p.L + kTT - 1) / kTT;
  p.n_blocks = p.n_ft * p.n_tt * p.B;
  p.group_f = p.n_blocks < kSmallGrid ? kGroupFSmall : kGroupFLarge;
  return launch_1d(reinterpret_cast<const void*>(&proj_bf16_kernel<kT, kTF, kTK>), p.n_blocks, kThreads, p,
                   stream);
}

// Workgroups of the 256-feature tiling (each factor bounded by the host checks).
int64_t wide_grid(const ProjProblem& p) {
  const int64_t F = (int64_t)p.n_out * p.H * p.d;
  return ((F + 255) / 256) * (((int64_t)p.L + kTT - 1) / kTT) * p.B;
}

}  // namespace

hipError_t launch_proj(const ProjProblem& p, hipStream_t stream) {
  // At most kNarrowGrid wide workgroups would leave half the CUs or more idle:
  // 128-feature tiles double the workgroups (the frozen tiles' 128-wide hidden
  // step needs D % 128 == 0; otherwise the wide tiles run).
  const bool narrow = wide_grid(p) <= kNarrowGrid;
  if (p.tx) return narrow ? launch<true, 128, 64>(p, stream) : launch<true, 256, 64>(p, stream);
  return narrow && p.D % 128 == 0 ? launch<false, 128, 128>(p, stream) : launch<false, 256, 64>(p, stream);
}

}  // namespace attnjvp
