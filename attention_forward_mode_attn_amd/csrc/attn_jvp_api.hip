// C ABI of the attention forward + JVP library: argument checks on the host,
// then one kernel launch on the caller's stream.  See include/attn_jvp.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>

#include "attn_jvp.h"
#include "launch.h"

static_assert(ATTN_JVP_MAX_MERGE_PARTS == attnjvp::kMaxMergeParts, "merge part limit");

namespace {

thread_local char g_last_error[256] = "";

int fail(int status, const char* what) {
  std::snprintf(g_last_error, sizeof g_last_error, "%s", what);
  return status;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Every kernel runs a 1-D grid of 256-thread workgroups, and a launch must
// keep gridDim.x * blockDim.x below 2^32: at most 2^24 - 1 workgroups.
constexpr int64_t kMaxWorkgroups = (int64_t(1) << 24) - 1;

}  // namespace

extern "C" {

int attn_jvp_version(void) { return ATTN_JVP_VERSION; }

const char* attn_jvp_status_string(int status) {
  switch (status) {
    case ATTN_JVP_OK: return "ok";
    case ATTN_JVP_EINVAL: return "invalid argument";
    case ATTN_JVP_EUNSUPPORTED: return "unsupported head dimension or size";
    case ATTN_JVP_EALIGN: return "misaligned pointer";
    case ATTN_JVP_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

const char* attn_jvp_last_error(void) { return g_last_error; }

}  // extern "C"

namespace {

int fwd_impl(const void* q, const void* k, const void* v, const void* tq, const void* tk, const void* tv, void* o,
             void* to, float* lse, float* tlse, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t kv_rows,
             int64_t d, float scale, int dtype, void* stream) {
  g_last_error[0] = '\0';
  if (dtype != ATTN_JVP_FP32 && dtype != ATTN_JVP_BF16 && dtype != ATTN_JVP_BF16_F32OUT)
    return fail(ATTN_JVP_EINVAL, "dtype must be 0 (fp32), 1 (bf16) or 2 (bf16 in, fp32 out)");
  if (B < 0 || H < 0 || Lq < 0 || Lk < 0 || d < 0) return fail(ATTN_JVP_EINVAL, "negative size");
  if (d != 64 && d != 128) return fail(ATTN_JVP_EUNSUPPORTED, "head dimension must be 64 or 128");
  if (B == 0 || H == 0 || Lq == 0) return ATTN_JVP_OK;  // nothing to compute
  if (Lk == 0) return fail(ATTN_JVP_EINVAL, "Lk == 0: softmax over no keys");
  if (kv_rows < Lk) return fail(ATTN_JVP_EINVAL, "kv_rows < Lk");
  if (!std::isfinite(scale) || !(scale > 0.0f)) return fail(ATTN_JVP_EINVAL, "scale must be finite and > 0");
  if (!q || !k || !v || !tq || !o || !to || !lse) return fail(ATTN_JVP_EINVAL, "NULL pointer");
  if ((tk == nullptr) != (tv == nullptr)) return fail(ATTN_JVP_EINVAL, "tk and tv must both be NULL or both non-NULL");
  const void* t16[] = {q, k, v, tq, tk, tv, o, to};
  for (const void* x : t16)
    if (!aligned(x, 16)) return fail(ATTN_JVP_EALIGN, "tensor pointers must be 16-byte aligned");
  if (!aligned(lse, 4) || !aligned(tlse, 4)) return fail(ATTN_JVP_EALIGN, "lse and tlse must be 4-byte aligned");
  const int64_t lim = int64_t(1) << 29;  // elements per head: keeps byte offsets within 32 bits
  if (Lq >= lim / d || Lk >= lim / d) return fail(ATTN_JVP_EUNSUPPORTED, "sequence too long for one head");
  if (kv_rows > INT32_MAX) return fail(ATTN_JVP_EUNSUPPORTED, "kv_rows too large");
  const int64_t qtiles = (Lq + 127) / 128;
  if (B > kMaxWorkgroups || H > kMaxWorkgroups || B * H > kMaxWorkgroups || B * H * qtiles > kMaxWorkgroups)
    return fail(ATTN_JVP_EUNSUPPORTED, "too many workgroups: B*H*ceil(Lq/128) must stay below 2^24");

  attnjvp::Problem p;
  p.q = q; p.k = k; p.v = v; p.tq = tq; p.tk = tk; p.tv = tv;
  p.o = o; p.to = to; p.lse = lse; p.tlse = tlse;
  p.B = (int)B; p.H = (int)H; p.Lq = (int)Lq; p.Lk = (int)Lk; p.d = (int)d;
  p.kv_rows = (int)kv_rows;
  p.scale = scale;
  p.out_f32 = dtype == ATTN_JVP_BF16_F32OUT;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = dtype == ATTN_JVP_FP32 ? attnjvp::launch_fp32(p, s) : attnjvp::launch_bf16(p, s);
  if (e != hipSuccess) {
    std::snprintf(g_last_error, sizeof g_last_error, "HIP error %d: %s", (int)e, hipGetErrorString(e));
    return ATTN_JVP_ELAUNCH;
  }
  return ATTN_JVP_OK;
}

}  // namespace

extern "C" {

int attn_jvp_fwd(const void* q, const void* k, const void* v, const void* tq, const void* tk, const void* tv,
                 void* o, void* to, float* lse, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d,
                 float scale, int dtype, void* stream) {
  return fwd_impl(q, k, v, tq, tk, tv, o, to, lse, nullptr, B, H, Lq, Lk, Lk, d, scale, dtype, stream);
}

int attn_jvp_fwd_part(const void* q, const void* k, const void* v, const void* tq, const void* tk,
                      const void* tv, void* o, void* to, float* lse, float* tlse, int64_t B, int64_t H,
                      int64_t Lq, int64_t Lk, int64_t kv_rows, int64_t d, float scale, int dtype,
                      void* stream) {
  return fwd_impl(q, k, v, tq, tk, tv, o, to, lse, tlse, B, H, Lq, Lk, kv_rows, d, scale, dtype, stream);
}

int attn_jvp_merge(int n, const void* const* o_parts, const void* const* to_parts, const float* const* lse_parts,
                   const float* const* tlse_parts, void* o, void* to, float* lse, float* tlse, int64_t rows,
                   int64_t d, int dtype, void* stream) {
  g_last_error[0] = '\0';
  if (dtype != ATTN_JVP_FP32 && dtype != ATTN_JVP_BF16 && dtype != ATTN_JVP_BF16_F32OUT)
    return fail(ATTN_JVP_EINVAL, "dtype must be 0 (fp32), 1 (bf16) or 2 (fp32 parts, bf16 result)");
  if (n < 1 || n > ATTN_JVP_MAX_MERGE_PARTS) return fail(ATTN_JVP_EINVAL, "n must be in 1 .. ATTN_JVP_MAX_MERGE_PARTS");
  if (rows < 0 || d < 0) return fail(ATTN_JVP_EINVAL, "negative size");
  if (d != 64 && d != 128) return fail(ATTN_JVP_EUNSUPPORTED, "head dimension must be 64 or 128");
  if (rows == 0) return ATTN_JVP_OK;
  const int64_t rows_per_block = 256 / (d / 8);
  if (rows > kMaxWorkgroups * rows_per_block)  // more than kMaxWorkgroups workgroups
    return fail(ATTN_JVP_EUNSUPPORTED, "too many rows: ceil(rows*d/2048) must stay below 2^24");
  if (!o_parts || !to_parts || !lse_parts || !tlse_parts || !o || !to || !lse)
    return fail(ATTN_JVP_EINVAL, "NULL pointer");
  attnjvp::MergeProblem p{};
  p.n = n;
  for (int s = 0; s < n; ++s) {
    if (!o_parts[s] || !to_parts[s] || !lse_parts[s] || !tlse_parts[s]) return fail(ATTN_JVP_EINVAL, "NULL pointer");
    if (!aligned(o_parts[s], 16) || !aligned(to_parts[s], 16))
      return fail(ATTN_JVP_EALIGN, "tensor pointers must be 16-byte aligned");
    if (!aligned(lse_parts[s], 4) || !aligned(tlse_parts[s], 4))
      return fail(ATTN_JVP_EALIGN, "lse and tlse must be 4-byte aligned");
    p.o[s] = o_parts[s];
    p.to[s] = to_parts[s];
    p.lse[s] = lse_parts[s];
    p.tlse[s] = tlse_parts[s];
  }
  if (!aligned(o, 16) || !aligned(to, 16)) return fail(ATTN_JVP_EALIGN, "tensor pointers must be 16-byte aligned");
  if (!aligned(lse, 4) || !aligned(tlse, 4)) return fail(ATTN_JVP_EALIGN, "lse and tlse must be 4-byte aligned");
  p.out_o = o;
  p.out_to = to;
  p.out_lse = lse;
  p.out_tlse = tlse;
  p.rows = rows;
  p.d = (int)d;
  p.in_bf16 = dtype == ATTN_JVP_BF16;
  p.out_bf16 = dtype != ATTN_JVP_FP32;
  const hipError_t e = attnjvp::launch_merge(p, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    std::snprintf(g_last_error, sizeof g_last_error, "HIP error %d: %s", (int)e, hipGetErrorString(e));
    return ATTN_JVP_ELAUNCH;
  }
  return ATTN_JVP_OK;
}

int attn_jvp_proj(const void* x, const void* tx, const void* w, const void* bias, void* y, void* ty, int64_t B,
                  int64_t L, int64_t D, int64_t n_out, int64_t H, int64_t d, int dtype, void* stream) {
  g_last_error[0] = '\0';
  if (dtype != ATTN_JVP_FP32 && dtype != ATTN_JVP_BF16 && dtype != ATTN_JVP_BF16_F32OUT)
    return fail(ATTN_JVP_EINVAL, "dtype must be 0 (fp32), 1 (bf16) or 2 (bf16 in, fp32 out)");
  if (B < 0 || L < 0 || D < 0 || n_out < 0 || H < 0 || d < 0) return fail(ATTN_JVP_EINVAL, "negative size");
  if (dtype != ATTN_JVP_BF16) return fail(ATTN_JVP_EUNSUPPORTED, "the projection is bf16 only");
  if (d != 64 && d != 128) return fail(ATTN_JVP_EUNSUPPORTED, "head dimension must be 64 or 128");
  if (B == 0 || L == 0 || n_out == 0 || H == 0) return ATTN_JVP_OK;  // nothing to compute
  if (D == 0 || D % 64 != 0) return fail(ATTN_JVP_EUNSUPPORTED, "D must be a positive multiple of 64");
  if (!x || !w || !y) return fail(ATTN_JVP_EINVAL, "NULL pointer");
  if ((tx == nullptr) != (ty == nullptr)) return fail(ATTN_JVP_EINVAL, "tx and ty must both be NULL or both non-NULL");
  const void* p16[] = {x, tx, w, bias, y, ty};
  for (const void* q : p16)
    if (!aligned(q, 16)) return fail(ATTN_JVP_EALIGN, "pointers must be 16-byte aligned");
  // Every factor is bounded before it is multiplied, so no product below can
  // overflow 64 bits whatever the caller passes.
  const int64_t lim = int64_t(1) << 31;
  if (B >= lim || L >= lim || n_out >= lim || H >= lim || D >= (int64_t(1) << 22) || n_out * H >= lim)
    return fail(ATTN_JVP_EUNSUPPORTED, "size beyond the projection's limits");
  const int64_t F = n_out * H * d;
  if (F >= lim || L * D >= lim || F * D >= lim || L * d >= lim)
    return fail(ATTN_JVP_EUNSUPPORTED, "size beyond the projection's limits");
  const int64_t tiles = ((F + 255) / 256) * ((L + 127) / 128);  // < 2^23 * 2^24: no overflow
  if (B > kMaxWorkgroups || tiles > kMaxWorkgroups || tiles * B > kMaxWorkgroups)
    return fail(ATTN_JVP_EUNSUPPORTED, "too many workgroups: B*ceil(L/128)*ceil(n_out*H*d/256) must stay below 2^24");
  attnjvp::ProjProblem p;
  p.x = x; p.tx = tx; p.w = w; p.bias = bias; p.y = y; p.ty = ty;
  p.B = (int)B; p.L = (int)L; p.D = (int)D; p.n_out = (int)n_out; p.H = (int)H; p.d = (int)d;
  const hipError_t e = attnjvp::launch_proj(p, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    std::snprintf(g_last_error, sizeof g_last_error, "HIP error %d: %s", (int)e, hipGetErrorString(e));
    return ATTN_JVP_ELAUNCH;
  }
  return ATTN_JVP_OK;
}

int attn_jvp_rmsnorm_rope(const void* x, const void* tx, void* y, void* ty, const void* gamma, const float* rope_cos,
                          const float* rope_sin, int64_t B, int64_t H, int64_t L, int64_t d, float eps, int dtype,
                          void* stream) {
  g_last_error[0] = '\0';
  if (dtype != ATTN_JVP_FP32 && dtype != ATTN_JVP_BF16 && dtype != ATTN_JVP_BF16_F32OUT)
    return fail(ATTN_JVP_EINVAL, "dtype must be 0 (fp32), 1 (bf16) or 2 (bf16 in, fp32 out)");
  if (B < 0 || H < 0 || L < 0 || d < 0) return fail(ATTN_JVP_EINVAL, "negative size");
  if (d != 64 && d != 128) return fail(ATTN_JVP_EUNSUPPORTED, "head dimension must be 64 or 128");
  if (dtype == ATTN_JVP_BF16_F32OUT) return fail(ATTN_JVP_EUNSUPPORTED, "float32 outputs apply to the attention outputs only");
  if (B == 0 || H == 0 || L == 0) return ATTN_JVP_OK;  // nothing to compute
  if (!std::isfinite(eps) || eps < 0.0f) return fail(ATTN_JVP_EINVAL, "eps must be finite and >= 0");
  if (!x || !y) return fail(ATTN_JVP_EINVAL, "NULL pointer");
  if ((tx == nullptr) != (ty == nullptr)) return fail(ATTN_JVP_EINVAL, "tx and ty must both be NULL or both non-NULL");
  if ((rope_cos == nullptr) != (rope_sin == nullptr))
    return fail(ATTN_JVP_EINVAL, "rope_cos and rope_sin must both be NULL or both non-NULL");
  const void* p16[] = {x, tx, y, ty, gamma, rope_cos, rope_sin};
  for (const void* q : p16)
    if (!aligned(q, 16)) return fail(ATTN_JVP_EALIGN, "pointers must be 16-byte aligned");
  // Every factor is bounded before it is multiplied.
  if (B > kMaxWorkgroups || H > kMaxWorkgroups || B * H > kMaxWorkgroups || L > INT32_MAX)
    return fail(ATTN_JVP_EUNSUPPORTED, "size beyond the limits");
  const int64_t rows_per_block = 256 / (d * (dtype == ATTN_JVP_BF16 ? 2 : 4) / 16);
  if (((L + rows_per_block - 1) / rows_per_block) * (B * H) > kMaxWorkgroups)
    return fail(ATTN_JVP_EUNSUPPORTED, "too many workgroups: B*H*ceil(L/rows per workgroup) must stay below 2^24");
  attnjvp::NormRopeProblem p{};
  p.x = x; p.tx = tx; p.y = y; p.ty = ty; p.gamma = gamma; p.cos = rope_cos; p.sin = rope_sin;
  p.BH = (int)(B * H); p.L = (int)L; p.d = (int)d; p.eps = eps; p.bf16 = dtype == ATTN_JVP_BF16;
  const hipError_t e = attnjvp::launch_norm_rope(p, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    std::snprintf(g_last_error, sizeof g_last_error, "HIP error %d: %s", (int)e, hipGetErrorString(e));
    return ATTN_JVP_ELAUNCH;
  }
  return ATTN_JVP_OK;
}

}  // extern "C"

