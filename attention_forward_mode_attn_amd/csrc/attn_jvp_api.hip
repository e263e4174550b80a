// C ABI of the attention forward + JVP library: argument checks on the host,
// then one kernel launch on the caller's stream.  See include/attn_jvp.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>

#include "attn_jvp.h"
#include "launch.h"

namespace {

thread_local char g_last_error[256] = "";

int fail(int status, const char* what) {
  std::snprintf(g_last_error, sizeof g_last_error, "%s", what);
  return status;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

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

int attn_jvp_fwd(const void* q, const void* k, const void* v, const void* tq, const void* tk, const void* tv,
                 void* o, void* to, float* lse, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d,
                 float scale, int dtype, void* stream) {
  g_last_error[0] = '\0';
  if (dtype != ATTN_JVP_FP32 && dtype != ATTN_JVP_BF16) return fail(ATTN_JVP_EINVAL, "dtype must be 0 (fp32) or 1 (bf16)");
  if (B < 0 || H < 0 || Lq < 0 || Lk < 0 || d < 0) return fail(ATTN_JVP_EINVAL, "negative size");
  if (d != 64 && d != 128) return fail(ATTN_JVP_EUNSUPPORTED, "head dimension must be 64 or 128");
  if (B == 0 || H == 0 || Lq == 0) return ATTN_JVP_OK;  // nothing to compute
  if (Lk == 0) return fail(ATTN_JVP_EINVAL, "Lk == 0: softmax over no keys");
  if (!std::isfinite(scale) || !(scale > 0.0f)) return fail(ATTN_JVP_EINVAL, "scale must be finite and > 0");
  if (!q || !k || !v || !tq || !tk || !tv || !o || !to || !lse) return fail(ATTN_JVP_EINVAL, "NULL pointer");
  const void* t16[] = {q, k, v, tq, tk, tv, o, to};
  for (const void* x : t16)
    if (!aligned(x, 16)) return fail(ATTN_JVP_EALIGN, "tensor pointers must be 16-byte aligned");
  if (!aligned(lse, 4)) return fail(ATTN_JVP_EALIGN, "lse must be 4-byte aligned");
  const int64_t lim = int64_t(1) << 29;  // elements per head: keeps byte offsets within 32 bits
  if (Lq * d >= lim || Lk * d >= lim) return fail(ATTN_JVP_EUNSUPPORTED, "sequence too long for one head");
  const int64_t qtiles = (Lq + 127) / 128;
  if (B > INT32_MAX || H > INT32_MAX || B * H > INT32_MAX || B * H * qtiles >= (int64_t(1) << 31))
    return fail(ATTN_JVP_EUNSUPPORTED, "too many workgroups");

  attnjvp::Problem p;
  p.q = q; p.k = k; p.v = v; p.tq = tq; p.tk = tk; p.tv = tv;
  p.o = o; p.to = to; p.lse = lse;
  p.B = (int)B; p.H = (int)H; p.Lq = (int)Lq; p.Lk = (int)Lk; p.d = (int)d;
  p.scale = scale;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = dtype == ATTN_JVP_BF16 ? attnjvp::launch_bf16(p, s) : attnjvp::launch_fp32(p, s);
  if (e != hipSuccess) {
    std::snprintf(g_last_error, sizeof g_last_error, "HIP error %d: %s", (int)e, hipGetErrorString(e));
    return ATTN_JVP_ELAUNCH;
  }
  return ATTN_JVP_OK;
}

}  // extern "C"
