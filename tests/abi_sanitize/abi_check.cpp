// Host-side check of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer (test infrastructure; built with the stub
// launchers, no GPU).  Every entry point is called over an argument matrix
// that includes the stated limits, one past them and 64-bit extremes; the
// checks must reject what the header rejects, pass what it accepts to the
// launcher unchanged, never launch after a failed check, and do all of it
// without undefined behaviour (signed overflow, out-of-bounds reads of the
// caller's pointer arrays).  Prints "ALL OK" and exits 0 when every check holds.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <thread>
#include <vector>

#include "attn_jvp.h"
#include "stub_launch.h"

static int failures = 0;
#define CHECK(cond)                                                       \
  do {                                                                    \
    if (!(cond)) {                                                        \
      std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);         \
      ++failures;                                                         \
    }                                                                     \
  } while (0)

static void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }
static float* F(uintptr_t a) { return reinterpret_cast<float*>(a); }
static const uintptr_t A0 = 0x10000;  // 16-byte aligned, never dereferenced

static const int64_t I64MAX = std::numeric_limits<int64_t>::max();
static const int64_t I64MIN = std::numeric_limits<int64_t>::min();
static const int64_t EXTREMES[] = {I64MIN, -1, 0, 1, (int64_t(1) << 24) - 1, int64_t(1) << 24, (int64_t(1) << 31) - 1,
                                   int64_t(1) << 31, (int64_t(1) << 62) + 3, I64MAX - 127, I64MAX};

static int fwd(int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d, float scale = 0.125f, int dtype = 1,
               bool frozen = false) {
  return attn_jvp_fwd(P(A0), P(A0 + 16), P(A0 + 32), P(A0 + 48), frozen ? nullptr : P(A0 + 64),
                      frozen ? nullptr : P(A0 + 80), P(A0 + 96), P(A0 + 112), F(A0 + 128), B, H, Lq, Lk, d, scale,
                      dtype, P(0x5000));
}

static int part(int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t kv, int64_t d, float* tlse = F(A0 + 144)) {
  return attn_jvp_fwd_part(P(A0), P(A0 + 16), P(A0 + 32), P(A0 + 48), P(A0 + 64), P(A0 + 80), P(A0 + 96),
                           P(A0 + 112), F(A0 + 128), tlse, B, H, Lq, Lk, kv, d, 0.125f, 1, nullptr);
}

static int merge(int n, int64_t rows, int64_t d, int dtype = 1) {
  // exactly n entries per array, on the heap: a read past them is an ASan error
  const int m = n > 0 ? n : 1;
  auto* o = new const void*[m];
  auto* to = new const void*[m];
  auto* l = new const float*[m];
  auto* tl = new const float*[m];
  for (int i = 0; i < m; ++i) {
    o[i] = P(A0 + 0x1000 * i);
    to[i] = P(A0 + 0x1000 * i + 16);
    l[i] = F(A0 + 0x1000 * i + 32);
    tl[i] = F(A0 + 0x1000 * i + 48);
  }
  const int s = attn_jvp_merge(n, o, to, l, tl, P(A0 + 0x100000), P(A0 + 0x100010), F(A0 + 0x100020),
                               F(A0 + 0x100030), rows, d, dtype, nullptr);
  delete[] o;
  delete[] to;
  delete[] l;
  delete[] tl;
  return s;
}

static int proj(int64_t B, int64_t L, int64_t D, int64_t n_out, int64_t H, int64_t d, bool tangent = true) {
  return attn_jvp_proj(P(A0), tangent ? P(A0 + 16) : nullptr, P(A0 + 32), P(A0 + 48), P(A0 + 64),
                       tangent ? P(A0 + 80) : nullptr, B, L, D, n_out, H, d, 1, nullptr);
}

static int norm_rope(int64_t B, int64_t H, int64_t L, int64_t d, float eps = 1e-6f, int dtype = 1,
                     bool tangent = true, bool tables = true) {
  return attn_jvp_rmsnorm_rope(P(A0), tangent ? P(A0 + 16) : nullptr, P(A0 + 32), tangent ? P(A0 + 48) : nullptr,
                               P(A0 + 64), tables ? F(A0 + 80) : nullptr, tables ? F(A0 + 96) : nullptr, B, H, L, d,
                               eps, dtype, nullptr);
}

// The workgroup count each launcher derives from an accepted problem.
static int64_t attn_blocks(const attnjvp::Problem& p) { return int64_t(p.B) * p.H * ((int64_t(p.Lq) + 127) / 128); }

int main() {
  // --- accepted calls reach the launcher with the values passed ---------------
  int c0 = stub::calls;
  CHECK(fwd(2, 3, 300, 77, 128) == ATTN_JVP_OK);
  CHECK(stub::calls == c0 + 1 && stub::last_kind == stub::Kind::bf16);
  CHECK(stub::last_problem.B == 2 && stub::last_problem.H == 3 && stub::last_problem.Lq == 300 &&
        stub::last_problem.Lk == 77 && stub::last_problem.kv_rows == 77 && stub::last_problem.d == 128);
  CHECK(stub::last_problem.tlse == nullptr && stub::last_problem.scale == 0.125f);
  CHECK(fwd(1, 1, 5, 5, 64, 0.5f, 0) == ATTN_JVP_OK && stub::last_kind == stub::Kind::fp32);
  CHECK(fwd(1, 1, 5, 5, 64, 0.5f, 1, true) == ATTN_JVP_OK && stub::last_problem.tk == nullptr &&
        stub::last_problem.tv == nullptr);
  CHECK(part(1, 2, 10, 7, 100, 128) == ATTN_JVP_OK && stub::last_problem.kv_rows == 100 &&
        stub::last_problem.Lk == 7 && stub::last_problem.tlse == F(A0 + 144));
  CHECK(merge(16, 1000, 64) == ATTN_JVP_OK && stub::last_kind == stub::Kind::merge &&
        stub::last_merge.n == 16 && stub::last_merge.rows == 1000 && stub::last_merge.d == 64);
  CHECK(stub::last_merge.in_bf16 && stub::last_merge.out_bf16);
  CHECK(merge(3, 10, 128, 2) == ATTN_JVP_OK && !stub::last_merge.in_bf16 && stub::last_merge.out_bf16);
  CHECK(merge(3, 10, 128, 0) == ATTN_JVP_OK && !stub::last_merge.in_bf16 && !stub::last_merge.out_bf16);
  CHECK(fwd(1, 2, 10, 10, 64, 0.1f, 2) == ATTN_JVP_OK && stub::last_kind == stub::Kind::bf16 &&
        stub::last_problem.out_f32);
  CHECK(fwd(1, 2, 10, 10, 64, 0.1f, 1) == ATTN_JVP_OK && !stub::last_problem.out_f32);
  CHECK(fwd(1, 2, 10, 10, 64, 0.1f, 3) == ATTN_JVP_EINVAL);
  CHECK(norm_rope(1, 1, 8, 64, 0.0f, 2) == ATTN_JVP_EUNSUPPORTED);
  CHECK(proj(2, 100, 256, 3, 4, 64) == ATTN_JVP_OK && stub::last_kind == stub::Kind::proj &&
        stub::last_proj.L == 100 && stub::last_proj.D == 256 && stub::last_proj.n_out == 3);
  CHECK(proj(2, 100, 256, 2, 4, 128, false) == ATTN_JVP_OK && stub::last_proj.tx == nullptr);

  CHECK(norm_rope(2, 3, 100, 128) == ATTN_JVP_OK && stub::last_kind == stub::Kind::norm_rope &&
        stub::last_norm_rope.BH == 6 && stub::last_norm_rope.L == 100 && stub::last_norm_rope.d == 128 &&
        stub::last_norm_rope.bf16 && stub::last_norm_rope.eps == 1e-6f);
  CHECK(norm_rope(1, 1, 7, 64, 0.0f, 0, false, false) == ATTN_JVP_OK && stub::last_norm_rope.tx == nullptr &&
        stub::last_norm_rope.cos == nullptr && !stub::last_norm_rope.bf16);

  // --- the largest accepted grids, and one workgroup more -----------------------
  const int64_t wg = (int64_t(1) << 24) - 1;
  CHECK(fwd(1, wg, 1, 1, 64) == ATTN_JVP_OK && attn_blocks(stub::last_problem) == wg);
  CHECK(fwd(1, wg + 1, 1, 1, 64) == ATTN_JVP_EUNSUPPORTED);
  CHECK(fwd(wg, 1, 128, 1, 64) == ATTN_JVP_OK && attn_blocks(stub::last_problem) == wg);
  CHECK(fwd(wg, 1, 129, 1, 64) == ATTN_JVP_EUNSUPPORTED);
  CHECK(merge(2, wg * 16, 128) == ATTN_JVP_OK);
  CHECK(merge(2, wg * 16 + 1, 128) == ATTN_JVP_EUNSUPPORTED);
  CHECK(merge(2, wg * 32, 64) == ATTN_JVP_OK);
  CHECK(merge(2, wg * 32 + 1, 64) == ATTN_JVP_EUNSUPPORTED);
  CHECK(proj(wg, 1, 64, 1, 2, 128) == ATTN_JVP_OK);
  CHECK(proj(wg + 1, 1, 64, 1, 2, 128) == ATTN_JVP_EUNSUPPORTED);

  CHECK(norm_rope(1, wg, 16, 128) == ATTN_JVP_OK);            // 16 rows per workgroup (bf16, d = 128)
  CHECK(norm_rope(1, wg, 17, 128) == ATTN_JVP_EUNSUPPORTED);
  CHECK(norm_rope(1, wg, 8, 128, 0.0f, 0) == ATTN_JVP_OK);     // 8 rows per workgroup (fp32, d = 128)
  CHECK(norm_rope(1, wg, 9, 128, 0.0f, 0) == ATTN_JVP_EUNSUPPORTED);

  // --- stated size limits ---------------------------------------------------------
  CHECK(fwd(1, 1, (int64_t(1) << 22) - 1, 8, 128) == ATTN_JVP_OK);  // Lq*d just below 2^29
  CHECK(fwd(1, 1, int64_t(1) << 22, 8, 128) == ATTN_JVP_EUNSUPPORTED);
  CHECK(fwd(1, 1, 8, (int64_t(1) << 23) - 1, 64) == ATTN_JVP_OK);
  CHECK(fwd(1, 1, 8, int64_t(1) << 23, 64) == ATTN_JVP_EUNSUPPORTED);
  CHECK(part(1, 1, 8, 8, (int64_t(1) << 31) - 1, 64) == ATTN_JVP_OK);
  CHECK(part(1, 1, 8, 8, int64_t(1) << 31, 64) == ATTN_JVP_EUNSUPPORTED);
  CHECK(proj(1, (int64_t(1) << 18) - 1, 8192, 1, 2, 128) == ATTN_JVP_OK);
  CHECK(proj(1, int64_t(1) << 18, 8192, 1, 2, 128) == ATTN_JVP_EUNSUPPORTED);

  // --- a failed check never launches ------------------------------------------------
  c0 = stub::calls;
  CHECK(fwd(1, 1, 8, 8, 96) == ATTN_JVP_EUNSUPPORTED);
  CHECK(fwd(1, 1, 8, 0, 64) == ATTN_JVP_EINVAL);
  CHECK(fwd(1, 1, 8, 8, 64, std::nanf("")) == ATTN_JVP_EINVAL);
  CHECK(fwd(1, 1, 8, 8, 64, -1.0f) == ATTN_JVP_EINVAL);
  CHECK(fwd(1, 1, 8, 8, 64, 0.1f, 7) == ATTN_JVP_EINVAL);
  CHECK(attn_jvp_fwd(P(A0 + 8), P(A0), P(A0), P(A0), P(A0), P(A0), P(A0), P(A0), F(A0), 1, 1, 8, 8, 64, 0.1f, 1,
                     nullptr) == ATTN_JVP_EALIGN);
  CHECK(attn_jvp_fwd(P(A0), P(A0), P(A0), P(A0), nullptr, P(A0), P(A0), P(A0), F(A0), 1, 1, 8, 8, 64, 0.1f, 1,
                     nullptr) == ATTN_JVP_EINVAL);
  CHECK(part(1, 1, 8, 8, 7, 64) == ATTN_JVP_EINVAL);
  CHECK(part(1, 1, 8, 8, 8, 64, F(A0 + 2)) == ATTN_JVP_EALIGN);
  CHECK(merge(0, 8, 64) == ATTN_JVP_EINVAL && merge(17, 8, 64) == ATTN_JVP_EINVAL);
  CHECK(merge(2, 8, 100) == ATTN_JVP_EUNSUPPORTED && merge(2, -1, 64) == ATTN_JVP_EINVAL);
  CHECK(proj(1, 8, 96, 3, 2, 64) == ATTN_JVP_EUNSUPPORTED);
  CHECK(norm_rope(1, 1, 8, 64, -1.0f) == ATTN_JVP_EINVAL && norm_rope(1, 1, 8, 64, INFINITY) == ATTN_JVP_EINVAL);
  CHECK(attn_jvp_rmsnorm_rope(P(A0), P(A0), P(A0), nullptr, nullptr, nullptr, nullptr, 1, 1, 8, 64, 0.0f, 1,
                              nullptr) == ATTN_JVP_EINVAL);
  CHECK(attn_jvp_rmsnorm_rope(P(A0), nullptr, P(A0), nullptr, nullptr, F(A0), nullptr, 1, 1, 8, 64, 0.0f, 1,
                              nullptr) == ATTN_JVP_EINVAL);
  CHECK(stub::calls == c0);
  CHECK(std::strlen(attn_jvp_last_error()) > 0);

  // --- zero-size calls are no-ops -----------------------------------------------------
  c0 = stub::calls;
  CHECK(attn_jvp_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 1, 8, 8,
                     64, 0.1f, 1, nullptr) == ATTN_JVP_OK);
  CHECK(attn_jvp_merge(2, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 64, 1,
                       nullptr) == ATTN_JVP_OK);
  CHECK(attn_jvp_proj(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 8, 64, 3, 2, 64, 1, nullptr) ==
        ATTN_JVP_OK);
  CHECK(stub::calls == c0 && attn_jvp_last_error()[0] == '\0');

  // --- every size argument at 64-bit extremes: rejected or accepted, never UB -----------
  for (int64_t x : EXTREMES) {
    for (int arg = 0; arg < 5; ++arg) {
      int64_t v[5] = {1, 2, 130, 70, 128};
      v[arg] = x;
      const int s = fwd(v[0], v[1], v[2], v[3], v[4]);
      CHECK(s == ATTN_JVP_OK || s == ATTN_JVP_EINVAL || s == ATTN_JVP_EUNSUPPORTED);
      if (s == ATTN_JVP_OK && v[0] * v[1] * v[2] > 0) CHECK(attn_blocks(stub::last_problem) <= wg);
    }
    for (int arg = 0; arg < 6; ++arg) {
      int64_t v[6] = {1, 2, 130, 70, 100, 128};
      v[arg] = x;
      const int s = part(v[0], v[1], v[2], v[3], v[4], v[5]);
      CHECK(s == ATTN_JVP_OK || s == ATTN_JVP_EINVAL || s == ATTN_JVP_EUNSUPPORTED);
    }
    for (int64_t d : {int64_t(64), int64_t(128), x}) {
      const int s = merge(3, x, d);
      CHECK(s == ATTN_JVP_OK || s == ATTN_JVP_EINVAL || s == ATTN_JVP_EUNSUPPORTED);
    }
    for (int arg = 0; arg < 6; ++arg) {
      int64_t v[6] = {2, 100, 256, 3, 4, 64};
      v[arg] = x;
      const int s = proj(v[0], v[1], v[2], v[3], v[4], v[5]);
      CHECK(s == ATTN_JVP_OK || s == ATTN_JVP_EINVAL || s == ATTN_JVP_EUNSUPPORTED);
    }
    for (int arg = 0; arg < 4; ++arg) {
      int64_t v[4] = {2, 3, 100, 128};
      v[arg] = x;
      const int s = norm_rope(v[0], v[1], v[2], v[3]);
      CHECK(s == ATTN_JVP_OK || s == ATTN_JVP_EINVAL || s == ATTN_JVP_EUNSUPPORTED);
    }
    for (int64_t y : EXTREMES) {  // pairs of large factors
      int s = fwd(x, y, 1 << 20, 8, 64);
      CHECK(s != ATTN_JVP_OK || attn_blocks(stub::last_problem) <= wg);
      s = proj(x, y, 64, 1, 2, 128);
      CHECK(s == ATTN_JVP_OK || s == ATTN_JVP_EINVAL || s == ATTN_JVP_EUNSUPPORTED);
      s = proj(1, 1 << 20, 64, x, y, 128);
      CHECK(s == ATTN_JVP_OK || s == ATTN_JVP_EINVAL || s == ATTN_JVP_EUNSUPPORTED);
      s = norm_rope(x, y, 1 << 20, 64);
      CHECK(s == ATTN_JVP_OK || s == ATTN_JVP_EINVAL || s == ATTN_JVP_EUNSUPPORTED);
      s = norm_rope(1, x, y, 128, 0.0f, 0);
      CHECK(s == ATTN_JVP_OK || s == ATTN_JVP_EINVAL || s == ATTN_JVP_EUNSUPPORTED);
      s = proj(x, 1 << 24, 64, 1, y, 128);
      CHECK(s == ATTN_JVP_OK || s == ATTN_JVP_EINVAL || s == ATTN_JVP_EUNSUPPORTED);
    }
  }
  // many workgroups spread over every factor of the projection grid
  CHECK(proj(int64_t(1) << 30, int64_t(1) << 24, 64, 1, int64_t(1) << 17, 128) == ATTN_JVP_EUNSUPPORTED);

  // --- a failed launch is reported, with the HIP message ------------------------------
  stub::next_status = hipErrorNoDevice;
  CHECK(fwd(1, 1, 8, 8, 64) == ATTN_JVP_ELAUNCH && std::strstr(attn_jvp_last_error(), "HIP error") != nullptr);
  CHECK(merge(2, 8, 64) == ATTN_JVP_ELAUNCH && proj(1, 8, 64, 1, 2, 64) == ATTN_JVP_ELAUNCH);
  stub::next_status = hipSuccess;

  // --- the last error is per host thread --------------------------------------------------
  CHECK(fwd(1, 1, 8, 8, 96) == ATTN_JVP_EUNSUPPORTED);
  std::thread t([] {
    CHECK(attn_jvp_last_error()[0] == '\0');
    CHECK(fwd(1, 1, 8, 0, 64) == ATTN_JVP_EINVAL && std::strstr(attn_jvp_last_error(), "Lk") != nullptr);
  });
  t.join();
  CHECK(std::strstr(attn_jvp_last_error(), "head dimension") != nullptr);

  CHECK(std::strcmp(attn_jvp_status_string(ATTN_JVP_OK), "ok") == 0);
  CHECK(std::strcmp(attn_jvp_status_string(12345), "unknown status") == 0);
  CHECK(attn_jvp_version() == ATTN_JVP_VERSION);

  if (failures == 0) std::printf("ALL OK\n");
  return failures ? 1 : 0;
}
