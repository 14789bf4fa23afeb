// C ABI of the library: argument validation and launch (see include/dbs.h).
//
// Every entry point validates its arguments on the host before launching
// anything, records a message for dbs_last_error() on failure and returns a
// status code; no exception leaves this file.
#include "dbs.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <exception>
#include <mutex>
#include <string>
#include <vector>

#include "dbs_internal.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

dbs_status fail(dbs_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

dbs_status ok() {
  g_last_error.clear();
  return DBS_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

dbs_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(DBS_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
}

#define DBS_GUARD_BEGIN try {
#define DBS_GUARD_END                                                     \
  }                                                                       \
  catch (const std::exception& ex) {                                      \
    return fail(DBS_ERR_INVALID_ARG, "internal error: %s", ex.what());    \
  }                                                                       \
  catch (...) {                                                           \
    return fail(DBS_ERR_INVALID_ARG, "internal error");                   \
  }

#define REQUIRE(cond, st, ...) \
  do {                         \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

dbs_status check_grid(int T, int H, int W, int prefix, int32_t* out) {
  REQUIRE(out != nullptr, DBS_ERR_INVALID_ARG, "perm_out is NULL");
  REQUIRE(T >= 1 && H >= 1 && W >= 1, DBS_ERR_INVALID_ARG, "grid sides must be >= 1 (got %d x %d x %d)", T, H, W);
  REQUIRE(prefix >= 0, DBS_ERR_INVALID_ARG, "prefix must be >= 0");
  const int64_t n = (int64_t)prefix + (int64_t)T * H * W;
  REQUIRE(n <= INT32_MAX, DBS_ERR_INVALID_ARG, "sequence length %lld exceeds int32", (long long)n);
  return DBS_OK;
}

// Shared checks for the token-geometry arguments of the device calls.
dbs_status check_geometry(int B, int Hh, int N, int Npad, int d, int b) {
  REQUIRE(B >= 1 && Hh >= 1, DBS_ERR_INVALID_ARG, "B and Hh must be >= 1 (got %d, %d)", B, Hh);
  REQUIRE(N >= 1, DBS_ERR_INVALID_ARG, "N must be >= 1 (got %d)", N);
  REQUIRE(d == 64 || d == 128, DBS_ERR_UNSUPPORTED, "head dim d=%d unsupported (64 or 128)", d);
  REQUIRE(b == 64 || b == 128, DBS_ERR_UNSUPPORTED, "block size b=%d unsupported (64 or 128)", b);
  REQUIRE(Npad >= N && Npad % b == 0, DBS_ERR_INVALID_ARG, "Npad=%d must be >= N=%d and a multiple of b=%d", Npad, N, b);
  REQUIRE(Npad - N < b, DBS_ERR_INVALID_ARG, "Npad=%d holds a whole empty block beyond N=%d", Npad, N);
  REQUIRE((int64_t)B * Hh * Npad * d <= ((int64_t)1 << 40), DBS_ERR_INVALID_ARG, "tensor too large");
  return DBS_OK;
}

dbs_status check_strides(int64_t sb, int64_t sn, int64_t sh, dbs_dtype dt) {
  const int64_t q = dt == DBS_BF16 ? 8 : 4;   // elements per 16 bytes
  REQUIRE(sb >= 0 && sn >= 0 && sh >= 0, DBS_ERR_INVALID_ARG, "strides must be >= 0");
  REQUIRE(sb % q == 0 && sn % q == 0 && sh % q == 0, DBS_ERR_ALIGNMENT,
          "strides (%lld, %lld, %lld) must keep rows 16-byte aligned", (long long)sb, (long long)sn,
          (long long)sh);
  return DBS_OK;
}

}  // namespace

extern "C" {

int dbs_abi_version(void) { return DBS_ABI_VERSION; }

const char* dbs_last_error(void) { return g_last_error.c_str(); }

dbs_status dbs_perm_gilbert3d(int T, int H, int W, int prefix, int32_t* perm_out) {
  DBS_GUARD_BEGIN
  dbs_status st = check_grid(T, H, W, prefix, perm_out);
  if (st != DBS_OK) return st;
  dbs::gilbert3d(T, H, W, prefix, perm_out);
  return ok();
  DBS_GUARD_END
}

dbs_status dbs_perm_cuboid(int T, int H, int W, int ct, int ch, int cw, int prefix, int32_t* perm_out) {
  DBS_GUARD_BEGIN
  dbs_status st = check_grid(T, H, W, prefix, perm_out);
  if (st != DBS_OK) return st;
  REQUIRE(ct >= 1 && ch >= 1 && cw >= 1, DBS_ERR_INVALID_ARG, "cuboid sides must be >= 1");
  dbs::cuboid_order(T, H, W, ct, ch, cw, prefix, perm_out);
  return ok();
  DBS_GUARD_END
}

dbs_status dbs_perm_invert(const int32_t* perm, int n, int32_t* inv_out) {
  DBS_GUARD_BEGIN
  REQUIRE(perm != nullptr && inv_out != nullptr, DBS_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(n >= 1, DBS_ERR_INVALID_ARG, "n must be >= 1");
  for (int i = 0; i < n; ++i) inv_out[i] = -1;
  for (int i = 0; i < n; ++i) {
    const int32_t p = perm[i];
    REQUIRE(p >= 0 && p < n && inv_out[p] == -1, DBS_ERR_INVALID_ARG,
            "not a permutation: entry %d is %d", i, p);
    inv_out[p] = i;
  }
  return ok();
  DBS_GUARD_END
}

dbs_status dbs_prune_anchors(int T, int H, int W, int prefix, int wt, int wh, int ww, const int32_t* perm,
                             int32_t* anchor_out) {
  DBS_GUARD_BEGIN
  dbs_status st = check_grid(T, H, W, prefix, anchor_out);
  if (st != DBS_OK) return st;
  REQUIRE(perm != nullptr, DBS_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(wt >= 1 && wh >= 1 && ww >= 1, DBS_ERR_INVALID_ARG, "window sides must be >= 1");
  const int n = prefix + T * H * W;
  std::vector<int32_t> inv(n, -1);
  for (int i = 0; i < n; ++i) {
    const int32_t p = perm[i];
    REQUIRE(p >= 0 && p < n && inv[p] == -1, DBS_ERR_INVALID_ARG, "not a permutation: entry %d is %d", i, p);
    inv[p] = i;
  }
  // centre of the window holding x along an axis of n cells: offset (e - 1) / 2 in
  // a window of extent e (windows tile from the origin; the last may be cut)
  auto centre = [](int x, int w, int len) {
    const int x0 = x / w * w;
    const int e = (x0 + w < len ? x0 + w : len) - x0;
    return x0 + (e - 1) / 2;
  };
  for (int i = 0; i < n; ++i) {
    const int tok = perm[i];
    int a = tok;
    if (tok >= prefix) {
      const int r = tok - prefix;
      const int t = r / (H * W), h = r / W % H, w = r % W;
      a = prefix + (centre(t, wt, T) * H + centre(h, wh, H)) * W + centre(w, ww, W);
    }
    anchor_out[i] = inv[a];
  }
  return ok();
  DBS_GUARD_END
}

dbs_status dbs_reorder(const void* x, dbs_dtype x_dt, int64_t sb, int64_t sn, int64_t sh, void* y,
                       dbs_dtype y_dt, dbs_layout y_layout, const int32_t* perm, int perm_per_head,
                       int B, int Hh, int N, int Npad, int d, int b, hipStream_t stream) {
  DBS_GUARD_BEGIN
  REQUIRE(x && y && perm, DBS_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(aligned16(x) && aligned16(y) && ((uintptr_t)perm & 3u) == 0, DBS_ERR_ALIGNMENT, "misaligned pointer");
  REQUIRE(x_dt == DBS_BF16 || x_dt == DBS_FP32, DBS_ERR_INVALID_ARG, "bad x dtype");
  REQUIRE(y_dt == DBS_BF16 || y_dt == DBS_FP32, DBS_ERR_INVALID_ARG, "bad y dtype");
  REQUIRE(!(x_dt == DBS_BF16 && y_dt == DBS_FP32), DBS_ERR_UNSUPPORTED, "bf16 -> fp32 reorder not offered");
  REQUIRE(y_layout == DBS_ROWS || y_layout == DBS_TILES_T, DBS_ERR_INVALID_ARG, "bad layout");
  REQUIRE(!(y_layout == DBS_TILES_T && y_dt != DBS_BF16), DBS_ERR_UNSUPPORTED, "tiles layout is bf16 only");
  REQUIRE(perm_per_head == 0 || perm_per_head == 1, DBS_ERR_INVALID_ARG, "perm_per_head must be 0 or 1");
  dbs_status st = check_geometry(B, Hh, N, Npad, d, b);
  if (st != DBS_OK) return st;
  st = check_strides(sb, sn, sh, x_dt);
  if (st != DBS_OK) return st;
  dbs::ReorderArgs a{};
  a.x = x; a.y = y; a.sb = sb; a.sn = sn; a.sh = sh; a.perm = perm;
  a.perm_h_stride = perm_per_head ? N : 0;
  a.B = B; a.Hh = Hh; a.N = N; a.Npad = Npad; a.d = d; a.b = b;
  a.x_f32 = x_dt == DBS_FP32; a.y_f32 = y_dt == DBS_FP32; a.tiles_t = y_layout == DBS_TILES_T;
  a.stream = stream;
  return from_hip(dbs::launch_reorder(a), "dbs_reorder launch");
  DBS_GUARD_END
}

dbs_status dbs_reorder_kv(const void* k, const void* v, dbs_dtype x_dt, int64_t sb, int64_t sn, int64_t sh,
                          void* k_r, void* v_t, const int32_t* perm, int perm_per_head, int B, int Hh, int N,
                          int Npad, int d, int b, hipStream_t stream) {
  DBS_GUARD_BEGIN
  REQUIRE(k && v && k_r && v_t && perm, DBS_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(aligned16(k) && aligned16(v) && aligned16(k_r) && aligned16(v_t) && ((uintptr_t)perm & 3u) == 0,
          DBS_ERR_ALIGNMENT, "misaligned pointer");
  REQUIRE(x_dt == DBS_BF16 || x_dt == DBS_FP32, DBS_ERR_INVALID_ARG, "bad k/v dtype");
  REQUIRE(perm_per_head == 0 || perm_per_head == 1, DBS_ERR_INVALID_ARG, "perm_per_head must be 0 or 1");
  dbs_status st = check_geometry(B, Hh, N, Npad, d, b);
  if (st != DBS_OK) return st;
  st = check_strides(sb, sn, sh, x_dt);
  if (st != DBS_OK) return st;
  dbs::ReorderArgs a{};
  a.x = k; a.x2 = v; a.y = k_r; a.y2 = v_t; a.sb = sb; a.sn = sn; a.sh = sh; a.perm = perm;
  a.perm_h_stride = perm_per_head ? N : 0;
  a.B = B; a.Hh = Hh; a.N = N; a.Npad = Npad; a.d = d; a.b = b;
  a.x_f32 = x_dt == DBS_FP32; a.y_f32 = false; a.tiles_t = true;
  a.stream = stream;
  return from_hip(dbs::launch_reorder_kv(a), "dbs_reorder_kv launch");
  DBS_GUARD_END
}

dbs_status dbs_reorder_kv_pool(const void* k, const void* v, dbs_dtype x_dt, int64_t sb, int64_t sn, int64_t sh,
                               void* k_r, void* v_t, const int32_t* perm, int perm_per_head, int B, int Hh, int N,
                               int Npad, int d, int b, int n, void* k_g, void* v_g, hipStream_t stream) {
  DBS_GUARD_BEGIN
  REQUIRE(k_g && v_g, DBS_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(aligned16(k_g) && aligned16(v_g), DBS_ERR_ALIGNMENT, "misaligned pointer");
  REQUIRE(n >= 1 && n <= N, DBS_ERR_INVALID_ARG, "n=%d must be in [1, N]", n);
  if (b % n != 0) {   // windows cross tiles: the two passes
    dbs_status st = dbs_reorder_kv(k, v, x_dt, sb, sn, sh, k_r, v_t, perm, perm_per_head, B, Hh, N, Npad, d, b,
                                   stream);
    if (st != DBS_OK) return st;
    return dbs_meanpool_kv(k_r, v_t, DBS_BF16, B, Hh, N, Npad, d, b, n, k_g, v_g, stream);
  }
  REQUIRE(k && v && k_r && v_t && perm, DBS_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(aligned16(k) && aligned16(v) && aligned16(k_r) && aligned16(v_t) && ((uintptr_t)perm & 3u) == 0,
          DBS_ERR_ALIGNMENT, "misaligned pointer");
  REQUIRE(x_dt == DBS_BF16 || x_dt == DBS_FP32, DBS_ERR_INVALID_ARG, "bad k/v dtype");
  REQUIRE(perm_per_head == 0 || perm_per_head == 1, DBS_ERR_INVALID_ARG, "perm_per_head must be 0 or 1");
  dbs_status st = check_geometry(B, Hh, N, Npad, d, b);
  if (st != DBS_OK) return st;
  st = check_strides(sb, sn, sh, x_dt);
  if (st != DBS_OK) return st;
  dbs::ReorderArgs a{};
  a.x = k; a.x2 = v; a.y = k_r; a.y2 = v_t; a.sb = sb; a.sn = sn; a.sh = sh; a.perm = perm;
  a.perm_h_stride = perm_per_head ? N : 0;
  a.B = B; a.Hh = Hh; a.N = N; a.Npad = Npad; a.d = d; a.b = b;
  a.x_f32 = x_dt == DBS_FP32; a.y_f32 = false; a.tiles_t = true;
  a.k_g = k_g; a.v_g = v_g; a.n_pool = n;
  a.stream = stream;
  return from_hip(dbs::launch_reorder_kv(a), "dbs_reorder_kv_pool launch");
  DBS_GUARD_END
}

dbs_status dbs_inverse_reorder(const void* y, dbs_dtype y_dt, void* x, dbs_dtype x_dt, int64_t sb,
                               int64_t sn, int64_t sh, const int32_t* perm, int perm_per_head, int B,
                               int Hh, int N, int Npad, int d, hipStream_t stream) {
  DBS_GUARD_BEGIN
  REQUIRE(x && y && perm, DBS_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(aligned16(x) && aligned16(y) && ((uintptr_t)perm & 3u) == 0, DBS_ERR_ALIGNMENT, "misaligned pointer");
  REQUIRE(y_dt == DBS_BF16 || y_dt == DBS_FP32, DBS_ERR_INVALID_ARG, "bad y dtype");
  REQUIRE(x_dt == DBS_BF16 || x_dt == DBS_FP32, DBS_ERR_INVALID_ARG, "bad x dtype");
  REQUIRE(!(y_dt == DBS_FP32 && x_dt == DBS_BF16), DBS_ERR_UNSUPPORTED, "float32 -> bf16 inverse not offered");
  REQUIRE(perm_per_head == 0 || perm_per_head == 1, DBS_ERR_INVALID_ARG, "perm_per_head must be 0 or 1");
  REQUIRE(B >= 1 && Hh >= 1 && N >= 1 && Npad >= N, DBS_ERR_INVALID_ARG, "bad sizes");
  REQUIRE(d == 64 || d == 128, DBS_ERR_UNSUPPORTED, "head dim d=%d unsupported", d);
  dbs_status st = check_strides(sb, sn, sh, x_dt);
  if (st != DBS_OK) return st;
  dbs::ReorderArgs a{};
  a.y = const_cast<void*>(y); a.x_out = x; a.sb = sb; a.sn = sn; a.sh = sh; a.perm = perm;
  a.perm_h_stride = perm_per_head ? N : 0;
  a.B = B; a.Hh = Hh; a.N = N; a.Npad = Npad; a.d = d; a.b = 0;
  a.x_f32 = x_dt == DBS_FP32; a.y_f32 = y_dt == DBS_FP32;
  a.stream = stream;
  return from_hip(dbs::launch_inverse_reorder(a), "dbs_inverse_reorder launch");
  DBS_GUARD_END
}

size_t dbs_estimate_workspace_bytes(int B, int Hh, int N, int d, int b, int k) {
  if (B < 1 || Hh < 1 || N < 1 || b < 1 || k < 1 || (d != 64 && d != 128)) return 0;
  const int nb = (N + b - 1) / b;
  return dbs::estimate_workspace_bytes(B, Hh, nb, k, d);
}

size_t dbs_estimate_kvtok_workspace_bytes(int B, int Hh, int N, int d, int b, int k) {
  if (B < 1 || Hh < 1 || N < 1 || b < 1 || k < 1 || (d != 64 && d != 128)) return 0;
  const int nb = (N + b - 1) / b;
  return dbs::estimate_kvtok_workspace_bytes(B, Hh, nb, k, d);
}

}  // extern "C"

namespace {

// Token-order Q operand: element (b, i, h, :) at b * sb + i * sn + h * sh.
dbs_status check_tok(const void* x, dbs_dtype dt, int64_t sb, int64_t sn, int64_t sh, const int32_t* perm,
                     int perm_per_head) {
  REQUIRE(x && perm, DBS_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(aligned16(x) && ((uintptr_t)perm & 3u) == 0, DBS_ERR_ALIGNMENT, "misaligned pointer");
  REQUIRE(dt == DBS_BF16 || dt == DBS_FP32, DBS_ERR_INVALID_ARG, "bad dtype");
  REQUIRE(perm_per_head == 0 || perm_per_head == 1, DBS_ERR_INVALID_ARG, "perm_per_head must be 0 or 1");
  return check_strides(sb, sn, sh, dt);
}

// The selection rule and its parameter into a, checked (rule values of dbs_mask_rule).
dbs_status rule_args(int rule, double param, int nb, dbs::MaskArgs& a) {
  REQUIRE(std::isfinite(param), DBS_ERR_INVALID_ARG, "param must be finite");
  if (rule == DBS_RULE_CUMULATIVE) {
    REQUIRE(param > 0.0 && param <= 1.0, DBS_ERR_INVALID_ARG, "tau=%g must be in (0, 1]", param);
    a.rule = 0; a.tau = (float)param;
    REQUIRE(a.tau > 0.f, DBS_ERR_INVALID_ARG, "tau=%g rounds to 0 in float32", param);
  } else if (rule == DBS_RULE_TOPK) {
    REQUIRE(param >= 1.0 && param == std::floor(param) && param <= 1e9, DBS_ERR_INVALID_ARG,
            "top-k count %g must be an integer >= 1", param);
    a.rule = 1; a.topk = param >= nb ? nb : (int)param;
  } else if (rule == DBS_RULE_STAT) {
    a.rule = 2; a.u = param;
  } else if (rule == DBS_RULE_STAT_K) {
    REQUIRE(param > 0.0 && param < (double)nb, DBS_ERR_INVALID_ARG, "expected count %g must be in (0, nb=%d)",
            param, nb);
    a.rule = 2; a.u = dbs::normal_quantile(1.0 - param / nb);
  } else {
    return fail(DBS_ERR_INVALID_ARG, "unknown rule %d", rule);
  }
  return DBS_OK;
}

// Float32 operands (reordered rows): the VALU estimator writes P_imp (into the
// workspace when the fused call is given no p_imp), then the selection runs on it.
dbs_status estimate_f32_impl(const void* q_r, const void* k_r, int B, int Hh, int N, int Npad, int d, int b,
                             int k, float scale, float* p_imp, void* workspace, size_t workspace_bytes,
                             hipStream_t stream, const dbs::MaskArgs* fuse = nullptr) {
  REQUIRE(q_r && k_r && (p_imp || fuse) && workspace, DBS_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(aligned16(q_r) && aligned16(k_r) && aligned16(p_imp) && aligned16(workspace), DBS_ERR_ALIGNMENT,
          "misaligned pointer");
  dbs_status st = check_geometry(B, Hh, N, Npad, d, b);
  if (st != DBS_OK) return st;
  REQUIRE(k >= 1 && k <= b, DBS_ERR_INVALID_ARG, "k=%d must be in [1, b=%d]", k, b);
  REQUIRE(std::isfinite(scale) && scale > 0.f, DBS_ERR_INVALID_ARG, "scale must be finite and > 0");
  const size_t need = dbs_estimate_workspace_bytes(B, Hh, N, d, b, k);
  REQUIRE(workspace_bytes >= need, DBS_ERR_INVALID_ARG, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  const int nb = Npad / b;
  REQUIRE(nb <= 4096, DBS_ERR_UNSUPPORTED, "nb=%d must be in [1, 4096]", nb);
  REQUIRE((int64_t)B * Hh * nb <= INT32_MAX, DBS_ERR_INVALID_ARG, "too many rows");
  float* P = p_imp;
  if (P == nullptr) {
    REQUIRE(workspace_bytes >= (size_t)B * Hh * nb * nb * sizeof(float), DBS_ERR_INVALID_ARG,
            "workspace too small to hold P_imp");
    P = reinterpret_cast<float*>(workspace);
  }
  dbs::EstimateArgs a{};
  a.q_r = q_r; a.k_r = k_r; a.p_imp = P; a.workspace = workspace;
  a.B = B; a.Hh = Hh; a.N = N; a.Npad = Npad; a.d = d; a.b = b; a.k = k; a.nb = nb;
  a.scale = scale; a.stream = stream;
  hipError_t e = dbs::launch_estimate_f32(a);
  if (e != hipSuccess || fuse == nullptr) return from_hip(e, "dbs_estimate_blocks launch");
  dbs::MaskArgs m = *fuse;
  m.p_imp = P; m.rows = B * Hh * nb; m.nb = nb; m.stream = stream;
  return from_hip(dbs::launch_build_mask(m), "dbs_estimate_mask launch");
}

// The token-order K of dbs_estimate_mask_kvtok (element (b, i, h, :) at
// b * sb + i * sn + h * sh); unset for the calls that read k_r.
struct KeyTok {
  const void* k = nullptr;
  int f32 = 0;
  int64_t sb = 0, sn = 0, sh = 0;
};

// fuse set: P_imp rows go straight into the block selection (p_imp nullable).
// key.k set: K is read in token order (tok.perm) and k_r is not used.
dbs_status estimate_impl(const void* q_r, const void* k_r, int B, int Hh, int N, int Npad, int d, int b, int k,
                         float scale, float* p_imp, void* workspace, size_t workspace_bytes,
                         const dbs::TokIO& tok, hipStream_t stream, const dbs::MaskArgs* fuse = nullptr,
                         const KeyTok& key = KeyTok{}) {
  REQUIRE((k_r || key.k) && (p_imp || fuse) && workspace, DBS_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(aligned16(k_r) && aligned16(p_imp) && aligned16(workspace), DBS_ERR_ALIGNMENT, "misaligned pointer");
  dbs_status st = check_geometry(B, Hh, N, Npad, d, b);
  if (st != DBS_OK) return st;
  REQUIRE(k >= 1 && k <= b, DBS_ERR_INVALID_ARG, "k=%d must be in [1, b=%d]", k, b);
  REQUIRE(std::isfinite(scale) && scale > 0.f, DBS_ERR_INVALID_ARG, "scale must be finite and > 0");
  const size_t need = key.k ? dbs_estimate_kvtok_workspace_bytes(B, Hh, N, d, b, k)
                            : dbs_estimate_workspace_bytes(B, Hh, N, d, b, k);
  REQUIRE(workspace_bytes >= need, DBS_ERR_INVALID_ARG, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  const int nb = Npad / b;
  REQUIRE((int64_t)nb * k <= INT32_MAX / 2, DBS_ERR_INVALID_ARG, "too many sampled tokens");
  dbs::EstimateArgs a{};
  a.q_r = q_r; a.k_r = k_r; a.p_imp = p_imp; a.workspace = workspace;
  a.B = B; a.Hh = Hh; a.N = N; a.Npad = Npad; a.d = d; a.b = b; a.k = k; a.nb = nb;
  a.scale = scale; a.tok = tok; a.stream = stream;
  a.k_tok = key.k; a.k_f32 = key.f32; a.ksb = key.sb; a.ksn = key.sn; a.ksh = key.sh;
  if (fuse != nullptr) {
    REQUIRE(nb <= 4096, DBS_ERR_UNSUPPORTED, "nb=%d must be in [1, 4096]", nb);
    REQUIRE((int64_t)B * Hh * nb <= INT32_MAX, DBS_ERR_INVALID_ARG, "too many rows");
    dbs::MaskArgs m = *fuse;
    m.rows = B * Hh * nb; m.nb = nb; m.stream = stream;
    a.fuse = &m;
    return from_hip(dbs::launch_estimate(a), "dbs_estimate_mask launch");
  }
  return from_hip(dbs::launch_estimate(a), "dbs_estimate_blocks launch");
}

// The kept-block outputs of the fused calls, checked, with the rule.
dbs_status fuse_args(int rule, double param, int32_t* kv_count, int32_t* kv_idx, uint8_t* mask, int32_t* order,
                     int Npad, int b, dbs::MaskArgs& m) {
  REQUIRE(kv_count && kv_idx, DBS_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(((uintptr_t)kv_count & 3u) == 0 && ((uintptr_t)kv_idx & 3u) == 0 && ((uintptr_t)order & 3u) == 0,
          DBS_ERR_ALIGNMENT, "misaligned pointer");
  m.kv_count = kv_count; m.kv_idx = kv_idx; m.mask = mask; m.order = order;
  return rule_args(rule, param, b > 0 ? Npad / b : 1, m);
}

}  // namespace

extern "C" {

dbs_status dbs_estimate_blocks(const void* q_r, const void* k_r, dbs_dtype dt, int B, int Hh, int N,
                               int Npad, int d, int b, int k, float scale, float* p_imp,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  DBS_GUARD_BEGIN
  REQUIRE(q_r, DBS_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(aligned16(q_r), DBS_ERR_ALIGNMENT, "misaligned pointer");
  REQUIRE(dt == DBS_BF16 || dt == DBS_FP32, DBS_ERR_INVALID_ARG, "bad dtype");
  if (dt == DBS_FP32)
    return estimate_f32_impl(q_r, k_r, B, Hh, N, Npad, d, b, k, scale, p_imp, workspace, workspace_bytes, stream);
  return estimate_impl(q_r, k_r, B, Hh, N, Npad, d, b, k, scale, p_imp, workspace, workspace_bytes, dbs::TokIO{},
                       stream);
  DBS_GUARD_END
}

dbs_status dbs_estimate_blocks_tok(const void* q, dbs_dtype q_dt, int64_t sb, int64_t sn, int64_t sh,
                                   const int32_t* perm, int perm_per_head, const void* k_r, int B, int Hh,
                                   int N, int Npad, int d, int b, int k, float scale, float* p_imp,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  DBS_GUARD_BEGIN
  dbs_status st = check_tok(q, q_dt, sb, sn, sh, perm, perm_per_head);
  if (st != DBS_OK) return st;
  dbs::TokIO tok{};
  tok.q = q; tok.q_f32 = q_dt == DBS_FP32; tok.qsb = sb; tok.qsn = sn; tok.qsh = sh;
  tok.perm = perm; tok.perm_h_stride = perm_per_head ? N : 0;
  return estimate_impl(nullptr, k_r, B, Hh, N, Npad, d, b, k, scale, p_imp, workspace, workspace_bytes, tok,
                       stream);
  DBS_GUARD_END
}

dbs_status dbs_estimate_mask(const void* q_r, const void* k_r, dbs_dtype dt, int B, int Hh, int N, int Npad,
                             int d, int b, int k, float scale, int rule, double param, float* p_imp,
                             int32_t* kv_count, int32_t* kv_idx, uint8_t* mask, int32_t* order, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  DBS_GUARD_BEGIN
  REQUIRE(q_r, DBS_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(aligned16(q_r), DBS_ERR_ALIGNMENT, "misaligned pointer");
  REQUIRE(dt == DBS_BF16 || dt == DBS_FP32, DBS_ERR_INVALID_ARG, "bad dtype");
  dbs::MaskArgs m{};
  dbs_status st = fuse_args(rule, param, kv_count, kv_idx, mask, order, Npad, b, m);
  if (st != DBS_OK) return st;
  if (dt == DBS_FP32)
    return estimate_f32_impl(q_r, k_r, B, Hh, N, Npad, d, b, k, scale, p_imp, workspace, workspace_bytes, stream,
                             &m);
  return estimate_impl(q_r, k_r, B, Hh, N, Npad, d, b, k, scale, p_imp, workspace, workspace_bytes, dbs::TokIO{},
                       stream, &m);
  DBS_GUARD_END
}

dbs_status dbs_estimate_mask_tok(const void* q, dbs_dtype q_dt, int64_t sb, int64_t sn, int64_t sh,
                                 const int32_t* perm, int perm_per_head, const void* k_r, int B, int Hh, int N,
                                 int Npad, int d, int b, int k, float scale, int rule, double param, float* p_imp,
                                 int32_t* kv_count, int32_t* kv_idx, uint8_t* mask, int32_t* order,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  DBS_GUARD_BEGIN
  dbs_status st = check_tok(q, q_dt, sb, sn, sh, perm, perm_per_head);
  if (st != DBS_OK) return st;
  dbs::MaskArgs m{};
  st = fuse_args(rule, param, kv_count, kv_idx, mask, order, Npad, b, m);
  if (st != DBS_OK) return st;
  dbs::TokIO tok{};
  tok.q = q; tok.q_f32 = q_dt == DBS_FP32; tok.qsb = sb; tok.qsn = sn; tok.qsh = sh;
  tok.perm = perm; tok.perm_h_stride = perm_per_head ? N : 0;
  return estimate_impl(nullptr, k_r, B, Hh, N, Npad, d, b, k, scale, p_imp, workspace, workspace_bytes, tok,
                       stream, &m);
  DBS_GUARD_END
}

dbs_status dbs_estimate_mask_kvtok(const void* q, dbs_dtype q_dt, int64_t qsb, int64_t qsn, int64_t qsh,
                                   const void* key, dbs_dtype key_dt, int64_t ksb, int64_t ksn, int64_t ksh,
                                   const int32_t* perm, int perm_per_head, int B, int Hh, int N, int Npad, int d,
                                   int b, int k, float scale, int rule, double param, float* p_imp,
                                   int32_t* kv_count, int32_t* kv_idx, uint8_t* mask, int32_t* order,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  DBS_GUARD_BEGIN
  dbs_status st = check_tok(q, q_dt, qsb, qsn, qsh, perm, perm_per_head);
  if (st != DBS_OK) return st;
  st = check_tok(key, key_dt, ksb, ksn, ksh, perm, perm_per_head);
  if (st != DBS_OK) return st;
  dbs::MaskArgs m{};
  st = fuse_args(rule, param, kv_count, kv_idx, mask, order, Npad, b, m);
  if (st != DBS_OK) return st;
  dbs::TokIO tok{};
  tok.q = q; tok.q_f32 = q_dt == DBS_FP32; tok.qsb = qsb; tok.qsn = qsn; tok.qsh = qsh;
  tok.perm = perm; tok.perm_h_stride = perm_per_head ? N : 0;
  KeyTok kt;
  kt.k = key; kt.f32 = key_dt == DBS_FP32; kt.sb = ksb; kt.sn = ksn; kt.sh = ksh;
  return estimate_impl(nullptr, nullptr, B, Hh, N, Npad, d, b, k, scale, p_imp, workspace, workspace_bytes, tok,
                       stream, &m, kt);
  DBS_GUARD_END
}

}  // extern "C"

// ---- the estimate-and-mask call without a workspace argument ----------------------------
// Its workspace is this array; each device holds its own copy at its own
// address.  In host code `scratch` names a host-side stand-in, never the
// device memory: only the address from hipGetSymbolAddress is passed on.
static __device__ __align__(256) unsigned char scratch[DBS_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;

// The device address of `scratch` on the device of `stream` (looked up once per
// device, with that device current).
dbs_status scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = stream != nullptr ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  REQUIRE(e == hipSuccess, DBS_ERR_HIP, "device of the stream: %s", hipGetErrorString(e));
  REQUIRE(dev >= 0 && dev < kMaxScratchDevices, DBS_ERR_UNSUPPORTED, "device %d: at most %d devices", dev,
          kMaxScratchDevices);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      int cur = -1;
      e = hipGetDevice(&cur);
      REQUIRE(e == hipSuccess, DBS_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
      if (cur != dev) {
        e = hipSetDevice(dev);
        REQUIRE(e == hipSuccess, DBS_ERR_HIP, "hipSetDevice(%d): %s", dev, hipGetErrorString(e));
      }
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
      REQUIRE(e == hipSuccess && p != nullptr, DBS_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
              hipGetErrorString(e));
      REQUIRE(e2 == hipSuccess, DBS_ERR_HIP, "hipSetDevice(%d): %s", cur, hipGetErrorString(e2));
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return DBS_OK;
}

}  // namespace

extern "C" {

dbs_status dbs_estimate_mask_tok_noalloc(const void* q, dbs_dtype q_dt, int64_t sb, int64_t sn, int64_t sh,
                                         const int32_t* perm, int perm_per_head, const void* k_r, int B, int Hh,
                                         int N, int Npad, int d, int b, int k, float scale, int rule, double param,
                                         float* p_imp, int32_t* kv_count, int32_t* kv_idx, uint8_t* mask,
                                         int32_t* order, hipStream_t stream) {
  DBS_GUARD_BEGIN
  dbs_status st = check_tok(q, q_dt, sb, sn, sh, perm, perm_per_head);
  if (st != DBS_OK) return st;
  dbs::MaskArgs m{};
  st = fuse_args(rule, param, kv_count, kv_idx, mask, order, Npad, b, m);
  if (st != DBS_OK) return st;
  st = check_geometry(B, Hh, N, Npad, d, b);
  if (st != DBS_OK) return st;
  const size_t need = dbs_estimate_workspace_bytes(B, Hh, N, d, b, k);
  REQUIRE(need <= DBS_NOALLOC_SCRATCH_BYTES, DBS_ERR_UNSUPPORTED,
          "this shape needs %zu bytes of scratch; the static scratch holds %zu (pass a workspace to "
          "dbs_estimate_mask_tok instead)",
          need, (size_t)DBS_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  st = scratch_address(stream, &ws);
  if (st != DBS_OK) return st;
  dbs::TokIO tok{};
  tok.q = q; tok.q_f32 = q_dt == DBS_FP32; tok.qsb = sb; tok.qsn = sn; tok.qsh = sh;
  tok.perm = perm; tok.perm_h_stride = perm_per_head ? N : 0;
  return estimate_impl(nullptr, k_r, B, Hh, N, Npad, d, b, k, scale, p_imp, ws, DBS_NOALLOC_SCRATCH_BYTES, tok,
                       stream, &m);
  DBS_GUARD_END
}

dbs_status dbs_build_mask(const float* p_imp, int B, int Hh, int nb, float tau, int32_t* kv_count,
                          int32_t* kv_idx, uint8_t* mask, int32_t* order, hipStream_t stream) {
  DBS_GUARD_BEGIN
  REQUIRE(p_imp && kv_count && kv_idx, DBS_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(((uintptr_t)p_imp & 3u) == 0 && ((uintptr_t)kv_count & 3u) == 0 && ((uintptr_t)kv_idx & 3u) == 0 &&
              ((uintptr_t)order & 3u) == 0,
          DBS_ERR_ALIGNMENT, "misaligned pointer");
  REQUIRE(B >= 1 && Hh >= 1, DBS_ERR_INVALID_ARG, "B and Hh must be >= 1");
  REQUIRE(nb >= 1 && nb <= 4096, DBS_ERR_UNSUPPORTED, "nb=%d must be in [1, 4096]", nb);
  REQUIRE(tau > 0.f && tau <= 1.f, DBS_ERR_INVALID_ARG, "tau=%g must be in (0, 1]", (double)tau);
  REQUIRE((int64_t)B * Hh * nb <= INT32_MAX, DBS_ERR_INVALID_ARG, "too many rows");
  dbs::MaskArgs a{};
  a.p_imp = p_imp; a.kv_count = kv_count; a.kv_idx = kv_idx; a.mask = mask; a.order = order;
  a.rows = B * Hh * nb; a.nb = nb; a.tau = tau; a.stream = stream;
  return from_hip(dbs::launch_build_mask(a), "dbs_build_mask launch");
  DBS_GUARD_END
}

dbs_status dbs_build_mask_rule(const float* p_imp, int B, int Hh, int nb, int rule, double param,
                               int32_t* kv_count, int32_t* kv_idx, uint8_t* mask, int32_t* order,
                               hipStream_t stream) {
  DBS_GUARD_BEGIN
  REQUIRE(p_imp && kv_count && kv_idx, DBS_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(((uintptr_t)p_imp & 3u) == 0 && ((uintptr_t)kv_count & 3u) == 0 && ((uintptr_t)kv_idx & 3u) == 0 &&
              ((uintptr_t)order & 3u) == 0,
          DBS_ERR_ALIGNMENT, "misaligned pointer");
  REQUIRE(B >= 1 && Hh >= 1, DBS_ERR_INVALID_ARG, "B and Hh must be >= 1");
  REQUIRE(nb >= 1 && nb <= 4096, DBS_ERR_UNSUPPORTED, "nb=%d must be in [1, 4096]", nb);
  REQUIRE((int64_t)B * Hh * nb <= INT32_MAX, DBS_ERR_INVALID_ARG, "too many rows");
  dbs::MaskArgs a{};
  a.p_imp = p_imp; a.kv_count = kv_count; a.kv_idx = kv_idx; a.mask = mask; a.order = order;
  a.rows = B * Hh * nb; a.nb = nb; a.stream = stream;
  dbs_status st = rule_args(rule, param, nb, a);
  if (st != DBS_OK) return st;
  return from_hip(dbs::launch_build_mask(a), "dbs_build_mask_rule launch");
  DBS_GUARD_END
}

dbs_status dbs_meanpool_kv(const void* k_r, const void* v_r, dbs_dtype dt, int B, int Hh, int N, int Npad,
                           int d, int b, int n, void* k_g, void* v_g, hipStream_t stream) {
  DBS_GUARD_BEGIN
  REQUIRE(k_r && v_r && k_g && v_g, DBS_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(aligned16(k_r) && aligned16(v_r) && aligned16(k_g) && aligned16(v_g), DBS_ERR_ALIGNMENT,
          "misaligned pointer");
  REQUIRE(dt == DBS_BF16, DBS_ERR_UNSUPPORTED, "meanpool_kv is bf16 only");
  dbs_status st = check_geometry(B, Hh, N, Npad, d, b);
  if (st != DBS_OK) return st;
  REQUIRE(n >= 1 && n <= N, DBS_ERR_INVALID_ARG, "pool window n=%d must be in [1, N]", n);
  dbs::MeanpoolArgs a{};
  a.k_r = k_r; a.v_t = v_r; a.k_g = k_g; a.v_g = v_g;
  a.B = B; a.Hh = Hh; a.N = N; a.Npad = Npad; a.d = d; a.b = b; a.n = n; a.Ng = (N + n - 1) / n;
  a.stream = stream;
  return from_hip(dbs::launch_meanpool(a), "dbs_meanpool_kv launch");
  DBS_GUARD_END
}

}  // extern "C"

namespace {

dbs_status attn_impl(const void* q_r, const void* k_r, const void* v_r, int B, int Hh, int N, int Npad, int d,
                     int b, float scale, const int32_t* kv_count, const int32_t* kv_idx, const int32_t* order,
                     const void* k_g, const void* v_g, int Ng, int n_pool, void* o_r, float* lse,
                     const dbs::TokIO& tok, hipStream_t stream, const int32_t* q_count = nullptr,
                     const int32_t* rowsel = nullptr, bool f32 = false) {
  REQUIRE(k_r && v_r && kv_count && kv_idx, DBS_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(aligned16(k_r) && aligned16(v_r), DBS_ERR_ALIGNMENT, "misaligned pointer");
  REQUIRE(((uintptr_t)kv_count & 3u) == 0 && ((uintptr_t)kv_idx & 3u) == 0 && ((uintptr_t)lse & 3u) == 0 &&
              ((uintptr_t)order & 3u) == 0,
          DBS_ERR_ALIGNMENT, "misaligned pointer");
  dbs_status st = check_geometry(B, Hh, N, Npad, d, b);
  if (st != DBS_OK) return st;
  REQUIRE(std::isfinite(scale), DBS_ERR_INVALID_ARG, "scale must be finite");
  REQUIRE((k_g == nullptr) == (v_g == nullptr), DBS_ERR_INVALID_ARG, "k_g and v_g must both be set or both NULL");
  if (k_g != nullptr) {
    REQUIRE(aligned16(k_g) && aligned16(v_g), DBS_ERR_ALIGNMENT, "misaligned pointer");
    REQUIRE(n_pool >= 1 && n_pool <= N, DBS_ERR_INVALID_ARG, "n_pool=%d must be in [1, N]", n_pool);
    REQUIRE(Ng == (N + n_pool - 1) / n_pool, DBS_ERR_INVALID_ARG, "Ng=%d must equal ceil(N/n_pool)=%d", Ng,
            (N + n_pool - 1) / n_pool);
  }
  dbs::AttnArgs a{};
  a.q_r = q_r; a.k_r = k_r; a.v_t = v_r; a.kv_count = kv_count; a.kv_idx = kv_idx; a.order = order;
  a.k_g = k_g; a.v_g = v_g; a.o_r = o_r; a.lse = lse;
  a.B = B; a.Hh = Hh; a.N = N; a.Npad = Npad; a.d = d; a.b = b; a.nb = Npad / b;
  a.Ng = k_g ? Ng : 0; a.n_pool = k_g ? n_pool : 1; a.scale = scale; a.tok = tok; a.stream = stream;
  a.q_count = q_count; a.rowsel = rowsel;
  REQUIRE(a.nb <= 4096, DBS_ERR_UNSUPPORTED, "nb=%d must be <= 4096", a.nb);
  REQUIRE((int64_t)B * Hh * a.nb <= INT32_MAX, DBS_ERR_INVALID_ARG, "too many query blocks");
  if (f32) return from_hip(dbs::launch_attn_fwd_f32(a), "dbs_sparse_attn_fwd launch");
  return from_hip(dbs::launch_attn_fwd(a), "dbs_sparse_attn_fwd launch");
}

}  // namespace

extern "C" {

dbs_status dbs_sparse_attn_fwd(const void* q_r, const void* k_r, const void* v_r, dbs_dtype dt, int B,
                               int Hh, int N, int Npad, int d, int b, float scale,
                               const int32_t* kv_count, const int32_t* kv_idx, const int32_t* order,
                               const void* k_g, const void* v_g, int Ng, int n_pool, void* o_r, float* lse,
                               hipStream_t stream) {
  DBS_GUARD_BEGIN
  REQUIRE(q_r && o_r, DBS_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(aligned16(q_r) && aligned16(o_r), DBS_ERR_ALIGNMENT, "misaligned pointer");
  REQUIRE(dt == DBS_BF16 || dt == DBS_FP32, DBS_ERR_INVALID_ARG, "bad dtype");
  if (dt == DBS_FP32) {
    REQUIRE(k_g == nullptr && v_g == nullptr, DBS_ERR_UNSUPPORTED, "float32 attention takes no global tokens");
    return attn_impl(q_r, k_r, v_r, B, Hh, N, Npad, d, b, scale, kv_count, kv_idx, order, nullptr, nullptr, 0, 0,
                     o_r, lse, dbs::TokIO{}, stream, nullptr, nullptr, true);
  }
  return attn_impl(q_r, k_r, v_r, B, Hh, N, Npad, d, b, scale, kv_count, kv_idx, order, k_g, v_g, Ng, n_pool,
                   o_r, lse, dbs::TokIO{}, stream);
  DBS_GUARD_END
}

dbs_status dbs_sparse_attn_fwd_tok(const void* q, dbs_dtype q_dt, int64_t qsb, int64_t qsn, int64_t qsh,
                                   const int32_t* perm, int perm_per_head, const void* k_r, const void* v_r,
                                   int B, int Hh, int N, int Npad, int d, int b, float scale,
                                   const int32_t* kv_count, const int32_t* kv_idx, const int32_t* order,
                                   const void* k_g, const void* v_g, int Ng, int n_pool, void* out,
                                   dbs_dtype out_dt, int64_t osb, int64_t osn, int64_t osh, float* lse,
                                   hipStream_t stream) {
  DBS_GUARD_BEGIN
  dbs_status st = check_tok(q, q_dt, qsb, qsn, qsh, perm, perm_per_head);
  if (st != DBS_OK) return st;
  st = check_tok(out, out_dt, osb, osn, osh, perm, perm_per_head);
  if (st != DBS_OK) return st;
  dbs::TokIO tok{};
  tok.q = q; tok.q_f32 = q_dt == DBS_FP32; tok.qsb = qsb; tok.qsn = qsn; tok.qsh = qsh;
  tok.out = out; tok.out_f32 = out_dt == DBS_FP32; tok.osb = osb; tok.osn = osn; tok.osh = osh;
  tok.perm = perm; tok.perm_h_stride = perm_per_head ? N : 0;
  return attn_impl(nullptr, k_r, v_r, B, Hh, N, Npad, d, b, scale, kv_count, kv_idx, order, k_g, v_g, Ng, n_pool,
                   nullptr, lse, tok, stream);
  DBS_GUARD_END
}

}  // extern "C"

extern "C" {

dbs_status dbs_query_prune(const void* q, dbs_dtype q_dt, int64_t sb, int64_t sn, int64_t sh, const int32_t* perm,
                           int perm_per_head, const int32_t* anchor, int B, int Hh, int N, int Npad, int d, int b,
                           double r, int32_t* q_count, int32_t* rowsel, uint8_t* keep, hipStream_t stream) {
  DBS_GUARD_BEGIN
  dbs_status st = check_tok(q, q_dt, sb, sn, sh, perm, perm_per_head);
  if (st != DBS_OK) return st;
  REQUIRE(anchor && q_count && rowsel && keep, DBS_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(((uintptr_t)anchor & 3u) == 0 && ((uintptr_t)q_count & 3u) == 0 && ((uintptr_t)rowsel & 3u) == 0,
          DBS_ERR_ALIGNMENT, "misaligned pointer");
  st = check_geometry(B, Hh, N, Npad, d, b);
  if (st != DBS_OK) return st;
  REQUIRE(std::isfinite(r) && r > 0.0 && r <= 1.0, DBS_ERR_INVALID_ARG, "keep ratio r=%g must be in (0, 1]", r);
  REQUIRE((int64_t)B * Hh * (Npad / b) <= INT32_MAX / 2, DBS_ERR_INVALID_ARG, "too many query blocks");
  dbs::PruneArgs a{};
  a.q = q; a.qsb = sb; a.qsn = sn; a.qsh = sh; a.q_f32 = q_dt == DBS_FP32;
  a.perm = perm; a.anchor = anchor; a.perm_h_stride = perm_per_head ? N : 0;
  a.B = B; a.Hh = Hh; a.N = N; a.Npad = Npad; a.d = d; a.b = b; a.nb = Npad / b; a.r = r;
  a.q_count = q_count; a.rowsel = rowsel; a.keep = keep; a.stream = stream;
  return from_hip(dbs::launch_query_prune(a), "dbs_query_prune launch");
  DBS_GUARD_END
}

dbs_status dbs_sparse_attn_fwd_pruned_tok(const void* q, dbs_dtype q_dt, int64_t qsb, int64_t qsn, int64_t qsh,
                                          const int32_t* perm, int perm_per_head, const void* k_r, const void* v_r,
                                          int B, int Hh, int N, int Npad, int d, int b, float scale,
                                          const int32_t* kv_count, const int32_t* kv_idx, const int32_t* order,
                                          const int32_t* q_count, const int32_t* rowsel, const int32_t* anchor,
                                          const uint8_t* keep, void* out, dbs_dtype out_dt, int64_t osb,
                                          int64_t osn, int64_t osh, float* lse, hipStream_t stream) {
  DBS_GUARD_BEGIN
  dbs_status st = check_tok(q, q_dt, qsb, qsn, qsh, perm, perm_per_head);
  if (st != DBS_OK) return st;
  st = check_tok(out, out_dt, osb, osn, osh, perm, perm_per_head);
  if (st != DBS_OK) return st;
  REQUIRE(q_count && rowsel && anchor && keep, DBS_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(((uintptr_t)q_count & 3u) == 0 && ((uintptr_t)rowsel & 3u) == 0 && ((uintptr_t)anchor & 3u) == 0,
          DBS_ERR_ALIGNMENT, "misaligned pointer");
  dbs::TokIO tok{};
  tok.q = q; tok.q_f32 = q_dt == DBS_FP32; tok.qsb = qsb; tok.qsn = qsn; tok.qsh = qsh;
  tok.out = out; tok.out_f32 = out_dt == DBS_FP32; tok.osb = osb; tok.osn = osn; tok.osh = osh;
  tok.perm = perm; tok.perm_h_stride = perm_per_head ? N : 0;
  st = attn_impl(nullptr, k_r, v_r, B, Hh, N, Npad, d, b, scale, kv_count, kv_idx, order, nullptr, nullptr, 0, 1,
                 nullptr, lse, tok, stream, q_count, rowsel);
  if (st != DBS_OK) return st;
  dbs::FillArgs f{};
  f.out = out; f.osb = osb; f.osn = osn; f.osh = osh; f.out_f32 = out_dt == DBS_FP32;
  f.row_bytes = d * (out_dt == DBS_FP32 ? 4 : 2);
  f.perm = perm; f.anchor = anchor; f.perm_h_stride = perm_per_head ? N : 0; f.keep = keep; f.lse = lse;
  f.B = B; f.Hh = Hh; f.N = N; f.Npad = Npad; f.stream = stream;
  return from_hip(dbs::launch_fill_pruned(f), "token filling launch");
  DBS_GUARD_END
}

size_t dbs_pooled_workspace_bytes(int B, int Hh, int N, int d, int b) {
  if (B < 1 || Hh < 1 || N < 1 || (d != 64 && d != 128) || (b != 64 && b != 128)) return 0;
  return dbs::pooled_workspace_bytes(B, Hh, (N + b - 1) / b, d);
}

dbs_status dbs_estimate_pooled_tok(const void* q, dbs_dtype q_dt, int64_t sb, int64_t sn, int64_t sh,
                                   const int32_t* perm, int perm_per_head, const void* k_r, int B, int Hh, int N,
                                   int Npad, int d, int b, int kind, float* p_imp, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  DBS_GUARD_BEGIN
  dbs_status st = check_tok(q, q_dt, sb, sn, sh, perm, perm_per_head);
  if (st != DBS_OK) return st;
  REQUIRE(k_r && p_imp && workspace, DBS_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(aligned16(k_r) && aligned16(p_imp) && aligned16(workspace), DBS_ERR_ALIGNMENT, "misaligned pointer");
  st = check_geometry(B, Hh, N, Npad, d, b);
  if (st != DBS_OK) return st;
  REQUIRE(kind == DBS_POOL_MEAN || kind == DBS_POOL_TRIP, DBS_ERR_INVALID_ARG, "unknown pooling kind %d", kind);
  const size_t need = dbs_pooled_workspace_bytes(B, Hh, N, d, b);
  REQUIRE(workspace_bytes >= need, DBS_ERR_INVALID_ARG, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  dbs::PooledArgs a{};
  a.k_r = k_r; a.p_imp = p_imp; a.workspace = workspace;
  a.tok.q = q; a.tok.q_f32 = q_dt == DBS_FP32; a.tok.qsb = sb; a.tok.qsn = sn; a.tok.qsh = sh;
  a.tok.perm = perm; a.tok.perm_h_stride = perm_per_head ? N : 0;
  a.B = B; a.Hh = Hh; a.N = N; a.Npad = Npad; a.d = d; a.b = b; a.nb = Npad / b; a.kind = kind;
  a.stream = stream;
  return from_hip(dbs::launch_pooled(a), "dbs_estimate_pooled_tok launch");
  DBS_GUARD_END
}

dbs_status dbs_sics_tok(const void* q, dbs_dtype q_dt, int64_t sb, int64_t sn, int64_t sh, const int32_t* perm,
                        int perm_per_head, int B, int Hh, int N, int Npad, int d, int b, float* sics,
                        float* as_out, hipStream_t stream) {
  DBS_GUARD_BEGIN
  dbs_status st = check_tok(q, q_dt, sb, sn, sh, perm, perm_per_head);
  if (st != DBS_OK) return st;
  REQUIRE(sics && as_out, DBS_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(((uintptr_t)sics & 3u) == 0 && ((uintptr_t)as_out & 3u) == 0, DBS_ERR_ALIGNMENT, "misaligned pointer");
  st = check_geometry(B, Hh, N, Npad, d, b);
  if (st != DBS_OK) return st;
  dbs::SicsArgs a{};
  a.tok.q = q; a.tok.q_f32 = q_dt == DBS_FP32; a.tok.qsb = sb; a.tok.qsn = sn; a.tok.qsh = sh;
  a.tok.perm = perm; a.tok.perm_h_stride = perm_per_head ? N : 0;
  a.sics = sics; a.as = as_out;
  a.B = B; a.Hh = Hh; a.N = N; a.Npad = Npad; a.d = d; a.b = b; a.nb = Npad / b; a.stream = stream;
  return from_hip(dbs::launch_sics(a), "dbs_sics_tok launch");
  DBS_GUARD_END
}

dbs_status dbs_sics_choose(const void* q, const void* k, dbs_dtype dt, int64_t sb, int64_t sn, int64_t sh,
                           const int32_t* perms, int n_cand, int B, int Hh, int N, int Npad, int d, int b,
                           float* block_scores, float* scores, int32_t* choice, hipStream_t stream) {
  DBS_GUARD_BEGIN
  dbs_status st = check_tok(q, dt, sb, sn, sh, perms, 0);
  if (st != DBS_OK) return st;
  REQUIRE(k == nullptr || aligned16(k), DBS_ERR_ALIGNMENT, "misaligned pointer");
  REQUIRE(block_scores && scores && choice, DBS_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(((uintptr_t)block_scores & 3u) == 0 && ((uintptr_t)scores & 3u) == 0 && ((uintptr_t)choice & 3u) == 0,
          DBS_ERR_ALIGNMENT, "misaligned pointer");
  REQUIRE(n_cand >= 1 && n_cand <= 64, DBS_ERR_INVALID_ARG, "n_cand=%d must be in [1, 64]", n_cand);
  st = check_geometry(B, Hh, N, Npad, d, b);
  if (st != DBS_OK) return st;
  dbs::SicsArgs a{};
  a.tok.q = q; a.tok.q_f32 = dt == DBS_FP32; a.tok.qsb = sb; a.tok.qsn = sn; a.tok.qsh = sh;
  a.tok.perm = perms; a.tok.perm_h_stride = 0;
  a.sics = block_scores; a.as = scores; a.choice = choice;
  a.k = k; a.perms = perms; a.n_cand = n_cand; a.tensors = k != nullptr ? 2 : 1;
  a.B = B; a.Hh = Hh; a.N = N; a.Npad = Npad; a.d = d; a.b = b; a.nb = Npad / b; a.stream = stream;
  return from_hip(dbs::launch_sics(a), "dbs_sics_choose launch");
  DBS_GUARD_END
}

double dbs_normal_quantile(double p) { return dbs::normal_quantile(p); }

dbs_status dbs_transpose_lists(const int32_t* kv_count, const int32_t* kv_idx, int B, int Hh, int nb,
                               int32_t* kvT_count, int32_t* kvT_idx, hipStream_t stream) {
  DBS_GUARD_BEGIN
  REQUIRE(kv_count && kv_idx && kvT_count && kvT_idx, DBS_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(((uintptr_t)kv_count & 3u) == 0 && ((uintptr_t)kv_idx & 3u) == 0 && ((uintptr_t)kvT_count & 3u) == 0 &&
              ((uintptr_t)kvT_idx & 3u) == 0,
          DBS_ERR_ALIGNMENT, "misaligned pointer");
  REQUIRE(B >= 1 && Hh >= 1 && nb >= 1, DBS_ERR_INVALID_ARG, "bad sizes");
  REQUIRE(nb <= 4096, DBS_ERR_UNSUPPORTED, "nb=%d must be <= 4096", nb);
  REQUIRE((int64_t)B * Hh * nb * nb <= ((int64_t)1 << 40), DBS_ERR_INVALID_ARG, "lists too large");
  dbs::TransposeListsArgs a{};
  a.kv_count = kv_count; a.kv_idx = kv_idx; a.kvT_count = kvT_count; a.kvT_idx = kvT_idx;
  a.B = B; a.Hh = Hh; a.nb = nb; a.stream = stream;
  return from_hip(dbs::launch_transpose_lists(a), "dbs_transpose_lists launch");
  DBS_GUARD_END
}

size_t dbs_attn_bwd_workspace_bytes(int B, int Hh, int Npad, int d) {
  if (B < 1 || Hh < 1 || Npad < 1 || (d != 64 && d != 128)) return 0;
  return dbs::attn_bwd_workspace_bytes(B, Hh, Npad, d);
}

dbs_status dbs_sparse_attn_bwd(const void* q_r, const void* k_r, const void* v_r, const void* o_r,
                               const void* do_r, const float* lse, int B, int Hh, int N, int Npad, int d, int b,
                               float scale, const int32_t* kv_count, const int32_t* kv_idx,
                               const int32_t* kvT_count, const int32_t* kvT_idx, float* dq_r, float* dk_r,
                               float* dv_r, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  DBS_GUARD_BEGIN
  REQUIRE(q_r && k_r && v_r && o_r && do_r && lse && kv_count && kv_idx && kvT_count && kvT_idx && dq_r && dk_r &&
              dv_r && workspace,
          DBS_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(aligned16(q_r) && aligned16(k_r) && aligned16(v_r) && aligned16(o_r) && aligned16(do_r) &&
              aligned16(dq_r) && aligned16(dk_r) && aligned16(dv_r) && aligned16(workspace),
          DBS_ERR_ALIGNMENT, "misaligned pointer");
  REQUIRE(((uintptr_t)lse & 3u) == 0 && ((uintptr_t)kv_count & 3u) == 0 && ((uintptr_t)kv_idx & 3u) == 0 &&
              ((uintptr_t)kvT_count & 3u) == 0 && ((uintptr_t)kvT_idx & 3u) == 0,
          DBS_ERR_ALIGNMENT, "misaligned pointer");
  dbs_status st = check_geometry(B, Hh, N, Npad, d, b);
  if (st != DBS_OK) return st;
  REQUIRE(std::isfinite(scale), DBS_ERR_INVALID_ARG, "scale must be finite");
  const int nb = Npad / b;
  REQUIRE(nb <= 4096, DBS_ERR_UNSUPPORTED, "nb=%d must be <= 4096", nb);
  REQUIRE((int64_t)B * Hh * nb <= INT32_MAX, DBS_ERR_INVALID_ARG, "too many blocks");
  const size_t need = dbs::attn_bwd_workspace_bytes(B, Hh, Npad, d);
  REQUIRE(workspace_bytes >= need, DBS_ERR_INVALID_ARG, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  dbs::AttnBwdArgs a{};
  a.q_r = q_r; a.k_r = k_r; a.v_r = v_r; a.o_r = o_r; a.do_r = do_r; a.lse = lse;
  a.kv_count = kv_count; a.kv_idx = kv_idx; a.kvT_count = kvT_count; a.kvT_idx = kvT_idx;
  a.dq = dq_r; a.dk = dk_r; a.dv = dv_r; a.workspace = workspace;
  a.B = B; a.Hh = Hh; a.N = N; a.Npad = Npad; a.d = d; a.b = b; a.nb = nb; a.scale = scale; a.stream = stream;
  return from_hip(dbs::launch_attn_bwd(a), "dbs_sparse_attn_bwd launch");
  DBS_GUARD_END
}

}  // extern "C"
