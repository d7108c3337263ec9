// C ABI of libcsa: argument validation, launch configuration, workspace
// sizing.  Every check runs before anything is enqueued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "../../include/csa.h"
#include "kernels.hpp"

namespace {

thread_local char g_err[512] = "";

csa_status_t fail(csa_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

csa_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) {
    g_err[0] = '\0';
    return CSA_OK;
  }
  return fail(CSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE(cond, ...)                                  \
  do {                                                      \
    if (!(cond)) return fail(CSA_ERR_INVALID_ARG, __VA_ARGS__); \
  } while (0)
#define REQUIRE_PTR(p)                                                       \
  do {                                                                       \
    if ((p) == nullptr) return fail(CSA_ERR_INVALID_ARG, "%s is NULL", #p);  \
    if (!aligned16(p)) return fail(CSA_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p); \
  } while (0)
#define OPT_PTR(p)                                                           \
  do {                                                                       \
    if ((p) != nullptr && !aligned16(p))                                     \
      return fail(CSA_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p);    \
  } while (0)

bool dtype_ok(csa_dtype_t dt) { return dt == CSA_F32 || dt == CSA_BF16 || dt == CSA_FP8 || dt == CSA_MXFP4; }
csa::Dt to_dt(csa_dtype_t dt) { return static_cast<csa::Dt>(static_cast<int>(dt)); }

csa_status_t compress_common(const void* x_a, const void* z_a, const void* x_b, const void* z_b,
                             const float* bias, void* out, int64_t B, int64_t n, int64_t D,
                             int64_t m, int64_t p0, int64_t n_raw, int64_t e0, int64_t e1,
                             int64_t out_ld, csa_dtype_t dt, void* stream) {
  REQUIRE(dtype_ok(dt), "unknown dtype %d", static_cast<int>(dt));
  REQUIRE(B >= 0 && n >= 1 && m >= 1 && D >= 8 && D % 8 == 0,
          "need B >= 0, n >= 1, m >= 1, D a positive multiple of 8 (B=%lld n=%lld m=%lld D=%lld)",
          (long long)B, (long long)n, (long long)m, (long long)D);
  REQUIRE(dt != CSA_MXFP4 || D % 32 == 0, "MXFP4 entries need D a multiple of 32 (D=%lld)", (long long)D);
  const int64_t L = (n + m - 1) / m;
  REQUIRE(e0 >= 0 && e0 <= e1 && e1 <= L, "entry range [%lld, %lld) outside [0, %lld]",
          (long long)e0, (long long)e1, (long long)L);
  REQUIRE(out_ld >= e1 - e0, "out_ld %lld < e1-e0", (long long)out_ld);
  REQUIRE((x_b == nullptr) == (z_b == nullptr), "x_b and z_b must both be given or both be NULL");
  if (B == 0 || e1 == e0) return CSA_OK;
  REQUIRE_PTR(x_a);
  REQUIRE_PTR(z_a);
  OPT_PTR(x_b);
  OPT_PTR(z_b);
  REQUIRE_PTR(out);
  if (bias != nullptr && (reinterpret_cast<uintptr_t>(bias) & 3u))
    return fail(CSA_ERR_INVALID_ARG, "bias is not 4-byte aligned");
  const bool two = x_b != nullptr;
  const int64_t lo = (two && e0 >= 1) ? (e0 - 1) * m : e0 * m;
  const int64_t hi = e1 * m < n ? e1 * m : n;
  REQUIRE(p0 >= 0 && n_raw >= 0 && p0 <= lo && p0 + n_raw >= hi && p0 + n_raw <= n,
          "raw rows [%lld, %lld) do not cover the positions [%lld, %lld) the entries read",
          (long long)p0, (long long)(p0 + n_raw), (long long)lo, (long long)hi);
  csa::CompressArgs a{x_a, z_a, x_b, z_b, bias, out, B, n, D, m, p0, n_raw, e0, e1, out_ld};
  return hip_status(csa::launch_compress(a, to_dt(dt), static_cast<hipStream_t>(stream)),
                    "compress launch");
}

csa_status_t index_common(const void* q_idx, const float* w_idx, const void* k_idx, int64_t B,
                          int64_t T, int64_t n_ctx, int64_t L, int64_t HI, int64_t dI, int64_t m,
                          csa_dtype_t dt) {
  REQUIRE(dtype_ok(dt), "unknown dtype %d", static_cast<int>(dt));
  REQUIRE(B >= 0 && T >= 1 && n_ctx >= T && L >= 0 && m >= 1 && HI >= 1 && dI >= 1,
          "need B >= 0, 1 <= T <= n_ctx, L >= 0, m >= 1, H_I >= 1, d_I >= 1");
  if (!csa::index_shape_supported(HI, dI, to_dt(dt)))
    return fail(CSA_ERR_UNSUPPORTED, "no indexer kernel for H_I=%lld d_I=%lld dtype=%d", (long long)HI,
                (long long)dI, static_cast<int>(dt));
  if (B == 0) return CSA_OK;
  REQUIRE_PTR(q_idx);
  if (L > 0) REQUIRE_PTR(k_idx);
  if (w_idx != nullptr && (reinterpret_cast<uintptr_t>(w_idx) & 3u))
    return fail(CSA_ERR_INVALID_ARG, "w_idx is not 4-byte aligned");
  return CSA_OK;
}

csa_status_t attn_common(const void* q, const void* kc, const void* vc, int64_t L, const void* kr,
                         const void* vr, int64_t R, int64_t W, const float* sink, float scale,
                         int64_t B, int64_t T, int64_t n_ctx, int64_t H, int64_t d, void* out,
                         float* lse, csa_dtype_t dt) {
  REQUIRE(dtype_ok(dt), "unknown dtype %d", static_cast<int>(dt));
  if (dt == CSA_MXFP4) return fail(CSA_ERR_UNSUPPORTED, "attention has no MXFP4 kernels");
  REQUIRE(B >= 0 && T >= 1 && n_ctx >= T && L >= 0 && H >= 1 && d >= 1 && W >= 0,
          "need B >= 0, 1 <= T <= n_ctx, L >= 0, H >= 1, d >= 1, W >= 0");
  REQUIRE(std::isfinite(scale), "scale is not finite");
  REQUIRE(L <= (int64_t(1) << 30) && R <= (int64_t(1) << 30) && W <= (int64_t(1) << 30),
          "L, R and W must not exceed 2^30 rows");
  if (!csa::attn_shape_supported(H, d, to_dt(dt)))
    return fail(CSA_ERR_UNSUPPORTED, "no attention kernel for H=%lld d=%lld dtype=%d", (long long)H,
                (long long)d, static_cast<int>(dt));
  if (W > 0) {
    REQUIRE(R >= T + W - 1 || R == n_ctx, "window needs R >= T+W-1 raw rows (R=%lld)", (long long)R);
    REQUIRE(R <= n_ctx, "R=%lld exceeds n_ctx", (long long)R);
  }
  if (B == 0) return CSA_OK;
  REQUIRE_PTR(q);
  REQUIRE_PTR(out);
  if (L > 0) {
    REQUIRE_PTR(kc);
    REQUIRE_PTR(vc);
  }
  if (W > 0) {
    REQUIRE_PTR(kr);
    REQUIRE_PTR(vr);
  }
  if (sink != nullptr && (reinterpret_cast<uintptr_t>(sink) & 3u))
    return fail(CSA_ERR_INVALID_ARG, "sink is not 4-byte aligned");
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(CSA_ERR_INVALID_ARG, "lse is not 4-byte aligned");
  return CSA_OK;
}

int64_t dense_max_rows(int64_t L, int64_t m, int64_t n_ctx, int64_t W) {
  int64_t nv = (n_ctx - 1) / m;
  if (nv > L) nv = L;
  return nv + W;
}

// Checks a serving layout against a call (L: cache capacity in entries; W, R:
// window) and converts it; NULL is the plain layout.
csa_status_t layout_from(const csa_layout_t* l, int64_t T, int64_t L, int64_t W, int64_t R, csa::SeqLayout* out) {
  *out = csa::SeqLayout{};
  if (l == nullptr) return CSA_OK;
  if (l->seq_len != nullptr) {
    REQUIRE((reinterpret_cast<uintptr_t>(l->seq_len) & 7u) == 0, "layout seq_len is not 8-byte aligned");
    out->lens = l->seq_len;
  }
  if (l->block_table != nullptr) {
    REQUIRE((reinterpret_cast<uintptr_t>(l->block_table) & 3u) == 0, "layout block_table is not 4-byte aligned");
    REQUIRE(l->page >= 16 && l->page % 16 == 0 && l->page <= (int64_t(1) << 30),
            "layout page=%lld must be a positive multiple of 16", (long long)l->page);
    REQUIRE(l->num_pages >= 1 && l->num_pages <= ((int64_t(1) << 31) - 1) / l->page,
            "layout num_pages=%lld: the pool must hold fewer than 2^31 rows", (long long)l->num_pages);
    REQUIRE(l->bt_stride >= (L + l->page - 1) / l->page, "layout bt_stride=%lld below ceil(L / page)",
            (long long)l->bt_stride);
    out->bt = l->block_table;
    out->bt_ld = l->bt_stride;
    out->page = l->page;
    out->npages = l->num_pages;
  }
  REQUIRE(l->window_ring == 0 || l->window_ring == 1, "layout window_ring must be 0 or 1");
  if (l->window_ring) {
    if (W > 0) REQUIRE(R >= T + W - 1 && R >= W, "a ring window needs R >= T+W-1 and R >= W (R=%lld)", (long long)R);
    out->ring = 1;
  }
  return CSA_OK;
}

}  // namespace

extern "C" {

csa_status_t csa_compress(const void* x_a, const void* z_a, const void* x_b, const void* z_b,
                          const float* bias, void* out, int64_t B, int64_t n, int64_t D, int64_t m,
                          int64_t p0, int64_t n_raw, int64_t e0, int64_t e1, int64_t out_ld,
                          csa_dtype_t dtype, void* stream) {
  return compress_common(x_a, z_a, x_b, z_b, bias, out, B, n, D, m, p0, n_raw, e0, e1, out_ld, dtype,
                         stream);
}

csa_status_t hca_compress(const void* x, const void* z, const float* bias, void* out, int64_t B,
                          int64_t n, int64_t D, int64_t m, int64_t p0, int64_t n_raw, int64_t e0,
                          int64_t e1, int64_t out_ld, csa_dtype_t dtype, void* stream) {
  return compress_common(x, z, nullptr, nullptr, bias, out, B, n, D, m, p0, n_raw, e0, e1, out_ld,
                         dtype, stream);
}

csa_status_t csa_index_score(const void* q_idx, const float* w_idx, const void* k_idx, int64_t B,
                             int64_t T, int64_t n_ctx, int64_t L, int64_t H_I, int64_t d_I,
                             int64_t m, float* score, csa_dtype_t dtype, void* stream) {
  csa_status_t st = index_common(q_idx, w_idx, k_idx, B, T, n_ctx, L, H_I, d_I, m, dtype);
  if (st != CSA_OK || B == 0 || L == 0) return st;
  REQUIRE_PTR(score);
  csa::IndexScoreArgs a{q_idx, w_idx, k_idx, score, L, 0, B * T, B, T, n_ctx, L, H_I, d_I, m, to_dt(dtype)};
  return hip_status(csa::launch_index_score(a, static_cast<hipStream_t>(stream)), "index score launch");
}

size_t csa_topk_select_workspace(int64_t B, int64_t T, int64_t L, int64_t k) {
  if (B <= 0 || T <= 0 || k <= 0) return 0;
  return static_cast<size_t>(B) * T * csa::topk_ws_bytes_per_row(L, k);
}

csa_status_t csa_topk_select(const float* score, int64_t B, int64_t T, int64_t n_ctx, int64_t L,
                             int64_t m, int64_t k, int32_t* idx, float* out_score, void* ws,
                             size_t ws_bytes, void* stream) {
  REQUIRE(B >= 0 && T >= 1 && n_ctx >= T && L >= 0 && m >= 1, "need B >= 0, 1 <= T <= n_ctx, L >= 0, m >= 1");
  REQUIRE(k >= 1 && k <= (1 << 20), "k=%lld outside [1, 2^20]", (long long)k);
  if (B == 0) return CSA_OK;
  if (L > 0) REQUIRE_PTR(score);
  REQUIRE_PTR(idx);
  OPT_PTR(out_score);
  const size_t need = csa_topk_select_workspace(B, T, L, k);
  if (ws == nullptr || ws_bytes < need)
    return fail(CSA_ERR_WORKSPACE, "top-k needs %zu workspace bytes, got %zu", need, ws_bytes);
  if (!aligned16(ws)) return fail(CSA_ERR_INVALID_ARG, "ws is not 16-byte aligned");
  csa::TopkArgs a{score, L, 0, B * T, T, n_ctx, L, m, k, idx, out_score};
  return hip_status(csa::launch_topk(a, ws, static_cast<hipStream_t>(stream)), "top-k launch");
}

static size_t index_topk_row_bytes(int64_t L, int64_t k) {
  const size_t sc = (static_cast<size_t>(L > 0 ? L : 0) * sizeof(float) + 255) / 256 * 256;
  return sc + csa::topk_ws_bytes_per_row(L, k);
}

size_t csa_index_topk_workspace(int64_t B, int64_t T, int64_t L, int64_t H_I, int64_t k) {
  (void)H_I;
  if (B <= 0 || T <= 0 || k <= 0) return 0;
  const size_t chunked = static_cast<size_t>(B) * T * index_topk_row_bytes(L, k);
  const size_t fused = L > 0 ? csa::index_topk_fused_ws_bytes(B * T, L, k) : 0;
  const size_t listed = L > 0 ? csa::index_topk_listed_ws_bytes(B * T, L, k) : 0;
  const size_t most = chunked > fused ? chunked : fused;
  return most > listed ? most : listed;
}

}  // extern "C"

namespace {

// Validation shared by csa_index_topk and csa_index_topk_noalloc.
csa_status_t index_topk_check(const void* q_idx, const float* w_idx, const void* k_idx, int64_t B, int64_t T,
                              int64_t n_ctx, int64_t L, int64_t H_I, int64_t d_I, int64_t m, int64_t k,
                              int32_t* idx, float* out_score, csa_dtype_t dtype) {
  csa_status_t st = index_common(q_idx, w_idx, k_idx, B, T, n_ctx, L, H_I, d_I, m, dtype);
  if (st != CSA_OK) return st;
  REQUIRE(k >= 1 && k <= (1 << 20), "k=%lld outside [1, 2^20]", (long long)k);
  if (B == 0) return CSA_OK;
  REQUIRE_PTR(idx);
  OPT_PTR(out_score);
  return CSA_OK;
}

// Index + top-k with a validated call and a workspace of ws_bytes at ws (the
// caller's, or the static scratch of the allocation-free entry point).
csa_status_t index_topk_run(const csa::SeqLayout& lay, const void* q_idx, const float* w_idx, const void* k_idx,
                            int64_t B, int64_t T, int64_t n_ctx, int64_t L, int64_t H_I, int64_t d_I, int64_t m,
                            int64_t k, int32_t* idx, float* out_score, void* ws, size_t ws_bytes, csa_dtype_t dtype,
                            void* stream) {
  csa_status_t st = CSA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t rows = B * T;
  // Many queries per sequence (prefill): the 16-row scoring kernel reads each
  // key once per 16 queries; it writes scores, so the stand-alone top-k follows.
  const bool multi = (dtype == CSA_BF16 || dtype == CSA_FP8 || dtype == CSA_MXFP4) && d_I == 128 && !lay.bt &&
                     csa::index_multi_rows(T, H_I, 0, rows);
  if (!multi && ws != nullptr && L > 0 && csa::index_topk_fusable(rows, L, H_I, d_I, k, to_dt(dtype)) &&
      ws_bytes >= csa::index_topk_fused_ws_bytes(rows, L, k)) {
    // The scan's workgroups keep their parts' candidates; no score matrix.
    if (!aligned16(ws)) return fail(CSA_ERR_INVALID_ARG, "ws is not 16-byte aligned");
    csa::IndexScoreArgs a{q_idx, w_idx, k_idx, nullptr, L, 0, rows, B, T, n_ctx, L, H_I, d_I, m, to_dt(dtype), lay};
    csa::TopkArgs t{nullptr, L, 0, rows, T, n_ctx, L, m, k, idx, out_score, lay.lens};
    return hip_status(csa::launch_index_topk_fused(a, t, ws, s), "fused index/top-k launch");
  }
  if (!multi && ws != nullptr && L > 0 && csa::index_topk_listable(rows, L, H_I, d_I, k, to_dt(dtype)) &&
      ws_bytes >= csa::index_topk_listed_ws_bytes(rows, L, k)) {
    // More parts than the fused path takes: scores plus exact per-part lists,
    // a list merge per row, the stand-alone top-k only for unsettled rows.
    if (!aligned16(ws)) return fail(CSA_ERR_INVALID_ARG, "ws is not 16-byte aligned");
    csa::IndexScoreArgs a{q_idx, w_idx, k_idx, nullptr, L, 0, rows, B, T, n_ctx, L, H_I, d_I, m, to_dt(dtype), lay};
    csa::TopkArgs t{nullptr, L, 0, rows, T, n_ctx, L, m, k, idx, out_score, lay.lens};
    return hip_status(csa::launch_index_topk_listed(a, t, ws, s), "listed index/top-k launch");
  }
  const size_t per_row = index_topk_row_bytes(L, k);
  if (ws == nullptr || ws_bytes < per_row)
    return fail(CSA_ERR_WORKSPACE, "workspace of %zu bytes is below the one-query minimum %zu", ws_bytes, per_row);
  if (!aligned16(ws)) return fail(CSA_ERR_INVALID_ARG, "ws is not 16-byte aligned");
  int64_t chunk = static_cast<int64_t>(ws_bytes / per_row);
  if (chunk > rows) chunk = rows;
  if (multi && chunk >= 16) chunk -= chunk % 16;  // keep the 16-row blocks whole
  const size_t sc_bytes = (static_cast<size_t>(chunk) * (L > 0 ? L : 0) * sizeof(float) + 255) / 256 * 256;
  float* sc = static_cast<float*>(ws);
  void* sel_ws = static_cast<char*>(ws) + sc_bytes;
  for (int64_t r0 = 0; r0 < rows; r0 += chunk) {
    const int64_t nr = r0 + chunk < rows ? chunk : rows - r0;
    if (L > 0) {
      csa::IndexScoreArgs a{q_idx, w_idx, k_idx, sc, L, r0, nr, B, T, n_ctx, L, H_I, d_I, m, to_dt(dtype), lay};
      st = hip_status(csa::launch_index_score(a, s), "index score launch");
      if (st != CSA_OK) return st;
    }
    csa::TopkArgs t{sc, L, r0, nr, T, n_ctx, L, m, k, idx + r0 * k,
                    out_score ? out_score + r0 * k : nullptr, lay.lens};
    st = hip_status(csa::launch_topk(t, sel_ws, s), "top-k launch");
    if (st != CSA_OK) return st;
  }
  return CSA_OK;
}

// Static scratch of the allocation-free index + top-k: one array per device
// (the code object's globals are per device), zero at load.  Host code uses
// the per-device address from hipGetSymbolAddress, never the array's name.
constexpr size_t kScratchBytes = size_t(32) << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of `scratch` on the calling thread's current device, looked up on
// the first call made on that device.
csa_status_t scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(CSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(CSA_ERR_UNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(CSA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CSA_OK;
}

}  // namespace

extern "C" {

csa_status_t csa_index_topk(const void* q_idx, const float* w_idx, const void* k_idx, int64_t B,
                            int64_t T, int64_t n_ctx, int64_t L, int64_t H_I, int64_t d_I, int64_t m,
                            int64_t k, int32_t* idx, float* out_score, void* ws, size_t ws_bytes,
                            csa_dtype_t dtype, void* stream) {
  const csa_status_t st = index_topk_check(q_idx, w_idx, k_idx, B, T, n_ctx, L, H_I, d_I, m, k, idx, out_score,
                                           dtype);
  if (st != CSA_OK || B == 0) return st;
  return index_topk_run(csa::SeqLayout{}, q_idx, w_idx, k_idx, B, T, n_ctx, L, H_I, d_I, m, k, idx, out_score, ws,
                        ws_bytes, dtype, stream);
}

csa_status_t csa_index_topk_ex(const csa_layout_t* layout, const void* q_idx, const float* w_idx,
                               const void* k_idx, int64_t B, int64_t T, int64_t n_ctx, int64_t L, int64_t H_I,
                               int64_t d_I, int64_t m, int64_t k, int32_t* idx, float* out_score, void* ws,
                               size_t ws_bytes, csa_dtype_t dtype, void* stream) {
  csa_status_t st = index_topk_check(q_idx, w_idx, k_idx, B, T, n_ctx, L, H_I, d_I, m, k, idx, out_score, dtype);
  if (st != CSA_OK) return st;
  csa::SeqLayout lay;
  st = layout_from(layout, T, L, 0, 0, &lay);
  if (st != CSA_OK || B == 0) return st;
  return index_topk_run(lay, q_idx, w_idx, k_idx, B, T, n_ctx, L, H_I, d_I, m, k, idx, out_score, ws, ws_bytes,
                        dtype, stream);
}

size_t csa_index_topk_noalloc_max_bytes(void) { return kScratchBytes; }

csa_status_t csa_index_topk_noalloc(const void* q_idx, const float* w_idx, const void* k_idx, int64_t B,
                                    int64_t T, int64_t n_ctx, int64_t L, int64_t H_I, int64_t d_I, int64_t m,
                                    int64_t k, int32_t* idx, float* out_score, csa_dtype_t dtype,
                                    void* stream) {
  csa_status_t st = index_topk_check(q_idx, w_idx, k_idx, B, T, n_ctx, L, H_I, d_I, m, k, idx, out_score, dtype);
  if (st != CSA_OK || B == 0) return st;
  // The scratch must hold at least one query row (its scores and selection
  // state); larger calls are processed in groups of rows that fit.
  const size_t one_row = index_topk_row_bytes(L, k);
  if (one_row > kScratchBytes)
    return fail(CSA_ERR_UNSUPPORTED,
                "one query row of L=%lld, k=%lld needs %zu bytes of scratch; the static scratch holds %zu",
                (long long)L, (long long)k, one_row, kScratchBytes);
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != CSA_OK) return st;
  return index_topk_run(csa::SeqLayout{}, q_idx, w_idx, k_idx, B, T, n_ctx, L, H_I, d_I, m, k, idx, out_score, ws,
                        kScratchBytes, dtype, stream);
}

size_t csa_sparse_attn_workspace(int64_t B, int64_t T, int64_t H, int64_t d, int64_t k, int64_t W,
                                 csa_dtype_t dtype) {
  if (B <= 0 || T <= 0) return 0;
  const int ns = csa::attn_splits(B, T, H, d, k + W, to_dt(dtype), true);
  return csa::attn_ws_bytes(B, T, H, d, ns);
}

size_t hca_dense_attn_workspace(int64_t B, int64_t T, int64_t H, int64_t d, int64_t L, int64_t m,
                                int64_t n_ctx, int64_t W, csa_dtype_t dtype) {
  if (B <= 0 || T <= 0 || m <= 0) return 0;
  const int ns = csa::attn_splits(B, T, H, d, dense_max_rows(L, m, n_ctx, W), to_dt(dtype), false);
  return csa::attn_ws_bytes(B, T, H, d, ns);
}

size_t csa_attn_workspace(int64_t B, int64_t T, int64_t H, int64_t d, int64_t n_rows) {
  if (B <= 0 || T <= 0 || n_rows < 0) return 0;
  // The split plan depends on the row count and on whether rows are gathered;
  // the bf16 plan covers FP8 too, and fp32 needs none.
  const int ns_s = csa::attn_splits(B, T, H, d, n_rows, csa::kBF16, true);
  const int ns_d = csa::attn_splits(B, T, H, d, n_rows, csa::kBF16, false);
  const size_t a = csa::attn_ws_bytes(B, T, H, d, ns_s), b = csa::attn_ws_bytes(B, T, H, d, ns_d);
  return a > b ? a : b;
}

static csa_status_t attn_launch(const csa::AttnArgs& a, bool sparse, int64_t max_rows, csa_dtype_t dt,
                                void* ws, size_t ws_bytes, void* stream) {
  // MFMA kernels cache gathered rows as 32-bit cache-row numbers
  if (dt != CSA_F32 && sparse && !a.lay.bt && a.B * a.L >= (int64_t(1) << 31))
    return fail(CSA_ERR_UNSUPPORTED, "B * L = %lld cache rows exceed 2^31", (long long)(a.B * a.L));
  const int ns = csa::attn_splits(a.B, a.T, a.H, a.d, max_rows, to_dt(dt), sparse);
  const size_t need = csa::attn_ws_bytes(a.B, a.T, a.H, a.d, ns);
  if (need > 0) {
    if (ws == nullptr || ws_bytes < need)
      return fail(CSA_ERR_WORKSPACE, "attention needs %zu workspace bytes, got %zu", need, ws_bytes);
    if (!aligned16(ws)) return fail(CSA_ERR_INVALID_ARG, "ws is not 16-byte aligned");
  }
  csa::AttnArgs b = a;
  b.ws = static_cast<float*>(ws);
  b.ws_bytes = ws_bytes;
  return hip_status(csa::launch_attn(b, sparse, to_dt(dt), ns, static_cast<hipStream_t>(stream)),
                    "attention launch");
}

csa_status_t csa_sparse_attn_ex(const csa_layout_t* layout, const void* q, const void* kc, const void* vc, int64_t L,
                                const int32_t* idx, int64_t k, const void* kr, const void* vr, int64_t R,
                                int64_t W, const float* sink, float scale, int64_t B, int64_t T,
                                int64_t n_ctx, int64_t H, int64_t d, void* out, float* lse, void* ws,
                                size_t ws_bytes, csa_dtype_t dtype, void* stream) {
  csa_status_t st = attn_common(q, kc, vc, L, kr, vr, R, W, sink, scale, B, T, n_ctx, H, d, out, lse, dtype);
  if (st != CSA_OK) return st;
  csa::SeqLayout lay;
  st = layout_from(layout, T, L, W, R, &lay);
  if (st != CSA_OK) return st;
  REQUIRE(k >= 0, "k < 0");
  if (dtype != CSA_F32 && k + W > csa::kAttnMaxRows)
    return fail(CSA_ERR_UNSUPPORTED, "MFMA sparse attention supports k + W <= %lld rows (got %lld)",
                (long long)csa::kAttnMaxRows, (long long)(k + W));
  if (B == 0) return CSA_OK;
  if (k > 0) REQUIRE_PTR(idx);
  csa::AttnArgs a{q, kc, vc, L, 1, idx, k, kr, vr, R, W, sink, scale, B, T, n_ctx, H, d, out, lse,
                  nullptr, 0, lay};
  return attn_launch(a, true, k + W, dtype, ws, ws_bytes, stream);
}

csa_status_t csa_sparse_attn(const void* q, const void* kc, const void* vc, int64_t L,
                             const int32_t* idx, int64_t k, const void* kr, const void* vr, int64_t R,
                             int64_t W, const float* sink, float scale, int64_t B, int64_t T,
                             int64_t n_ctx, int64_t H, int64_t d, void* out, float* lse, void* ws,
                             size_t ws_bytes, csa_dtype_t dtype, void* stream) {
  return csa_sparse_attn_ex(nullptr, q, kc, vc, L, idx, k, kr, vr, R, W, sink, scale, B, T, n_ctx, H, d, out, lse,
                            ws, ws_bytes, dtype, stream);
}

csa_status_t hca_dense_attn_ex(const csa_layout_t* layout, const void* q, const void* kc, const void* vc, int64_t L,
                               int64_t m, const void* kr, const void* vr, int64_t R, int64_t W, const float* sink,
                               float scale, int64_t B, int64_t T, int64_t n_ctx, int64_t H, int64_t d,
                               void* out, float* lse, void* ws, size_t ws_bytes, csa_dtype_t dtype,
                               void* stream) {
  csa_status_t st = attn_common(q, kc, vc, L, kr, vr, R, W, sink, scale, B, T, n_ctx, H, d, out, lse, dtype);
  if (st != CSA_OK) return st;
  REQUIRE(m >= 1, "m < 1");
  csa::SeqLayout lay;
  st = layout_from(layout, T, L, W, R, &lay);
  if (st != CSA_OK) return st;
  const int64_t rows = dense_max_rows(L, m, n_ctx, W);
  if (dtype != CSA_F32 && lay.bt && rows > csa::kAttnMaxRows)
    return fail(CSA_ERR_UNSUPPORTED, "paged dense attention supports at most %lld rows per query (got %lld)",
                (long long)csa::kAttnMaxRows, (long long)rows);
  if (B == 0) return CSA_OK;
  csa::AttnArgs a{q, kc, vc, L, m, nullptr, 0, kr, vr, R, W, sink, scale, B, T, n_ctx, H, d, out, lse,
                  nullptr, 0, lay};
  // A paged cache is read through the gathering kernel, over the implicit
  // list of every visible entry.
  return attn_launch(a, lay.bt != nullptr, rows, dtype, ws, ws_bytes, stream);
}

csa_status_t hca_dense_attn(const void* q, const void* kc, const void* vc, int64_t L, int64_t m,
                            const void* kr, const void* vr, int64_t R, int64_t W, const float* sink,
                            float scale, int64_t B, int64_t T, int64_t n_ctx, int64_t H, int64_t d,
                            void* out, float* lse, void* ws, size_t ws_bytes, csa_dtype_t dtype,
                            void* stream) {
  return hca_dense_attn_ex(nullptr, q, kc, vc, L, m, kr, vr, R, W, sink, scale, B, T, n_ctx, H, d, out, lse, ws,
                           ws_bytes, dtype, stream);
}

csa_status_t csa_compress_append(const csa_layout_t* layout, const void* x_a, const void* z_a, const void* x_b,
                                 const void* z_b, const float* bias, void* ring_xa, void* ring_za, void* ring_xb,
                                 void* ring_zb, int64_t S, const int64_t* pos, void* cache, int64_t L, int64_t B,
                                 int64_t D, int64_t m, csa_dtype_t dtype, void* stream) {
  REQUIRE(dtype_ok(dtype), "unknown dtype %d", static_cast<int>(dtype));
  REQUIRE(B >= 0 && m >= 1 && L >= 0 && D >= 8 && D % 8 == 0,
          "need B >= 0, m >= 1, L >= 0, D a positive multiple of 8");
  REQUIRE(dtype != CSA_MXFP4 || D % 32 == 0, "MXFP4 entries need D a multiple of 32 (D=%lld)", (long long)D);
  REQUIRE((x_b == nullptr) == (z_b == nullptr), "x_b and z_b must both be given or both be NULL");
  const bool two = x_b != nullptr;
  REQUIRE(S >= (two ? 2 * m : m), "staging rings of %lld rows: need at least %lld", (long long)S,
          (long long)(two ? 2 * m : m));
  csa::SeqLayout lay;
  csa_status_t st = layout_from(layout, 1, L, 0, 0, &lay);
  if (st != CSA_OK) return st;
  if (B == 0) return CSA_OK;
  REQUIRE_PTR(x_a);
  REQUIRE_PTR(z_a);
  REQUIRE_PTR(ring_xa);
  REQUIRE_PTR(ring_za);
  if (two) {
    REQUIRE_PTR(x_b);
    REQUIRE_PTR(z_b);
    REQUIRE_PTR(ring_xb);
    REQUIRE_PTR(ring_zb);
  }
  REQUIRE_PTR(pos);
  if (L > 0) REQUIRE_PTR(cache);
  if (bias != nullptr && (reinterpret_cast<uintptr_t>(bias) & 3u))
    return fail(CSA_ERR_INVALID_ARG, "bias is not 4-byte aligned");
  csa::CompressArgs a{x_a, z_a, x_b, z_b, bias, cache, B, int64_t(1) << 62, D, m, 0, S, 0, 0, L};
  a.pos = pos;
  a.ring_xa = ring_xa;
  a.ring_za = ring_za;
  a.ring_xb = ring_xb;
  a.ring_zb = ring_zb;
  a.lay = lay;
  return hip_status(csa::launch_compress_append(a, to_dt(dtype), static_cast<hipStream_t>(stream)),
                    "compress append launch");
}

csa_status_t csa_window_append(const void* k_new, const void* v_new, void* kr, void* vr, const int64_t* pos,
                               int64_t B, int64_t R, int64_t d, csa_dtype_t dtype, void* stream) {
  REQUIRE(dtype == CSA_F32 || dtype == CSA_BF16 || dtype == CSA_FP8, "window rows are fp32, bf16 or FP8");
  REQUIRE(B >= 0 && R >= 1 && d >= 1, "need B >= 0, R >= 1, d >= 1");
  const int64_t eb = dtype == CSA_F32 ? 4 : (dtype == CSA_BF16 ? 2 : 1);
  REQUIRE((d * eb) % 16 == 0, "a row of d=%lld elements must be a multiple of 16 bytes", (long long)d);
  if (B == 0) return CSA_OK;
  REQUIRE_PTR(k_new);
  REQUIRE_PTR(v_new);
  REQUIRE_PTR(kr);
  REQUIRE_PTR(vr);
  REQUIRE_PTR(pos);
  return hip_status(csa::launch_window_append(k_new, v_new, kr, vr, pos, B, R, d * eb,
                                              static_cast<hipStream_t>(stream)),
                    "window append launch");
}

const char* csa_status_string(csa_status_t status) {
  switch (status) {
    case CSA_OK: return "CSA_OK";
    case CSA_ERR_INVALID_ARG: return "CSA_ERR_INVALID_ARG";
    case CSA_ERR_UNSUPPORTED: return "CSA_ERR_UNSUPPORTED";
    case CSA_ERR_WORKSPACE: return "CSA_ERR_WORKSPACE";
    case CSA_ERR_HIP: return "CSA_ERR_HIP";
  }
  return "CSA_ERR_UNKNOWN";
}

csa_status_t csa_time_next_scan(void* start_event, void* stop_event) {
  REQUIRE((start_event == nullptr) == (stop_event == nullptr), "give both events or neither");
  csa::time_next_scan(static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event));
  return CSA_OK;
}

const char* csa_last_error(void) { return g_err; }

}  // extern "C"
