// C ABI entry points: host-side argument checks (before anything is enqueued), then launches.
#include <hip/hip_runtime_api.h>
#include <math.h>

#include <algorithm>
#include <cmath>

#include "../../include/rkv.h"
#include "rkv_launch.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool head_dim_ok(int D) { return D == 64 || D == 128; }
bool dtype_ok(int dtype) { return dtype == RKV_F32 || dtype == RKV_BF16; }
int ceil_div(int a, int b) { return (a + b - 1) / b; }
int launch_status(hipError_t e) { return e == hipSuccess ? RKV_OK : RKV_ERR_LAUNCH; }
constexpr int kFusedMaxPages = 8192;       // pages one block can rank in registers
constexpr int kAttendMaxPages = 256 * 1024;  // splits x LDS page slots of the attention kernel

// Every element count handed to a kernel must fit a signed 32-bit index per row and a size_t
// overall; these bounds keep all products below 2^62.
bool dims_ok(long a, long b, long c, long d) {
  const long lim = 1L << 31;
  return a >= 1 && b >= 1 && c >= 1 && d >= 1 && a < lim && b < lim && c < lim && d < lim &&
         a * b < lim && c * d < lim;
}

int check_evict(const void* q_win, const void* k, const void* v, int B, int Hq, int Hkv, int L,
                int D, int W, int keep, int pool_kernel, int pool_type, float scale, int dtype,
                const int32_t* kept_idx, const void* k_out, const void* v_out) {
  if (!q_win || !k || !v || !kept_idx) return RKV_ERR_NULL;
  if ((k_out == nullptr) != (v_out == nullptr)) return RKV_ERR_NULL;
  if (!dtype_ok(dtype)) return RKV_ERR_DTYPE;
  if (B < 1 || Hq < 1 || Hkv < 1 || L < 1 || W < 1 || keep < 1) return RKV_ERR_SHAPE;
  if (Hq % Hkv != 0 || W > L || keep < W) return RKV_ERR_SHAPE;
  if (pool_kernel < 1 || pool_kernel % 2 == 0) return RKV_ERR_SHAPE;
  if (pool_type != RKV_POOL_AVG && pool_type != RKV_POOL_MAX) return RKV_ERR_SHAPE;
  if (!(scale > 0.f) || !isfinite(scale)) return RKV_ERR_SHAPE;
  if (!dims_ok((long)B * Hkv, L, (long)L, D) || !dims_ok((long)B * Hq, W, (long)W * Hq / Hkv, D))
    return RKV_ERR_SHAPE;
  if (!head_dim_ok(D)) return RKV_ERR_UNSUPPORTED;
  if (pool_kernel > 127) return RKV_ERR_UNSUPPORTED;
  const long GW = (long)(Hq / Hkv) * W;
  if (dtype == RKV_BF16 && GW > 512) return RKV_ERR_UNSUPPORTED;  // window rows live in LDS
  if (dtype == RKV_F32 && GW > 2048) return RKV_ERR_UNSUPPORTED;
  if (!aligned16(q_win) || !aligned16(k) || !aligned16(v)) return RKV_ERR_SHAPE;
  if (k_out && (!aligned16(k_out) || !aligned16(v_out))) return RKV_ERR_SHAPE;
  return RKV_OK;
}

}  // namespace

extern "C" {

int rkv_version(void) { return RKV_VERSION; }

int rkv_plan_budget(int L, int D, int W, int token_budget, int* keep, int* page_size, int* r,
                    int* topk, int* pool_kernel, int* approx_tokens) {
  if (!keep || !page_size || !r || !topk || !pool_kernel || !approx_tokens) return RKV_ERR_NULL;
  if (L < 1 || D < 1 || W < 1 || W > L || token_budget < 1) return RKV_ERR_SHAPE;
  const int pool = L <= 4096 ? 7 : L <= 16384 ? 15 : L <= 65536 ? 31 : 63;
  if (token_budget >= L) {
    *keep = L;
    *page_size = 1;
    *r = D;
    *topk = L;
    *pool_kernel = pool;
    *approx_tokens = 0;
    return RKV_OK;
  }
  const double stage = std::sqrt((double)L / (double)token_budget);  // each stage's ratio
  const double dim = std::sqrt(stage);  // each dimension's share of the second stage
  const int kp = std::min(std::max((int)std::lround((double)L / stage), W), L);
  const int ps = std::max(1, (int)std::lround(dim));
  const int rr = std::min(std::max((int)std::lround((double)D / dim), 1), D);
  const long num = (long)kp * rr, den = (long)ps * 2 * D;
  const int approx = (int)((num + den - 1) / den);
  const int kcap = ceil_div(kp, ps) * ps;
  int tk = (token_budget - approx) / ps * ps;
  tk = std::min(std::max(tk, ps), kcap);
  *keep = kp;
  *page_size = ps;
  *r = rr;
  *topk = tk;
  *pool_kernel = pool;
  *approx_tokens = approx;
  return RKV_OK;
}

const char* rkv_status_string(int status) {
  switch (status) {
    case RKV_OK:
      return "success";
    case RKV_ERR_NULL:
      return "a required pointer is NULL";
    case RKV_ERR_SHAPE:
      return "a size or parameter is out of range, inconsistent, or a pointer is misaligned";
    case RKV_ERR_DTYPE:
      return "unknown dtype";
    case RKV_ERR_WORKSPACE:
      return "workspace missing or too small";
    case RKV_ERR_UNSUPPORTED:
      return "unsupported configuration (head dim must be 64 or 128; see header limits)";
    case RKV_ERR_LAUNCH:
      return "the HIP runtime failed to enqueue a kernel";
    case RKV_ERR_SCRATCH:
      return "the shape needs more than the library's fixed scratch (RKV_NOALLOC_SCRATCH_BYTES)";
    default:
      return "unknown status";
  }
}

int rkv_snapkvpp_workspace_bytes(int B, int Hq, int Hkv, int L, int D, int W, int keep,
                                 int dtype, size_t* bytes) {
  if (!bytes) return RKV_ERR_NULL;
  if (!dtype_ok(dtype)) return RKV_ERR_DTYPE;
  if (B < 1 || Hq < 1 || Hkv < 1 || L < 1 || W < 1 || keep < W || Hq % Hkv || W > L)
    return RKV_ERR_SHAPE;
  if (!head_dim_ok(D)) return RKV_ERR_UNSUPPORTED;
  *bytes = rkv::evict_ws_bytes(B, Hq, Hkv, L, D, W, keep, dtype);
  return RKV_OK;
}

int rkv_snapkvpp_evict(const void* q_win, const void* k, const void* v, int B, int Hq, int Hkv,
                       int L, int D, int W, int keep, int pool_kernel, int pool_type, float scale,
                       int dtype, int32_t* kept_idx, void* k_out, void* v_out, float* pooled_out,
                       void* ws, size_t ws_bytes, void* stream) {
  int st = check_evict(q_win, k, v, B, Hq, Hkv, L, D, W, keep, pool_kernel, pool_type, scale,
                       dtype, kept_idx, k_out, v_out);
  if (st != RKV_OK) return st;
  const size_t need = rkv::evict_ws_bytes(B, Hq, Hkv, L, D, W, keep, dtype);
  if (need > 0 && (ws == nullptr || ws_bytes < need || !aligned16(ws))) return RKV_ERR_WORKSPACE;
  return launch_status(rkv::launch_evict(q_win, k, v, B, Hq, Hkv, L, D, W, keep, pool_kernel,
                                         pool_type, scale, dtype, kept_idx, k_out, v_out,
                                         keep >= L ? nullptr : pooled_out, ws,
                                         static_cast<hipStream_t>(stream)));
}

int rkv_build_page_summaries(const void* k_c, int B, int Hkv, int Lc, int D, int page_size,
                             int dtype, void* kmin_t, void* kmax_t, void* stream) {
  if (!k_c || !kmin_t || !kmax_t) return RKV_ERR_NULL;
  if (!dtype_ok(dtype)) return RKV_ERR_DTYPE;
  if (B < 1 || Hkv < 1 || Lc < 1 || page_size < 1 || D < 1) return RKV_ERR_SHAPE;
  if (!dims_ok((long)B * Hkv, Lc, Lc, D)) return RKV_ERR_SHAPE;
  if (!head_dim_ok(D)) return RKV_ERR_UNSUPPORTED;
  if (!aligned16(k_c)) return RKV_ERR_SHAPE;
  return launch_status(rkv::launch_page_minmax(k_c, nullptr, B * Hkv, Lc, Lc, Lc, D, page_size,
                                               dtype, kmin_t, kmax_t,
                                               static_cast<hipStream_t>(stream)));
}

int rkv_build_page_summaries_cap(const void* k_c, int B, int Hkv, int Lc, int cap, int D,
                                 int page_size, int dtype, void* kmin_t, void* kmax_t,
                                 void* stream) {
  if (!k_c || !kmin_t || !kmax_t) return RKV_ERR_NULL;
  if (!dtype_ok(dtype)) return RKV_ERR_DTYPE;
  if (B < 1 || Hkv < 1 || Lc < 1 || cap < Lc || page_size < 1 || D < 1) return RKV_ERR_SHAPE;
  if (!dims_ok((long)B * Hkv, cap, cap, D)) return RKV_ERR_SHAPE;
  if (!head_dim_ok(D)) return RKV_ERR_UNSUPPORTED;
  if (!aligned16(k_c)) return RKV_ERR_SHAPE;
  return launch_status(rkv::launch_page_minmax(k_c, nullptr, B * Hkv, Lc, cap, cap, D, page_size,
                                               dtype, kmin_t, kmax_t,
                                               static_cast<hipStream_t>(stream)));
}

int rkv_build_page_summaries_indexed(const void* k, const int32_t* kept_idx, int B, int Hkv,
                                     int L, int Lc, int D, int page_size, int dtype, void* kmin_t,
                                     void* kmax_t, void* stream) {
  if (!k || !kept_idx || !kmin_t || !kmax_t) return RKV_ERR_NULL;
  if (!dtype_ok(dtype)) return RKV_ERR_DTYPE;
  if (B < 1 || Hkv < 1 || L < 1 || Lc < 1 || page_size < 1 || D < 1) return RKV_ERR_SHAPE;
  if (!dims_ok((long)B * Hkv, L, L, D) || !dims_ok((long)B * Hkv, Lc, 1, 1)) return RKV_ERR_SHAPE;
  if (!head_dim_ok(D)) return RKV_ERR_UNSUPPORTED;
  if (!aligned16(k)) return RKV_ERR_SHAPE;
  return launch_status(rkv::launch_page_minmax(k, kept_idx, B * Hkv, Lc, L, Lc, D, page_size,
                                               dtype, kmin_t, kmax_t,
                                               static_cast<hipStream_t>(stream)));
}

int rkv_kv_append(const void* k_new, const void* v_new, int B, int Hkv, int Lc, int cap, int D,
                  int page_size, int dtype, void* k_c, void* v_c, void* kmin_t, void* kmax_t,
                  void* stream) {
  if (!k_new || !v_new || !k_c || !v_c || !kmin_t || !kmax_t) return RKV_ERR_NULL;
  if (!dtype_ok(dtype)) return RKV_ERR_DTYPE;
  if (B < 1 || Hkv < 1 || Lc < 0 || cap < 1 || Lc >= cap || page_size < 1) return RKV_ERR_SHAPE;
  if (!dims_ok((long)B * Hkv, cap, cap, D)) return RKV_ERR_SHAPE;
  if (!head_dim_ok(D)) return RKV_ERR_UNSUPPORTED;
  return launch_status(rkv::launch_kv_append(k_new, v_new, B * Hkv, Lc, cap, D, page_size, dtype,
                                             k_c, v_c, kmin_t, kmax_t,
                                             static_cast<hipStream_t>(stream)));
}

int rkv_hybrid_approx_scores(const void* q, const void* kmin_t, const void* kmax_t, int B,
                             int Hq, int Hkv, int D, int P, int r, int dtype, int32_t* chan_idx,
                             float* page_scores, void* stream) {
  if (!q || !kmin_t || !kmax_t || !page_scores) return RKV_ERR_NULL;
  if (!dtype_ok(dtype)) return RKV_ERR_DTYPE;
  if (B < 1 || Hq < 1 || Hkv < 1 || P < 1 || Hq % Hkv || r < 1 || r > D) return RKV_ERR_SHAPE;
  if (!dims_ok((long)B * Hkv, D, D, P)) return RKV_ERR_SHAPE;
  if (!head_dim_ok(D) || Hq / Hkv > 8) return RKV_ERR_UNSUPPORTED;
  if (!aligned16(kmin_t) || !aligned16(kmax_t)) return RKV_ERR_SHAPE;
  return launch_status(rkv::launch_approx_scores(q, kmin_t, kmax_t, B, Hq, Hkv, D, P, r, dtype,
                                                 chan_idx, page_scores,
                                                 static_cast<hipStream_t>(stream)));
}

int rkv_topk_workspace_bytes(int rows, int n, int k, size_t* bytes) {
  if (!bytes) return RKV_ERR_NULL;
  if (rows < 1 || n < 1 || k < 0) return RKV_ERR_SHAPE;
  *bytes = rkv::topk_ws_bytes(rows, n, k);
  return RKV_OK;
}

int rkv_topk_select(const float* scores, int rows, int n, int k, int32_t* idx_out, void* ws,
                    size_t ws_bytes, void* stream) {
  if (!scores) return RKV_ERR_NULL;
  if (rows < 1 || n < 1 || k < 0 || !dims_ok(rows, n, 1, 1)) return RKV_ERR_SHAPE;
  if (k == 0) return RKV_OK;  // nothing selected; idx_out may be NULL
  if (!idx_out) return RKV_ERR_NULL;
  const size_t need = rkv::topk_ws_bytes(rows, n, k);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return RKV_ERR_WORKSPACE;
  const int kk = k < n ? k : n;
  return launch_status(rkv::launch_topk(scores, rows, n, kk, idx_out, kk, ws,
                                        static_cast<hipStream_t>(stream)));
}

int rkv_sparse_attend_workspace_bytes(int B, int Hq, int Hkv, int D, int page_size, int n_pages,
                                      int dtype, size_t* bytes) {
  if (!bytes) return RKV_ERR_NULL;
  if (!dtype_ok(dtype)) return RKV_ERR_DTYPE;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || page_size < 1 || n_pages < 1)
    return RKV_ERR_SHAPE;
  if (!head_dim_ok(D) || Hq / Hkv > 8 || n_pages > kAttendMaxPages) return RKV_ERR_UNSUPPORTED;
  *bytes = rkv::attend_ws_bytes(B, Hq, Hkv, D, page_size, n_pages, dtype);
  return RKV_OK;
}

int rkv_sparse_attend_decode(const void* q, const void* k_c, const void* v_c,
                             const int32_t* page_idx, int B, int Hq, int Hkv, int Lc, int D,
                             int page_size, int n_pages, float scale, int dtype, void* out,
                             void* ws, size_t ws_bytes, void* stream) {
  if (!q || !k_c || !v_c || !page_idx || !out) return RKV_ERR_NULL;
  if (!dtype_ok(dtype)) return RKV_ERR_DTYPE;
  if (B < 1 || Hq < 1 || Hkv < 1 || Lc < 1 || page_size < 1 || n_pages < 1 || Hq % Hkv)
    return RKV_ERR_SHAPE;
  if (n_pages > ceil_div(Lc, page_size) || !isfinite(scale)) return RKV_ERR_SHAPE;
  if (!dims_ok((long)B * Hkv, Lc, Lc, D) || (long)n_pages * page_size >= (1L << 31))
    return RKV_ERR_SHAPE;
  if (!head_dim_ok(D) || Hq / Hkv > 8 || n_pages > kAttendMaxPages) return RKV_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k_c) || !aligned16(v_c)) return RKV_ERR_SHAPE;
  const size_t need = rkv::attend_ws_bytes(B, Hq, Hkv, D, page_size, n_pages, dtype);
  if (need > 0 && (ws == nullptr || ws_bytes < need || !aligned16(ws))) return RKV_ERR_WORKSPACE;
  return launch_status(rkv::launch_sparse_attend(q, k_c, v_c, page_idx, B, Hq, Hkv, Lc, D,
                                                 page_size, n_pages, scale, dtype, out, ws,
                                                 static_cast<hipStream_t>(stream)));
}

int rkv_hybrid_decode_workspace_bytes(int B, int Hq, int Hkv, int Lc, int D, int page_size,
                                      int n_pages, int dtype, size_t* bytes) {
  if (!bytes) return RKV_ERR_NULL;
  if (!dtype_ok(dtype)) return RKV_ERR_DTYPE;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || Lc < 1 || page_size < 1 || n_pages < 1 ||
      n_pages > ceil_div(Lc, page_size))
    return RKV_ERR_SHAPE;
  if (!head_dim_ok(D) || Hq / Hkv > 8 || ceil_div(Lc, page_size) > kFusedMaxPages)
    return RKV_ERR_UNSUPPORTED;
  *bytes = rkv::decode_ws_bytes(B, Hq, Hkv, Lc, D, page_size, n_pages, dtype);
  return RKV_OK;
}

int rkv_hybrid_decode_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws) return RKV_ERR_NULL;
  if (ws_bytes < 256 || !aligned16(ws)) return RKV_ERR_WORKSPACE;
  return launch_status(rkv::launch_decode_ws_init(ws, ws_bytes, static_cast<hipStream_t>(stream)));
}

int rkv_hybrid_decode_status(void* ws, size_t ws_bytes, int clear, uint32_t* status,
                             void* stream) {
  if (!ws || !status) return RKV_ERR_NULL;
  if (ws_bytes < 256 || !aligned16(ws)) return RKV_ERR_WORKSPACE;
  return launch_status(rkv::read_decode_status(ws, clear, status, static_cast<hipStream_t>(stream)));
}

int rkv_hybrid_decode_step(const void* q, const void* kmin_t, const void* kmax_t,
                           const void* k_c, const void* v_c, int B, int Hq, int Hkv, int Lc,
                           int D, int page_size, int r, int n_pages, float scale, int dtype,
                           int32_t* chan_idx, float* page_scores, int32_t* page_idx, void* out,
                           void* ws, size_t ws_bytes, void* stream) {
  if (!q || !kmin_t || !kmax_t || !k_c || !v_c || !out) return RKV_ERR_NULL;
  if (!dtype_ok(dtype)) return RKV_ERR_DTYPE;
  if (B < 1 || Hq < 1 || Hkv < 1 || Lc < 1 || page_size < 1 || n_pages < 1 || Hq % Hkv)
    return RKV_ERR_SHAPE;
  const int P = ceil_div(Lc, page_size);
  if (n_pages > P || r < 1 || r > D || !isfinite(scale)) return RKV_ERR_SHAPE;
  if (!dims_ok((long)B * Hkv, Lc, Lc, D)) return RKV_ERR_SHAPE;
  if (!head_dim_ok(D) || Hq / Hkv > 8 || P > kFusedMaxPages) return RKV_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k_c) || !aligned16(v_c) || !aligned16(kmin_t) ||
      !aligned16(kmax_t))
    return RKV_ERR_SHAPE;
  const size_t need = rkv::decode_ws_bytes(B, Hq, Hkv, Lc, D, page_size, n_pages, dtype);
  if (ws == nullptr || ws_bytes < need || !aligned16(ws)) return RKV_ERR_WORKSPACE;
  return launch_status(rkv::launch_decode_step(q, kmin_t, kmax_t, k_c, v_c, nullptr, B, Hq, Hkv,
                                               Lc, Lc, Lc, D, page_size, r, n_pages, scale, dtype,
                                               chan_idx, page_scores, page_idx, out, ws,
                                               static_cast<hipStream_t>(stream)));
}

int rkv_hybrid_decode_step_noalloc(const void* q, const void* kmin_t, const void* kmax_t,
                                   const void* k_c, const void* v_c, int B, int Hq, int Hkv,
                                   int Lc, int D, int page_size, int r, int n_pages, float scale,
                                   int dtype, int32_t* chan_idx, float* page_scores,
                                   int32_t* page_idx, void* out, uint32_t* status, void* stream) {
  static_assert(rkv::kNoAllocScratchBytes == RKV_NOALLOC_SCRATCH_BYTES, "scratch size");
  if (!q || !kmin_t || !kmax_t || !k_c || !v_c || !out) return RKV_ERR_NULL;
  if (!dtype_ok(dtype)) return RKV_ERR_DTYPE;
  if (B < 1 || Hq < 1 || Hkv < 1 || Lc < 1 || page_size < 1 || n_pages < 1 || Hq % Hkv)
    return RKV_ERR_SHAPE;
  const int P = ceil_div(Lc, page_size);
  if (n_pages > P || r < 1 || r > D || !isfinite(scale)) return RKV_ERR_SHAPE;
  if (!dims_ok((long)B * Hkv, Lc, Lc, D)) return RKV_ERR_SHAPE;
  if (!head_dim_ok(D) || Hq / Hkv > 8 || P > kFusedMaxPages) return RKV_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k_c) || !aligned16(v_c) || !aligned16(kmin_t) ||
      !aligned16(kmax_t) || (status != nullptr && !aligned16(status)))
    return RKV_ERR_SHAPE;
  if (rkv::decode_ws_bytes(B, Hq, Hkv, Lc, D, page_size, n_pages, dtype) >
      rkv::kNoAllocScratchBytes)
    return RKV_ERR_SCRATCH;
  return launch_status(rkv::launch_decode_step_noalloc(
      q, kmin_t, kmax_t, k_c, v_c, B, Hq, Hkv, Lc, D, page_size, r, n_pages, scale, dtype,
      chan_idx, page_scores, page_idx, out, status, static_cast<hipStream_t>(stream)));
}

int rkv_hybrid_decode_step_indexed(const void* q, const void* kmin_t, const void* kmax_t,
                                   const void* k, const void* v, const int32_t* kept_idx, int B,
                                   int Hq, int Hkv, int L, int Lc, int D, int page_size, int r,
                                   int n_pages, float scale, int dtype, int32_t* chan_idx,
                                   float* page_scores, int32_t* page_idx, void* out, void* ws,
                                   size_t ws_bytes, void* stream) {
  if (!q || !kmin_t || !kmax_t || !k || !v || !kept_idx || !out) return RKV_ERR_NULL;
  if (!dtype_ok(dtype)) return RKV_ERR_DTYPE;
  if (B < 1 || Hq < 1 || Hkv < 1 || L < 1 || Lc < 1 || page_size < 1 || n_pages < 1 || Hq % Hkv)
    return RKV_ERR_SHAPE;
  const int P = ceil_div(Lc, page_size);
  if (n_pages > P || r < 1 || r > D || !isfinite(scale)) return RKV_ERR_SHAPE;
  if (!dims_ok((long)B * Hkv, L, L, D) || !dims_ok((long)B * Hkv, Lc, 1, 1)) return RKV_ERR_SHAPE;
  if (!head_dim_ok(D) || Hq / Hkv > 8 || P > kFusedMaxPages) return RKV_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(kmin_t) ||
      !aligned16(kmax_t))
    return RKV_ERR_SHAPE;
  const size_t need = rkv::decode_ws_bytes(B, Hq, Hkv, Lc, D, page_size, n_pages, dtype);
  if (ws == nullptr || ws_bytes < need || !aligned16(ws)) return RKV_ERR_WORKSPACE;
  return launch_status(rkv::launch_decode_step(q, kmin_t, kmax_t, k, v, kept_idx, B, Hq, Hkv, Lc,
                                               L, Lc, D, page_size, r, n_pages, scale, dtype,
                                               chan_idx, page_scores, page_idx, out, ws,
                                               static_cast<hipStream_t>(stream)));
}

int rkv_hybrid_decode_step_cap(const void* q, const void* kmin_t, const void* kmax_t,
                               const void* k_c, const void* v_c, int B, int Hq, int Hkv, int Lc,
                               int cap, int D, int page_size, int r, int n_pages, float scale,
                               int dtype, int32_t* chan_idx, float* page_scores,
                               int32_t* page_idx, void* out, void* ws, size_t ws_bytes,
                               void* stream) {
  if (!q || !kmin_t || !kmax_t || !k_c || !v_c || !out) return RKV_ERR_NULL;
  if (!dtype_ok(dtype)) return RKV_ERR_DTYPE;
  if (B < 1 || Hq < 1 || Hkv < 1 || Lc < 1 || cap < Lc || page_size < 1 || n_pages < 1 ||
      Hq % Hkv)
    return RKV_ERR_SHAPE;
  const int P = ceil_div(Lc, page_size);
  if (n_pages > P || r < 1 || r > D || !isfinite(scale)) return RKV_ERR_SHAPE;
  if (!dims_ok((long)B * Hkv, cap, cap, D)) return RKV_ERR_SHAPE;
  if (!head_dim_ok(D) || Hq / Hkv > 8 || ceil_div(cap, page_size) > kFusedMaxPages)
    return RKV_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k_c) || !aligned16(v_c) || !aligned16(kmin_t) ||
      !aligned16(kmax_t))
    return RKV_ERR_SHAPE;
  const size_t need = rkv::decode_ws_bytes(B, Hq, Hkv, cap, D, page_size, n_pages, dtype);
  if (ws == nullptr || ws_bytes < need || !aligned16(ws)) return RKV_ERR_WORKSPACE;
  return launch_status(rkv::launch_decode_step(q, kmin_t, kmax_t, k_c, v_c, nullptr, B, Hq, Hkv,
                                               Lc, cap, cap, D, page_size, r, n_pages, scale,
                                               dtype, chan_idx, page_scores, page_idx, out, ws,
                                               static_cast<hipStream_t>(stream)));
}

}  // extern "C"
