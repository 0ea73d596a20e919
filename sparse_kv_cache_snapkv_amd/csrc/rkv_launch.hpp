// Internal launchers behind the C ABI. Arguments are validated by the caller (rkv_api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rkv {

// Compute units of the current device (at most 256), cached per device.
int device_cus();

// Element-wise page min/max of the first Lc slots of k_c [BH, kv_pitch, D] into channel-major
// [BH, D, ceil(cap/page_size)] (its first ceil(Lc/page_size) pages). rows (may be null): slot t
// of head bh is row rows[bh*Lc + t] of k_c.
hipError_t launch_page_minmax(const void* k_c, const int32_t* rows, int BH, int Lc, int kv_pitch,
                              int cap, int D, int page_size, int dtype, void* kmin_t,
                              void* kmax_t, hipStream_t stream);

// One token per (b, h) into slot Lc of caches of capacity cap, folded into its page summary.
hipError_t launch_kv_append(const void* k_new, const void* v_new, int BH, int Lc, int cap, int D,
                            int page_size, int dtype, void* k_c, void* v_c, void* kmin_t,
                            void* kmax_t, hipStream_t stream);

// Channel selection and sign-selected page bounds. The pitched form reads summary rows `pitch`
// pages apart (pitch >= P; a cache laid out for a larger capacity) and writes rows of P scores.
hipError_t launch_approx_scores_pitched(const void* q, const void* kmin_t, const void* kmax_t,
                                        int B, int Hq, int Hkv, int D, int P, int pitch, int r,
                                        int dtype, int32_t* chan_idx, float* page_scores,
                                        hipStream_t stream);
hipError_t launch_approx_scores(const void* q, const void* kmin_t, const void* kmax_t, int B,
                                int Hq, int Hkv, int D, int P, int r, int dtype,
                                int32_t* chan_idx, float* page_scores, hipStream_t stream);

// Per-row top-k (ties to the lower index), ascending, rows of out spaced out_stride apart.
size_t topk_ws_bytes(int rows, int n, int k);
hipError_t launch_topk(const float* scores, int rows, int n, int k, int32_t* out, int out_stride,
                       void* ws, hipStream_t stream);
// Rows that take the multi-block path keep their digit histograms in the first
// topk_hist_words(rows) 32-bit words of the top-k workspace, kTopkHistRowWords per row; a row's
// first level counts the keys' top bits (order key >> kTopkLevel0Shift) in its first
// kTopkLevel0Bins words. A caller that has already cleared them (in a launch of its own, as
// SnapKV++ eviction does) calls launch_topk_cleared, which skips the clearing launch; one whose
// producing kernel has also counted the first level (the eviction's pooling) passes
// level0_counted, which skips that pass too.
constexpr int kTopkHistRowWords = 3 * 2048;
constexpr int kTopkLevel0Shift = 21;
constexpr int kTopkLevel0Bins = 2048;
bool topk_multiblock(int n, int k);
size_t topk_hist_words(int rows);
hipError_t launch_topk_cleared(const float* scores, int rows, int n, int k, int32_t* out,
                               int out_stride, void* ws, bool level0_counted, hipStream_t stream);

// Exact attention over the selected pages.
size_t attend_ws_bytes(int B, int Hq, int Hkv, int D, int page_size, int n_pages, int dtype);
hipError_t launch_sparse_attend(const void* q, const void* k_c, const void* v_c,
                                const int32_t* page_idx, int B, int Hq, int Hkv, int Lc, int D,
                                int page_size, int n_pages, float scale, int dtype, void* out,
                                void* ws, hipStream_t stream);
// The same over caches of kv_pitch token rows per head, optionally through a row map (slot t of
// head bh is row rows[bh*Lc + t], clamped into [0, kv_pitch)).
hipError_t launch_sparse_attend_view(const void* q, const void* k, const void* v,
                                     const int32_t* rows, const int32_t* page_idx, int B, int Hq,
                                     int Hkv, int Lc, int kv_pitch, int D, int page_size,
                                     int n_pages, float scale, int dtype, void* out, void* ws,
                                     hipStream_t stream);

// One fused decode step in a single kernel: approximate page scores, page top-k, attention and
// split merge; the blocks of a head take their roles from their block index and exchange
// call-tagged words through the workspace.
size_t decode_ws_bytes(int B, int Hq, int Hkv, int Lc, int D, int page_size, int n_pages,
                       int dtype);
hipError_t launch_decode_ws_init(void* ws, size_t bytes, hipStream_t stream);
// Copies the workspace's status word to *status (host memory), optionally clears it, and
// synchronises the stream.
hipError_t read_decode_status(void* ws, int clear, uint32_t* status, hipStream_t stream);
// Caches of kv_pitch rows per head (slot t is row t, or rows[bh*Lc + t] when rows is given),
// summaries of ceil(cap/page_size) pages per channel row (the first ceil(Lc/page_size) valid);
// the workspace is laid out for cap.
hipError_t launch_decode_step(const void* q, const void* kmin_t, const void* kmax_t,
                              const void* k_c, const void* v_c, const int32_t* rows, int B, int Hq,
                              int Hkv, int Lc, int kv_pitch, int cap, int D, int page_size, int r,
                              int n_pages, float scale, int dtype, int32_t* chan_idx,
                              float* page_scores, int32_t* page_idx, void* out, void* ws,
                              hipStream_t stream);

// The same step with the library's own per-device scratch in place of a workspace, for callers
// that cannot allocate: a layout of more than kNoAllocScratchBytes is refused (by the caller of
// launch_decode_step_noalloc), the scratch is cleared whenever the layout differs from the
// previous call's on the device, and when status is not NULL the status word is moved there
// (device memory) after the step.
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
hipError_t launch_decode_step_noalloc(const void* q, const void* kmin_t, const void* kmax_t,
                                      const void* k_c, const void* v_c, int B, int Hq, int Hkv,
                                      int Lc, int D, int page_size, int r, int n_pages,
                                      float scale, int dtype, int32_t* chan_idx,
                                      float* page_scores, int32_t* page_idx, void* out,
                                      uint32_t* status, hipStream_t stream);

// SnapKV++ eviction.
size_t evict_ws_bytes(int B, int Hq, int Hkv, int L, int D, int W, int keep, int dtype);
hipError_t launch_evict(const void* q_win, const void* k, const void* v, int B, int Hq, int Hkv,
                        int L, int D, int W, int keep, int pool_kernel, int pool_type, float scale,
                        int dtype, int32_t* kept_idx, void* k_out, void* v_out, float* pooled_out,
                        void* ws, hipStream_t stream);

}  // namespace rkv
