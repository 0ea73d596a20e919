// Page summaries: element-wise min/max of K over pages of consecutive slots, written
// channel-major so a decode step reads each selected channel's page row contiguously.
// (RocketKV rebuttal, "Explanation of Calculating Approximate Attention Scores", Figure 3.)
// Also the decode-time append of one token per (b, h), which folds the new K row into the
// summary of its page (the tail page grows; a token at a page boundary starts a new page).
#include "rkv_common.hpp"
#include "rkv_launch.hpp"

namespace rkv {

namespace {

constexpr int kPagesPerBlock = 64;
constexpr int kThreads = 256;

// One block: kPagesPerBlock pages of one (b, h). Reads token rows as 16-byte chunks, reduces
// over each page's slots, transposes through LDS and writes [D][pages] rows. The cache holds
// kv_pitch token slots per head (the first Lc valid) and a summary row s_pitch pages. rows (may
// be null): slot t of head bh is row rows[bh*Lc + t] of the cache, clamped into [0, kv_pitch).
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void k_page_minmax(const T* __restrict__ k_c,
                                                          const int32_t* __restrict__ rows,
                                                          T* __restrict__ kmin_t,
                                                          T* __restrict__ kmax_t, int Lc, int P,
                                                          int ps, int kv_pitch, int s_pitch) {
  constexpr int V = vec16<T>::n;
  constexpr int CH = D / V;  // 16-byte chunks per token row
  __shared__ float smin[D][kPagesPerBlock + 1];
  __shared__ float smax[D][kPagesPerBlock + 1];
  const int bh = blockIdx.y;
  const int p0 = blockIdx.x * kPagesPerBlock;
  const T* kb = k_c + (size_t)bh * kv_pitch * D;
  const int32_t* rb = rows != nullptr ? rows + (size_t)bh * Lc : nullptr;
  auto row = [&](int t) { return rb != nullptr ? min(max(rb[t], 0), kv_pitch - 1) : t; };
  for (int idx = threadIdx.x; idx < kPagesPerBlock * CH; idx += kThreads) {
    const int pl = idx / CH, ch = idx % CH, p = p0 + pl;
    if (p >= P) continue;
    const int t0 = p * ps, t1 = min(t0 + ps, Lc);
    float mn[V], mx[V];
    unpack16<T>(load16(kb + (size_t)row(t0) * D + ch * V), mn);
#pragma unroll
    for (int e = 0; e < V; ++e) mx[e] = mn[e];
    for (int t = t0 + 1; t < t1; ++t) {
      float x[V];
      unpack16<T>(load16(kb + (size_t)row(t) * D + ch * V), x);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        mn[e] = x[e] < mn[e] ? x[e] : mn[e];
        mx[e] = x[e] > mx[e] ? x[e] : mx[e];
      }
    }
#pragma unroll
    for (int e = 0; e < V; ++e) {
      smin[ch * V + e][pl] = mn[e];
      smax[ch * V + e][pl] = mx[e];
    }
  }
  __syncthreads();
  const int np = min(kPagesPerBlock, P - p0);
  T* mnb = kmin_t + (size_t)bh * D * s_pitch + p0;
  T* mxb = kmax_t + (size_t)bh * D * s_pitch + p0;
  for (int idx = threadIdx.x; idx < D * kPagesPerBlock; idx += kThreads) {
    const int c = idx / kPagesPerBlock, pl = idx % kPagesPerBlock;
    if (pl >= np) continue;
    mnb[(size_t)c * s_pitch + pl] = from_f32<T>(smin[c][pl]);
    mxb[(size_t)c * s_pitch + pl] = from_f32<T>(smax[c][pl]);
  }
}

// Block = one (b, h), thread = one channel: the new token's K and V rows go to slot Lc, and its
// K value folds into the page's (min, max) with the comparison order of k_page_minmax (the
// running value is replaced only by a strictly smaller / larger one), so appending tokens one
// by one gives the same bits as summarising the grown cache.
template <typename T>
__global__ void k_kv_append(const T* __restrict__ k_new, const T* __restrict__ v_new, int D,
                            int Lc, int ps, int kv_pitch, int s_pitch, T* __restrict__ k_c,
                            T* __restrict__ v_c, T* __restrict__ kmin_t, T* __restrict__ kmax_t) {
  const int bh = blockIdx.x, c = threadIdx.x;
  if (c >= D) return;
  const T k = k_new[(size_t)bh * D + c];
  const size_t slot = ((size_t)bh * kv_pitch + Lc) * D + c;
  k_c[slot] = k;
  v_c[slot] = v_new[(size_t)bh * D + c];
  const size_t s = ((size_t)bh * D + c) * s_pitch + Lc / ps;
  if (Lc % ps == 0) {
    kmin_t[s] = k;
    kmax_t[s] = k;
  } else {
    const float x = to_f32(k), mn = to_f32(kmin_t[s]), mx = to_f32(kmax_t[s]);
    if (x < mn) kmin_t[s] = k;
    if (x > mx) kmax_t[s] = k;
  }
}

template <typename T, int D>
hipError_t launch_t(const void* k_c, const int32_t* rows, int BH, int Lc, int kv_pitch, int cap,
                    int ps, void* kmin_t, void* kmax_t, hipStream_t stream) {
  const int P = (Lc + ps - 1) / ps;
  dim3 grid((P + kPagesPerBlock - 1) / kPagesPerBlock, BH);
  hipLaunchKernelGGL((k_page_minmax<T, D>), grid, dim3(kThreads), 0, stream,
                     static_cast<const T*>(k_c), rows, static_cast<T*>(kmin_t),
                     static_cast<T*>(kmax_t), Lc, P, ps, kv_pitch, (cap + ps - 1) / ps);
  return hipGetLastError();
}

template <typename T>
hipError_t append_t(const void* k_new, const void* v_new, int BH, int Lc, int cap, int D, int ps,
                    void* k_c, void* v_c, void* kmin_t, void* kmax_t, hipStream_t stream) {
  hipLaunchKernelGGL((k_kv_append<T>), dim3(BH), dim3(D), 0, stream,
                     static_cast<const T*>(k_new), static_cast<const T*>(v_new), D, Lc, ps, cap,
                     (cap + ps - 1) / ps, static_cast<T*>(k_c), static_cast<T*>(v_c),
                     static_cast<T*>(kmin_t), static_cast<T*>(kmax_t));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_page_minmax(const void* k_c, const int32_t* rows, int BH, int Lc, int kv_pitch,
                              int cap, int D, int page_size, int dtype, void* kmin_t,
                              void* kmax_t, hipStream_t stream) {
  if (dtype == 0)
    return D == 64 ? launch_t<float, 64>(k_c, rows, BH, Lc, kv_pitch, cap, page_size, kmin_t,
                                         kmax_t, stream)
                   : launch_t<float, 128>(k_c, rows, BH, Lc, kv_pitch, cap, page_size, kmin_t,
                                          kmax_t, stream);
  return D == 64 ? launch_t<bf16_t, 64>(k_c, rows, BH, Lc, kv_pitch, cap, page_size, kmin_t,
                                        kmax_t, stream)
                 : launch_t<bf16_t, 128>(k_c, rows, BH, Lc, kv_pitch, cap, page_size, kmin_t,
                                         kmax_t, stream);
}

hipError_t launch_kv_append(const void* k_new, const void* v_new, int BH, int Lc, int cap, int D,
                            int page_size, int dtype, void* k_c, void* v_c, void* kmin_t,
                            void* kmax_t, hipStream_t stream) {
  if (dtype == 0)
    return append_t<float>(k_new, v_new, BH, Lc, cap, D, page_size, k_c, v_c, kmin_t, kmax_t,
                           stream);
  return append_t<bf16_t>(k_new, v_new, BH, Lc, cap, D, page_size, k_c, v_c, kmin_t, kmax_t,
                          stream);
}

}  // namespace rkv
