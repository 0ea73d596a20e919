// Page summaries: element-wise min/max of K over pages of consecutive slots, written
// channel-major so a decode step reads each selected channel's page row contiguously.
// (RocketKV rebuttal, "Explanation of Calculating Approximate Attention Scores", Figure 3.)
#include "rkv_common.hpp"
#include "rkv_launch.hpp"

namespace rkv {

namespace {

constexpr int kPagesPerBlock = 64;
constexpr int kThreads = 256;

// One block: kPagesPerBlock pages of one (b, h). Reads token rows as 16-byte chunks, reduces
// over each page's slots, transposes through LDS and writes [D][pages] rows.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void k_page_minmax(const T* __restrict__ k_c,
                                                          T* __restrict__ kmin_t,
                                                          T* __restrict__ kmax_t, int Lc, int P,
                                                          int ps) {
  constexpr int V = vec16<T>::n;
  constexpr int CH = D / V;  // 16-byte chunks per token row
  __shared__ float smin[D][kPagesPerBlock + 1];
  __shared__ float smax[D][kPagesPerBlock + 1];
  const int bh = blockIdx.y;
  const int p0 = blockIdx.x * kPagesPerBlock;
  const T* kb = k_c + (size_t)bh * Lc * D;
  for (int idx = threadIdx.x; idx < kPagesPerBlock * CH; idx += kThreads) {
    const int pl = idx / CH, ch = idx % CH, p = p0 + pl;
    if (p >= P) continue;
    const int t0 = p * ps, t1 = min(t0 + ps, Lc);
    float mn[V], mx[V];
    unpack16<T>(load16(kb + (size_t)t0 * D + ch * V), mn);
#pragma unroll
    for (int e = 0; e < V; ++e) mx[e] = mn[e];
    for (int t = t0 + 1; t < t1; ++t) {
      float x[V];
      unpack16<T>(load16(kb + (size_t)t * D + ch * V), x);
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
  T* mnb = kmin_t + (size_t)bh * D * P + p0;
  T* mxb = kmax_t + (size_t)bh * D * P + p0;
  for (int idx = threadIdx.x; idx < D * kPagesPerBlock; idx += kThreads) {
    const int c = idx / kPagesPerBlock, pl = idx % kPagesPerBlock;
    if (pl >= np) continue;
    mnb[(size_t)c * P + pl] = from_f32<T>(smin[c][pl]);
    mxb[(size_t)c * P + pl] = from_f32<T>(smax[c][pl]);
  }
}

template <typename T, int D>
hipError_t launch_t(const void* k_c, int BH, int Lc, int ps, void* kmin_t, void* kmax_t,
                    hipStream_t stream) {
  const int P = (Lc + ps - 1) / ps;
  dim3 grid((P + kPagesPerBlock - 1) / kPagesPerBlock, BH);
  hipLaunchKernelGGL((k_page_minmax<T, D>), grid, dim3(kThreads), 0, stream,
                     static_cast<const T*>(k_c), static_cast<T*>(kmin_t),
                     static_cast<T*>(kmax_t), Lc, P, ps);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_page_minmax(const void* k_c, int BH, int Lc, int D, int page_size, int dtype,
                              void* kmin_t, void* kmax_t, hipStream_t stream) {
  if (dtype == 0)
    return D == 64 ? launch_t<float, 64>(k_c, BH, Lc, page_size, kmin_t, kmax_t, stream)
                   : launch_t<float, 128>(k_c, BH, Lc, page_size, kmin_t, kmax_t, stream);
  return D == 64 ? launch_t<bf16_t, 64>(k_c, BH, Lc, page_size, kmin_t, kmax_t, stream)
                 : launch_t<bf16_t, 128>(k_c, BH, Lc, page_size, kmin_t, kmax_t, stream);
}

}  // namespace rkv
