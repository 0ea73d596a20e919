// Page summaries: element-wise min/max of K over pages of consecutive slots, written
// channel-major so a decode step reads each selected channel's page row contiguously.
// (RocketKV rebuttal, "Explanation of Calculating Approximate Attention Scores", Figure 3.)
// Also the decode-time append of one token per (b, h), which folds the new K row into the
// summary of its page (the tail page grows; a token at a page boundary starts a new page).
#include "rkv_common.hpp"
#include "rkv_launch.hpp"

namespace rkv {

namespace {

constexpr int kPagesPerBlock = 32;
constexpr int kThreads = 256;

// One block: kPagesPerBlock pages of one (b, h). Reads token rows as 16-byte chunks, reduces
// over each page's slots, transposes through LDS and writes [D][pages] rows. The cache holds
// kv_pitch token slots per head (the first Lc valid) and a summary row s_pitch pages. rows (may
// be null): slot t of head bh is row rows[bh*Lc + t] of the cache, clamped into [0, kv_pitch).
// A thread owns kItems (page, chunk) items; the loads of kSlots slots of all of them are issued
// before any is folded (the slots of a page fold in slot order, keeping the first of equal
// values, as the append does).
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void k_page_minmax(const T* __restrict__ k_c,
                                                          const int32_t* __restrict__ rows,
                                                          T* __restrict__ kmin_t,
                                                          T* __restrict__ kmax_t, int Lc, int P,
                                                          int ps, int kv_pitch, int s_pitch) {
  constexpr int V = vec16<T>::n;
  constexpr int CH = D / V;  // 16-byte chunks per token row
  constexpr int kItems = kPagesPerBlock * CH / kThreads;
  constexpr int kSlots = 4;
  static_assert(kItems * kThreads == kPagesPerBlock * CH, "items must tile the block");
  __shared__ float smin[D][kPagesPerBlock + 1];
  __shared__ float smax[D][kPagesPerBlock + 1];
  const int bh = blockIdx.y;
  const int p0 = blockIdx.x * kPagesPerBlock;
  const T* kb = k_c + (size_t)bh * kv_pitch * D;
  const int32_t* rb = rows != nullptr ? rows + (size_t)bh * Lc : nullptr;
  int t0[kItems], nt[kItems];
  float mn[kItems][V], mx[kItems][V];
#pragma unroll
  for (int i = 0; i < kItems; ++i) {
    const int p = p0 + (i * kThreads + threadIdx.x) / CH;
    t0[i] = p * ps;
    nt[i] = p < P ? min(ps, Lc - t0[i]) : 0;  // >= 1 for a page of the cache
  }
  for (int base = 0; base < ps; base += kSlots) {
    uint4 raw[kItems][kSlots];
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const int ch = (i * kThreads + threadIdx.x) % CH;
#pragma unroll
      for (int s = 0; s < kSlots; ++s) {
        raw[i][s] = make_uint4(0, 0, 0, 0);
        if (base + s < nt[i]) {
          const int t = t0[i] + base + s;
          const int r = rb != nullptr ? min(max(rb[t], 0), kv_pitch - 1) : t;
          raw[i][s] = load16(kb + (size_t)r * D + ch * V);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
#pragma unroll
      for (int s = 0; s < kSlots; ++s) {
        if (base + s >= nt[i]) continue;
        float x[V];
        unpack16<T>(raw[i][s], x);
        if (base + s == 0) {
#pragma unroll
          for (int e = 0; e < V; ++e) mn[i][e] = mx[i][e] = x[e];
        } else {
#pragma unroll
          for (int e = 0; e < V; ++e) {
            mn[i][e] = x[e] < mn[i][e] ? x[e] : mn[i][e];
            mx[i][e] = x[e] > mx[i][e] ? x[e] : mx[i][e];
          }
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kItems; ++i) {
    if (nt[i] <= 0) continue;
    const int idx = i * kThreads + threadIdx.x, pl = idx / CH, ch = idx % CH;
#pragma unroll
    for (int e = 0; e < V; ++e) {
      smin[ch * V + e][pl] = mn[i][e];
      smax[ch * V + e][pl] = mx[i][e];
    }
  }
  __syncthreads();
  // each thread writes kVecP consecutive pages of a channel row with one 16-byte store where the
  // row segment is whole and aligned (element stores otherwise)
  constexpr int kVecP = 16 / sizeof(T), kSegs = kPagesPerBlock / kVecP;
  const int np = min(kPagesPerBlock, P - p0);
  T* mnb = kmin_t + (size_t)bh * D * s_pitch + p0;
  T* mxb = kmax_t + (size_t)bh * D * s_pitch + p0;
  for (int idx = threadIdx.x; idx < D * kSegs; idx += kThreads) {
    const int c = idx / kSegs, pv = (idx % kSegs) * kVecP;
    if (pv >= np) continue;
    T* dmn = mnb + (size_t)c * s_pitch + pv;
    T* dmx = mxb + (size_t)c * s_pitch + pv;
    if (pv + kVecP <= np && ((reinterpret_cast<uintptr_t>(dmn) | reinterpret_cast<uintptr_t>(dmx)) & 15) == 0) {
      T vmn[kVecP], vmx[kVecP];
#pragma unroll
      for (int e = 0; e < kVecP; ++e) {
        vmn[e] = from_f32<T>(smin[c][pv + e]);
        vmx[e] = from_f32<T>(smax[c][pv + e]);
      }
      uint4 wmn, wmx;
      __builtin_memcpy(&wmn, vmn, 16);
      __builtin_memcpy(&wmx, vmx, 16);
      store16_stream(dmn, wmn);
      store16_stream(dmx, wmx);
    } else {
      for (int e = 0; e < kVecP && pv + e < np; ++e) {
        dmn[e] = from_f32<T>(smin[c][pv + e]);
        dmx[e] = from_f32<T>(smax[c][pv + e]);
      }
    }
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
