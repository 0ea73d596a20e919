// Standalone exact softmax attention over the selected pages (RocketKV rebuttal, "Lack of Direct
// Latency Comparison": Step 3 sparse attention; "Explanation of Calculating Approximate Attention
// Scores": one selection per GQA group). Block = (split of the head's page list, b*Hkv+h), 4
// waves; the block copies its slice of page_idx into LDS, attends with the per-wave state of
// rkv_attend.hpp, and several splits per head are combined by k_attend_merge (log-sum-exp form).
#include <math.h>

#include <algorithm>

#include "rkv_attend.hpp"
#include "rkv_common.hpp"
#include "rkv_launch.hpp"

namespace rkv {

namespace {

// ------------------------------------------------------------------------------ standalone call

struct AttendArgs {
  const void* q;
  const void* k_c;
  const void* v_c;
  const int32_t* page_idx;  // [BH, n_pages]
  const int32_t* rows;      // [BH, Lc] or null: slot t of head bh is row rows[bh*Lc + t]
  int Lc, kv_pitch, ps, n_pages, P, pps, nsplit;  // kv_pitch: token rows per head of k_c, v_c
  float scale2;
  float* part;              // [BH, nsplit, G, D+2]
  void* out;
};

template <typename T, int D, int G>
__global__ __launch_bounds__(kAttThreads) void k_attend(AttendArgs a) {
  __shared__ AttendShared<D, G> sh;
  const int tid = threadIdx.x;
  const int bh = blockIdx.y, split = blockIdx.x;
  const int p_lo = split * a.pps;
  const int p_hi = min(p_lo + a.pps, a.n_pages);
  const int np_blk = max(p_hi - p_lo, 0);
  const int32_t* pb = a.page_idx + (size_t)bh * a.n_pages + p_lo;
  for (int i = tid; i < np_blk; i += kAttThreads) sh.pages[i] = pb[i];
  __syncthreads();
  const T* kc_bh = static_cast<const T*>(a.k_c) + (size_t)bh * a.kv_pitch * D;
  const T* vc_bh = static_cast<const T*>(a.v_c) + (size_t)bh * a.kv_pitch * D;
  const int32_t* rows_bh = a.rows != nullptr ? a.rows + (size_t)bh * a.Lc : nullptr;
  const T* q_bh = static_cast<const T*>(a.q) + (size_t)bh * G * D;
  AttendWave<T, D, G> st;
  st.init(q_bh, a.scale2);
  st.run(kc_bh, vc_bh, sh.pages, np_blk * a.ps, a.ps, a.P, a.Lc, rows_bh, a.kv_pitch - 1, sh);
  st.publish(sh);
  __syncthreads();
  T* out = static_cast<T*>(a.out);
  for (int idx = tid; idx < G * D; idx += kAttThreads) {
    const int g = idx / D, c = idx % D;
    float M, lsum, o;
    wave_merge<D, G>(sh, g, c, M, lsum, o);
    if (a.nsplit == 1) {
      out[((size_t)bh * G + g) * D + c] = from_f32<T>(lsum > 0.f ? o / lsum : 0.f);
    } else {
      float* pp = a.part + (((size_t)bh * a.nsplit + split) * G + g) * (D + 2);
      pp[c] = o;
      if (c == 0) {
        pp[D] = M;
        pp[D + 1] = lsum;
      }
    }
  }
}

// Split merge: block = (b*Hkv+h); each wave reduces the splits' (max, sum) of its heads into
// per-split weights in LDS, then every output element sums its splits with independent loads.
template <typename T, int G>
__global__ __launch_bounds__(kAttThreads) void k_attend_merge(const float* __restrict__ part,
                                                          int nsplit, int D,
                                                          T* __restrict__ out) {
  constexpr int kMaxSplits = 256;
  __shared__ float s_w[kMaxSplits][G];
  __shared__ float s_inv[G];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const size_t stride = (size_t)G * (D + 2);
  const float* hp = part + (size_t)bh * nsplit * stride;
  for (int g = tid / kWave; g < G; g += kAttWaves) {
    const int lane = tid % kWave;
    float M = -INFINITY;
    for (int s = lane; s < nsplit; s += kWave) M = fmaxf(M, hp[s * stride + g * (D + 2) + D]);
    M = group_max<64>(M);
    float lsum = 0.f;
    for (int s = lane; s < nsplit; s += kWave) {
      const float ms = hp[s * stride + g * (D + 2) + D];
      const float w = ms == -INFINITY ? 0.f : exp2_hw(ms - M);
      s_w[s][g] = w;
      lsum = fmaf(hp[s * stride + g * (D + 2) + D + 1], w, lsum);
    }
    lsum = group_sum<64>(lsum);
    if (lane == 0) s_inv[g] = lsum > 0.f ? 1.f / lsum : 0.f;
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += kAttThreads) {
    const int g = idx / D, c = idx % D;
    const float* pc = hp + (size_t)g * (D + 2) + c;
    float o = 0.f;
#pragma unroll 8
    for (int s = 0; s < nsplit; ++s) o = fmaf(pc[s * stride], s_w[s][g], o);
    out[((size_t)bh * G + g) * D + c] = from_f32<T>(o * s_inv[g]);
  }
}

// ------------------------------------------------------------------------------ plans

constexpr int kTargetBlocks = 256;  // one block per CU of an MI355X
constexpr int kAttSoloTokens = 128;  // budgets up to this many tokens: one block per head

struct Plan {
  int nsplit, pps;
};

template <typename T, int D>
Plan plan_attend(int BH, int ps, int n_pages) {
  const int ntok = n_pages * ps;
  const int chunk = kAttWaves * Geo<T, D>::WTOK;
  int ns = (2 * kTargetBlocks + BH - 1) / BH;
  // a small budget goes to one block per head: its output is written without a merge launch
  ns = ntok <= kAttSoloTokens ? 1 : min(ns, (ntok + chunk - 1) / chunk);
  ns = max(ns, (n_pages + kMaxPagesPerSplit - 1) / kMaxPagesPerSplit);
  ns = max(min(ns, 256), 1);
  int pps = (n_pages + ns - 1) / ns;
  ns = (n_pages + pps - 1) / pps;
  return {ns, pps};
}

template <typename T, int D, int G>
hipError_t attend_g(AttendArgs a, int BH, hipStream_t stream) {
  hipLaunchKernelGGL((k_attend<T, D, G>), dim3(a.nsplit, BH), dim3(kAttThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  hipLaunchKernelGGL((k_attend_merge<T, G>), dim3(BH), dim3(kAttThreads), 0, stream, a.part,
                     a.nsplit, D, static_cast<T*>(a.out));
  return hipGetLastError();
}

#define RKV_DISPATCH_G(FN, ...)                      \
  switch (G) {                                       \
    case 1: return FN<T, D, 1>(__VA_ARGS__);         \
    case 2: return FN<T, D, 2>(__VA_ARGS__);         \
    case 3: return FN<T, D, 3>(__VA_ARGS__);         \
    case 4: return FN<T, D, 4>(__VA_ARGS__);         \
    case 5: return FN<T, D, 5>(__VA_ARGS__);         \
    case 6: return FN<T, D, 6>(__VA_ARGS__);         \
    case 7: return FN<T, D, 7>(__VA_ARGS__);         \
    case 8: return FN<T, D, 8>(__VA_ARGS__);         \
    default: return hipErrorInvalidValue;            \
  }

template <typename T, int D>
hipError_t attend_d(int G, AttendArgs a, int BH, hipStream_t s) { RKV_DISPATCH_G(attend_g, a, BH, s) }

Plan plan_attend_any(int dtype, int D, int BH, int ps, int n_pages) {
  if (dtype == 0)
    return D == 64 ? plan_attend<float, 64>(BH, ps, n_pages) : plan_attend<float, 128>(BH, ps, n_pages);
  return D == 64 ? plan_attend<bf16_t, 64>(BH, ps, n_pages) : plan_attend<bf16_t, 128>(BH, ps, n_pages);
}

}  // namespace

int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kTargetBlocks;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = kTargetBlocks;
    cache[dev] = n;
  }
  return min(cache[dev], kTargetBlocks);
}


size_t attend_ws_bytes(int B, int Hq, int Hkv, int D, int page_size, int n_pages, int dtype) {
  const Plan pl = plan_attend_any(dtype, D, B * Hkv, page_size, n_pages);
  if (pl.nsplit == 1) return 0;
  return (size_t)B * Hkv * pl.nsplit * (Hq / Hkv) * (D + 2) * sizeof(float);
}

hipError_t launch_sparse_attend_view(const void* q, const void* k, const void* v,
                                     const int32_t* rows, const int32_t* page_idx, int B, int Hq,
                                     int Hkv, int Lc, int kv_pitch, int D, int page_size,
                                     int n_pages, float scale, int dtype, void* out, void* ws,
                                     hipStream_t stream) {
  const int BH = B * Hkv;
  const Plan pl = plan_attend_any(dtype, D, BH, page_size, n_pages);
  AttendArgs a{q,        k,          v,         page_idx, rows,   Lc,
               kv_pitch, page_size,  n_pages,   (Lc + page_size - 1) / page_size,
               pl.pps,   pl.nsplit,  scale * kLog2e, static_cast<float*>(ws), out};
  const int G = Hq / Hkv;
  if (dtype == 0)
    return D == 64 ? attend_d<float, 64>(G, a, BH, stream) : attend_d<float, 128>(G, a, BH, stream);
  return D == 64 ? attend_d<bf16_t, 64>(G, a, BH, stream) : attend_d<bf16_t, 128>(G, a, BH, stream);
}

hipError_t launch_sparse_attend(const void* q, const void* k_c, const void* v_c,
                                const int32_t* page_idx, int B, int Hq, int Hkv, int Lc, int D,
                                int page_size, int n_pages, float scale, int dtype, void* out,
                                void* ws, hipStream_t stream) {
  return launch_sparse_attend_view(q, k_c, v_c, nullptr, page_idx, B, Hq, Hkv, Lc, Lc, D,
                                   page_size, n_pages, scale, dtype, out, ws, stream);
}

}  // namespace rkv
