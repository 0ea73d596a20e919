// Exact per-row top-k by radix select on order-preserving 32-bit keys (RocketKV rebuttal,
// "Explanation of Calculating Approximate Attention Scores": select the pages with higher
// scores; "Measurement of Exact-TopK": SnapKV's one-time top-k filter of the prompt).
//
// Rows of up to 8192 elements (page scores of a decode step): one 256-thread block per row holds
// the row in registers and runs the block select of rkv_select.hpp. Longer rows (prompt token
// scores): one 1024-thread block per row, four 8-bit digit passes over LDS histograms that
// re-read the row each pass (it is L2-resident after the first), then an ordered compaction.
#include "rkv_common.hpp"
#include "rkv_launch.hpp"
#include "rkv_select.hpp"

namespace rkv {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kTile = kThreads * 4;  // elements per tile: 4 consecutive per thread

struct TopkShared {
  uint32_t hist[256];
  uint32_t wave_a[kWaves];
  uint32_t wave_b[kWaves];
  uint32_t digit;
  uint32_t above;
};

// Exclusive block scan of two counters; also returns the block totals.
__device__ __forceinline__ void block_scan2(uint32_t a, uint32_t b, uint32_t& ea, uint32_t& eb,
                                            uint32_t& ta, uint32_t& tb, TopkShared& sh) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  uint32_t ia = a, ib = b;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t xa = __shfl_up(ia, o, kWave);
    const uint32_t xb = __shfl_up(ib, o, kWave);
    if (lane >= o) {
      ia += xa;
      ib += xb;
    }
  }
  if (lane == kWave - 1) {
    sh.wave_a[wave] = ia;
    sh.wave_b[wave] = ib;
  }
  __syncthreads();
  uint32_t pa = 0, pb = 0, sa = 0, sb = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t va = sh.wave_a[w], vb = sh.wave_b[w];
    if (w < wave) {
      pa += va;
      pb += vb;
    }
    sa += va;
    sb += vb;
  }
  ea = pa + ia - a;
  eb = pb + ib - b;
  ta = sa;
  tb = sb;
  __syncthreads();
}

__device__ __forceinline__ void load4(const float* __restrict__ s, int n, int i0, uint32_t (&key)[4],
                                      bool (&ok)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = i0 + e;
    ok[e] = i < n;
    key[e] = ok[e] ? order_key(s[i]) : 0u;
  }
}

template <int R>
__global__ __launch_bounds__(kThreads) void k_topk(const float* __restrict__ scores, int n, int k,
                                                   int32_t* __restrict__ out, int out_stride) {
  __shared__ TopkShared sh;
  const int tid = threadIdx.x;
  const float* s = scores + (size_t)blockIdx.x * n;
  int32_t* o = out + (size_t)blockIdx.x * out_stride;
  if (k >= n) {
    for (int i = tid; i < n; i += kThreads) o[i] = i;
    return;
  }
  if (k <= 0) return;
  const int ntiles = (n + kTile - 1) / kTile;

  uint32_t rkey[R > 0 ? R : 1][4];
  bool rok[R > 0 ? R : 1][4];
  if constexpr (R > 0) {
#pragma unroll
    for (int t = 0; t < R; ++t) load4(s, n, (t * kThreads + tid) * 4, rkey[t], rok[t]);
  }

  uint32_t prefix = 0, mask = 0;
  uint32_t krem = (uint32_t)k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) sh.hist[tid] = 0;
    __syncthreads();
    auto count4 = [&](const uint32_t (&key)[4], const bool (&ok)[4]) {
      // merge equal digits of the thread's four elements before touching LDS
      uint32_t d[4];
      uint32_t c[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool m = ok[e] && ((key[e] & mask) == prefix);
        d[e] = (key[e] >> shift) & 255u;
        c[e] = m ? 1u : 0u;
      }
#pragma unroll
      for (int e = 1; e < 4; ++e) {
#pragma unroll
        for (int f = 0; f < e; ++f) {
          if (c[e] && c[f] && d[f] == d[e]) {
            c[f] += c[e];
            c[e] = 0;
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (c[e]) atomicAdd(&sh.hist[d[e]], c[e]);
    };
    if constexpr (R > 0) {
#pragma unroll
      for (int t = 0; t < R; ++t) count4(rkey[t], rok[t]);
    } else {
      for (int t = 0; t < ntiles; ++t) {
        uint32_t key[4];
        bool ok[4];
        load4(s, n, (t * kThreads + tid) * 4, key, ok);
        count4(key, ok);
      }
    }
    __syncthreads();
    if (tid < kWave) {
      // lane l owns digits 255-4l .. 252-4l (descending); find the digit holding the krem-th key
      uint32_t c4 = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) c4 += sh.hist[255 - 4 * tid - j];
      uint32_t incl = c4;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t x = __shfl_up(incl, off, kWave);
        if (tid >= off) incl += x;
      }
      const uint32_t excl = incl - c4;
      if (excl < krem && krem <= incl) {
        uint32_t run = excl;
        for (int j = 0; j < 4; ++j) {
          const uint32_t dgt = 255 - 4 * tid - j;
          const uint32_t c = sh.hist[dgt];
          if (run + c >= krem) {
            sh.digit = dgt;
            sh.above = run;
            break;
          }
          run += c;
        }
      }
    }
    __syncthreads();
    prefix |= sh.digit << shift;
    mask |= 255u << shift;
    krem -= sh.above;
    __syncthreads();
  }
  const uint32_t T = prefix;
  const uint32_t need_eq = krem;  // elements equal to T that are taken (lowest indices first)

  uint32_t carry_gt = 0, carry_eq = 0;
  auto emit4 = [&](const uint32_t (&key)[4], const bool (&ok)[4], int i0) {
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ngt += (ok[e] && key[e] > T);
      neq += (ok[e] && key[e] == T);
    }
    uint32_t egt, eeq, tgt, teq;
    block_scan2(ngt, neq, egt, eeq, tgt, teq, sh);
    uint32_t bg = carry_gt + egt, be = carry_eq + eeq;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (!ok[e]) continue;
      if (key[e] > T) {
        const uint32_t pos = bg + (be < need_eq ? be : need_eq);
        if (pos < (uint32_t)k) o[pos] = i0 + e;
        ++bg;
      } else if (key[e] == T) {
        if (be < need_eq && bg + be < (uint32_t)k) o[bg + be] = i0 + e;
        ++be;
      }
    }
    carry_gt += tgt;
    carry_eq += teq;
  };
  if constexpr (R > 0) {
#pragma unroll
    for (int t = 0; t < R; ++t) emit4(rkey[t], rok[t], (t * kThreads + tid) * 4);
  } else {
    for (int t = 0; t < ntiles; ++t) {
      uint32_t key[4];
      bool ok[4];
      const int i0 = (t * kThreads + tid) * 4;
      load4(s, n, i0, key, ok);
      emit4(key, ok, i0);
    }
  }
}

constexpr int kBlockThreads = 256;

template <int E>
__global__ __launch_bounds__(kBlockThreads) void k_topk_block(const float* __restrict__ scores,
                                                             int n, int k,
                                                             int32_t* __restrict__ out,
                                                             int out_stride) {
  __shared__ SelectShared<kBlockThreads> sh;
  const float* row = scores + (size_t)blockIdx.x * n;
  int32_t* o = out + (size_t)blockIdx.x * out_stride;
  if (k >= n) {
    for (int i = threadIdx.x; i < n; i += kBlockThreads) o[i] = i;
    return;
  }
  if (k <= 0) return;
  uint32_t key[E];
  const int i0 = threadIdx.x * E;
  const int nv = load_keys<E>(row, n, i0, key);
  uint32_t T, need_eq;
  block_threshold<kBlockThreads, E>(key, nv, (uint32_t)k, T, need_eq, sh);
  block_compact<kBlockThreads, E>(key, nv, T, need_eq, i0, 0u, (uint32_t)k, sh,
                                  [&](uint32_t pos, int idx, bool take) {
                                    if (take && pos < (uint32_t)k) o[pos] = idx;
                                  });
}

}  // namespace

size_t topk_ws_bytes(int, int, int) { return 0; }

hipError_t launch_topk(const float* scores, int rows, int n, int k, int32_t* out, int out_stride,
                       void*, hipStream_t stream) {
  dim3 grid(rows);
  if (n <= 16 * kBlockThreads)
    hipLaunchKernelGGL(k_topk_block<16>, grid, dim3(kBlockThreads), 0, stream, scores, n, k, out,
                       out_stride);
  else if (n <= 32 * kBlockThreads)
    hipLaunchKernelGGL(k_topk_block<32>, grid, dim3(kBlockThreads), 0, stream, scores, n, k, out,
                       out_stride);
  else
    hipLaunchKernelGGL(k_topk<0>, grid, dim3(kThreads), 0, stream, scores, n, k, out, out_stride);
  return hipGetLastError();
}

}  // namespace rkv
