// Block-wide exact top-k over a row held in registers (RocketKV rebuttal, "Explanation of
// Calculating Approximate Attention Scores": select the pages with higher scores).
//
// Thread t holds elements [t*E, t*E+E) of the row as order-preserving 32-bit keys. The block
// first reduces the minimum and maximum key: bits above their highest differing bit are common
// to every element, so the 8-bit radix digits start right below them (the first digit then
// spreads over bins instead of piling onto one, which matters for LDS histogram atomics).
// Digit passes narrow the k-th largest key T; an ordered compaction then gives every element
// above T, and the lowest-index elements equal to T, its position in the ascending list.
#pragma once

#include "rkv_common.hpp"

namespace rkv {

template <int THREADS>
struct SelectShared {
  uint32_t hist[256];
  uint32_t wa[THREADS / kWave];
  uint32_t wb[THREADS / kWave];
  uint32_t digit, above;
};

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, kWave));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, kWave));
  return v;
}

// Exclusive scan of two counters over the block, plus the totals. Contains two barriers.
template <int THREADS>
__device__ __forceinline__ void block_scan2(uint32_t a, uint32_t b, uint32_t& ea, uint32_t& eb,
                                            uint32_t& ta, uint32_t& tb, SelectShared<THREADS>& sh) {
  constexpr int NW = THREADS / kWave;
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
    sh.wa[wave] = ia;
    sh.wb[wave] = ib;
  }
  __syncthreads();
  uint32_t pa = 0, pb = 0, sa = 0, sb = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t va = sh.wa[w], vb = sh.wb[w];
    pa += w < wave ? va : 0u;
    pb += w < wave ? vb : 0u;
    sa += va;
    sb += vb;
  }
  ea = pa + ia - a;
  eb = pb + ib - b;
  ta = sa;
  tb = sb;
  __syncthreads();
}

// Finds T (the k-th largest key) and need_eq (how many keys equal to T are taken), for
// 1 <= k < number of valid keys. Every thread of the block must call it.
template <int THREADS, int E>
__device__ __forceinline__ void block_threshold(const uint32_t (&key)[E], int nvalid,
                                                uint32_t k, uint32_t& T, uint32_t& need_eq,
                                                SelectShared<THREADS>& sh) {
  constexpr int NW = THREADS / kWave;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (e < nvalid) {
      lo = min(lo, key[e]);
      hi = max(hi, key[e]);
    }
  }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (lane == 0) {
    sh.wa[wave] = lo;
    sh.wb[wave] = hi;
  }
  __syncthreads();
  lo = sh.wa[0];
  hi = sh.wb[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    lo = min(lo, sh.wa[w]);
    hi = max(hi, sh.wb[w]);
  }
  __syncthreads();
  if (lo == hi) {  // all keys equal
    T = lo;
    need_eq = k;
    return;
  }
  int bits = 32 - __clz(lo ^ hi);  // low bits that still vary
  uint32_t prefix = bits >= 32 ? 0u : (lo >> bits) << bits;
  uint32_t mask = bits >= 32 ? 0u : ~((1u << bits) - 1u);
  uint32_t krem = k;
  while (bits > 0) {
    const int shift = bits > 8 ? bits - 8 : 0;
    if (tid < 256) sh.hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (e < nvalid && (key[e] & mask) == prefix) atomicAdd(&sh.hist[(key[e] >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < kWave) {
      // lane l owns digits 255-4l .. 252-4l (descending)
      uint32_t c[4], c4 = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = sh.hist[255 - 4 * tid - j];
        c4 += c[j];
      }
      uint32_t incl = c4;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t x = __shfl_up(incl, off, kWave);
        if (tid >= off) incl += x;
      }
      const uint32_t excl = incl - c4;
      if (excl < krem && krem <= incl) {
        uint32_t run = excl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (run < krem && krem <= run + c[j]) {
            sh.digit = 255 - 4 * tid - j;
            sh.above = run;
          }
          run += c[j];
        }
      }
    }
    __syncthreads();
    prefix |= sh.digit << shift;
    mask |= 255u << shift;
    krem -= sh.above;
    bits = shift;
    __syncthreads();
  }
  T = prefix;
  need_eq = krem;
}

// Ascending positions of the selected elements. emit(pos, index) is called once per selected
// element (pos < k). Contains barriers; every thread of the block must call it.
template <int THREADS, int E, typename Emit>
__device__ __forceinline__ void block_compact(const uint32_t (&key)[E], int nvalid, uint32_t T,
                                              uint32_t need_eq, int base_index,
                                              SelectShared<THREADS>& sh, Emit&& emit) {
  uint32_t ngt = 0, neq = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    ngt += (e < nvalid && key[e] > T);
    neq += (e < nvalid && key[e] == T);
  }
  uint32_t bg, be, tg, te;
  block_scan2<THREADS>(ngt, neq, bg, be, tg, te, sh);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (e >= nvalid) continue;
    if (key[e] > T) {
      emit(bg + (be < need_eq ? be : need_eq), base_index + e);
      ++bg;
    } else if (key[e] == T) {
      if (be < need_eq) emit(bg + be, base_index + e);
      ++be;
    }
  }
}

// Loads the E consecutive scores of a row starting at i0 (blocked layout) as keys; returns how
// many of them exist (0..E).
template <int E>
__device__ __forceinline__ int load_keys(const float* __restrict__ row, int n, int i0,
                                         uint32_t (&key)[E]) {
  if ((((uintptr_t)(row + i0)) & 15u) == 0 && i0 + E <= n) {
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      const float4 v = *reinterpret_cast<const float4*>(row + i0 + e);
      key[e] = order_key(v.x);
      key[e + 1] = order_key(v.y);
      key[e + 2] = order_key(v.z);
      key[e + 3] = order_key(v.w);
    }
    return E;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) key[e] = i0 + e < n ? order_key(row[i0 + e]) : 0u;
  return n - i0 < 0 ? 0 : (n - i0 > E ? E : n - i0);
}

// Same, reading through device-coherent loads (scores written by other blocks of the grid).
template <int E>
__device__ __forceinline__ int load_keys_coherent(const float* __restrict__ row, int n, int i0,
                                                  uint32_t (&key)[E]) {
#pragma unroll
  for (int e = 0; e < E; ++e)
    key[e] = i0 + e < n ? order_key(__hip_atomic_load(row + i0 + e, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT))
                        : 0u;
  return n - i0 < 0 ? 0 : (n - i0 > E ? E : n - i0);
}

}  // namespace rkv
