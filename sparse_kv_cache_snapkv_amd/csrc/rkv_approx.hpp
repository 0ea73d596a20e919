// Block-level pieces of the hybrid approximate page scores (RocketKV rebuttal, "Explanation of
// Calculating Approximate Attention Scores": bound max(q*Kmin, q*Kmax) on the channels where
// |q| is large, one of Kmin/Kmax fetched per channel by the sign of q, GQA-consistent through
// the group sums of q and |q|).
#pragma once

#include "rkv_common.hpp"

namespace rkv {

constexpr int kApproxMaxD = 128;

struct ChannelShared {
  int chan[kApproxMaxD];  // j-th chosen channel, ascending
  float qc[kApproxMaxD];  // sum_g q_g of the j-th chosen channel
};

// Chooses the r channels with the largest sum_g |q_g[c]| of group (b, h) (ties: lower channel)
// and lists them ascending in sh.chan, with sum_g q_g[c] in sh.qc. Wave 0 does the work: lane l
// holds channels 2l and 2l+1 (D even, at most 128); the r-th largest sum is found exactly by a
// bitwise search over ballot counts of the sums' bit patterns (non-negative floats order like
// their bits), then the channels above it and the lowest-index ones equal to it are placed by
// ballot prefix counts. Both sums run over g in ascending order. Contains one barrier; every
// thread of the block must call it.
template <typename T, int G>
__device__ __forceinline__ void select_channels_block(const T* __restrict__ q, int b, int h,
                                                      int Hkv, int D, int r, ChannelShared& sh) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int c0 = 2 * lane;
    const bool valid = c0 < D;
    const T* qg = q + ((size_t)b * Hkv + h) * G * D + (valid ? c0 : 0);
    float x0[G], x1[G];
    if constexpr (sizeof(T) == 2) {
      uint32_t raw[G];  // every load in flight before the first use
#pragma unroll
      for (int g = 0; g < G; ++g) raw[g] = *reinterpret_cast<const uint32_t*>(qg + (size_t)g * D);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        x0[g] = __uint_as_float(raw[g] << 16);
        x1[g] = __uint_as_float(raw[g] & 0xffff0000u);
      }
    } else {
      float2 raw[G];
#pragma unroll
      for (int g = 0; g < G; ++g) raw[g] = *reinterpret_cast<const float2*>(qg + (size_t)g * D);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        x0[g] = raw[g].x;
        x1[g] = raw[g].y;
      }
    }
    float a0 = 0.f, a1 = 0.f, s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      a0 += fabsf(x0[g]);
      a1 += fabsf(x1[g]);
      s0 += x0[g];
      s1 += x1[g];
    }
    // keys: a real channel sets the top bit above its sum's bits, padding lanes stay 0
    const uint32_t k0 = valid ? (__float_as_uint(a0) | 0x80000000u) : 0u;
    const uint32_t k1 = valid ? (__float_as_uint(a1) | 0x80000000u) : 0u;
    uint32_t thr = 0x80000000u;  // at least D >= r keys are >= it
#pragma unroll
    for (int bit = 30; bit >= 0; --bit) {
      const uint32_t cand = thr | (1u << bit);
      const int cnt = __popcll(__ballot(k0 >= cand)) + __popcll(__ballot(k1 >= cand));
      if (cnt >= r) thr = cand;
    }
    const uint64_t eq0 = __ballot(k0 == thr), eq1 = __ballot(k1 == thr);
    const int need = r - (__popcll(__ballot(k0 > thr)) + __popcll(__ballot(k1 > thr)));
    const uint64_t below = (1ull << lane) - 1ull;
    const int eq_below0 = __popcll(eq0 & below) + __popcll(eq1 & below);
    const int eq_below1 = eq_below0 + (int)((eq0 >> lane) & 1ull);
    const bool t0 = k0 > thr || (k0 == thr && eq_below0 < need);
    const bool t1 = k1 > thr || (k1 == thr && eq_below1 < need);
    const uint64_t b0 = __ballot(t0), b1 = __ballot(t1);
    const int pos0 = __popcll(b0 & below) + __popcll(b1 & below);
    const int pos1 = pos0 + (t0 ? 1 : 0);
    if (t0) {
      sh.chan[pos0] = c0;
      sh.qc[pos0] = s0;
    }
    if (t1) {
      sh.chan[pos1] = c0 + 1;
      sh.qc[pos1] = s1;
    }
  }
  __syncthreads();
}

// Channel partition of the page-score sum: group g sums chosen channels g, g+4, g+8, ... in
// ascending order, and the four group sums are combined as (s0 + s1) + (s2 + s3). Every kernel
// that scores pages uses this order, so they all produce the same bits.
constexpr int kScoreGroups = 4;
constexpr int kScoreBatch = 8;  // row loads a lane has in flight at once

// Thread layout: lane = 4 * vector + group. VEC: a vector is 16 bytes of consecutive pages
// (p_begin a multiple of the vector width, P a multiple of it); otherwise one page per vector.
// Scores pages [p_begin, p_end) of one (b, h) and hands each score to sink(page, value), called
// by one lane per page. No barrier; the whole quad of a vector must be active together.
template <typename T, bool VEC, typename Sink>
__device__ __forceinline__ void score_page_range(const T* __restrict__ kmin_bh,
                                                 const T* __restrict__ kmax_bh, int D, int P,
                                                 int r, int p_begin, int p_end,
                                                 const ChannelShared& ch, Sink&& sink) {
  constexpr int V = VEC ? vec16<T>::n : 1;
  const int grp = threadIdx.x % kScoreGroups;
  const int nvec_pass = blockDim.x / kScoreGroups;
  const int nvec = (p_end - p_begin + V - 1) / V;
  const int nj = (r - grp + kScoreGroups - 1) / kScoreGroups;  // channels of this group
  for (int v0 = 0; v0 < nvec; v0 += nvec_pass) {  // uniform trip count across the block
    const int vi = v0 + (int)threadIdx.x / kScoreGroups;
    const bool active = vi < nvec;
    const int p = p_begin + (active ? vi : 0) * V;
    float acc[V];
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] = 0.f;
    for (int t0 = 0; t0 < nj; t0 += kScoreBatch) {
      // all of the batch's loads are issued before the first multiply
      float qcv[kScoreBatch];
      const T* rows[kScoreBatch];
#pragma unroll
      for (int u = 0; u < kScoreBatch; ++u) {
        const int t = t0 + u;
        const int j = grp + (t < nj ? t : 0) * kScoreGroups;
        qcv[u] = t < nj ? ch.qc[j] : 0.f;
        const int c = min(max(ch.chan[j], 0), D - 1);
        rows[u] = (qcv[u] >= 0.f ? kmax_bh : kmin_bh) + (size_t)c * P + p;
      }
      if constexpr (VEC) {
        uint4 raw[kScoreBatch];
#pragma unroll
        for (int u = 0; u < kScoreBatch; ++u) raw[u] = load16(rows[u]);
#pragma unroll
        for (int u = 0; u < kScoreBatch; ++u) {
          float x[V];
          unpack16<T>(raw[u], x);
          const bool use = t0 + u < nj;
#pragma unroll
          for (int e = 0; e < V; ++e) acc[e] = use ? fmaf(qcv[u], x[e], acc[e]) : acc[e];
        }
      } else {
        T raw[kScoreBatch];
#pragma unroll
        for (int u = 0; u < kScoreBatch; ++u) raw[u] = rows[u][0];
#pragma unroll
        for (int u = 0; u < kScoreBatch; ++u)
          acc[0] = t0 + u < nj ? fmaf(qcv[u], to_f32(raw[u]), acc[0]) : acc[0];
      }
    }
#pragma unroll
    for (int e = 0; e < V; ++e) {
      acc[e] += dpp<kDppXor1>(acc[e]);
      acc[e] += dpp<kDppXor2>(acc[e]);
    }
    if (active) {
      // lane `grp` of the quad hands over pages grp, grp+4 of its vector (all lanes hold the sums)
#pragma unroll
      for (int e = 0; e < V; ++e)
        if (e % kScoreGroups == grp && p + e < p_end) sink(p + e, acc[e]);
    }
  }
}

}  // namespace rkv
