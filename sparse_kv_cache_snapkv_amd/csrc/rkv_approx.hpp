// Block-level pieces of the hybrid approximate page scores (RocketKV rebuttal, "Explanation of
// Calculating Approximate Attention Scores": bound max(q*Kmin, q*Kmax) on the channels where
// |q| is large, one of Kmin/Kmax fetched per channel by the sign of q, GQA-consistent through
// the group sums of q and |q|).
#pragma once

#include "rkv_common.hpp"

namespace rkv {

constexpr int kApproxMaxD = 128;

struct ChannelShared {
  __align__(16) float a[kApproxMaxD];  // sum_g |q_g[c]|
  float qb[kApproxMaxD];               // sum_g q_g[c]
  float qc[kApproxMaxD];               // qbar of the j-th chosen channel
  int chan[kApproxMaxD];               // j-th chosen channel, ascending
  unsigned cnt[2];
};

// Chooses the r channels with the largest sum |q| (ties: lower channel) of group (b, h) and
// lists them ascending in sh.chan / sh.qc. Works for any block of >= 64 threads; contains three
// barriers, every thread must call it.
template <typename T>
__device__ __forceinline__ void select_channels_block(const T* __restrict__ q, int b, int h,
                                                      int Hkv, int G, int D, int r,
                                                      ChannelShared& sh) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int nthr = blockDim.x, nw = nthr / kWave;
  for (int c = tid; c < kApproxMaxD; c += nthr) {
    float a = 0.f, sq = 0.f;
    if (c < D) {
      const T* qg = q + ((size_t)b * Hkv * G + (size_t)h * G) * D + c;
      for (int g = 0; g < G; ++g) {
        const float x = to_f32(qg[(size_t)g * D]);
        a += fabsf(x);
        sq += x;
      }
    }
    sh.a[c] = c < D ? a : -1.f;  // padding ranks below every real channel (a >= 0)
    sh.qb[c] = sq;
    sh.chan[c] = 0;              // every slot valid even if ranks were not a permutation
    sh.qc[c] = 0.f;
  }
  __syncthreads();
  // wave w ranks channel chunks w, w+nw (of 64 channels each)
  unsigned long long ball[2] = {0ull, 0ull};
  for (int ck = wave; ck < 2; ck += nw) {
    const int c = ck * kWave + lane;
    bool sel = false;
    if (c < D) {
      const float a = sh.a[c];
      int rank = 0;
#pragma unroll
      for (int o = 0; o < kApproxMaxD; o += 4) {
        const float4 v = *reinterpret_cast<const float4*>(&sh.a[o]);
        rank += (v.x > a) || (v.x == a && o < c);
        rank += (v.y > a) || (v.y == a && o + 1 < c);
        rank += (v.z > a) || (v.z == a && o + 2 < c);
        rank += (v.w > a) || (v.w == a && o + 3 < c);
      }
      sel = rank < r;
    }
    ball[ck] = __ballot(sel);
    if (lane == 0) sh.cnt[ck] = (unsigned)__popcll(ball[ck]);
  }
  __syncthreads();
  for (int ck = wave; ck < 2; ck += nw) {
    const int c = ck * kWave + lane;
    if ((ball[ck] >> lane) & 1ull) {
      const unsigned pos = (unsigned)__popcll(ball[ck] & ((1ull << lane) - 1ull)) +
                           (ck == 1 ? sh.cnt[0] : 0u);
      sh.chan[pos] = c;
      sh.qc[pos] = sh.qb[c];
    }
  }
  __syncthreads();
}

// Channel partition of the page-score sum: group g sums chosen channels g, g+4, g+8, ... in
// ascending order, and the four group sums are combined as (s0 + s1) + (s2 + s3). Every kernel
// that scores pages uses this order, so they all produce the same bits.
constexpr int kScoreGroups = 4;

// Thread layout: lane = 4 * vector + group. Scores the VMAX consecutive pages of vector
// `pv` = p_begin/V + tid/4 of one (b, h) over [p_begin, p_end) (p_begin a multiple of VMAX when
// `vec`; `vec` requires P to be a multiple of VMAX, otherwise one page per vector).
// COHERENT: store with device-coherent (write-through) stores for other blocks to read.
// No barrier; the whole quad of a vector must be active together.
template <typename T, bool COHERENT>
__device__ __forceinline__ void score_page_range(const T* __restrict__ kmin_bh,
                                                 const T* __restrict__ kmax_bh, int D, int P,
                                                 int r, int p_begin, int p_end, bool vec,
                                                 const ChannelShared& ch,
                                                 float* __restrict__ scores_row) {
  constexpr int VMAX = vec16<T>::n;
  const int V = vec ? VMAX : 1;
  const int grp = threadIdx.x % kScoreGroups;
  const int nvec_pass = blockDim.x / kScoreGroups;
  const int nvec = (p_end - p_begin + V - 1) / V;
  const int nj = (r - grp + kScoreGroups - 1) / kScoreGroups;  // channels of this group
  for (int v0 = 0; v0 < nvec; v0 += nvec_pass) {  // uniform trip count across the block
    const int vi = v0 + (int)threadIdx.x / kScoreGroups;
    const bool active = vi < nvec;
    const int p = p_begin + (active ? vi : 0) * V;
    float acc[VMAX];
#pragma unroll
    for (int e = 0; e < VMAX; ++e) acc[e] = 0.f;
    if (active) {
#pragma unroll 8
      for (int t = 0; t < nj; ++t) {
        const int j = grp + t * kScoreGroups;
        const float qc = ch.qc[j];
        const int c = min(max(ch.chan[j], 0), D - 1);
        const T* row = (qc >= 0.f ? kmax_bh : kmin_bh) + (size_t)c * P + p;
        if (vec) {
          float x[VMAX];
          unpack16<T>(load16(row), x);
#pragma unroll
          for (int e = 0; e < VMAX; ++e) acc[e] = fmaf(qc, x[e], acc[e]);
        } else {
          acc[0] = fmaf(qc, to_f32(row[0]), acc[0]);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < VMAX; ++e) {
      acc[e] += dpp<kDppXor1>(acc[e]);
      acc[e] += dpp<kDppXor2>(acc[e]);
    }
    if (active) {
      // lane `grp` of the quad stores pages grp, grp+4 of its vector (all lanes hold the sums)
      for (int e = grp; e < V; e += kScoreGroups) {
        if (p + e < p_end) {
          if constexpr (COHERENT)
            __hip_atomic_store(scores_row + p + e, acc[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          else
            scores_row[p + e] = acc[e];
        }
      }
    }
  }
}

}  // namespace rkv
