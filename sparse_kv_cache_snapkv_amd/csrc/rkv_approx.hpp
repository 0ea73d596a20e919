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

// Bound of the VMAX consecutive pages starting at p (of one (b, h); P a multiple of VMAX when
// `vec`, else one page in out[0]). The chosen channels are summed in ascending order, so every
// kernel that scores pages produces the same bits.
template <typename T>
__device__ __forceinline__ void score_page_vector(const T* __restrict__ kmin_bh,
                                                  const T* __restrict__ kmax_bh, int D, int P,
                                                  int r, int p, bool vec, const ChannelShared& ch,
                                                  float (&out)[vec16<T>::n]) {
  constexpr int VMAX = vec16<T>::n;
#pragma unroll
  for (int e = 0; e < VMAX; ++e) out[e] = 0.f;
#pragma unroll 8
  for (int j = 0; j < r; ++j) {
    const float qc = ch.qc[j];
    const int c = min(max(ch.chan[j], 0), D - 1);
    const T* row = (qc >= 0.f ? kmax_bh : kmin_bh) + (size_t)c * P + p;
    if (vec) {
      float x[VMAX];
      unpack16<T>(load16(row), x);
#pragma unroll
      for (int e = 0; e < VMAX; ++e) out[e] = fmaf(qc, x[e], out[e]);
    } else {
      out[0] = fmaf(qc, to_f32(row[0]), out[0]);
    }
  }
}

// Scores pages [p_begin, p_end) of one (b, h) into scores_row, one page vector per thread per
// pass. No barrier.
template <typename T>
__device__ __forceinline__ void score_page_range(const T* __restrict__ kmin_bh,
                                                 const T* __restrict__ kmax_bh, int D, int P,
                                                 int r, int p_begin, int p_end, bool vec,
                                                 const ChannelShared& ch,
                                                 float* __restrict__ scores_row) {
  constexpr int VMAX = vec16<T>::n;
  const int V = vec ? VMAX : 1;
  for (int p = p_begin + (int)threadIdx.x * V; p < p_end; p += (int)blockDim.x * V) {
    float s[VMAX];
    score_page_vector<T>(kmin_bh, kmax_bh, D, P, r, p, vec, ch, s);
    if (vec && p + VMAX <= p_end) {
      float4* dst = reinterpret_cast<float4*>(scores_row + p);
#pragma unroll
      for (int e = 0; e < VMAX; e += 4) dst[e / 4] = make_float4(s[e], s[e + 1], s[e + 2], s[e + 3]);
    } else {
      for (int e = 0; e < V && p + e < p_end; ++e) scores_row[p + e] = s[e];
    }
  }
}

}  // namespace rkv
