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
  __align__(16) uint64_t key[kApproxMaxD];  // {sum |q| bits, 127 - channel}: distinct, ordered
  float qb[kApproxMaxD];
  unsigned rank[8][kApproxMaxD];            // partial ranks over the parts of the keys
};

// Chooses the r channels with the largest sum_g |q_g[c]| of group (b, h) (ties: lower channel)
// and lists them ascending in sh.chan, with sum_g q_g[c] in sh.qc. Both sums run over g in
// ascending order. Each channel gets a distinct 64-bit key (the sum's bits, which order like the
// value for non-negative floats, above 127 - c, so equal sums rank the lower channel higher);
// the keys split into PARTS parts and each of the block's THREADS threads counts, for
// 128 * PARTS / THREADS channels, the keys of one part above that channel's key (more parts, a
// shorter chain of LDS reads per thread: 16 keys each with 8 parts in 512 threads, 32 with 4 in
// 256); the parts add up to each channel's rank. Wave 0 then places the channels of rank < r in
// ascending channel order by ballot prefix counts. The block must have exactly THREADS threads
// and every thread must take every step: load, then phase 1 (which ends with a barrier), then
// phase 2 (two barriers). The load is separate so that a kernel can issue its other first loads before
// any of them is waited for.
template <typename T, int G>
struct ChannelQ {
  float x[G];  // q_g[c] of this thread's channel c = tid % kApproxMaxD (clamped into the row)
  __device__ __forceinline__ void load(const T* __restrict__ q, int b, int h, int Hkv, int D) {
    const int c = (int)threadIdx.x % kApproxMaxD;
    const T* qg = q + ((size_t)b * Hkv + h) * G * D + (c < D ? c : 0);
#pragma unroll
    for (int g = 0; g < G; ++g) x[g] = to_f32(qg[(size_t)g * D]);
  }
};

template <typename T, int G>
__device__ __forceinline__ void select_channels_phase1(const ChannelQ<T, G>& cq, int D,
                                                       ChannelShared& sh) {
  const int tid = threadIdx.x;
  if (tid < kApproxMaxD) {
    const int c = tid;
    float a = 0.f, sq = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      a += fabsf(cq.x[g]);
      sq += cq.x[g];
    }
    // padding channels (c >= D) get key 0, below every real one
    sh.key[c] = c < D ? (((uint64_t)__float_as_uint(a) + 1ull) << 7) | (uint64_t)(127 - c) : 0ull;
    sh.qb[c] = sq;
  }
  lds_barrier();
}

struct NoHook {
  __device__ void operator()() const {}
};

// before_last_barrier() runs (in every thread) just before the final barrier, so that what it
// writes to LDS is visible to the whole block on return.
template <int PARTS = 2, int THREADS = 256, typename Hook = NoHook>
__device__ __forceinline__ void select_channels_phase2(int D, int r, ChannelShared& sh,
                                                       Hook&& before_last_barrier = Hook{}) {
  static_assert(PARTS >= 2 && PARTS <= 8 && kApproxMaxD % PARTS == 0, "parts of the keys");
  constexpr int PK = kApproxMaxD / PARTS;             // keys per part
  constexpr int CPT = kApproxMaxD * PARTS / THREADS;  // channels per thread
  constexpr int CS = kApproxMaxD / CPT;               // stride between a thread's channels
  static_assert(CPT >= 1 && CPT * THREADS == kApproxMaxD * PARTS, "threads per part");
  const int tid = threadIdx.x;
  const int part = tid / CS, c0 = tid % CS;
  uint64_t kc[CPT];
  unsigned above[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    kc[i] = sh.key[c0 + i * CS];
    above[i] = 0u;
  }
#pragma unroll
  for (int j = 0; j < PK; j += 2) {
    const ulonglong2 kk = *reinterpret_cast<const ulonglong2*>(&sh.key[part * PK + j]);
#pragma unroll
    for (int i = 0; i < CPT; ++i) above[i] += (kk.x > kc[i]) + (kk.y > kc[i]);
  }
#pragma unroll
  for (int i = 0; i < CPT; ++i) sh.rank[part][c0 + i * CS] = above[i];
  lds_barrier();
  if (tid < kWave) {
    const int lane = tid;
    unsigned r0 = 0, r1 = 0;
#pragma unroll
    for (int q = 0; q < PARTS; ++q) {
      r0 += sh.rank[q][lane];
      r1 += sh.rank[q][lane + kWave];
    }
    const bool t0 = lane < D && r0 < (unsigned)r;
    const bool t1 = lane + kWave < D && r1 < (unsigned)r;
    const uint64_t b0 = __ballot(t0), b1 = __ballot(t1);
    const uint64_t below = (1ull << lane) - 1ull;
    if (t0) {
      const int pos = __popcll(b0 & below);
      sh.chan[pos] = lane;
      sh.qc[pos] = sh.qb[lane];
    }
    if (t1) {
      const int pos = __popcll(b0) + __popcll(b1 & below);
      sh.chan[pos] = lane + kWave;
      sh.qc[pos] = sh.qb[lane + kWave];
    }
  }
  before_last_barrier();
  lds_barrier();
}

template <typename T, int G>
__device__ __forceinline__ void select_channels_block(const T* __restrict__ q, int b, int h,
                                                      int Hkv, int D, int r, ChannelShared& sh) {
  ChannelQ<T, G> cq;
  cq.load(q, b, h, Hkv, D);
  select_channels_phase1<T, G>(cq, D, sh);
  select_channels_phase2<4, 256>(D, r, sh);
}

// Channel partition of the page-score sum: group g (of 16) sums chosen channels g, g+16, g+32,
// ... in ascending order, and the group sums are combined by a fixed tree inside a row of 16
// lanes (pairs, quads, halves of 8, then the two halves). Every kernel that scores pages uses
// this order, so they all produce the same bits.
constexpr int kScoreGroups = 16;
constexpr int kScoreBatch = kApproxMaxD / kScoreGroups;  // every row load of a lane in flight

// Thread layout: lane = 16 * vector + group. VEC: a vector is 16 bytes of consecutive pages
// (p_begin and the row pitch multiples of the vector width); otherwise one page per vector.
// Scores pages [p_begin, p_end) of one (b, h), whose summary rows are `pitch` pages apart, and
// hands each score to sink(page, value), called by one lane per page. No barrier; the whole row
// of a vector must be active together. BATCH: row loads a lane can hold per pass (at least the
// group's channel count, ceil(r / 16)); PASSES: passes whose loads are all issued before the
// first of them is summed, so a long range keeps PASSES * BATCH loads per lane in flight.
template <typename T, bool VEC, int BATCH, int PASSES, typename Sink>
__device__ __forceinline__ void score_pages(const T* __restrict__ kmin_bh,
                                            const T* __restrict__ kmax_bh, int D, int pitch,
                                            int r, int p_begin, int p_end,
                                            const ChannelShared& ch, Sink&& sink) {
  constexpr int V = VEC ? vec16<T>::n : 1;
  const int grp = threadIdx.x % kScoreGroups;
  const int nvec_pass = blockDim.x / kScoreGroups;
  const int nvec = (p_end - p_begin + V - 1) / V;
  const int nj = (r - grp + kScoreGroups - 1) / kScoreGroups;  // channels of this group
  // the lane's channel rows (its group's channels grp, grp + 16, ...) and their q-bar factors
  float qcv[BATCH];
  const T* rows[BATCH];
#pragma unroll
  for (int u = 0; u < BATCH; ++u) {
    const int j = grp + (u < nj ? u : 0) * kScoreGroups;
    qcv[u] = u < nj ? ch.qc[j] : 0.f;
    const int c = min(max(ch.chan[j], 0), D - 1);
    rows[u] = (qcv[u] >= 0.f ? kmax_bh : kmin_bh) + (size_t)c * pitch;
  }
  for (int v0 = 0; v0 < nvec; v0 += nvec_pass * PASSES) {  // uniform trip count across the block
    int pg[PASSES];
    bool act[PASSES];
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int vi = v0 + ps * nvec_pass + (int)threadIdx.x / kScoreGroups;
      act[ps] = vi < nvec;
      pg[ps] = p_begin + (act[ps] ? vi : 0) * V;
    }
    if constexpr (VEC) {
      uint4 raw[PASSES][BATCH];
#pragma unroll
      for (int ps = 0; ps < PASSES; ++ps)
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
          raw[ps][u] = make_uint4(0u, 0u, 0u, 0u);
          if (u < nj && (ps == 0 || act[ps])) raw[ps][u] = load16(rows[u] + pg[ps]);
        }
#pragma unroll
      for (int ps = 0; ps < PASSES; ++ps) {
        if (ps > 0 && v0 + ps * nvec_pass >= nvec) break;  // block-uniform: no vector left
        float acc[V];
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] = 0.f;
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
          float x[V];
          unpack16<T>(raw[ps][u], x);
          const bool use = u < nj;
#pragma unroll
          for (int e = 0; e < V; ++e) acc[e] = use ? fmaf(qcv[u], x[e], acc[e]) : acc[e];
        }
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] = group_sum<kScoreGroups>(acc[e]);
        if (act[ps]) {
          // lane `grp` of the row hands over page grp of its vector (all lanes hold the sums)
#pragma unroll
          for (int e = 0; e < V; ++e)
            if (e % kScoreGroups == grp && pg[ps] + e < p_end) sink(pg[ps] + e, acc[e]);
        }
      }
    } else {
      float raw[PASSES][BATCH];
#pragma unroll
      for (int ps = 0; ps < PASSES; ++ps)
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
          raw[ps][u] = 0.f;
          if (u < nj && (ps == 0 || act[ps])) raw[ps][u] = to_f32(rows[u][pg[ps]]);
        }
#pragma unroll
      for (int ps = 0; ps < PASSES; ++ps) {
        if (ps > 0 && v0 + ps * nvec_pass >= nvec) break;
        float acc = 0.f;
#pragma unroll
        for (int u = 0; u < BATCH; ++u) acc = u < nj ? fmaf(qcv[u], raw[ps][u], acc) : acc;
        acc = group_sum<kScoreGroups>(acc);
        if (act[ps] && grp == 0 && pg[ps] < p_end) sink(pg[ps], acc);
      }
    }
  }
}

// score_pages for any r <= kApproxMaxD; a range of more than one pass with at most two channels
// per group (r <= 32) keeps four passes' loads in flight.
template <typename T, bool VEC, typename Sink>
__device__ __forceinline__ void score_page_range(const T* __restrict__ kmin_bh,
                                                 const T* __restrict__ kmax_bh, int D, int pitch,
                                                 int r, int p_begin, int p_end,
                                                 const ChannelShared& ch, Sink&& sink) {
  constexpr int V = VEC ? vec16<T>::n : 1;
  const bool long_range = p_end - p_begin > (int)(blockDim.x / kScoreGroups) * V;
  if (r <= 2 * kScoreGroups && long_range)
    score_pages<T, VEC, 2, 4>(kmin_bh, kmax_bh, D, pitch, r, p_begin, p_end, ch, sink);
  else
    score_pages<T, VEC, kScoreBatch, 1>(kmin_bh, kmax_bh, D, pitch, r, p_begin, p_end, ch, sink);
}

}  // namespace rkv
