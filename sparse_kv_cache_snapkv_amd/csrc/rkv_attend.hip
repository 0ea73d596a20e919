// Exact softmax attention over the tokens of the selected pages, shared by the G query heads of
// a GQA group (RocketKV rebuttal, "Lack of Direct Latency Comparison": Step 3 sparse attention;
// "Explanation of Calculating Approximate Attention Scores": one selection per group).
//
// Work split: block = (split of the head's page list, b*Hkv+h), 4 waves. A token row of D
// elements is spread over LPT lanes, 16 bytes each, so one load instruction fetches TPL = 64/LPT
// whole rows; per chunk a wave issues all its K and V loads (SLOTS of each) before reducing in
// registers (DPP inside a row of 16 lanes), with an online softmax across chunks. The four waves
// merge (max, sum, P.V) through LDS.
//
// The standalone call copies its slice of page_idx into LDS; several splits per head are combined
// by k_attend_merge (log-sum-exp form). The fused decode step (k_decode_step) is one kernel:
//   1. each block scores its share of its head's pages (rkv_approx.hpp) into the workspace and
//      arrives on a per-head counter; the blocks of a head wait for each other (bounded spin;
//      the grid never exceeds one block per CU, so all of them are resident at once). Data that
//      crosses blocks (scores, partial results) moves only through device-coherent stores and
//      loads ordered by s_waitcnt, so no fence has to write back or invalidate the L2;
//   2. each block runs the exact block top-k (rkv_select.hpp) on all of its head's page scores
//      and keeps its slice of the ascending page list;
//   3. attention over that slice;
//   4. the last block of the head to finish merges the splits and resets the counters.
#include <math.h>

#include <algorithm>

#include "rkv_approx.hpp"
#include "rkv_common.hpp"
#include "rkv_launch.hpp"
#include "rkv_select.hpp"

namespace rkv {

namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kSlots = 4;            // row loads per wave per chunk
constexpr int kMaxPagesPerSplit = 1024;

constexpr int kSpinLimit = 1 << 20;  // polls before a head's cross-block wait gives up

template <typename T, int D>
struct Geo {
  static constexpr int V = vec16<T>::n;
  static constexpr int LPT = D / V;
  static constexpr int TPL = kWave / LPT;
  static constexpr int WTOK = kSlots * TPL;  // tokens per wave per chunk
};

template <int D, int G>
struct AttendShared {
  int pages[kMaxPagesPerSplit + 1];  // the last slot takes discarded writes
  float m[kWavesPerBlock][G], l[kWavesPerBlock][G];
  float o[kWavesPerBlock][G][D];
};

// Per-wave online-softmax state of the G heads of a group.
template <typename T, int D, int G>
struct WaveState {
  float qf[G][Geo<T, D>::V];
  float m[G], l[G], acc[G][Geo<T, D>::V];

  __device__ __forceinline__ void init(const T* __restrict__ q_bh, float scale2) {
    constexpr int V = Geo<T, D>::V, LPT = Geo<T, D>::LPT;
    const int li = (threadIdx.x & (kWave - 1)) % LPT;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      unpack16<T>(load16(q_bh + (size_t)g * D + li * V), qf[g]);
#pragma unroll
      for (int e = 0; e < V; ++e) qf[g][e] *= scale2;
      m[g] = -INFINITY;
      l[g] = 0.f;
#pragma unroll
      for (int e = 0; e < V; ++e) acc[g][e] = 0.f;
    }
  }

  // Tokens [0, ntok) of the page list `pages` (LDS): this wave takes chunks wave, wave+4, ...
  __device__ __forceinline__ void run(const T* __restrict__ kc_bh, const T* __restrict__ vc_bh,
                                      const int* pages, int ntok, int ps, int P, int Lc) {
    constexpr int V = Geo<T, D>::V, LPT = Geo<T, D>::LPT, TPL = Geo<T, D>::TPL;
    constexpr int WTOK = Geo<T, D>::WTOK;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int lg = lane / LPT, li = lane % LPT;
    const T* kb = kc_bh + li * V;
    const T* vb = vc_bh + li * V;
    for (int c0 = wave * WTOK; c0 < ntok; c0 += kWavesPerBlock * WTOK) {
      int tok[kSlots];
      bool ok[kSlots];
#pragma unroll
      for (int s = 0; s < kSlots; ++s) {
        const int ti = c0 + s * TPL + lg;
        bool valid = ti < ntok;
        const int page = valid ? pages[ti / ps] : 0;
        const int t = page * ps + ti % ps;
        valid = valid && page >= 0 && page < P && t < Lc;
        ok[s] = valid;
        tok[s] = valid ? t : 0;
      }
      uint4 kr[kSlots], vr[kSlots];
#pragma unroll
      for (int s = 0; s < kSlots; ++s) {
        kr[s] = load16_stream(kb + (size_t)tok[s] * D);
        vr[s] = load16_stream(vb + (size_t)tok[s] * D);
      }
      float sc[kSlots][G];
#pragma unroll
      for (int s = 0; s < kSlots; ++s) {
        float kf[V];
        unpack16<T>(kr[s], kf);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < V; ++e) d = fmaf(qf[g][e], kf[e], d);
          d = group_sum<LPT>(d);
          sc[s][g] = ok[s] ? d : -INFINITY;
        }
      }
      float mu[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float x = sc[0][g];
#pragma unroll
        for (int s = 1; s < kSlots; ++s) x = fmaxf(x, sc[s][g]);
        x = across_max<LPT>(x);
        const float mn = fmaxf(m[g], x);
        const float f = mn == -INFINITY ? 1.f : exp2f(m[g] - mn);
        mu[g] = mn == -INFINITY ? 0.f : mn;
        m[g] = mn;
        l[g] *= f;
#pragma unroll
        for (int e = 0; e < V; ++e) acc[g][e] *= f;
      }
#pragma unroll
      for (int s = 0; s < kSlots; ++s) {
        float vf[V];
        unpack16<T>(vr[s], vf);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float p = exp2f(sc[s][g] - mu[g]);
          l[g] += p;
#pragma unroll
          for (int e = 0; e < V; ++e) acc[g][e] = fmaf(p, vf[e], acc[g][e]);
        }
      }
    }
  }

  // Reduces over the wave's lane groups and stores (m, l, o) of this wave in sh.
  __device__ __forceinline__ void publish(AttendShared<D, G>& sh) {
    constexpr int V = Geo<T, D>::V, LPT = Geo<T, D>::LPT;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int lg = lane / LPT, li = lane % LPT;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      l[g] = across_sum<LPT>(l[g]);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[g][e] = across_sum<LPT>(acc[g][e]);
    }
    if (lg == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int e = 0; e < V; ++e) sh.o[wave][g][li * V + e] = acc[g][e];
        if (li == 0) {
          sh.m[wave][g] = m[g];
          sh.l[wave][g] = l[g];
        }
      }
    }
  }
};

// Combines the four waves' (m, l, o) for output element idx = g*D + c.
template <int D, int G>
__device__ __forceinline__ void wave_merge(const AttendShared<D, G>& sh, int g, int c, float& M,
                                           float& lsum, float& o) {
  M = sh.m[0][g];
#pragma unroll
  for (int w = 1; w < kWavesPerBlock; ++w) M = fmaxf(M, sh.m[w][g]);
  lsum = 0.f;
  o = 0.f;
  if (M == -INFINITY) return;
#pragma unroll
  for (int w = 0; w < kWavesPerBlock; ++w) {
    const float fw = exp2f(sh.m[w][g] - M);
    lsum = fmaf(sh.l[w][g], fw, lsum);
    o = fmaf(sh.o[w][g][c], fw, o);
  }
}

// ------------------------------------------------------------------------------ standalone call

struct AttendArgs {
  const void* q;
  const void* k_c;
  const void* v_c;
  const int32_t* page_idx;  // [BH, n_pages]
  int Lc, ps, n_pages, P, pps, nsplit;
  float scale2;
  float* part;              // [BH, nsplit, G, D+2]
  void* out;
};

template <typename T, int D, int G>
__global__ __launch_bounds__(kThreads) void k_attend(AttendArgs a) {
  __shared__ AttendShared<D, G> sh;
  const int tid = threadIdx.x;
  const int bh = blockIdx.y, split = blockIdx.x;
  const int p_lo = split * a.pps;
  const int p_hi = min(p_lo + a.pps, a.n_pages);
  const int np_blk = max(p_hi - p_lo, 0);
  const int32_t* pb = a.page_idx + (size_t)bh * a.n_pages + p_lo;
  for (int i = tid; i < np_blk; i += kThreads) sh.pages[i] = pb[i];
  __syncthreads();
  WaveState<T, D, G> st;
  st.init(static_cast<const T*>(a.q) + (size_t)bh * G * D, a.scale2);
  st.run(static_cast<const T*>(a.k_c) + (size_t)bh * a.Lc * D,
         static_cast<const T*>(a.v_c) + (size_t)bh * a.Lc * D, sh.pages, np_blk * a.ps, a.ps, a.P,
         a.Lc);
  st.publish(sh);
  __syncthreads();
  T* out = static_cast<T*>(a.out);
  for (int idx = tid; idx < G * D; idx += kThreads) {
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
__global__ __launch_bounds__(kThreads) void k_attend_merge(const float* __restrict__ part,
                                                          int nsplit, int D,
                                                          T* __restrict__ out) {
  constexpr int kMaxSplits = 256;
  __shared__ float s_w[kMaxSplits][G];
  __shared__ float s_inv[G];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const size_t stride = (size_t)G * (D + 2);
  const float* hp = part + (size_t)bh * nsplit * stride;
  for (int g = tid / kWave; g < G; g += kWavesPerBlock) {
    const int lane = tid % kWave;
    float M = -INFINITY;
    for (int s = lane; s < nsplit; s += kWave) M = fmaxf(M, hp[s * stride + g * (D + 2) + D]);
    M = group_max<64>(M);
    float lsum = 0.f;
    for (int s = lane; s < nsplit; s += kWave) {
      const float ms = hp[s * stride + g * (D + 2) + D];
      const float w = ms == -INFINITY ? 0.f : exp2f(ms - M);
      s_w[s][g] = w;
      lsum = fmaf(hp[s * stride + g * (D + 2) + D + 1], w, lsum);
    }
    lsum = group_sum<64>(lsum);
    if (lane == 0) s_inv[g] = lsum > 0.f ? 1.f / lsum : 0.f;
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int g = idx / D, c = idx % D;
    const float* pc = hp + (size_t)g * (D + 2) + c;
    float o = 0.f;
#pragma unroll 8
    for (int s = 0; s < nsplit; ++s) o = fmaf(pc[s * stride], s_w[s][g], o);
    out[((size_t)bh * G + g) * D + c] = from_f32<T>(o * s_inv[g]);
  }
}

// ------------------------------------------------------------------------------ fused step

constexpr int kMaxSplit = 64;  // blocks per head in the fused step (one wave polls their flags)

struct StepArgs {
  const void* q;
  const void* kmin_t;
  const void* kmax_t;
  const void* k_c;
  const void* v_c;
  int BH, Hkv, Lc, ps, n_pages, P, r, pps, ppb1, nsplit, nsplit_att, vec;
  float scale2;
  int32_t* chan_idx;  // optional [BH, r]
  float* scores;      // [BH, P]
  int32_t* page_idx;  // optional [BH, n_pages]
  float* part;        // [BH, nsplit_att, G, D+2]
  unsigned* sync;     // [0] status; arrive flags [BH][kMaxSplit]; done flags [BH][kMaxSplit]
  void* out;
};

__device__ __forceinline__ unsigned ld_coherent(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename V>
__device__ __forceinline__ void st_coherent(V* p, V v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave 0 polls flags[lo..hi) (one lane each, one coherent load per poll) until all are set;
// bounded, on give-up the status word is set. Call from wave 0 only.
__device__ __forceinline__ void wave_wait_flags(const unsigned* flags, int lo, int hi,
                                                unsigned* status) {
  const int lane = threadIdx.x & (kWave - 1);
  for (int polls = 0;; ++polls) {
    const bool mine = lane >= lo && lane < hi;
    const unsigned f = mine ? ld_coherent(flags + lane) : 1u;
    if (__all(f != 0u)) return;
    if (polls > kSpinLimit) {
      if (lane == 0) __hip_atomic_fetch_or(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

template <typename T, int D, int G, int E>
__global__ __launch_bounds__(kThreads) void k_decode_step(StepArgs a) {
  __shared__ ChannelShared ch;
  // The head's scores are dead once the keys are in registers (block_threshold passes a barrier
  // before any page-list or attention write), so they share LDS with the attention scratch.
  __shared__ union {
    __align__(16) float scores[E * kThreads];
    AttendShared<D, G> att;
  } u;
  AttendShared<D, G>& sh = u.att;
  float* s_scores = u.scores;
  __shared__ SelectShared<kThreads> sel;
  __shared__ float s_w[kMaxSplit][G], s_l[kMaxSplit][G];
  __shared__ float s_inv[G];
  const int tid = threadIdx.x, wave = tid / kWave;
  const int bh = blockIdx.y, split = blockIdx.x, b = bh / a.Hkv, h = bh % a.Hkv;
  const T* q = static_cast<const T*>(a.q);
  unsigned* arrive = a.sync + 16 + (size_t)bh * kMaxSplit;
  unsigned* done = a.sync + 16 + (size_t)a.BH * kMaxSplit + (size_t)bh * kMaxSplit;
  const bool attends = split < a.nsplit_att;

  WaveState<T, D, G> st;  // the queries' loads overlap the channel selection
  if (attends) st.init(q + (size_t)bh * G * D, a.scale2);

  // 1. this block's share of the head's approximate page scores
  select_channels_block<T>(q, b, h, a.Hkv, G, D, a.r, ch);
  if (a.chan_idx != nullptr && split == 0)
    for (int j = tid; j < a.r; j += kThreads) a.chan_idx[(size_t)bh * a.r + j] = ch.chan[j];
  float* srow = a.scores + (size_t)bh * a.P;
  {
    const int pb_lo = split * a.ppb1, pb_hi = min(a.P, pb_lo + a.ppb1);
    const size_t sbase = (size_t)bh * D * a.P;
    // device-coherent stores: the other blocks of the head read them
    score_page_range<T, true>(static_cast<const T*>(a.kmin_t) + sbase,
                              static_cast<const T*>(a.kmax_t) + sbase, D, a.P, a.r, pb_lo, pb_hi,
                              a.vec != 0, ch, srow);
  }
  if (a.nsplit > 1) {
    // Exchange through device-coherent accesses only: wait until this block's score stores are
    // complete, raise this block's flag, then wait for every block of the head.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) st_coherent(arrive + split, 1u);
    if (!attends) return;  // a scoring-only block
    if (wave == 0) wave_wait_flags(arrive, 0, a.nsplit, a.sync);
  }
  __syncthreads();

  // 2. the head's scores into LDS (coalesced), then the top pages of this block's slice
  if (a.nsplit > 1) {
    float v[E];  // every load issued before the first use
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int i = j * kThreads + tid;
      v[j] = i < a.P ? ld_coherent(srow + i) : 0.f;
    }
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int i = j * kThreads + tid;
      if (i < a.P) s_scores[i] = v[j];
    }
  } else {
    for (int i = tid; i < a.P; i += kThreads) s_scores[i] = srow[i];
  }
  __syncthreads();
  const int p_lo = split * a.pps;
  const int p_hi = min(p_lo + a.pps, a.n_pages);
  const T* kc_bh = static_cast<const T*>(a.k_c) + (size_t)bh * a.Lc * D;
  const T* vc_bh = static_cast<const T*>(a.v_c) + (size_t)bh * a.Lc * D;
  int32_t* pout = (a.page_idx != nullptr && split == 0) ? a.page_idx + (size_t)bh * a.n_pages
                                                        : nullptr;
  if (a.n_pages >= a.P) {
    for (int i = tid; pout != nullptr && i < a.n_pages; i += kThreads) pout[i] = i;
    for (int w0 = p_lo; w0 < p_hi; w0 += kMaxPagesPerSplit) {
      const int nw = min(kMaxPagesPerSplit, p_hi - w0);
      __syncthreads();
      for (int i = tid; i < nw; i += kThreads) sh.pages[i] = w0 + i;
      __syncthreads();
      st.run(kc_bh, vc_bh, sh.pages, nw * a.ps, a.ps, a.P, a.Lc);
    }
  } else {
    uint32_t key[E];
    const int i0 = tid * E;
    const int nv = load_keys<E>(s_scores, a.P, i0, key);
    uint32_t thr, need_eq;
    block_threshold<kThreads, E>(key, nv, (uint32_t)a.n_pages, thr, need_eq, sel);
    int w0 = p_lo;
    do {  // the first window also writes the full page list when asked
      const int nw = min(kMaxPagesPerSplit, max(p_hi - w0, 0));
      const bool write_out = pout != nullptr && w0 == p_lo;
      __syncthreads();
      block_compact<kThreads, E>(key, nv, thr, need_eq, i0, sel,
                                 [&](uint32_t pos, int idx, bool take) {
        const int p = (int)pos;
        // branch-free: elements outside the window go to the spare slot
        sh.pages[(take && p >= w0 && p < w0 + nw) ? p - w0 : kMaxPagesPerSplit] = idx;
        if (write_out && take && p < a.n_pages) pout[p] = idx;
      });
      __syncthreads();
      st.run(kc_bh, vc_bh, sh.pages, nw * a.ps, a.ps, a.P, a.Lc);
      w0 += kMaxPagesPerSplit;
    } while (w0 < p_hi);
  }

  // 3. attention partial of this block
  st.publish(sh);
  __syncthreads();
  T* out = static_cast<T*>(a.out);
  const int nsa = a.nsplit_att;
  float* hp = a.part + (size_t)bh * nsa * G * (D + 2);
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int g = idx / D, c = idx % D;
    float M, lsum, o;
    wave_merge<D, G>(sh, g, c, M, lsum, o);
    if (nsa == 1) {
      out[((size_t)bh * G + g) * D + c] = from_f32<T>(lsum > 0.f ? o / lsum : 0.f);
    } else {
      float* pp = hp + ((size_t)split * G + g) * (D + 2);
      st_coherent(pp + c, o);
      if (c == 0) {
        st_coherent(pp + D, M);
        st_coherent(pp + D + 1, lsum);
      }
    }
  }
  if (nsa > 1) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (split != 0) {
      if (tid == 0) st_coherent(done + split, 1u);
      return;
    }
    // 4. split 0 waits for the other attending blocks, then merges every split
    if (wave == 0) wave_wait_flags(done, 1, nsa, a.sync);
    __syncthreads();
    const size_t stride = (size_t)G * (D + 2);
    {  // (max, sum) of every split and head into LDS, all loads in flight at once
      constexpr int kPer = (kMaxSplit * G + kThreads - 1) / kThreads;
      float mv[kPer], lv[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int i = j * kThreads + tid;
        const bool ok = i < nsa * G;
        const float* pp = hp + (ok ? (i / G) * stride + (i % G) * (D + 2) : 0);
        mv[j] = ok ? ld_coherent(pp + D) : 0.f;
        lv[j] = ok ? ld_coherent(pp + D + 1) : 0.f;
      }
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int i = j * kThreads + tid;
        if (i < nsa * G) {
          s_w[i / G][i % G] = mv[j];
          s_l[i / G][i % G] = lv[j];
        }
      }
    }
    __syncthreads();
    if (tid < G) {
      float M = -INFINITY;
      for (int s = 0; s < nsa; ++s) M = fmaxf(M, s_w[s][tid]);
      float lsum = 0.f;
      for (int s = 0; s < nsa; ++s) {
        const float ms = s_w[s][tid];
        const float wgt = ms == -INFINITY ? 0.f : exp2f(ms - M);
        lsum = fmaf(s_l[s][tid], wgt, lsum);
        s_w[s][tid] = wgt;
      }
      s_inv[tid] = lsum > 0.f ? 1.f / lsum : 0.f;
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += kThreads) {
      const int g = idx / D, c = idx % D;
      const float* pc = hp + (size_t)g * (D + 2) + c;
      float o = 0.f;
      for (int s0 = 0; s0 < nsa; s0 += 16) {
        float x[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) x[j] = s0 + j < nsa ? ld_coherent(pc + (s0 + j) * stride) : 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (s0 + j < nsa) o = fmaf(x[j], s_w[s0 + j][g], o);
      }
      out[((size_t)bh * G + g) * D + c] = from_f32<T>(o * s_inv[g]);
    }
  }
  // every block of the head has passed its flags: leave them zero for the next call
  if (a.nsplit > 1 && tid < a.nsplit) {
    st_coherent(arrive + tid, 0u);
    st_coherent(done + tid, 0u);
  }
}

__global__ void k_zero_u32(unsigned* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// ------------------------------------------------------------------------------ plans

constexpr int kTargetBlocks = 256;  // one block per CU of an MI355X

struct Plan {
  int nsplit, pps;
};

template <typename T, int D>
Plan plan_attend(int BH, int ps, int n_pages) {
  const int ntok = n_pages * ps;
  const int chunk = kWavesPerBlock * Geo<T, D>::WTOK;
  int ns = (2 * kTargetBlocks + BH - 1) / BH;
  ns = min(ns, (ntok + chunk - 1) / chunk);
  ns = max(ns, (n_pages + kMaxPagesPerSplit - 1) / kMaxPagesPerSplit);
  ns = max(min(ns, 256), 1);
  int pps = (n_pages + ns - 1) / ns;
  ns = (n_pages + pps - 1) / pps;
  return {ns, pps};
}

// Fused step: scoring blocks per head while the whole grid fits one block per CU (the blocks of
// a head wait for each other), at most kMaxSplit; the first of them also attend, each to at
// least one chunk of tokens.
struct StepPlan {
  int nsplit, nsplit_att, pps;
};

template <typename T, int D>
StepPlan plan_step(int BH, int ps, int n_pages, int ncu) {
  const int ntok = n_pages * ps;
  const int chunk = kWavesPerBlock * Geo<T, D>::WTOK;
  const int ns = max(min(ncu / BH, kMaxSplit), 1);
  int na = max(min(ns, (ntok + chunk - 1) / chunk), 1);
  const int pps = (n_pages + na - 1) / na;
  na = (n_pages + pps - 1) / pps;
  return {ns, na, pps};
}

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

template <typename T, int D, int G>
hipError_t attend_g(AttendArgs a, int BH, hipStream_t stream) {
  hipLaunchKernelGGL((k_attend<T, D, G>), dim3(a.nsplit, BH), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  hipLaunchKernelGGL((k_attend_merge<T, G>), dim3(BH), dim3(kThreads), 0, stream, a.part,
                     a.nsplit, D, static_cast<T*>(a.out));
  return hipGetLastError();
}

template <typename T, int D, int G>
hipError_t step_g(StepArgs a, int BH, hipStream_t stream) {
  if (a.P <= 16 * kThreads)
    hipLaunchKernelGGL((k_decode_step<T, D, G, 16>), dim3(a.nsplit, BH), dim3(kThreads), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((k_decode_step<T, D, G, 32>), dim3(a.nsplit, BH), dim3(kThreads), 0,
                       stream, a);
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
template <typename T, int D>
hipError_t step_d(int G, StepArgs a, int BH, hipStream_t s) { RKV_DISPATCH_G(step_g, a, BH, s) }

Plan plan_attend_any(int dtype, int D, int BH, int ps, int n_pages) {
  if (dtype == 0)
    return D == 64 ? plan_attend<float, 64>(BH, ps, n_pages) : plan_attend<float, 128>(BH, ps, n_pages);
  return D == 64 ? plan_attend<bf16_t, 64>(BH, ps, n_pages) : plan_attend<bf16_t, 128>(BH, ps, n_pages);
}

StepPlan plan_step_any(int dtype, int D, int BH, int ps, int n_pages, int ncu) {
  if (dtype == 0)
    return D == 64 ? plan_step<float, 64>(BH, ps, n_pages, ncu) : plan_step<float, 128>(BH, ps, n_pages, ncu);
  return D == 64 ? plan_step<bf16_t, 64>(BH, ps, n_pages, ncu) : plan_step<bf16_t, 128>(BH, ps, n_pages, ncu);
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct StepLayout {
  size_t off_scores, off_part, off_sync, total;
};

// Sized for the largest split count any device can get (kTargetBlocks CUs).
StepLayout step_layout(int B, int Hq, int Hkv, int D, int P, int nsplit_max) {
  const size_t BH = (size_t)B * Hkv;
  StepLayout lo{};
  lo.off_sync = 0;
  lo.off_scores = align256((16 + 2 * BH * kMaxSplit) * sizeof(unsigned));
  lo.off_part = align256(lo.off_scores + BH * P * sizeof(float));
  lo.total = align256(lo.off_part + BH * nsplit_max * (Hq / Hkv) * (D + 2) * sizeof(float));
  return lo;
}

}  // namespace

size_t attend_ws_bytes(int B, int Hq, int Hkv, int D, int page_size, int n_pages, int dtype) {
  const Plan pl = plan_attend_any(dtype, D, B * Hkv, page_size, n_pages);
  if (pl.nsplit == 1) return 0;
  return (size_t)B * Hkv * pl.nsplit * (Hq / Hkv) * (D + 2) * sizeof(float);
}

hipError_t launch_sparse_attend(const void* q, const void* k_c, const void* v_c,
                                const int32_t* page_idx, int B, int Hq, int Hkv, int Lc, int D,
                                int page_size, int n_pages, float scale, int dtype, void* out,
                                void* ws, hipStream_t stream) {
  const int BH = B * Hkv;
  const Plan pl = plan_attend_any(dtype, D, BH, page_size, n_pages);
  AttendArgs a{q, k_c, v_c, page_idx, Lc, page_size, n_pages, (Lc + page_size - 1) / page_size,
               pl.pps, pl.nsplit, scale * kLog2e, static_cast<float*>(ws), out};
  const int G = Hq / Hkv;
  if (dtype == 0)
    return D == 64 ? attend_d<float, 64>(G, a, BH, stream) : attend_d<float, 128>(G, a, BH, stream);
  return D == 64 ? attend_d<bf16_t, 64>(G, a, BH, stream) : attend_d<bf16_t, 128>(G, a, BH, stream);
}

size_t decode_ws_bytes(int B, int Hq, int Hkv, int Lc, int D, int page_size, int n_pages,
                       int dtype) {
  const int P = (Lc + page_size - 1) / page_size;
  const StepPlan pl = plan_step_any(dtype, D, B * Hkv, page_size, n_pages, kTargetBlocks);
  return step_layout(B, Hq, Hkv, D, P, pl.nsplit_att).total;
}

hipError_t launch_decode_ws_init(void* ws, size_t bytes, hipStream_t stream) {
  const size_t n = bytes / sizeof(unsigned);
  const int blocks = (int)std::min<size_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(k_zero_u32, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, stream,
                     static_cast<unsigned*>(ws), n);
  return hipGetLastError();
}

hipError_t launch_decode_step(const void* q, const void* kmin_t, const void* kmax_t,
                              const void* k_c, const void* v_c, int B, int Hq, int Hkv, int Lc,
                              int D, int page_size, int r, int n_pages, float scale, int dtype,
                              int32_t* chan_idx, float* page_scores, int32_t* page_idx, void* out,
                              void* ws, hipStream_t stream) {
  const int BH = B * Hkv;
  const int P = (Lc + page_size - 1) / page_size;
  const StepPlan pmax = plan_step_any(dtype, D, BH, page_size, n_pages, kTargetBlocks);
  const StepPlan pl = plan_step_any(dtype, D, BH, page_size, n_pages, device_cus());
  const StepLayout lo = step_layout(B, Hq, Hkv, D, P, pmax.nsplit_att);
  char* w = static_cast<char*>(ws);
  const int vmax = dtype == 0 ? vec16<float>::n : vec16<bf16_t>::n;
  int ppb1 = (P + pl.nsplit - 1) / pl.nsplit;
  ppb1 = (ppb1 + vmax - 1) / vmax * vmax;
  StepArgs a{q, kmin_t, kmax_t, k_c, v_c, BH, Hkv, Lc, page_size, n_pages, P, r, pl.pps, ppb1,
             pl.nsplit, pl.nsplit_att, P % vmax == 0, scale * kLog2e, chan_idx,
             page_scores != nullptr ? page_scores : reinterpret_cast<float*>(w + lo.off_scores),
             page_idx, reinterpret_cast<float*>(w + lo.off_part),
             reinterpret_cast<unsigned*>(w + lo.off_sync), out};
  const int G = Hq / Hkv;
  if (dtype == 0)
    return D == 64 ? step_d<float, 64>(G, a, BH, stream) : step_d<float, 128>(G, a, BH, stream);
  return D == 64 ? step_d<bf16_t, 64>(G, a, BH, stream) : step_d<bf16_t, 128>(G, a, BH, stream);
}

}  // namespace rkv
