// Exact softmax attention over the tokens of the selected pages, shared by the G query heads of
// a GQA group (RocketKV rebuttal, "Lack of Direct Latency Comparison": Step 3 sparse attention;
// "Explanation of Calculating Approximate Attention Scores": one selection per group).
//
// Work split: block = (split of the head's page list, b*Hkv+h), 4 waves (8 in the fused step). A
// token row of D elements is spread over LPT lanes, 16 bytes each, so one load instruction
// fetches TPL = 64/LPT whole rows; per chunk a wave issues all its K and V loads (SLOTS of each)
// before reducing in registers (DPP inside a row of 16 lanes), with an online softmax across
// chunks. The waves merge (max, sum, P.V) through LDS.
//
// The standalone call copies its slice of page_idx into LDS; several splits per head are combined
// by k_attend_merge (log-sum-exp form). The fused decode step (k_decode_step) is one kernel:
//   1. each block scores its share of its head's pages (rkv_approx.hpp) and publishes them as
//      epoch-tagged 64-bit words; the attending blocks of the head poll those words until every
//      tag is current (bounded spin; the grid never exceeds one block per CU, so all of them are
//      resident at once). Data that crosses blocks moves only through device-coherent loads and
//      stores, and a tag travels in the same single-copy-atomic word as its value, so no fence
//      or flag has to order anything;
//   2. each attending block runs the exact block top-k (rkv_select.hpp, strided layout: the
//      scores go from the exchanged words straight into registers) on all of its head's page
//      scores and keeps its slice of the ascending page list;
//   3. attention over that slice, published as a tagged partial (max, sum, P.V);
//   4. every attending block merges a slice of the head's outputs over all partials, and split 0
//      advances the head's epoch for the next call.
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
constexpr int kSlots = 4;            // row loads per wave per chunk (standalone attention)
constexpr int kMaxPagesPerSplit = 1024;

constexpr int kSpinLimit = 1 << 20;  // polls before a head's cross-block wait gives up

template <typename T, int D, int SLOTS = kSlots>
struct Geo {
  static constexpr int V = vec16<T>::n;
  static constexpr int LPT = D / V;
  static constexpr int TPL = kWave / LPT;
  static constexpr int WTOK = SLOTS * TPL;  // tokens per wave per chunk
};

template <int D, int G, int NW = kWavesPerBlock>
struct AttendShared {
  int pages[kMaxPagesPerSplit + kWave];  // slots from kMaxPagesPerSplit: discarded writes, per lane
  float m[NW][G], l[NW][G];
  float o[NW][G][D];
};

// Per-wave online-softmax state of the G heads of a group; NW waves share a block's page list and
// each issues SLOTS K and V row loads per chunk. bf16 scores are packed bf16 dot products of the
// raw query and key bits, scaled after the lane reduction; fp32 scores use the pre-scaled query.
template <typename T, int D, int G, int NW = kWavesPerBlock, int SLOTS = kSlots>
struct WaveState {
  static constexpr bool kBf16 = elem<T>::bytes == 2;
  float qf[G][Geo<T, D, SLOTS>::V];  // fp32 only: the query times scale * log2(e)
  float m[G], l[G], acc[G][Geo<T, D, SLOTS>::V];
  uint4 qraw[G];
  float sc2;     // scale * log2(e)
  bool started;  // a chunk has been accumulated (before it, rescaling zeros is skipped)

  // The lane's slices of the G queries, as loaded; init(scale2) converts them.
  __device__ __forceinline__ void load_q(const T* __restrict__ q_bh) {
    constexpr int V = Geo<T, D, SLOTS>::V, LPT = Geo<T, D, SLOTS>::LPT;
    const int li = (threadIdx.x & (kWave - 1)) % LPT;
#pragma unroll
    for (int g = 0; g < G; ++g) qraw[g] = load16(q_bh + (size_t)g * D + li * V);
  }

  __device__ __forceinline__ void init(const T* __restrict__ q_bh, float scale2) {
    load_q(q_bh);
    init(scale2);
  }

  __device__ __forceinline__ void init(float scale2) {
    constexpr int V = Geo<T, D, SLOTS>::V;
    sc2 = scale2;
    started = false;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if constexpr (!kBf16) {
        unpack16<T>(qraw[g], qf[g]);
#pragma unroll
        for (int e = 0; e < V; ++e) qf[g][e] *= scale2;
      }
      m[g] = -INFINITY;
      l[g] = 0.f;
#pragma unroll
      for (int e = 0; e < V; ++e) acc[g][e] = 0.f;
    }
  }

  // Tokens [0, ntok) of the page list `pages` (LDS): this wave takes chunks wave, wave+4, ...
  // rows (may be null): slot t of the compressed view is row rows[t] of kc_bh / vc_bh, clamped
  // into [0, row_hi] (the multi-turn variant keeps the whole cache and indexes its kept rows).
  __device__ __forceinline__ void run(const T* __restrict__ kc_bh, const T* __restrict__ vc_bh,
                                      const int* pages, int ntok, int ps, int P, int Lc,
                                      const int32_t* __restrict__ rows = nullptr,
                                      int row_hi = 0) {
    constexpr int V = Geo<T, D, SLOTS>::V, LPT = Geo<T, D, SLOTS>::LPT, TPL = Geo<T, D, SLOTS>::TPL;
    constexpr int WTOK = Geo<T, D, SLOTS>::WTOK;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int lg = lane / LPT, li = lane % LPT;
    const T* kb = kc_bh + li * V;
    const T* vb = vc_bh + li * V;
    for (int c0 = wave * WTOK; c0 < ntok; c0 += NW * WTOK) {
      int tok[SLOTS];
      bool ok[SLOTS];
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        const int ti = c0 + s * TPL + lg;
        bool valid = ti < ntok;
        const int page = valid ? pages[ti / ps] : 0;
        const int t = page * ps + ti % ps;
        valid = valid && page >= 0 && page < P && t < Lc;
        ok[s] = valid;
        tok[s] = valid ? t : 0;
      }
      if (rows != nullptr) {
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) tok[s] = min(max(rows[tok[s]], 0), row_hi);
      }
      uint4 kr[SLOTS], vr[SLOTS];
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        kr[s] = load16_stream(kb + (size_t)tok[s] * D);
        vr[s] = load16_stream(vb + (size_t)tok[s] * D);
      }
      float sc[SLOTS][G];
      if constexpr (kBf16) {
        float d[SLOTS * G];
#pragma unroll
        for (int s = 0; s < SLOTS; ++s)
#pragma unroll
          for (int g = 0; g < G; ++g) d[s * G + g] = dot8_bf16(qraw[g], kr[s]);
        group_sum_n<LPT>(d);
#pragma unroll
        for (int s = 0; s < SLOTS; ++s)
#pragma unroll
          for (int g = 0; g < G; ++g) sc[s][g] = ok[s] ? d[s * G + g] * sc2 : -INFINITY;
      } else {
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
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
      }
      float mu[G], f[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float x = sc[0][g];
#pragma unroll
        for (int s = 1; s < SLOTS; ++s) x = fmaxf(x, sc[s][g]);
        x = across_max<LPT>(x);
        const float mn = fmaxf(m[g], x);
        f[g] = mn == -INFINITY ? 1.f : exp2_hw(m[g] - mn);
        mu[g] = mn == -INFINITY ? 0.f : mn;
        m[g] = mn;
      }
      // `started` is the same in every lane; until the first chunk, l and acc are zero
      if (__builtin_amdgcn_readfirstlane((int)started)) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          l[g] *= f[g];
#pragma unroll
          for (int e = 0; e < V; ++e) acc[g][e] *= f[g];
        }
      }
      started = true;
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        float vf[V];
        unpack16<T>(vr[s], vf);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float p = exp2_hw(sc[s][g] - mu[g]);
          l[g] += p;
#pragma unroll
          for (int e = 0; e < V; ++e) acc[g][e] = fmaf(p, vf[e], acc[g][e]);
        }
      }
    }
  }

  // Reduces over the wave's lane groups and stores (m, l, o) of this wave in sh.
  __device__ __forceinline__ void publish(AttendShared<D, G, NW>& sh) {
    constexpr int V = Geo<T, D, SLOTS>::V, LPT = Geo<T, D, SLOTS>::LPT;
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

// Combines the NW waves' (m, l, o) for output element idx = g*D + c.
template <int D, int G, int NW = kWavesPerBlock>
__device__ __forceinline__ void wave_merge(const AttendShared<D, G, NW>& sh, int g, int c, float& M,
                                           float& lsum, float& o) {
  M = sh.m[0][g];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = fmaxf(M, sh.m[w][g]);
  lsum = 0.f;
  o = 0.f;
  if (M == -INFINITY) return;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float fw = exp2_hw(sh.m[w][g] - M);
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
      const float w = ms == -INFINITY ? 0.f : exp2_hw(ms - M);
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

constexpr int kMaxSplit = 64;  // blocks per head in the fused step
constexpr int kStepThreads = 512;  // threads of a fused-step block: two waves per SIMD
constexpr int kStepWaves = kStepThreads / kWave;
constexpr int kStepSlots = 4;       // row loads per wave per chunk in the fused step
constexpr int kStepSoloTokens = 128;  // budgets up to this many tokens: one attending block
constexpr int kStepTokensPerBlock = 64;  // attending blocks: one per this many budget tokens,
constexpr int kMaxAttending = 16;        // at most this many per head (each reads every score)

// Cross-block data of the fused step is exchanged as 64-bit words {value bits, epoch}: every
// block of a head reads the head's epoch word at the start, tags what it publishes with
// epoch + 1, and readers poll a word until its tag matches, so no flag or counter has to be
// raised after the data and cleared afterwards. Split 0 stores the new epoch once the merge has
// seen every split's partial, by which time every block of the head has read the old one.
struct StepArgs {
  const void* q;
  const void* kmin_t;
  const void* kmax_t;
  const void* k_c;
  const void* v_c;
  int BH, Hkv, Lc, ps, n_pages, P, r, pps, ppb1, nsplit, nsplit_att, part_cap, vec;
  int kv_pitch;  // token slots per head of k_c, v_c (>= Lc; the full length L with rows)
  const int32_t* rows;  // optional [BH, Lc]: slot t of head bh is row rows[bh*Lc + t] of k_c, v_c
  int s_pitch;   // pages per channel row of the summaries (>= P)
  float scale2;
  int32_t* chan_idx;     // optional [BH, r]
  float* page_scores;    // optional [BH, P]
  int32_t* page_idx;     // optional [BH, n_pages]
  uint64_t* xscores;     // [BH, P] tagged page scores
  uint64_t* xpart;       // [BH, part_cap, G*D + 2G] tagged partials: o[G*D], M[G], l[G]
  unsigned* sync;        // [0] status, [16 + bh] epoch of head bh
  void* out;
};

__device__ __forceinline__ unsigned ld_coherent(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_coherent(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename V>
__device__ __forceinline__ void st_coherent(V* p, V v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t tagged(float v, unsigned epoch) {
  return ((uint64_t)epoch << 32) | __float_as_uint(v);
}
__device__ __forceinline__ bool tag_is(uint64_t w, unsigned epoch) {
  return (unsigned)(w >> 32) == epoch;
}
__device__ __forceinline__ float tag_value(uint64_t w) { return __uint_as_float((unsigned)w); }

// Loads N tagged words (addr(j) for j with use(j)) until every tag is `epoch`: a waiting wave
// re-reads only its stale words, after a short sleep, so a word is seen one L2 round trip after
// it lands. Bounded: on give-up the status word is set and the stale values are used. Call with
// the whole wave (the exit is wave-uniform).
template <int N>
__device__ __forceinline__ void load_tagged(uint64_t (&w)[N], const bool (&use)[N],
                                            const uint64_t* const (&ptr)[N], unsigned epoch,
                                            unsigned* status) {
#pragma unroll
  for (int j = 0; j < N; ++j) w[j] = use[j] ? ld_coherent(ptr[j]) : 0ull;
  for (int polls = 0;; ++polls) {
    bool stale = false;
#pragma unroll
    for (int j = 0; j < N; ++j) stale = stale || (use[j] && !tag_is(w[j], epoch));
    if (__ballot(stale) == 0ull) return;
    if (polls > kSpinLimit) {
      if (stale) __hip_atomic_fetch_or(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int j = 0; j < N; ++j)
      if (use[j] && !tag_is(w[j], epoch)) w[j] = ld_coherent(ptr[j]);
  }
}

template <int D, int G>
struct MergeShared {
  float o[G * D + kMaxSplit];  // [split][element of this block's range]
  float m[kMaxSplit][G];       // max, then the split's weight
  float l[kMaxSplit][G];
  float inv[G];
};

constexpr int kMergePer = 8;  // tagged words a thread loads per round of the merge

template <typename T, int D, int G, int E>
__global__ __launch_bounds__(kStepThreads) void k_decode_step(StepArgs a) {
  __shared__ ChannelShared ch;
  // A block's own scores (single-block heads) are dead once its keys are in registers, which
  // happens before the selection's first barrier and so before any page-list or attention write;
  // they share LDS with the attention scratch, and the merge scratch comes after the attention's
  // last read of it.
  __shared__ union {
    __align__(16) float scores[E * kStepThreads];
    AttendShared<D, G, kStepWaves> att;
    MergeShared<D, G> mg;
  } u;
  AttendShared<D, G, kStepWaves>& sh = u.att;
  float* s_scores = u.scores;
  __shared__ SelectShared<kStepThreads> sel;  // the radix passes for clustered scores
  __shared__ StridedShared<kStepThreads, E> ssel;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  // grid (BH, nsplit): consecutive blocks belong to different heads, so the round-robin
  // placement of blocks on the XCDs keeps every block of a head on one XCD when BH is a
  // multiple of 8 (its summaries rows and exchanged words then stay in that XCD's L2)
  const int bh = blockIdx.x, split = blockIdx.y, b = bh / a.Hkv, h = bh % a.Hkv;
  const T* q = static_cast<const T*>(a.q);
  const bool multi = a.nsplit > 1;
  const bool attends = split < a.nsplit_att;
  unsigned* epoch_word = a.sync + 16 + bh;

  // The first loads (the head's epoch word, which every workspace holds, and the queries for the
  // attention and for the channel choice) are all issued before any of them is waited for.
  const unsigned epoch_prev = ld_coherent(epoch_word);
  WaveState<T, D, G, kStepWaves, kStepSlots> st;
  st.load_q(q + (size_t)bh * G * D);
  ChannelQ<T, G> cq;
  cq.load(q, b, h, a.Hkv, D);
  if (attends) strided_clear(ssel);  // ordered before its use by the channel choice's barriers

  // 1. this block's share of the head's approximate page scores
  select_channels_phase1<T, G>(cq, D, ch);
  select_channels_phase2(D, a.r, ch);
  unsigned epoch = 0;
  if (multi) {
    epoch = epoch_prev + 1u;
    if (epoch == 0u) epoch = 1u;  // tag 0 is what a cleared workspace holds
  }
  if (attends) st.init(a.scale2);
  if (a.chan_idx != nullptr && split == 0)
    for (int j = tid; j < a.r; j += kStepThreads) a.chan_idx[(size_t)bh * a.r + j] = ch.chan[j];
  {
    const int pb_lo = split * a.ppb1, pb_hi = min(a.P, pb_lo + a.ppb1);
    const size_t sbase = (size_t)bh * D * a.s_pitch;
    const T* kmin_bh = static_cast<const T*>(a.kmin_t) + sbase;
    const T* kmax_bh = static_cast<const T*>(a.kmax_t) + sbase;
    float* pso = a.page_scores != nullptr ? a.page_scores + (size_t)bh * a.P : nullptr;
    uint64_t* xs = a.xscores + (size_t)bh * a.P;
    auto sink = [&](int p, float v) {
      if (multi)
        st_coherent(xs + p, tagged(v, epoch));
      else
        s_scores[p] = v;
      if (pso != nullptr) pso[p] = v;
    };
    if (a.vec)
      score_page_range<T, true>(kmin_bh, kmax_bh, D, a.s_pitch, a.r, pb_lo, pb_hi, ch, sink);
    else
      score_page_range<T, false>(kmin_bh, kmax_bh, D, a.s_pitch, a.r, pb_lo, pb_hi, ch, sink);
  }
  if (!attends) return;  // a scoring-only block

  // 2. the top pages of the head (every attending block finds them) and this block's slice.
  // Strided keys: thread t holds pages j * kStepThreads + t, straight from coalesced loads. In a
  // head of several blocks every attending block reads all the scores even when it needs none of
  // them: that wait orders every block's read of the epoch word before split 0 advances it.
  uint32_t key[E];
  const int nv = tid < a.P ? min(E, (a.P - 1 - tid) / kStepThreads + 1) : 0;
  if (multi) {
    const uint64_t* xs = a.xscores + (size_t)bh * a.P;
    uint64_t w[E];
    bool use[E];
    const uint64_t* ptr[E];
#pragma unroll
    for (int j = 0; j < E; ++j) {
      use[j] = j < nv;
      ptr[j] = xs + min(j * kStepThreads + tid, a.P - 1);
    }
    load_tagged<E>(w, use, ptr, epoch, a.sync);
#pragma unroll
    for (int j = 0; j < E; ++j) key[j] = use[j] ? order_key(tag_value(w[j])) : 0u;
  }
  const int p_lo = split * a.pps;
  const int p_hi = min(p_lo + a.pps, a.n_pages);
  const T* kc_bh = static_cast<const T*>(a.k_c) + (size_t)bh * a.kv_pitch * D;
  const T* vc_bh = static_cast<const T*>(a.v_c) + (size_t)bh * a.kv_pitch * D;
  const int32_t* rows_bh = a.rows != nullptr ? a.rows + (size_t)bh * a.Lc : nullptr;
  int32_t* pout = (a.page_idx != nullptr && split == 0) ? a.page_idx + (size_t)bh * a.n_pages
                                                        : nullptr;
  if (a.n_pages >= a.P) {
    for (int i = tid; pout != nullptr && i < a.n_pages; i += kStepThreads) pout[i] = i;
    for (int w0 = p_lo; w0 < p_hi; w0 += kMaxPagesPerSplit) {
      const int nw = min(kMaxPagesPerSplit, p_hi - w0);
      __syncthreads();
      for (int i = tid; i < nw; i += kStepThreads) sh.pages[i] = w0 + i;
      __syncthreads();
      st.run(kc_bh, vc_bh, sh.pages, nw * a.ps, a.ps, a.P, a.Lc, rows_bh, a.kv_pitch - 1);
    }
  } else {
    if (!multi) {
      __syncthreads();  // the block's own scores are in LDS
#pragma unroll
      for (int j = 0; j < E; ++j)
        key[j] = j < nv ? order_key(s_scores[min(j * kStepThreads + tid, a.P - 1)]) : 0u;
    }
    uint32_t thr, need_eq, eq_total;
    strided_threshold<kStepThreads, E>(key, nv, (uint32_t)a.n_pages, thr, need_eq, eq_total,
                                       ssel, sel);
    uint32_t pos[E], take;
    strided_positions<kStepThreads, E>(key, nv, thr, need_eq, eq_total == need_eq, ssel, pos,
                                       take);
    int w0 = p_lo;
    do {  // the first window also writes the full page list when asked
      const int nw = min(kMaxPagesPerSplit, max(p_hi - w0, 0));
      const bool write_out = pout != nullptr && w0 == p_lo;
      if (w0 != p_lo) __syncthreads();  // the previous window's attention has read its pages
#pragma unroll
      for (int j = 0; j < E; ++j) {
        if ((take >> j) & 1u) {
          const int p = (int)pos[j], idx = j * kStepThreads + tid;
          if (p >= w0 && p < w0 + nw) sh.pages[p - w0] = idx;
          if (write_out && p < a.n_pages) pout[p] = idx;
        }
      }
      __syncthreads();
      st.run(kc_bh, vc_bh, sh.pages, nw * a.ps, a.ps, a.P, a.Lc, rows_bh, a.kv_pitch - 1);
      w0 += kMaxPagesPerSplit;
    } while (w0 < p_hi);
  }

  // 3. attention partial of this block
  st.publish(sh);
  __syncthreads();
  T* out = static_cast<T*>(a.out) + (size_t)bh * G * D;
  const int nsa = a.nsplit_att;
  constexpr int kStride = G * D + 2 * G;
  uint64_t* hp = a.xpart + (size_t)bh * a.part_cap * kStride;
  if (nsa == 1) {
    for (int idx = tid; idx < G * D; idx += kStepThreads) {
      float M, lsum, o;
      wave_merge<D, G, kStepWaves>(sh, idx / D, idx % D, M, lsum, o);
      out[idx] = from_f32<T>(lsum > 0.f ? o / lsum : 0.f);
    }
  } else {
    uint64_t* mine = hp + (size_t)split * kStride;
    for (int idx = tid; idx < G * D; idx += kStepThreads) {
      const int g = idx / D, c = idx % D;
      float M, lsum, o;
      wave_merge<D, G, kStepWaves>(sh, g, c, M, lsum, o);
      st_coherent(mine + idx, tagged(o, epoch));
      if (c == 0) {
        st_coherent(mine + G * D + g, tagged(M, epoch));
        st_coherent(mine + G * D + G + g, tagged(lsum, epoch));
      }
    }
  }
  if (!multi) return;
  if (nsa > 1) {
    // 4. this block merges output elements [e0, e0 + ne) over every split
    const int cpb = (G * D + nsa - 1) / nsa;
    const int e0 = split * cpb;
    const int ne = min(cpb, G * D - e0);
    if (ne <= 0) return;  // (never split 0)
    const int g0 = e0 / D, ng = (e0 + ne - 1) / D - g0 + 1;
    MergeShared<D, G>& mg = u.mg;
    __syncthreads();  // the attention scratch is dead from here on
    // Items, indexed without division: o of (split s, element e) at s * NEP + e for e < ne (NEP
    // = ne rounded up to a power of two), then (max, sum) of (split s, group gg) at
    // NO + (which * kMaxSplit + s) * 8 + gg for gg < ng.
    const int lne = 32 - __clz(ne - 1);  // log2 of NEP
    const int NO = nsa << lne;
    const int n_all = NO + 2 * kMaxSplit * 8;
    for (int base = 0; base < n_all; base += kMergePer * kStepThreads) {
      uint64_t w[kMergePer];
      bool use[kMergePer];
      const uint64_t* ptr[kMergePer];
      int dst[kMergePer];  // LDS slot: o index, or -1 - (which * kMaxSplit * G + s * G + gg)
#pragma unroll
      for (int j = 0; j < kMergePer; ++j) {
        const int i = base + j * kStepThreads + tid;
        bool u_ = false;
        const uint64_t* pp = hp;
        int d = 0;
        if (i < NO) {
          const int sp = i >> lne, e = i & ((1 << lne) - 1);
          u_ = e < ne;
          pp = hp + (size_t)sp * kStride + e0 + min(e, ne - 1);
          d = sp * ne + e;
        } else if (i < n_all) {
          const int t = i - NO, gg = t & 7, sp = (t >> 3) & (kMaxSplit - 1), which = t >> 9;
          u_ = sp < nsa && gg < ng;
          pp = hp + (size_t)min(sp, nsa - 1) * kStride + G * D + which * G + g0 + min(gg, ng - 1);
          d = -1 - ((which * kMaxSplit + sp) * G + gg);
        }
        use[j] = u_;
        ptr[j] = pp;
        dst[j] = d;
      }
      load_tagged<kMergePer>(w, use, ptr, epoch, a.sync);
#pragma unroll
      for (int j = 0; j < kMergePer; ++j) {
        if (!use[j]) continue;
        const float v = tag_value(w[j]);
        if (dst[j] >= 0) {
          mg.o[dst[j]] = v;
        } else {
          const int d = -1 - dst[j], which = d / (kMaxSplit * G), r = d % (kMaxSplit * G);
          (which == 0 ? mg.m : mg.l)[r / G][r % G] = v;
        }
      }
    }
    __syncthreads();
    if (split == 0 && tid == 0) st_coherent(epoch_word, epoch);  // every split has published
    for (int gg = wave; gg < ng; gg += kStepWaves) {  // lane = split
      const float ms = lane < nsa ? mg.m[lane][gg] : -INFINITY;
      const float M = group_max<kWave>(ms);
      const float wgt = (lane < nsa && ms != -INFINITY) ? exp2_hw(ms - M) : 0.f;
      const float lsum = group_sum<kWave>(lane < nsa ? mg.l[lane][gg] * wgt : 0.f);
      if (lane < nsa) mg.m[lane][gg] = wgt;
      if (lane == 0) mg.inv[gg] = lsum > 0.f ? 1.f / lsum : 0.f;
    }
    __syncthreads();
    for (int e = tid; e < ne; e += kStepThreads) {
      const int gg = (e0 + e) / D - g0;
      float o = 0.f;
      for (int s = 0; s < nsa; ++s) o = fmaf(mg.o[s * ne + e], mg.m[s][gg], o);
      out[e0 + e] = from_f32<T>(o * mg.inv[gg]);
    }
  } else if (split == 0) {
    // a single attending block: it has read every score, so every block has read the epoch
    if (tid == 0) st_coherent(epoch_word, epoch);
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
  // a small budget goes to one block per head: its output is written without a merge launch
  ns = ntok <= kStepSoloTokens ? 1 : min(ns, (ntok + chunk - 1) / chunk);
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
  const int chunk = kStepTokensPerBlock;
  const int ns = max(min(ncu / BH, kMaxSplit), 1);
  // a small budget goes to one block (no partials to merge across blocks)
  int na = ntok <= kStepSoloTokens ? 1
                                   : max(min(min(ns, kMaxAttending), (ntok + chunk - 1) / chunk), 1);
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
  if (a.P <= 8 * kStepThreads)
    hipLaunchKernelGGL((k_decode_step<T, D, G, 8>), dim3(BH, a.nsplit), dim3(kStepThreads), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((k_decode_step<T, D, G, 16>), dim3(BH, a.nsplit), dim3(kStepThreads), 0,
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
  size_t off_sync, off_xscores, off_xpart, total;
  int part_cap;
};

// Depends on the shape only (not on n_pages or the device), so one initialised workspace serves
// every top-k budget of a shape. Partial slots are sized for the largest split count any device
// can get (kTargetBlocks CUs); a plan with one block per head exchanges nothing.
StepLayout step_layout(int B, int Hq, int Hkv, int D, int P) {
  const size_t BH = (size_t)B * Hkv;
  const int G = Hq / Hkv;
  StepLayout lo{};
  lo.part_cap = max(min(kTargetBlocks / (int)std::min<size_t>(BH, kTargetBlocks), kMaxSplit), 1);
  lo.off_sync = 0;
  lo.off_xscores = align256((16 + BH) * sizeof(unsigned));
  if (lo.part_cap == 1) {
    lo.off_xpart = lo.total = lo.off_xscores;
    return lo;
  }
  lo.off_xpart = align256(lo.off_xscores + BH * P * sizeof(uint64_t));
  lo.total = align256(lo.off_xpart + BH * lo.part_cap * (size_t)G * (D + 2) * sizeof(uint64_t));
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

size_t decode_ws_bytes(int B, int Hq, int Hkv, int Lc, int D, int page_size, int, int) {
  const int P = (Lc + page_size - 1) / page_size;
  return step_layout(B, Hq, Hkv, D, P).total;
}

hipError_t launch_decode_ws_init(void* ws, size_t bytes, hipStream_t stream) {
  const size_t n = bytes / sizeof(unsigned);
  const int blocks = (int)std::min<size_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(k_zero_u32, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, stream,
                     static_cast<unsigned*>(ws), n);
  return hipGetLastError();
}

hipError_t launch_decode_step(const void* q, const void* kmin_t, const void* kmax_t,
                              const void* k_c, const void* v_c, const int32_t* rows, int B, int Hq,
                              int Hkv, int Lc, int kv_pitch, int cap, int D, int page_size, int r,
                              int n_pages, float scale, int dtype, int32_t* chan_idx,
                              float* page_scores, int32_t* page_idx, void* out, void* ws,
                              hipStream_t stream) {
  const int BH = B * Hkv;
  const int P = (Lc + page_size - 1) / page_size;
  const int Pcap = (cap + page_size - 1) / page_size;
  // laid out for the capacity, so a growing cache never moves a head's exchanged words
  const StepLayout lo = step_layout(B, Hq, Hkv, D, Pcap);
  StepPlan pl = plan_step_any(dtype, D, BH, page_size, n_pages, device_cus());
  if (pl.nsplit > lo.part_cap) return hipErrorInvalidValue;  // cannot happen: cap is the maximum
  char* w = static_cast<char*>(ws);
  const int vmax = dtype == 0 ? vec16<float>::n : vec16<bf16_t>::n;
  int ppb1 = (P + pl.nsplit - 1) / pl.nsplit;
  ppb1 = (ppb1 + vmax - 1) / vmax * vmax;
  StepArgs a{q, kmin_t, kmax_t, k_c, v_c, BH, Hkv, Lc, page_size, n_pages, P, r, pl.pps, ppb1,
             pl.nsplit, pl.nsplit_att, lo.part_cap, Pcap % vmax == 0, kv_pitch, rows, Pcap,
             scale * kLog2e, chan_idx,
             page_scores, page_idx, reinterpret_cast<uint64_t*>(w + lo.off_xscores),
             reinterpret_cast<uint64_t*>(w + lo.off_xpart),
             reinterpret_cast<unsigned*>(w + lo.off_sync), out};
  const int G = Hq / Hkv;
  if (dtype == 0)
    return D == 64 ? step_d<float, 64>(G, a, BH, stream) : step_d<float, 128>(G, a, BH, stream);
  return D == 64 ? step_d<bf16_t, 64>(G, a, BH, stream) : step_d<bf16_t, 128>(G, a, BH, stream);
}

}  // namespace rkv
