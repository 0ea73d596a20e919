// One hybrid decode step in one kernel launch (RocketKV rebuttal, "Lack of Direct Latency
// Comparison": Steps 1-2 approximate the attention scores and select, Step 3 attends to the
// selected tokens; "Explanation of Calculating Approximate Attention Scores": the page bound on
// the channels where |q| is large, one selection per GQA group).
//
// Roles. The grid is (B*Hkv, nb): nb blocks per head. A block's role comes from a ticket it draws
// from a per-head counter as it starts, not from its block index:
//   rank < ns            scorer: ranks the channels and scores share `rank` of the head's pages;
//   rank >= ns - 1       attender: waits for every score, selects the top pages and attends to
//                        slice rank - (ns - 1) of the ascending page list (the last scorer is also
//                        the first attender, so nb = ns + na - 1).
// A block only ever waits for data that blocks with a lower rank produce, and a block that holds a
// ticket has started, so every wait ends however the blocks are scheduled: no block needs another
// to be resident at the same time. Several attenders combine their partials through a counter:
// the one that arrives last merges them (nobody waits for a later arrival) and writes the output.
//
// Exchange. Scores and partials cross blocks as 64-bit words {value bits, epoch} written and read
// with device-coherent relaxed atomics; a reader re-reads a word until its tag is the current
// epoch, so no fence or flag orders anything. The block that finishes the head (the merger, or the
// only attender) resets the head's counters and stores the new epoch, after it has seen every
// block's output, hence after every block of the head has drawn its ticket and read the epoch.
// Every wait is bounded by wall-clock time: a wait that runs out (which only a block that stalls
// far beyond the step's own time can cause) sets a status bit and proceeds with what it has.
//
// One-block heads (large B*Hkv: nb = 1) score into LDS and exchange nothing.
#pragma once

#include <math.h>

#include <algorithm>

#include "rkv_approx.hpp"
#include "rkv_attend.hpp"
#include "rkv_common.hpp"
#include "rkv_select.hpp"

namespace rkv {
namespace step {

constexpr int kThreads = 512;  // two waves per SIMD
constexpr int kWaves = kThreads / kWave;
constexpr int kSlots = 4;            // row loads per wave per chunk of attention
constexpr int kSoloTokens = 128;     // budgets up to this many tokens: one attender per head
constexpr int kTokensPerBlock = 64;  // otherwise one attender per this many budget tokens,
constexpr int kMaxAttending = 16;    // at most this many per head
constexpr int kMaxScorers = 64;
constexpr int kTargetBlocks = 256;   // CUs of an MI355X: the grid of a waiting plan fits them
constexpr int kSyncHeader = 16;      // words before the per-head words; word 0 is the status
constexpr int kHeadWords = 4;        // per head: epoch, ticket counter, arrival counter, spare

enum : unsigned {
  kStatusScoreWait = 1u,    // an attender's wait for the scores ran out of time
  kStatusPartialWait = 2u,  // the merger's wait for the partials ran out of time
  kStatusTicket = 4u,       // a block drew a ticket beyond the plan (workspace state corrupt)
};

struct Args {
  const void* q;
  const void* kmin_t;
  const void* kmax_t;
  const void* k_c;
  const void* v_c;
  int BH, Hkv, Lc, ps, n_pages, P, r;
  int ns, na, nb;        // scorers, attenders and blocks per head
  int ppb1, pps, vec;    // pages per scorer (vector multiple), list pages per attender, vector rows
  int cap_s, cap_a;      // exchange slots per head for scorer extremes and attender partials
  int kv_pitch;          // token slots per head of k_c, v_c (>= Lc; the full length L with rows)
  const int32_t* rows;   // optional [BH, Lc]: slot t of head bh is row rows[bh*Lc + t] of k_c, v_c
  int s_pitch;           // pages per channel row of the summaries (>= P)
  float scale2;          // softmax scale * log2(e)
  long long wait_ticks;  // bound of one wait, in steady-counter ticks
  int32_t* chan_idx;     // optional [BH, r]
  float* page_scores;    // optional [BH, P]
  int32_t* page_idx;     // optional [BH, n_pages]
  uint64_t* xscores;     // [BH, P] tagged page scores
  uint64_t* xext;        // [BH, cap_s, 2] tagged (largest, smallest) score key of each share
  uint64_t* xpart;       // [BH, cap_a, G*D + 2G] tagged partials: o[G*D], M[G], l[G]
  unsigned* sync;        // [0] status; [kSyncHeader + kHeadWords*bh + 0/1/2] epoch/ticket/arrivals
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
__device__ __forceinline__ unsigned add_coherent(unsigned* p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t tagged(uint32_t bits, unsigned epoch) {
  return ((uint64_t)epoch << 32) | bits;
}
__device__ __forceinline__ bool tag_is(uint64_t w, unsigned epoch) {
  return (unsigned)(w >> 32) == epoch;
}
__device__ __forceinline__ uint32_t tag_bits(uint64_t w) { return (uint32_t)w; }

// Loads the N words addr(j) with use[j] until every tag is `epoch`: a waiting wave re-reads only
// its stale words, after a short sleep. Bounded by wall-clock time (wait_ticks): on running out,
// `flag` is or-ed into the status word and the stale values stay. Call with the whole wave.
template <int N, typename Addr>
__device__ __forceinline__ void poll_tagged(uint64_t (&w)[N], const bool (&use)[N], Addr&& addr,
                                            unsigned epoch, long long wait_ticks,
                                            unsigned* status, unsigned flag) {
#pragma unroll
  for (int j = 0; j < N; ++j) w[j] = use[j] ? ld_coherent(addr(j)) : 0ull;
  long long deadline = 0;
  for (bool first = true;; first = false) {
    bool stale = false;
#pragma unroll
    for (int j = 0; j < N; ++j) stale = stale || (use[j] && !tag_is(w[j], epoch));
    if (__ballot(stale) == 0ull) return;
    const long long now = wall_clock64();
    if (first) deadline = now + wait_ticks;
    if (now > deadline) {
      if (stale) __hip_atomic_fetch_or(status, flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int j = 0; j < N; ++j)
      if (use[j] && !tag_is(w[j], epoch)) w[j] = ld_coherent(addr(j));
  }
}

template <int G>
struct MergeShared {
  float m[kMaxAttending][G];
  float l[kMaxAttending][G];
};

template <typename T, int D, int G, int E>
__global__ __launch_bounds__(kThreads) void k_decode_step(Args a) {
  __shared__ ChannelShared ch;
  // A one-block head's own scores are dead once its keys are in registers, which happens before
  // the selection's first barrier and so before any page-list or attention write.
  __shared__ union {
    __align__(16) float scores[E * kThreads];
    AttendShared<D, G, kWaves> att;
  } u;
  __shared__ MergeShared<G> mg;
  __shared__ SelectShared<kThreads> sel;  // the radix passes for clustered scores
  __shared__ StridedShared<kThreads, E> ssel;
  __shared__ unsigned s_rank, s_arrival, s_kmax, s_kmin;
  AttendShared<D, G, kWaves>& sh = u.att;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  // grid (BH, nb): consecutive blocks belong to different heads, so the round-robin placement of
  // blocks on the XCDs keeps every block of a head on one XCD when BH is a multiple of 8
  const int bh = blockIdx.x, b = bh / a.Hkv, h = bh % a.Hkv;
  const T* q = static_cast<const T*>(a.q);
  const bool multi = a.nb > 1;
  unsigned* hw = a.sync + kSyncHeader + kHeadWords * bh;

  // First loads, all in flight together: the head's epoch, a ticket, the queries for the
  // attention and for the channel choice.
  const unsigned epoch_prev = multi ? ld_coherent(hw) : 0u;
  unsigned ticket = 0u;
  if (multi && tid == 0) ticket = add_coherent(hw + 1, 1u);
  WaveState<T, D, G, kWaves, kSlots> st;
  st.load_q(q + (size_t)bh * G * D);
  ChannelQ<T, G> cq;
  cq.load(q, b, h, a.Hkv, D);
  strided_clear(ssel);  // ordered before its use by the channel choice's barrier
  if (tid == 0) {
    s_rank = ticket;
    s_kmax = 0u;
    s_kmin = 0xffffffffu;
  }
  select_channels_phase1<T, G>(cq, D, ch);  // ends with a barrier
  const int rank = (int)s_rank;
  if (rank >= a.nb) {  // only a workspace left inconsistent by an earlier failure gets here
    if (tid == 0)
      __hip_atomic_fetch_or(a.sync, kStatusTicket, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  unsigned epoch = epoch_prev + 1u;
  if (epoch == 0u) epoch = 1u;  // tag 0 is what a cleared workspace holds
  const bool attends = rank >= a.ns - 1;

  // 1. scorer: its share of the head's approximate page scores
  if (rank < a.ns) {
    select_channels_phase2(D, a.r, ch);
    if (a.chan_idx != nullptr && rank == 0)
      for (int j = tid; j < a.r; j += kThreads) a.chan_idx[(size_t)bh * a.r + j] = ch.chan[j];
    const int pb_lo = rank * a.ppb1, pb_hi = min(a.P, pb_lo + a.ppb1);
    const size_t sbase = (size_t)bh * D * a.s_pitch;
    const T* kmin_bh = static_cast<const T*>(a.kmin_t) + sbase;
    const T* kmax_bh = static_cast<const T*>(a.kmax_t) + sbase;
    float* pso = a.page_scores != nullptr ? a.page_scores + (size_t)bh * a.P : nullptr;
    uint64_t* xs = a.xscores + (size_t)bh * a.P;
    uint32_t kmax = 0u, kmin = 0xffffffffu;
    auto sink = [&](int p, float v) {
      if (multi) {
        st_coherent(xs + p, tagged(__float_as_uint(v), epoch));
        const uint32_t k = order_key(v);
        kmax = max(kmax, k);
        kmin = min(kmin, k);
      } else {
        u.scores[p] = v;
      }
      if (pso != nullptr) pso[p] = v;
    };
    if (a.vec)
      score_page_range<T, true>(kmin_bh, kmax_bh, D, a.s_pitch, a.r, pb_lo, pb_hi, ch, sink);
    else
      score_page_range<T, false>(kmin_bh, kmax_bh, D, a.s_pitch, a.r, pb_lo, pb_hi, ch, sink);
    if (multi) {
      // the share's largest and smallest keys, so an attender needs no block reduction for them
      kmax = wave_reduce_u32(kmax, OpMaxU{});
      kmin = wave_reduce_u32(kmin, OpMinU{});
      if (lane == 0) {
        atomicMax(&s_kmax, kmax);
        atomicMin(&s_kmin, kmin);
      }
      __syncthreads();
      if (tid == 0) {
        uint64_t* xe = a.xext + ((size_t)bh * a.cap_s + rank) * 2;
        st_coherent(xe, tagged(s_kmax, epoch));
        st_coherent(xe + 1, tagged(s_kmin, epoch));
      }
    }
  }
  if (!attends) return;
  const int slice = rank - (a.ns - 1);

  // 2. the head's top pages (every attender finds them) and this attender's slice. Strided keys:
  // thread t holds pages j * kThreads + t, straight from coalesced loads. An attender reads every
  // score even when it needs none (every page selected): having seen them, it knows that every
  // scorer has drawn its ticket and read the epoch.
  st.init(a.scale2);
  uint32_t key[E];
  const int nv = tid < a.P ? min(E, (a.P - 1 - tid) / kThreads + 1) : 0;
  uint32_t lo = 0u, hi = 0u;
  if (multi) {
    const uint64_t* xs = a.xscores + (size_t)bh * a.P;
    const uint64_t* xe = a.xext + (size_t)bh * a.cap_s * 2;
    uint64_t w[E + 2];
    bool use[E + 2];
#pragma unroll
    for (int j = 0; j < E; ++j) use[j] = j < nv;
    use[E] = use[E + 1] = lane < a.ns;
    poll_tagged<E + 2>(
        w, use,
        [&](int j) {
          return j < E ? xs + min(j * kThreads + tid, a.P - 1)
                       : xe + min(lane, a.ns - 1) * 2 + (j - E);
        },
        epoch, a.wait_ticks, a.sync, kStatusScoreWait);
#pragma unroll
    for (int j = 0; j < E; ++j) key[j] = use[j] ? order_key(__uint_as_float(tag_bits(w[j]))) : 0u;
    hi = wave_max_u32(use[E] ? tag_bits(w[E]) : 0u);
    lo = wave_min_u32(use[E] ? tag_bits(w[E + 1]) : 0xffffffffu);
  }
  const int p_lo = slice * a.pps;
  const int p_hi = min(p_lo + a.pps, a.n_pages);
  const T* kc_bh = static_cast<const T*>(a.k_c) + (size_t)bh * a.kv_pitch * D;
  const T* vc_bh = static_cast<const T*>(a.v_c) + (size_t)bh * a.kv_pitch * D;
  const int32_t* rows_bh = a.rows != nullptr ? a.rows + (size_t)bh * a.Lc : nullptr;
  int32_t* pout = (a.page_idx != nullptr && slice == 0) ? a.page_idx + (size_t)bh * a.n_pages
                                                        : nullptr;
  if (a.n_pages >= a.P) {
    for (int i = tid; pout != nullptr && i < a.n_pages; i += kThreads) pout[i] = i;
    for (int w0 = p_lo; w0 < p_hi; w0 += kMaxPagesPerSplit) {
      const int nw = min(kMaxPagesPerSplit, p_hi - w0);
      __syncthreads();
      for (int i = tid; i < nw; i += kThreads) sh.pages[i] = w0 + i;
      __syncthreads();
      st.run(kc_bh, vc_bh, sh.pages, nw * a.ps, a.ps, a.P, a.Lc, rows_bh, a.kv_pitch - 1);
    }
  } else {
    if (!multi) {
      __syncthreads();  // the block's own scores are in LDS
#pragma unroll
      for (int j = 0; j < E; ++j)
        key[j] = j < nv ? order_key(u.scores[min(j * kThreads + tid, a.P - 1)]) : 0u;
    }
    uint32_t thr, need_eq, eq_total;
    strided_threshold<kThreads, E>(key, nv, (uint32_t)a.n_pages, thr, need_eq, eq_total, ssel, sel,
                                   multi, lo, hi);
    uint32_t pos[E], take;
    strided_positions<kThreads, E>(key, nv, thr, need_eq, eq_total == need_eq, ssel, pos, take);
    int w0 = p_lo;
    do {  // the first window also writes the full page list when asked
      const int nw = min(kMaxPagesPerSplit, max(p_hi - w0, 0));
      const bool write_out = pout != nullptr && w0 == p_lo;
      if (w0 != p_lo) __syncthreads();  // the previous window's attention has read its pages
#pragma unroll
      for (int j = 0; j < E; ++j) {
        if ((take >> j) & 1u) {
          const int p = (int)pos[j], idx = j * kThreads + tid;
          if (p >= w0 && p < w0 + nw) sh.pages[p - w0] = idx;
          if (write_out && p < a.n_pages) pout[p] = idx;
        }
      }
      __syncthreads();
      st.run(kc_bh, vc_bh, sh.pages, nw * a.ps, a.ps, a.P, a.Lc, rows_bh, a.kv_pitch - 1);
      w0 += kMaxPagesPerSplit;
    } while (w0 < p_hi);
  }

  // 3. this attender's partial
  st.publish(sh);
  __syncthreads();
  T* out = static_cast<T*>(a.out) + (size_t)bh * G * D;
  constexpr int kStride = G * D + 2 * G;
  if (a.na == 1) {
    for (int idx = tid; idx < G * D; idx += kThreads) {
      float M, lsum, o;
      wave_merge<D, G, kWaves>(sh, idx / D, idx % D, M, lsum, o);
      out[idx] = from_f32<T>(lsum > 0.f ? o / lsum : 0.f);
    }
    if (multi && tid == 0) {  // the head is finished: counters back to zero, the next epoch
      st_coherent(hw + 1, 0u);
      st_coherent(hw, epoch);
    }
    return;
  }
  uint64_t* hp = a.xpart + (size_t)bh * a.cap_a * kStride;
  {
    uint64_t* mine = hp + (size_t)slice * kStride;
    for (int idx = tid; idx < G * D; idx += kThreads) {
      const int g = idx / D, c = idx % D;
      float M, lsum, o;
      wave_merge<D, G, kWaves>(sh, g, c, M, lsum, o);
      st_coherent(mine + idx, tagged(__float_as_uint(o), epoch));
      if (c == 0) {
        st_coherent(mine + G * D + g, tagged(__float_as_uint(M), epoch));
        st_coherent(mine + G * D + G + g, tagged(__float_as_uint(lsum), epoch));
      }
    }
  }
  __syncthreads();  // every store of the partial is issued before the arrival is counted
  if (tid == 0) s_arrival = add_coherent(hw + 2, 1u);
  __syncthreads();
  if (s_arrival != (unsigned)(a.na - 1)) return;

  // 4. the last attender to arrive merges every partial of the head: the (max, sum) words of
  // every (attender, head) go to LDS, then each thread combines its output elements, one element
  // per round (a round's words are all in flight together)
  constexpr int NE = (G * D + kThreads - 1) / kThreads;  // output elements per thread
  const int nml = 2 * a.na * G;
#pragma unroll 1
  for (int e = 0; e < NE; ++e) {
    const int idx = tid + e * kThreads;
    constexpr int NW = kMaxAttending + 1;  // the element's words, then one (max or sum) word
    uint64_t w[NW];
    bool use[NW];
#pragma unroll
    for (int s = 0; s < kMaxAttending; ++s) use[s] = s < a.na && idx < G * D;
    use[NW - 1] = e == 0 && tid < nml;
    poll_tagged<NW>(
        w, use,
        [&](int j) {
          if (j == NW - 1) {
            const int t = min(tid, nml - 1), which = t / (a.na * G), rem = t % (a.na * G);
            return hp + (size_t)(rem / G) * kStride + G * D + which * G + rem % G;
          }
          return hp + (size_t)min(j, a.na - 1) * kStride + min(idx, G * D - 1);
        },
        epoch, a.wait_ticks, a.sync, kStatusPartialWait);
    if (e == 0) {
      if (use[NW - 1]) {
        const int which = tid / (a.na * G), rem = tid % (a.na * G);
        (which == 0 ? mg.m : mg.l)[rem / G][rem % G] = __uint_as_float(tag_bits(w[NW - 1]));
      }
      __syncthreads();
    }
    if (idx >= G * D) continue;
    const int g = idx / D;
    float M = -INFINITY;
    for (int s = 0; s < a.na; ++s) M = fmaxf(M, mg.m[s][g]);
    float lsum = 0.f, o = 0.f;
#pragma unroll
    for (int s = 0; s < kMaxAttending; ++s) {
      const int sc = min(s, a.na - 1);
      const float ms = mg.m[sc][g];
      const float wt = (s >= a.na || ms == -INFINITY) ? 0.f : exp2_hw(ms - M);
      lsum = fmaf(mg.l[sc][g], wt, lsum);
      o = fmaf(__uint_as_float(tag_bits(w[s])), wt, o);
    }
    out[idx] = from_f32<T>(lsum > 0.f ? o / lsum : 0.f);
  }
  if (tid == 0) {  // every block of the head is done with the counters and the epoch
    st_coherent(hw + 1, 0u);
    st_coherent(hw + 2, 0u);
    st_coherent(hw, epoch);
  }
}

// Blocks per head. A plan in which blocks wait keeps the whole grid within one block per CU, so
// that waiting never depends on a block that has yet to find room; the waits are correct without
// that (tickets), it only keeps the step from running in two rounds. Budgets of at most
// kSoloTokens tokens get one attender (no partials to merge); larger ones one per
// kTokensPerBlock tokens, at most kMaxAttending; the remaining blocks score.
struct Plan {
  int ns, na, nb, ppb1, pps;
};

inline Plan plan(int BH, int P, int ps, int n_pages, int ncu, int vmax) {
  const int budget = ncu / BH;  // blocks per head within one block per CU
  const int ntok = n_pages * ps;
  int na = 1, ns = 1;
  if (budget >= 2) {
    na = ntok <= kSoloTokens ? 1
                             : std::max(std::min(std::min(kMaxAttending, budget),
                                                 (ntok + kTokensPerBlock - 1) / kTokensPerBlock),
                                        1);
    ns = std::min(std::max(budget - na + 1, 1), kMaxScorers);
  }
  int pps = (n_pages + na - 1) / na;
  na = (n_pages + pps - 1) / pps;
  int ppb1 = (P + ns - 1) / ns;
  ppb1 = (ppb1 + vmax - 1) / vmax * vmax;
  ns = (P + ppb1 - 1) / ppb1;
  return {ns, na, ns + na - 1, ppb1, pps};
}

// Exchange slots per head, sized for the largest plan any device can get (kTargetBlocks CUs), so
// the layout depends on the shape only. A shape whose heads cannot get two blocks exchanges nothing.
struct Layout {
  size_t off_sync, off_xscores, off_xext, off_xpart, total;
  int cap_s, cap_a;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline Layout layout(int B, int Hq, int Hkv, int D, int Pcap) {
  const size_t BH = (size_t)B * Hkv;
  const int G = Hq / Hkv;
  Layout lo{};
  const int budget = BH >= (size_t)kTargetBlocks ? 0 : kTargetBlocks / (int)BH;
  lo.off_sync = 0;
  lo.off_xscores = align256((kSyncHeader + kHeadWords * BH) * sizeof(unsigned));
  if (budget < 2) {
    lo.cap_s = lo.cap_a = 1;
    lo.off_xext = lo.off_xpart = lo.total = lo.off_xscores;
    return lo;
  }
  lo.cap_s = std::min(budget, kMaxScorers);
  lo.cap_a = std::min(budget, kMaxAttending);
  lo.off_xext = align256(lo.off_xscores + BH * (size_t)Pcap * sizeof(uint64_t));
  lo.off_xpart = align256(lo.off_xext + BH * (size_t)lo.cap_s * 2 * sizeof(uint64_t));
  lo.total = align256(lo.off_xpart + BH * (size_t)lo.cap_a * (G * D + 2 * G) * sizeof(uint64_t));
  return lo;
}

template <typename T, int D, int G>
hipError_t launch_g(const Args& a, hipStream_t stream) {
  if (a.P <= 8 * kThreads)
    hipLaunchKernelGGL((k_decode_step<T, D, G, 8>), dim3(a.BH, a.nb), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((k_decode_step<T, D, G, 16>), dim3(a.BH, a.nb), dim3(kThreads), 0, stream,
                       a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(int G, const Args& a, hipStream_t s) {
  switch (G) {
    case 1: return launch_g<T, D, 1>(a, s);
    case 2: return launch_g<T, D, 2>(a, s);
    case 3: return launch_g<T, D, 3>(a, s);
    case 4: return launch_g<T, D, 4>(a, s);
    case 5: return launch_g<T, D, 5>(a, s);
    case 6: return launch_g<T, D, 6>(a, s);
    case 7: return launch_g<T, D, 7>(a, s);
    case 8: return launch_g<T, D, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace step

// Per-dtype launchers (one translation unit each).
hipError_t step_launch_f32(int D, int G, const step::Args& a, hipStream_t stream);
hipError_t step_launch_bf16(int D, int G, const step::Args& a, hipStream_t stream);

}  // namespace rkv
