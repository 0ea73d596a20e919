// One hybrid decode step in one kernel launch (RocketKV rebuttal, "Lack of Direct Latency
// Comparison": Steps 1-2 approximate the attention scores and select, Step 3 attends to the
// selected tokens; "Explanation of Calculating Approximate Attention Scores": the page bound on
// the channels where |q| is large, one selection per GQA group).
//
// Roles. The grid is (B*Hkv, nb): nb blocks per head. Block y scores share y of the head's pages
// (y < ns); blocks y < na also attend: each reads every score, selects the top pages, attends to
// slice y of the ascending page list and publishes its partial; with several attenders, each
// then merges a range of the head's outputs over every slice's partial.
// Progress without co-residency. A waiting block never depends on another block being resident:
// a wait that has not seen its data after a steal deadline (tens of microseconds, far beyond the
// step's own duration) computes the missing work itself. An attender scores the shares it is
// missing and attends the slices whose partials it is missing; the results are bit-identical to
// the owner's, so work done twice is harmless. So a call finishes however its blocks are
// scheduled, also while other kernels hold CUs, and it needs no counter on its critical path.
//
// Exchange. Scores and partials cross blocks as 64-bit words {value bits, epoch}, read with
// device-coherent relaxed atomic loads, which pass the CU's own cache; a reader re-reads a word
// until its tag is the current epoch, so no fence or flag orders anything. Where every block of a
// head runs on one XCD (a.xcd_local), the words are written with workgroup-scope stores: the CU's
// cache writes through into the XCD's L2, which those loads read, so no word travels past that L2.
// The memory model does not promise another block that visibility; the cache arrangement gives it,
// and a word that never showed up would only cost the steal deadline (below), not a wrong value: a
// block's re-reads of words its own threads wrote are within the stores' scope. Elsewhere the words
// are written device-coherently.
// Each block reads the head's stored epoch at its start and then counts itself as started; the
// block that finds it was the last to start (at its end, so the count's round trip delays nobody)
// stores the new epoch and clears the count: by then every block of the head has read the old
// epoch, and no block of the call reads it again.
//
// One-block heads (nb = 1: heads of at most 128 pages, or more heads than fit two blocks each)
// score into LDS and exchange nothing. Over kTargetBlocks heads the step does not use this kernel
// (pipelined(): the scoring, top-k and attention kernels of the separate calls, in turn).
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
constexpr int kSoloTokens = 256;     // budgets up to this many tokens: one attender per head
constexpr int kTokensPerBlock = 64;  // otherwise one attender per this many budget tokens,
constexpr int kMaxAttending = 16;    // at most this many per head
constexpr int kMaxScorers = 64;
// A score share never has fewer pages than this: a head of few pages is scored by few blocks
// (one for 128 pages, with no exchange at all), as each share costs a full exchange round trip.
constexpr int kMinScorePages = 128;
constexpr int kTargetBlocks = 256;   // CUs of an MI355X: the grid of a waiting plan fits them
constexpr int kXcds = 8;             // XCDs of an MI355X, dealt blocks round-robin by linear id
// Touching ahead (Args::pf): budgets up to kPrefetchTokens tokens, shares up to kPrefetchShare
// pages (the share is ranked in LDS, one page per thread against all), at most kPrefetchPages.
constexpr int kPrefetchTokens = 512;
constexpr int kPrefetchShare = 256;
constexpr int kPrefetchPages = 8;
constexpr int kSyncHeader = 16;      // words before the per-head words; word 0 is the status
constexpr int kHeadWords = 4;        // per head: epoch, started count, two spare

enum : unsigned {
  kStatusScoreWait = 1u,     // an attender's wait for score words ran out of time
  kStatusPartialWait = 2u,   // the merger's wait for partials ran out of time
  kStatusStoleShare = 16u,   // informational: an attender scored a share it found missing
  kStatusStoleSlice = 32u,   // informational: the merger attended a slice it found missing
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
  int cap_a;             // partial slots per head
  int kv_pitch;          // token slots per head of k_c, v_c (>= Lc; the full length L with rows)
  const int32_t* rows;   // optional [BH, Lc]: slot t of head bh is row rows[bh*Lc + t] of k_c, v_c
  int s_pitch;           // pages per channel row of the summaries (>= P)
  int xcd_local;         // every block of a head runs on one XCD (exchange words stay in its L2)
  int pf;                // pages of its own share whose K/V rows a block that only scores touches
                         // after scoring (0: none)
  float scale2;          // softmax scale * log2(e)
  long long steal_ticks; // wait before a block does missing work itself (steady-counter
                         // ticks); negative: it does all of it itself (a test mode)
  long long wait_ticks;  // bound of a wait for words that must already be on their way
  int32_t* chan_idx;     // optional [BH, r]
  float* page_scores;    // optional [BH, P]
  int32_t* page_idx;     // optional [BH, n_pages]
  uint64_t* xscores;     // [BH, P] tagged page scores
  uint64_t* xpart;       // [BH, cap_a, G*D + 2G] tagged partials: o[G*D], M[G], l[G]
  unsigned* sync;        // [0] status; [kSyncHeader + kHeadWords*bh + 0/1] epoch/started count
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
// An exchange word, written as described at the top of this file.
template <typename V>
__device__ __forceinline__ void st_exchange(V* p, V v, bool xcd_local) {
  if (xcd_local)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  else
    st_coherent(p, v);
}
// *p + 1, returning the old value. An increment rather than an add: the compiler turns a
// wave-uniform atomic add into a wave-wide one whose result it waits for at once, which would put
// the atomic's round trip in front of the block's next barrier.
__device__ __forceinline__ unsigned inc_coherent(unsigned* p) {
  return __builtin_amdgcn_atomic_inc32(p, 0xffffffffu, __ATOMIC_RELAXED, "agent");
}
__device__ __forceinline__ void set_status(unsigned* status, unsigned flag) {
  __hip_atomic_fetch_or(status, flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t tagged(uint32_t bits, unsigned epoch) {
  return ((uint64_t)epoch << 32) | bits;
}
__device__ __forceinline__ bool tag_is(uint64_t w, unsigned epoch) {
  return (unsigned)(w >> 32) == epoch;
}
__device__ __forceinline__ uint32_t tag_bits(uint64_t w) { return (uint32_t)w; }

// Loads the N words addr(j) with use[j] until every tag is `epoch` or `ticks` of wall-clock time
// have passed: a waiting wave re-reads only its stale words, after a short sleep. Returns whether
// any of this lane's words is still stale. Call with the whole wave (the exit is wave-uniform).
// With fresh, every used word is loaded first; otherwise w already holds earlier reads and only
// its stale words are loaded again.
template <int N, int SLEEP = 1, typename Addr>
__device__ __forceinline__ bool poll_tagged(uint64_t (&w)[N], const bool (&use)[N], Addr&& addr,
                                            unsigned epoch, long long ticks, bool fresh = true) {
#pragma unroll
  for (int j = 0; j < N; ++j)
    if (use[j] && (fresh || !tag_is(w[j], epoch))) w[j] = ld_coherent(addr(j));
  long long deadline = 0;
  for (bool first = true;; first = false) {
    bool stale = false;
#pragma unroll
    for (int j = 0; j < N; ++j) stale = stale || (use[j] && !tag_is(w[j], epoch));
    if (__ballot(stale) == 0ull) return false;
    const long long now = wall_clock64();
    if (first) deadline = now + ticks;
    if (now > deadline) return stale;
    __builtin_amdgcn_s_sleep(SLEEP);
#pragma unroll
    for (int j = 0; j < N; ++j)
      if (use[j] && !tag_is(w[j], epoch)) w[j] = ld_coherent(addr(j));
  }
}

template <int D, int G>
struct MergeShared {
  float o[G * D + kMaxAttending];  // [slice][element of this attender's range]
  float m[kMaxAttending][G];       // every slice's max of each head of the group
  float l[kMaxAttending][G];       // and its sum
  unsigned missing;                // slices with a stale word at the steal deadline
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
  __shared__ MergeShared<D, G> mg;
  __shared__ SelectShared<kThreads> sel;  // the radix passes for clustered scores
  __shared__ StridedShared<kThreads, E> ssel;
  __shared__ unsigned s_miss_lo, s_miss_hi;
  AttendShared<D, G, kWaves>& sh = u.att;
  const int tid = threadIdx.x;
  // grid (BH, nb): consecutive blocks belong to different heads, so the round-robin placement of
  // blocks on the XCDs keeps every block of a head on one XCD when BH is a multiple of 8
  const int bh = blockIdx.x, y = blockIdx.y, b = bh / a.Hkv, h = bh % a.Hkv;
  const T* q = static_cast<const T*>(a.q);
  const bool multi = a.nb > 1;
  unsigned* hw = a.sync + kSyncHeader + kHeadWords * bh;

  // First loads, all in flight together: the head's epoch and the queries for the attention and
  // for the channel choice.
  const unsigned epoch_prev = multi ? ld_coherent(hw) : 0u;
  WaveState<T, D, G, kWaves, kSlots> st;
  st.load_q(q + (size_t)bh * G * D);
  ChannelQ<T, G> cq;
  cq.load(q, b, h, a.Hkv, D);
  strided_clear(ssel);  // ordered before its use by the channel choice's barriers
  if (tid == 0) {
    s_miss_lo = s_miss_hi = 0u;
    mg.missing = 0u;
  }
  select_channels_phase1<T, G>(cq, D, ch);
  select_channels_phase2<8, kThreads>(D, a.r, ch);
  unsigned epoch = epoch_prev + 1u;
  if (epoch == 0u) epoch = 1u;  // tag 0 is what a cleared workspace holds
  const size_t sbase = (size_t)bh * D * a.s_pitch;
  const T* kmin_bh = static_cast<const T*>(a.kmin_t) + sbase;
  const T* kmax_bh = static_cast<const T*>(a.kmax_t) + sbase;
  float* pso = a.page_scores != nullptr ? a.page_scores + (size_t)bh * a.P : nullptr;
  uint64_t* xs = a.xscores + (size_t)bh * a.P;

  // Scores share j: published as tagged words, and kept in LDS (for a one-block head, its
  // selection's input; otherwise the touch ahead's, ahead of any other use of that LDS).
  const bool keep_share = multi && y >= a.na && y < a.ns && a.pf > 0 && a.ppb1 <= kPrefetchShare;
  auto score_share = [&](int j) {
    const int pb_lo = j * a.ppb1, pb_hi = min(a.P, pb_lo + a.ppb1);
    auto sink = [&](int p, float v) {
      if (multi) {
        st_exchange(xs + p, tagged(__float_as_uint(v), epoch), a.xcd_local != 0);
        u.scores[p - pb_lo] = v;  // read back only by a block that touches ahead
      } else {
        u.scores[p] = v;
      }
      if (pso != nullptr) pso[p] = v;
    };
    if (a.vec)
      score_page_range<T, true>(kmin_bh, kmax_bh, D, a.s_pitch, a.r, pb_lo, pb_hi, ch, sink);
    else
      score_page_range<T, false>(kmin_bh, kmax_bh, D, a.s_pitch, a.r, pb_lo, pb_hi, ch, sink);
  };

  // The block counts itself as started once it holds the epoch (the empty asm makes the loaded
  // value, hence the load's completion, a precondition of the count). The count is placed where
  // no later load of the block waits behind its round trip (a wave's memory operations complete
  // in order): a scorer counts at its end, an attender before its selection.
  unsigned started = 0u;
  auto count_started = [&]() {
    if (multi && tid == 0) {
      asm volatile("" ::"v"(epoch_prev));
      started = inc_coherent(hw + 1);
    }
  };

  // 1. the block's share of the head's approximate page scores
  if (y < a.ns) {
    if (a.chan_idx != nullptr && y == 0)
      for (int j = tid; j < a.r; j += kThreads) a.chan_idx[(size_t)bh * a.r + j] = ch.chan[j];
    score_share(y);
    if (keep_share) {
      // Touch ahead: the K/V rows of this share's pf best pages are loaded and dropped, so that
      // the attenders (on the same XCD) find them in its L2. The attention at small budgets waits
      // on its first loads; this block would otherwise idle until the step ends. A page's rank
      // counts the share's higher scores (and equal ones at lower index), so ranks are distinct.
      const int pb_lo = y * a.ppb1, nsh = min(a.P, pb_lo + a.ppb1) - pb_lo;
      const int m = min(nsh, a.pf);
      int* best = reinterpret_cast<int*>(mg.o);  // unused by a block that does not attend
      const int nsh4 = (nsh + 3) & ~3;  // read four at a time; the padding never outranks
      if (tid < nsh4 - nsh) u.scores[nsh + tid] = -INFINITY;
      lds_barrier();
      for (int t = tid; t < nsh; t += kThreads) {
        const float v = u.scores[t];
        int rank = 0;
#pragma unroll 2
        for (int i = 0; i < nsh4; i += 4) {
          const float4 w = *reinterpret_cast<const float4*>(&u.scores[i]);
          rank += (w.x > v || (w.x == v && i < t)) ? 1 : 0;
          rank += (w.y > v || (w.y == v && i + 1 < t)) ? 1 : 0;
          rank += (w.z > v || (w.z == v && i + 2 < t)) ? 1 : 0;
          rank += (w.w > v || (w.w == v && i + 3 < t)) ? 1 : 0;
        }
        if (rank < m) best[rank] = pb_lo + t;
      }
      lds_barrier();
      const T* kc_bh = static_cast<const T*>(a.k_c) + (size_t)bh * a.kv_pitch * D;
      const T* vc_bh = static_cast<const T*>(a.v_c) + (size_t)bh * a.kv_pitch * D;
      const int32_t* rows_bh = a.rows != nullptr ? a.rows + (size_t)bh * a.Lc : nullptr;
      constexpr int kChunks = (int)(D * sizeof(T) / 16);  // 16-byte pieces of a row
      const int wave = tid / kWave, lane = tid % kWave;
      uint32_t sink = 0u;
#pragma unroll 1
      for (int e = wave; e < m; e += kWaves) {
        const int p = best[e];
        if (p < pb_lo || p >= pb_lo + nsh) continue;  // a NaN score can leave a rank unfilled
#pragma unroll 1
        for (int i = lane; i < a.ps * kChunks; i += kWave) {
          const int t = p * a.ps + i / kChunks;
          if (t >= a.Lc) continue;
          const int row = rows_bh != nullptr ? min(max(rows_bh[t], 0), a.kv_pitch - 1) : t;
          const uint4 kx = load16(kc_bh + (size_t)row * D + (i % kChunks) * (16 / sizeof(T)));
          const uint4 vx = load16(vc_bh + (size_t)row * D + (i % kChunks) * (16 / sizeof(T)));
          sink ^= kx.x ^ kx.y ^ kx.z ^ kx.w ^ vx.x ^ vx.y ^ vx.z ^ vx.w;
        }
      }
      asm volatile("" ::"v"(sink));  // the loads stay: their values are consumed
    }
  }

  if (y < a.na) {
    // 2. the head's top pages (every attender finds them). Strided keys: thread t holds pages
    // j * kThreads + t, straight from coalesced loads.
    uint32_t key[E];
    const int nv = tid < a.P ? min(E, (a.P - 1 - tid) / kThreads + 1) : 0;
    if (multi) {
      // every score word, polled from the moment this block's own share is done; a word still
      // stale at the steal deadline marks its share as missing (scored here: the same bits its
      // owner would publish)
      uint64_t w[E];
      bool use[E];
#pragma unroll
      for (int j = 0; j < E; ++j) use[j] = j < nv;
      auto addr = [&](int j) { return xs + min(j * kThreads + tid, a.P - 1); };
      if (poll_tagged<E>(w, use, addr, epoch, a.steal_ticks)) {
#pragma unroll
        for (int j = 0; j < E; ++j)
          if (use[j] && !tag_is(w[j], epoch)) {
            const int share = (j * kThreads + tid) / a.ppb1;
            atomicOr(share < 32 ? &s_miss_lo : &s_miss_hi, 1u << (share & 31));
          }
      }
      lds_barrier();
      uint64_t missing = ((uint64_t)s_miss_hi << 32) | s_miss_lo;
      if (a.steal_ticks < 0) missing = a.ns >= 64 ? ~0ull : (1ull << a.ns) - 1ull;  // test mode
      if (missing != 0ull) {
        if (tid == 0) set_status(a.sync, kStatusStoleShare);
        while (missing != 0ull) {  // block-uniform
          const int j = __ffsll((long long)missing) - 1;
          missing &= missing - 1ull;
          score_share(j);
        }
        if (poll_tagged<E>(w, use, addr, epoch, a.wait_ticks, /*fresh=*/false))
          set_status(a.sync, kStatusScoreWait);
      }
#pragma unroll
      for (int j = 0; j < E; ++j)
        key[j] = use[j] ? order_key(__uint_as_float(tag_bits(w[j]))) : 0u;
    }
    count_started();
    const bool all_pages = a.n_pages >= a.P;
    uint32_t pos[E], take = 0u;
    if (!all_pages) {
      if (!multi) {
        lds_barrier();  // the block's own scores are in LDS
#pragma unroll
        for (int j = 0; j < E; ++j)
          key[j] = j < nv ? order_key(u.scores[min(j * kThreads + tid, a.P - 1)]) : 0u;
      }
      uint32_t thr, need_eq, eq_total;
      strided_threshold<kThreads, E>(key, nv, (uint32_t)a.n_pages, thr, need_eq, eq_total, ssel,
                                     sel);
      strided_positions<kThreads, E>(key, nv, thr, need_eq, eq_total == need_eq, ssel, pos, take);
    }
    const T* kc_bh = static_cast<const T*>(a.k_c) + (size_t)bh * a.kv_pitch * D;
    const T* vc_bh = static_cast<const T*>(a.v_c) + (size_t)bh * a.kv_pitch * D;
    const int32_t* rows_bh = a.rows != nullptr ? a.rows + (size_t)bh * a.Lc : nullptr;
    T* out = static_cast<T*>(a.out) + (size_t)bh * G * D;
    constexpr int kStride = G * D + 2 * G;
    uint64_t* hp = a.xpart + (size_t)bh * a.cap_a * kStride;

    // 3. attention over slice s of the page list, its partial published (or, with one
    // attender, the output written); pout: the full page list, written with the first window
    auto attend_slice = [&](int s, int32_t* pout) {
      st.init(a.scale2);
      const int p_lo = s * a.pps, p_hi = min(p_lo + a.pps, a.n_pages);
      if (all_pages) {
        for (int i = tid; pout != nullptr && i < a.n_pages; i += kThreads) pout[i] = i;
        for (int w0 = p_lo; w0 < p_hi; w0 += kMaxPagesPerSplit) {
          const int nw = min(kMaxPagesPerSplit, p_hi - w0);
          lds_barrier();
          for (int i = tid; i < nw; i += kThreads) sh.pages[i] = w0 + i;
          lds_barrier();
          st.run(kc_bh, vc_bh, sh.pages, nw * a.ps, a.ps, a.P, a.Lc, rows_bh, a.kv_pitch - 1, sh);
        }
      } else {
        int w0 = p_lo;
        do {
          const int nw = min(kMaxPagesPerSplit, max(p_hi - w0, 0));
          const bool write_out = pout != nullptr && w0 == p_lo;
          lds_barrier();  // the page slots are free (earlier window or earlier use of the LDS)
#pragma unroll
          for (int j = 0; j < E; ++j) {
            if ((take >> j) & 1u) {
              const int p = (int)pos[j], idx = j * kThreads + tid;
              if (p >= w0 && p < w0 + nw) sh.pages[p - w0] = idx;
              if (write_out && p < a.n_pages) pout[p] = idx;
            }
          }
          lds_barrier();
          st.run(kc_bh, vc_bh, sh.pages, nw * a.ps, a.ps, a.P, a.Lc, rows_bh, a.kv_pitch - 1, sh);
          w0 += kMaxPagesPerSplit;
        } while (w0 < p_hi);
      }
      st.publish(sh);
      lds_barrier();
      if (a.na == 1) {
        for (int idx = tid; idx < G * D; idx += kThreads) {
          float M, lsum, o;
          wave_merge<D, G, kWaves>(sh, idx / D, idx % D, M, lsum, o);
          out[idx] = from_f32<T>(lsum > 0.f ? o / lsum : 0.f);
        }
        return;
      }
      uint64_t* mine = hp + (size_t)s * kStride;
      for (int idx = tid; idx < G * D; idx += kThreads) {
        const int g = idx / D, c = idx % D;
        float M, lsum, o;
        wave_merge<D, G, kWaves>(sh, g, c, M, lsum, o);
        st_exchange(mine + idx, tagged(__float_as_uint(o), epoch), a.xcd_local != 0);
        if (c == 0) {
          st_exchange(mine + G * D + g, tagged(__float_as_uint(M), epoch), a.xcd_local != 0);
          st_exchange(mine + G * D + G + g, tagged(__float_as_uint(lsum), epoch), a.xcd_local != 0);
        }
      }
    };
    attend_slice(y, (a.page_idx != nullptr && y == 0) ? a.page_idx + (size_t)bh * a.n_pages
                                                      : nullptr);

    if (a.na > 1) {
      // 4. this attender merges output elements [e0, e0 + ne) over every slice's partial: the
      // words are all loaded together (o of (slice, element) at i < na * ne, three per thread;
      // (max, sum) of every (slice, head) at thread t < 2 * na * G), then combined from LDS.
      // Slices still missing at the steal deadline are attended here.
      const int cpb = (G * D + a.na - 1) / a.na;
      const int e0 = y * cpb, ne = min(cpb, G * D - e0);
      constexpr int NO = (G * D + kMaxAttending + kThreads - 1) / kThreads;  // o words per thread
      constexpr int NW = NO + 1;
      const int nml = 2 * a.na * G;
      const int no = ne > 0 ? a.na * ne : 0;
      uint64_t w[NW];
      bool use[NW];
      int slice_of[NW];
#pragma unroll
      for (int k = 0; k < NO; ++k) {
        const int i = tid + k * kThreads;
        use[k] = i < no;
        slice_of[k] = use[k] ? i / ne : 0;
      }
      use[NO] = tid < nml;
      slice_of[NO] = use[NO] ? (tid % (a.na * G)) / G : 0;
      auto addr = [&](int j) {
        if (j == NO) {
          const int t = min(tid, nml - 1), which = t / (a.na * G), rem = t % (a.na * G);
          return hp + (size_t)(rem / G) * kStride + G * D + which * G + rem % G;
        }
        const int i = min(tid + j * kThreads, max(no - 1, 0));
        const int sl = ne > 0 ? i / ne : 0, e = ne > 0 ? i - sl * ne : 0;
        return hp + (size_t)sl * kStride + min(e0 + e, G * D - 1);
      };
#pragma unroll
      for (int j = 0; j < NW; ++j) w[j] = 0ull;
      bool stale = poll_tagged<NW>(w, use, addr, epoch, a.steal_ticks);
      if (stale) {
#pragma unroll
        for (int j = 0; j < NW; ++j)
          if (use[j] && !tag_is(w[j], epoch)) atomicOr(&mg.missing, 1u << slice_of[j]);
      }
      lds_barrier();
      unsigned miss = mg.missing;
      if (a.steal_ticks < 0) miss = (1u << a.na) - 1u;  // test mode: every slice redone here
      if (miss != 0u) {
        if (tid == 0) set_status(a.sync, kStatusStoleSlice);
        while (miss != 0u) {  // block-uniform
          const int sl = __ffs((int)miss) - 1;
          miss &= miss - 1u;
          attend_slice(sl, nullptr);
        }
        if (poll_tagged<NW>(w, use, addr, epoch, a.wait_ticks, /*fresh=*/false))
          set_status(a.sync, kStatusPartialWait);
      }
#pragma unroll
      for (int k = 0; k < NO; ++k)
        if (use[k]) mg.o[tid + k * kThreads] = __uint_as_float(tag_bits(w[k]));
      if (use[NO]) {
        const int which = tid / (a.na * G), rem = tid % (a.na * G);
        (which == 0 ? mg.m : mg.l)[rem / G][rem % G] = __uint_as_float(tag_bits(w[NO]));
      }
      lds_barrier();
      for (int e = tid; e < ne; e += kThreads) {
        const int g = (e0 + e) / D;
        float M = -INFINITY;
        for (int sl = 0; sl < a.na; ++sl) M = fmaxf(M, mg.m[sl][g]);
        float lsum = 0.f, o = 0.f;
        for (int sl = 0; sl < a.na; ++sl) {
          const float ms = mg.m[sl][g];
          const float wt = ms == -INFINITY ? 0.f : exp2_hw(ms - M);
          lsum = fmaf(mg.l[sl][g], wt, lsum);
          o = fmaf(mg.o[sl * ne + e], wt, o);
        }
        out[e0 + e] = from_f32<T>(lsum > 0.f ? o / lsum : 0.f);
      }
    }
  } else {
    count_started();
  }

  // The last block of the head to start stores the next epoch and clears the count.
  if (multi && tid == 0 && started == (unsigned)(a.nb - 1)) {
    st_coherent(hw + 1, 0u);
    st_coherent(hw, epoch);
  }
}

// Blocks per head: as many as fit one block per CU (at most kMaxScorers), so that every block is
// resident from the start (the step is correct without that, through stealing; it only keeps the
// step from running in two rounds). Every block scores a share of the pages; the first na also
// attend: one for budgets of at most kSoloTokens tokens (no partials to merge), otherwise one per
// kTokensPerBlock tokens, at most kMaxAttending.
struct Plan {
  int ns, na, nb, ppb1, pps;
};

inline Plan plan(int BH, int P, int ps, int n_pages, int ncu, int vmax) {
  const int nb0 = std::max(std::min(ncu / BH, kMaxScorers), 1);
  const int ntok = n_pages * ps;
  int na = ntok <= kSoloTokens
               ? 1
               : std::max(std::min(std::min(kMaxAttending, nb0),
                                   (ntok + kTokensPerBlock - 1) / kTokensPerBlock),
                          1);
  const int pps = (n_pages + na - 1) / na;
  na = (n_pages + pps - 1) / pps;
  int ppb1 = std::max((P + nb0 - 1) / nb0, kMinScorePages);
  ppb1 = (ppb1 + vmax - 1) / vmax * vmax;
  const int ns = (P + ppb1 - 1) / ppb1;
  return {ns, na, std::max(ns, na), ppb1, pps};
}

// More heads than kTargetBlocks: one block per head would leave the grid in several rounds of
// long blocks, each running its phases one after another. Such a step runs as three launches
// instead (page scores, top-k, attention), each spread over many short blocks, with scores, pages
// and attention partials passing through the workspace.
inline bool pipelined(size_t BH) { return BH > (size_t)kTargetBlocks; }

// Exchange slots per head, sized for the largest plan any device can get (kTargetBlocks CUs), so
// the layout depends on the shape only. A shape whose heads cannot get two blocks exchanges nothing.
// A pipelined shape holds [BH, Pcap] scores, [BH, Pcap] pages and the attention partials of the
// largest split the attention plans for n_pages <= Pcap: at most max(ceil(2*kTargetBlocks/BH),
// ceil(Pcap/kMaxPagesPerSplit)) splits of G*(D+2) floats per head.
struct Layout {
  size_t off_sync, off_xscores, off_xpart, total;
  int cap_a;
  bool pipe;
  size_t off_pscores, off_ppages, off_ppart;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline Layout layout(int B, int Hq, int Hkv, int D, int Pcap) {
  const size_t BH = (size_t)B * Hkv;
  const int G = Hq / Hkv;
  Layout lo{};
  const int budget = BH >= (size_t)kTargetBlocks ? 0 : kTargetBlocks / (int)BH;
  lo.off_sync = 0;
  lo.off_xscores = align256((kSyncHeader + kHeadWords * BH) * sizeof(unsigned));
  if (pipelined(BH)) {
    const int splits = std::min(256, std::max((int)((2 * kTargetBlocks + BH - 1) / BH),
                                              (Pcap + kMaxPagesPerSplit - 1) / kMaxPagesPerSplit));
    lo.cap_a = 1;
    lo.pipe = true;
    lo.off_xpart = lo.off_xscores;
    lo.off_pscores = lo.off_xscores;
    lo.off_ppages = align256(lo.off_pscores + BH * (size_t)Pcap * sizeof(float));
    lo.off_ppart = align256(lo.off_ppages + BH * (size_t)Pcap * sizeof(int32_t));
    lo.total = align256(lo.off_ppart + BH * (size_t)splits * G * (D + 2) * sizeof(float));
    return lo;
  }
  if (budget < 2) {
    lo.cap_a = 1;
    lo.off_xpart = lo.total = lo.off_xscores;
    return lo;
  }
  lo.cap_a = std::min(budget, kMaxAttending);
  lo.off_xpart = align256(lo.off_xscores + BH * (size_t)Pcap * sizeof(uint64_t));
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
