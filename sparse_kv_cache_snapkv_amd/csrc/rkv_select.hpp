// Block-wide exact top-k over a row held in registers (RocketKV rebuttal, "Explanation of
// Calculating Approximate Attention Scores": select the pages with higher scores).
//
// Thread t holds elements [t*E, t*E+E) of the row as order-preserving 32-bit keys. The block
// first reduces the minimum and maximum key and counts the keys into kValueBins bins linear in
// value between them; a scan of the bins from the top finds the bin holding the k-th largest key
// T, and when that bin holds at most kSelectCandidates keys they are gathered and T is found by
// ranking them against each other directly. Crowded bins fall back to 8-bit radix passes that
// start below the bits common to the minimum and maximum, counting into per-wave histograms
// (double-buffered). An ordered compaction then gives every element above T, and the
// lowest-index elements equal to T, its position in the ascending list.
#pragma once

#include "rkv_common.hpp"

namespace rkv {

constexpr int kSelectCandidates = 256;  // a bin this small is finished by direct ranking
constexpr int kValueBins = 2048;       // bins of the first, value-linear counting pass

template <int THREADS>
struct SelectShared {
  static constexpr int NW = THREADS / kWave;
  union {
    uint32_t hist[2][NW][256 + kWave];  // bins 256.. take non-matching keys, one per lane (unread)
    uint32_t vbins[kValueBins];
  };
  __align__(16) uint32_t cand[kSelectCandidates + kWave];  // slots from 256: one spare per lane
  uint32_t wa[2][NW];  // per-wave partials, two slots so that consecutive scans need no barrier
  uint32_t wb[2][NW];
  uint32_t digit, above, binc, ncand, thr, need;
};

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return wave_reduce_u32(v, OpMinU{}); }
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) { return wave_reduce_u32(v, OpMaxU{}); }

// Exclusive scan of two counters over the block, plus the totals. One barrier; the same slot
// may be used again only after the block has passed another barrier.
template <int THREADS>
__device__ __forceinline__ void block_scan2(uint32_t a, uint32_t b, uint32_t& ea, uint32_t& eb,
                                            uint32_t& ta, uint32_t& tb, SelectShared<THREADS>& sh,
                                            int slot) {
  constexpr int NW = THREADS / kWave;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const uint32_t ia = wave_inclusive_scan(a), ib = wave_inclusive_scan(b);
  if (lane == kWave - 1) {
    sh.wa[slot][wave] = ia;
    sh.wb[slot][wave] = ib;
  }
  lds_barrier();
  uint32_t pa = 0, pb = 0, sa = 0, sb = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t va = sh.wa[slot][w], vb = sh.wb[slot][w];
    pa += w < wave ? va : 0u;
    pb += w < wave ? vb : 0u;
    sa += va;
    sb += vb;
  }
  ea = pa + ia - a;
  eb = pb + ib - b;
  ta = sa;
  tb = sb;
}

// The keys of one bin (match(e) true for element e of nbin <= kSelectCandidates keys over the
// whole block) are gathered into sh.cand, one wave-level slot reservation per wave, and ranked
// against each other: returns the krem-th largest of them (T) and how many keys equal to T are
// taken (need). Every thread must call it; two barriers.
template <int THREADS, int E, typename Match>
__device__ __forceinline__ void rank_bin(const uint32_t (&key)[E], int nvalid, uint32_t nbin,
                                         uint32_t krem, Match&& match, uint32_t& T,
                                         uint32_t& need, SelectShared<THREADS>& sh) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  bool m[E];
  uint32_t cnt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    m[e] = e < nvalid && match(e);
    cnt += m[e] ? 1u : 0u;
  }
  const uint32_t incl = wave_inclusive_scan(cnt);
  uint32_t base = 0;
  if (lane == kWave - 1 && incl != 0u) base = atomicAdd(&sh.ncand, incl);
  base = (uint32_t)__builtin_amdgcn_readlane((int)base, kWave - 1);
  uint32_t slot = base + incl - cnt;
#pragma unroll
  for (int e = 0; e < E; ++e) {  // branch-free: other keys go to the lane's spare slot
    sh.cand[m[e] ? slot : (uint32_t)(kSelectCandidates + lane)] = key[e];
    slot += m[e] ? 1u : 0u;
  }
  lds_barrier();
  for (uint32_t t = tid; t < nbin; t += THREADS) {
    const uint32_t kt = sh.cand[t];
    uint32_t gt = 0, ge = 0;
    for (uint32_t j = 0; j < nbin; j += 4) {
      const uint4 c = *reinterpret_cast<const uint4*>(&sh.cand[j]);
      gt += (c.x > kt) + (j + 1 < nbin && c.y > kt) + (j + 2 < nbin && c.z > kt) +
            (j + 3 < nbin && c.w > kt);
      ge += (c.x >= kt) + (j + 1 < nbin && c.y >= kt) + (j + 2 < nbin && c.z >= kt) +
            (j + 3 < nbin && c.w >= kt);
    }
    if (gt < krem && krem <= ge) {  // kt is the krem-th largest key of the bin
      sh.thr = kt;
      sh.need = krem - gt;
    }
  }
  lds_barrier();
  T = sh.thr;
  need = sh.need;
}

// Finds T (the k-th largest key) and need_eq (how many keys equal to T are taken), for
// 1 <= k < number of valid keys. Every thread of the block must call it. On return the block
// may run block_compact right away.
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
    sh.wa[0][wave] = lo;
    sh.wb[0][wave] = hi;
  }
  for (int i = tid; i < kValueBins; i += THREADS) sh.vbins[i] = 0u;
  if (tid == 0) sh.ncand = 0;
  lds_barrier();
  lo = sh.wa[0][0];
  hi = sh.wb[0][0];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    lo = min(lo, sh.wa[0][w]);
    hi = max(hi, sh.wb[0][w]);
  }
  if (lo == hi) {  // all keys equal
    T = lo;
    need_eq = k;
    return;
  }
  // Pass over value-linear bins between the block's minimum and maximum: the bin index is a
  // monotone function of the key, so the bin holding the k-th largest key is exact; its keys are
  // then ranked directly. Clustered values (a large bin) fall back to the radix passes below.
  const float flo = key_float(lo), fhi = key_float(hi);
  const float inv = (float)kValueBins / (fhi - flo);
  const bool value_pass = isfinite(flo) && isfinite(fhi) && isfinite(inv) && inv > 0.f;
  if (value_pass) {
    int bin[E];  // a monotone function of the key, computed once
#pragma unroll
    for (int e = 0; e < E; ++e) {
      bin[e] = min(max((int)((key_float(key[e]) - flo) * inv), 0), kValueBins - 1);
      if (e < nvalid) atomicAdd(&sh.vbins[bin[e]], 1u);
    }
    lds_barrier();
    // thread t owns the kValueBins/THREADS bins just below those of thread t-1 (descending)
    constexpr int BPT = kValueBins / THREADS;
    uint32_t c[BPT], local = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      c[j] = sh.vbins[kValueBins - 1 - (tid * BPT + j)];
      local += c[j];
    }
    uint32_t excl, unused, tot, unused2;
    block_scan2<THREADS>(local, 0u, excl, unused, tot, unused2, sh, 0);
    if (excl < k && k <= excl + local) {
      uint32_t run = excl;
#pragma unroll
      for (int j = 0; j < BPT; ++j) {
        if (run < k && k <= run + c[j]) {
          sh.digit = (uint32_t)(kValueBins - 1 - (tid * BPT + j));
          sh.above = run;
          sh.binc = c[j];
        }
        run += c[j];
      }
    }
    lds_barrier();
    const uint32_t nbin = sh.binc;
    if (nbin <= (uint32_t)kSelectCandidates) {
      const int bstar = (int)sh.digit;
      rank_bin<THREADS, E>(key, nvalid, nbin, k - sh.above,
                           [&](int e) { return bin[e] == bstar; }, T, need_eq, sh);
      return;
    }
  }
  // radix passes from clean histograms (they share LDS with the value bins)
  for (int i = tid; i < 2 * NW * (256 + kWave); i += THREADS) (&sh.hist[0][0][0])[i] = 0u;
  lds_barrier();
  int bits = 32 - __clz((int)(lo ^ hi));  // low bits that still vary
  uint32_t prefix = bits >= 32 ? 0u : (lo >> bits) << bits;
  uint32_t mask = bits >= 32 ? 0u : ~((1u << bits) - 1u);
  uint32_t krem = k;
  int buf = 0;
  while (bits > 0) {
    const int shift = bits > 8 ? bits - 8 : 0;
    uint32_t* hw = sh.hist[buf][wave];
#pragma unroll
    for (int e = 0; e < E; ++e) {  // branch-free: non-matching keys count into the lane's spare bin
      const bool m = e < nvalid && (key[e] & mask) == prefix;
      atomicAdd(&hw[m ? ((key[e] >> shift) & 255u) : 256u + lane], 1u);
    }
    // the other buffer (scanned in the previous pass) is cleared for the next one
    for (int i = tid; i < NW * (256 + kWave); i += THREADS) (&sh.hist[buf ^ 1][0][0])[i] = 0u;
    if (tid == 0) sh.ncand = 0;
    lds_barrier();
    if (tid < kWave) {
      // lane l owns digits 255-4l .. 252-4l (descending), summed over the waves' histograms
      uint32_t c[4], c4 = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t x = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) x += sh.hist[buf][w][255 - 4 * tid - j];
        c[j] = x;
        c4 += x;
      }
      const uint32_t incl = wave_inclusive_scan(c4);
      const uint32_t excl = incl - c4;
      if (excl < krem && krem <= incl) {
        uint32_t run = excl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (run < krem && krem <= run + c[j]) {
            sh.digit = 255 - 4 * tid - j;
            sh.above = run;
            sh.binc = c[j];
          }
          run += c[j];
        }
      }
    }
    lds_barrier();
    prefix |= sh.digit << shift;
    mask |= 255u << shift;
    krem -= sh.above;
    bits = shift;
    buf ^= 1;
    const uint32_t nbin = sh.binc;
    if (bits > 0 && nbin <= (uint32_t)kSelectCandidates) {
      const uint32_t pm = prefix, mk = mask;
      rank_bin<THREADS, E>(key, nvalid, nbin, krem, [&](int e) { return (key[e] & mk) == pm; },
                           prefix, krem, sh);
      break;
    }
  }
  T = prefix;
  need_eq = krem;
  lds_barrier();  // the last pass's reads of sh.digit / sh.above precede later writes
}

// Ascending positions of the selected elements. emit(pos, index, selected) is called for every
// element of a thread whose selected elements (which take consecutive positions) reach into
// [win_lo, win_hi), and for no element of the other threads; pos is meaningful only when
// `selected`. One barrier (scan slot 1, whose partials the threshold never touches); every
// thread of the block must call it, and a second call needs a barrier in between.
// gt_base / eq_base: elements above / equal to T that precede this block's elements in the row
// (when a row is spread over several blocks).
template <int THREADS, int E, typename Emit>
__device__ __forceinline__ void block_compact(const uint32_t (&key)[E], int nvalid, uint32_t T,
                                              uint32_t need_eq, int base_index, uint32_t win_lo,
                                              uint32_t win_hi, SelectShared<THREADS>& sh,
                                              Emit&& emit, uint32_t gt_base = 0,
                                              uint32_t eq_base = 0) {
  uint32_t ngt = 0, neq = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    ngt += (e < nvalid && key[e] > T);
    neq += (e < nvalid && key[e] == T);
  }
  uint32_t bg, be, tg, te;
  block_scan2<THREADS>(ngt, neq, bg, be, tg, te, sh, 1);
  bg += gt_base;
  be += eq_base;
  const uint32_t first = bg + min(be, need_eq);
  const uint32_t ntake = ngt + (be < need_eq ? min(neq, need_eq - be) : 0u);
  if (ntake == 0u || first >= win_hi || first + ntake <= win_lo) return;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool gt = e < nvalid && key[e] > T;
    const bool eq = e < nvalid && key[e] == T;
    const bool take = gt || (eq && be < need_eq);
    const uint32_t pos = bg + (gt ? min(be, need_eq) : be);
    emit(pos, base_index + e, take);
    bg += gt;
    be += eq;
  }
}

// Loads the E consecutive scores of a row starting at i0 (blocked layout) as keys; returns how
// many of them exist (0..E). Works for global and LDS rows.
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
  for (int e = 0; e < E; ++e) {
    const float x = row[min(i0 + e, n - 1)];  // every address inside the row
    key[e] = i0 + e < n ? order_key(x) : 0u;
  }
  return n - i0 < 0 ? 0 : (n - i0 > E ? E : n - i0);
}

// ------------------------------------------------------------------------- strided layout
// Thread t of a block of THREADS threads holds elements j*THREADS + t (j < E) of a row as keys;
// the valid ones are j < nvalid (a prefix, since the row end cuts every thread's j range). The
// keys come straight from coalesced loads, and the per-element work uses wave ballots where the
// blocked layout above needs block scans: the bin holding the k-th largest key is found by every
// wave from the per-wave totals, its keys are ranked by every wave, and positions come from a
// table of per-(j, wave) counts, so a selection passes four barriers and the positions one.

constexpr int kStridedCandidates = 256;  // bin size up to which the bin's keys are ranked directly

template <int THREADS, int E>
struct StridedShared {
  static constexpr int NW = THREADS / kWave;
  static constexpr int NTAB = E * NW;  // (j, wave) groups in index order
  uint32_t vbins[kValueBins];
  __align__(16) uint32_t cand[kStridedCandidates + 4];
  uint32_t wmin[NW], wmax[NW], wtot[NW];
  uint32_t ncand;
  uint32_t gtc[NTAB], eqc[NTAB];
};

// Lanes below this one whose bit is set in m.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
}

// Zeroes what strided_threshold expects to be zero; the block must pass a barrier afterwards.
template <int THREADS, int E>
__device__ __forceinline__ void strided_clear(StridedShared<THREADS, E>& sh) {
  for (int i = threadIdx.x; i < kValueBins; i += THREADS) sh.vbins[i] = 0u;
  if (threadIdx.x == 0) sh.ncand = 0u;
}

// T (the k-th largest key), need_eq (how many keys equal to T are taken) and eq_total (how many
// keys equal T, or 0xffffffff where the radix passes leave it uncounted), for 1 <= k < number of
// valid keys, with sh cleared by strided_clear (and a barrier passed) since its last use.
// Value-linear bins between the block's minimum and maximum locate the bin of the k-th largest
// key; a bin of at most kStridedCandidates keys is gathered and ranked, larger ones (clustered
// values) go to block_threshold's radix passes in fb. Every thread must call it.
template <int THREADS, int E>
__device__ __forceinline__ void strided_threshold(const uint32_t (&key)[E], int nvalid, uint32_t k,
                                                  uint32_t& T, uint32_t& need_eq,
                                                  uint32_t& eq_total,
                                                  StridedShared<THREADS, E>& sh,
                                                  SelectShared<THREADS>& fb) {
  constexpr int NW = THREADS / kWave;
  constexpr int BPT = kValueBins / THREADS;
  static_assert(BPT % 4 == 0, "bins per thread");
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = wave_id();
  uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    lo = e < nvalid ? min(lo, key[e]) : lo;
    hi = e < nvalid ? max(hi, key[e]) : hi;
  }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (lane == 0) {
    sh.wmin[wave] = lo;
    sh.wmax[wave] = hi;
  }
  lds_barrier();
  lo = sh.wmin[0];
  hi = sh.wmax[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    lo = min(lo, sh.wmin[w]);
    hi = max(hi, sh.wmax[w]);
  }
  if (lo == hi) {  // all keys equal
    T = lo;
    need_eq = k;
    eq_total = 0xffffffffu;
    return;
  }
  const float flo = key_float(lo), fhi = key_float(hi);
  const float inv = (float)kValueBins / (fhi - flo);
  if (isfinite(flo) && isfinite(fhi) && isfinite(inv) && inv > 0.f) {
    int bin[E];  // a monotone function of the key
#pragma unroll
    for (int e = 0; e < E; ++e) {
      bin[e] = min(max((int)((key_float(key[e]) - flo) * inv), 0), kValueBins - 1);
      if (e < nvalid) atomicAdd(&sh.vbins[bin[e]], 1u);
    }
    lds_barrier();
    // thread t owns bins kValueBins-1-(t*BPT+i), i < BPT (descending from the top)
    auto read_bins = [&](int t, uint32_t (&c)[BPT]) {
#pragma unroll
      for (int i = 0; i < BPT; i += 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(&sh.vbins[kValueBins - (t * BPT + i) - 4]);
        c[i] = v.w;
        c[i + 1] = v.z;
        c[i + 2] = v.y;
        c[i + 3] = v.x;
      }
    };
    uint32_t c[BPT], local = 0;
    read_bins(tid, c);
#pragma unroll
    for (int i = 0; i < BPT; ++i) local += c[i];
    const uint32_t incl = wave_inclusive_scan(local);
    if (lane == kWave - 1) sh.wtot[wave] = incl;
    lds_barrier();
    // the wave whose bins reach the k-th key, then (in every wave) the bin within it
    uint32_t before = 0, wabove = 0;
    int wstar = 0;
    bool found = false;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t t = sh.wtot[w];
      const bool here = !found && k <= before + t;
      wstar = here ? w : wstar;
      wabove = here ? before : wabove;
      found = found || here;
      before += t;
    }
    uint32_t cw[BPT], lw = 0;
    read_bins(wstar * kWave + lane, cw);
#pragma unroll
    for (int i = 0; i < BPT; ++i) lw += cw[i];
    uint32_t run = wabove + wave_inclusive_scan(lw) - lw;
    int bsel = 0;
    uint32_t asel = 0, csel = 0;
    bool has = false;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      const bool here = !has && run < k && k <= run + cw[i];
      bsel = here ? kValueBins - 1 - ((wstar * kWave + lane) * BPT + i) : bsel;
      asel = here ? run : asel;
      csel = here ? cw[i] : csel;
      has = has || here;
      run += cw[i];
    }
    const int src = __ffsll((long long)__ballot(has)) - 1;
    const int bstar = __builtin_amdgcn_readlane(bsel, src);
    const uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)asel, src);
    const uint32_t nbin = (uint32_t)__builtin_amdgcn_readlane((int)csel, src);
    if (nbin <= (uint32_t)kStridedCandidates) {
      bool m[E];
      uint32_t cnt = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        m[e] = e < nvalid && bin[e] == bstar;
        cnt += m[e] ? 1u : 0u;
      }
      const uint32_t wincl = wave_inclusive_scan(cnt);
      uint32_t base = 0;
      if (lane == kWave - 1 && wincl != 0u) base = atomicAdd(&sh.ncand, wincl);
      base = (uint32_t)__builtin_amdgcn_readlane((int)base, kWave - 1);
      uint32_t slot = base + wincl - cnt;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (m[e]) sh.cand[slot] = key[e];
        slot += m[e] ? 1u : 0u;
      }
      lds_barrier();
      // every wave ranks the bin's keys (lane l: keys l, l+64, ...) against each other
      const uint32_t krem = k - above;
      uint32_t tsel = 0, nsel = 0, esel = 0;
      bool ok = false;
      for (uint32_t i0 = 0; i0 < nbin; i0 += kWave) {
        const uint32_t ci = i0 + lane;
        const uint32_t kt = sh.cand[min(ci, nbin - 1)];
        uint32_t gt = 0, ge = 0;
        for (uint32_t j = 0; j < nbin; j += 4) {
          const uint4 c4 = *reinterpret_cast<const uint4*>(&sh.cand[j]);
          gt += (c4.x > kt) + (j + 1 < nbin && c4.y > kt) + (j + 2 < nbin && c4.z > kt) +
                (j + 3 < nbin && c4.w > kt);
          ge += (c4.x >= kt) + (j + 1 < nbin && c4.y >= kt) + (j + 2 < nbin && c4.z >= kt) +
                (j + 3 < nbin && c4.w >= kt);
        }
        const bool here = ci < nbin && gt < krem && krem <= ge;  // kt is the krem-th largest
        tsel = here ? kt : tsel;
        nsel = here ? krem - gt : nsel;
        esel = here ? ge - gt : esel;  // every key equal to T is in this bin
        ok = ok || here;
      }
      const int s2 = __ffsll((long long)__ballot(ok)) - 1;
      T = (uint32_t)__builtin_amdgcn_readlane((int)tsel, s2);
      need_eq = (uint32_t)__builtin_amdgcn_readlane((int)nsel, s2);
      eq_total = (uint32_t)__builtin_amdgcn_readlane((int)esel, s2);
      return;
    }
  }
  block_threshold<THREADS, E>(key, nvalid, k, T, need_eq, fb);
  eq_total = 0xffffffffu;
}

// Ascending positions of the selected elements: the elements above T and the need_eq
// lowest-index elements equal to T. pos[e] is meaningful where bit e of take is set. all_eq
// (block-uniform): every key equal to T is taken (need_eq equals their count), so no element's
// rank among the equal keys is needed. One barrier; every thread must call it.
template <int THREADS, int E>
__device__ __forceinline__ void strided_positions(const uint32_t (&key)[E], int nvalid, uint32_t T,
                                                  uint32_t need_eq, bool all_eq,
                                                  StridedShared<THREADS, E>& sh,
                                                  uint32_t (&pos)[E], uint32_t& take) {
  constexpr int NW = THREADS / kWave;
  constexpr int NTAB = E * NW;
  constexpr int R = (NTAB + kWave - 1) / kWave;  // table entries per lane
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  // base[e]: selected elements of the table entries (j, w) before entry (e, wave), in index order
  auto bases = [&](const uint32_t (&tk)[R], uint32_t (&b)[E]) {
    uint32_t lt = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) lt += tk[r];
    uint32_t bs[R], run = wave_inclusive_scan(lt) - lt;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      bs[r] = run;
      run += tk[r];
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int en = e * NW + wave;
      uint32_t v = 0;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t x = (uint32_t)__builtin_amdgcn_readlane((int)bs[r], en / R);
        v = r == en % R ? x : v;
      }
      b[e] = v;
    }
  };
  uint32_t b[E];
  take = 0u;
  if (all_eq) {
    uint64_t bt[E];
#pragma unroll
    for (int e = 0; e < E; ++e) bt[e] = __ballot(e < nvalid && key[e] >= T);
    if (lane == 0) {
#pragma unroll
      for (int e = 0; e < E; ++e) sh.gtc[e * NW + wave] = (uint32_t)__popcll(bt[e]);
    }
    lds_barrier();
    uint32_t tk[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int en = lane * R + r;
      tk[r] = en < NTAB ? sh.gtc[en] : 0u;
    }
    bases(tk, b);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      pos[e] = b[e] + lanes_below(bt[e]);
      take |= (e < nvalid && key[e] >= T) ? (1u << e) : 0u;
    }
    return;
  }
  uint64_t bg[E], be[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    bg[e] = __ballot(e < nvalid && key[e] > T);
    be[e] = __ballot(e < nvalid && key[e] == T);
  }
  if (lane == 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      sh.gtc[e * NW + wave] = (uint32_t)__popcll(bg[e]);
      sh.eqc[e * NW + wave] = (uint32_t)__popcll(be[e]);
    }
  }
  lds_barrier();
  // every wave scans the table: lane l holds entries l*R .. l*R+R-1
  uint32_t tg[R], te[R], le = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int en = lane * R + r;
    tg[r] = en < NTAB ? sh.gtc[en] : 0u;
    te[r] = en < NTAB ? sh.eqc[en] : 0u;
    le += te[r];
  }
  uint32_t run = wave_inclusive_scan(le) - le;  // keys equal to T in earlier entries
  uint32_t eqx[R], tk[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    eqx[r] = run;
    tk[r] = tg[r] + min(te[r], need_eq > run ? need_eq - run : 0u);
    run += te[r];
  }
  bases(tk, b);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int en = e * NW + wave;
    uint32_t x0 = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t vx = (uint32_t)__builtin_amdgcn_readlane((int)eqx[r], en / R);
      x0 = r == en % R ? vx : x0;
    }
    const bool gt = e < nvalid && key[e] > T;
    const bool eq = e < nvalid && key[e] == T;
    const bool tk_e = gt || (eq && x0 + lanes_below(be[e]) < need_eq);
    pos[e] = b[e] + lanes_below(__ballot(tk_e));
    take |= tk_e ? (1u << e) : 0u;
  }
}

}  // namespace rkv
