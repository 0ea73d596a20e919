// Exact softmax attention over the tokens of selected pages, shared by the G query heads of a GQA
// group (RocketKV rebuttal, "Lack of Direct Latency Comparison": Step 3 sparse attention;
// "Explanation of Calculating Approximate Attention Scores": one selection per group). The
// per-wave state below is used by the standalone attention call and by the fused decode step.
//
// A token row of D elements is spread over LPT lanes, 16 bytes each, so one load instruction
// fetches TPL = 64/LPT whole rows; per chunk a wave issues all its K and V loads (SLOTS of each)
// before reducing in registers (DPP inside a row of 16 lanes), with an online softmax across
// chunks. The waves of a block merge (max, sum, P.V) through LDS.
#pragma once

#include <math.h>

#include "rkv_common.hpp"

namespace rkv {

constexpr int kAttThreads = 256;
constexpr int kAttWaves = kAttThreads / kWave;
constexpr int kAttSlots = 4;            // row loads per wave per chunk (standalone attention)
constexpr int kMaxPagesPerSplit = 1024;

template <typename T, int D, int SLOTS = kAttSlots>
struct Geo {
  static constexpr int V = vec16<T>::n;
  static constexpr int LPT = D / V;
  static constexpr int TPL = kWave / LPT;
  static constexpr int WTOK = SLOTS * TPL;  // tokens per wave per chunk
};

template <int D, int G, int NW = kAttWaves>
struct AttendShared {
  int pages[kMaxPagesPerSplit + kWave];  // slots from kMaxPagesPerSplit: discarded writes, per lane
  float m[NW][G], l[NW][G];
  float o[NW][G][D];
  __align__(16) float px[NW][4][32];  // per wave and row of 16 lanes: a chunk's weights (RS path)
  __align__(16) float fx[NW][4][8];   // and its per-head rescaling factors
  __align__(16) int rowbuf[NW][32];   // MFMA path: cache rows of a wave's chunk (-1: no token)
};

// Reduce-scatter step inside a row of 16 lanes: lanes paired by the DPP pattern CTRL (an
// involution), the lane with `upper` set keeps the upper half of the N values, its partner the
// lower half, each adding the partner's copy of the half it keeps.
// Applies to the first NA values of v.
template <int CTRL, int NA, int N>
__device__ __forceinline__ void rs_step(float (&v)[N], bool upper) {
  static_assert(NA <= N && NA % 2 == 0, "values in the step");
#pragma unroll
  for (int i = 0; i < NA / 2; ++i) {
    const float send = upper ? v[i] : v[i + NA / 2];
    const float keep = upper ? v[i + NA / 2] : v[i];
    v[i] = keep + dpp<CTRL>(send);
  }
}

// Lanes i <- i + R (mod 16) inside each row.
template <int R>
__device__ __forceinline__ float dpp_ror(float v) {
  return dpp<0x120 + R>(v);
}

// Per-wave online-softmax state of the G heads of a group; NW waves share a block's page list and
// each issues SLOTS K and V row loads per chunk. bf16 scores are packed bf16 dot products of the
// raw query and key bits, scaled after the lane reduction; fp32 scores use the pre-scaled query.
template <typename T, int D, int G, int NW = kAttWaves, int SLOTS = kAttSlots>
struct WaveState {
  static constexpr bool kBf16 = elem<T>::bytes == 2;
  float qf[G][Geo<T, D, SLOTS>::V];  // fp32 only: the query times scale * log2(e)
  float m[G], l[G], acc[G][Geo<T, D, SLOTS>::V];
  uint4 qraw[G];
  float sc2;     // scale * log2(e)
  bool started;  // a chunk has been accumulated (before it, rescaling zeros is skipped)

  // Reduce-scatter path (bf16 rows of 16 lanes, SLOTS*G a multiple of 16): the SLOTS*G partial
  // dot products of a row are summed by a reduce-scatter, so that lane li finishes NH of them
  // (slot li / PG, heads (li % PG) * NH + t) and takes one exponential each instead of every
  // lane taking all of them; the weights reach the row through LDS. m and l below then hold the
  // running max and sum of the lane's NH heads.
  static constexpr bool kRS = kBf16 && Geo<T, D, SLOTS>::LPT == 16 && (SLOTS * G) % 16 == 0 &&
                              16 % SLOTS == 0 && G <= 8;
  static constexpr int NV = SLOTS * G;      // partial dot products per lane and chunk
  static constexpr int NH = NV / 16;        // of them finished by each lane
  static constexpr int PG = 16 / SLOTS;     // lanes of a row between two with the same heads

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
                                      const int32_t* __restrict__ rows, int row_hi,
                                      AttendShared<D, G, NW>& shared) {
    run(kc_bh, vc_bh, pages, ntok, ps, P, Lc, rows, row_hi, shared.px, shared.fx);
  }
  __device__ __forceinline__ void run(const T* __restrict__ kc_bh, const T* __restrict__ vc_bh,
                                      const int* pages, int ntok, int ps, int P, int Lc,
                                      const int32_t* __restrict__ rows, int row_hi,
                                      float (&px)[NW][4][32], float (&fx)[NW][4][8]) {
    constexpr int V = Geo<T, D, SLOTS>::V, LPT = Geo<T, D, SLOTS>::LPT, TPL = Geo<T, D, SLOTS>::TPL;
    constexpr int WTOK = Geo<T, D, SLOTS>::WTOK;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int lg = lane / LPT, li = lane % LPT;
    const T* kb = kc_bh + li * V;
    const T* vb = vc_bh + li * V;
    if constexpr (kRS) {
      run_rs(kb, vb, pages, ntok, ps, P, Lc, rows, row_hi, px, fx);
      return;
    }
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

  __device__ __forceinline__ void run_rs(const T* __restrict__ kb, const T* __restrict__ vb,
                                         const int* pages, int ntok, int ps, int P, int Lc,
                                         const int32_t* __restrict__ rows, int row_hi,
                                         float (&px)[NW][4][32], float (&fx)[NW][4][8]) {
    constexpr int V = Geo<T, D, SLOTS>::V, TPL = Geo<T, D, SLOTS>::TPL;
    constexpr int WTOK = Geo<T, D, SLOTS>::WTOK;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int lg = lane / 16, li = lane % 16;
    const int slot_l = li / PG;  // the slot whose scores this lane finishes
    float* prow = px[wave][lg];
    float* frow = fx[wave][lg];
    for (int c0 = wave * WTOK; c0 < ntok; c0 += NW * WTOK) {
      int tok[SLOTS];
      unsigned okmask = 0u;
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        const int ti = c0 + s * TPL + lg;
        bool valid = ti < ntok;
        const int page = valid ? pages[ti / ps] : 0;
        const int t = page * ps + ti % ps;
        valid = valid && page >= 0 && page < P && t < Lc;
        okmask |= valid ? (1u << s) : 0u;
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
      float d[NV];
#pragma unroll
      for (int s = 0; s < SLOTS; ++s)
#pragma unroll
        for (int g = 0; g < G; ++g) d[s * G + g] = dot8_bf16(qraw[g], kr[s]);
      // reduce-scatter over the row: lane li ends with the sums of d[li*NH .. li*NH + NH)
      rs_step<kDppRor8, NV>(d, (li & 8) != 0);
      rs_step<kDppHalfMirror, NV / 2>(d, (li & 4) != 0);
      rs_step<kDppXor2, NV / 4>(d, (li & 2) != 0);
      rs_step<kDppXor1, NV / 8>(d, (li & 1) != 0);
      const bool ok = (okmask >> slot_l) & 1u;
      float sc[NH], mx[NH];
#pragma unroll
      for (int t = 0; t < NH; ++t) {
        sc[t] = ok ? d[t] * sc2 : -INFINITY;
        mx[t] = sc[t];
      }
      // the chunk's max of each head: over the lanes of the row with the same heads (li mod PG),
      // then over the wave's four rows
#pragma unroll
      for (int t = 0; t < NH; ++t) {
        if constexpr (PG <= 4) mx[t] = fmaxf(mx[t], dpp_ror<(PG <= 4 ? 4 : 1)>(mx[t]));
        if constexpr (PG <= 2) mx[t] = fmaxf(mx[t], dpp_ror<(PG <= 2 ? 2 : 1)>(mx[t]));
        if constexpr (PG <= 1) mx[t] = fmaxf(mx[t], dpp_ror<1>(mx[t]));
        mx[t] = fmaxf(mx[t], dpp_ror<8>(mx[t]));
        mx[t] = xor16_step(mx[t], OpMax{});
        mx[t] = xor32_step(mx[t], OpMax{});
      }
      float p[NH], f[NH];
#pragma unroll
      for (int t = 0; t < NH; ++t) {
        const float mn = fmaxf(m[t], mx[t]);
        f[t] = mn == -INFINITY ? 1.f : exp2_hw(m[t] - mn);
        const float mu = mn == -INFINITY ? 0.f : mn;
        p[t] = exp2_hw(sc[t] - mu);
        l[t] = l[t] * f[t] + p[t];
        m[t] = mn;
      }
      // weights (slot, head) and the heads' rescaling factors to every lane of the row (a wave's
      // LDS accesses complete in order, so no barrier)
#pragma unroll
      for (int t = 0; t < NH; ++t) prow[li * NH + t] = p[t];
      if (li < PG) {
#pragma unroll
        for (int t = 0; t < NH; ++t) frow[li * NH + t] = f[t];
      }
      float pw[NV], fg[G];
#pragma unroll
      for (int v = 0; v < NV; v += 4) {
        const float4 x = *reinterpret_cast<const float4*>(prow + v);
        pw[v] = x.x;
        pw[v + 1] = x.y;
        pw[v + 2] = x.z;
        pw[v + 3] = x.w;
      }
      // `started` is the same in every lane; until the first chunk, acc is zero
      if (__builtin_amdgcn_readfirstlane((int)started)) {
#pragma unroll
        for (int g = 0; g < G; ++g) fg[g] = frow[g];
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int e = 0; e < V; ++e) acc[g][e] *= fg[g];
      }
      started = true;
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        float vf[V];
        unpack16<T>(vr[s], vf);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float w = pw[s * G + g];
#pragma unroll
          for (int e = 0; e < V; ++e) acc[g][e] = fmaf(w, vf[e], acc[g][e]);
        }
      }
    }
  }

  // Reduces over the wave's lane groups and stores (m, l, o) of this wave in sh.
  __device__ __forceinline__ void publish(AttendShared<D, G, NW>& sh) {
    if constexpr (kRS) {
      publish_rs(sh);
      return;
    }
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

  // Reduce-scatter publish: l summed over the lanes holding the same heads and over the rows;
  // acc summed over the four rows by permlane swaps that leave each lane a quarter of the sums.
  __device__ __forceinline__ void publish_rs(AttendShared<D, G, NW>& sh) {
    constexpr int V = Geo<T, D, SLOTS>::V;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int li = lane % 16;
#pragma unroll
    for (int t = 0; t < NH; ++t) {
      float x = l[t];
      if constexpr (PG <= 4) x += dpp_ror<(PG <= 4 ? 4 : 1)>(x);
      if constexpr (PG <= 2) x += dpp_ror<(PG <= 2 ? 2 : 1)>(x);
      if constexpr (PG <= 1) x += dpp_ror<1>(x);
      x += dpp_ror<8>(x);
      x = xor16_step(x, OpSum{});
      x = xor32_step(x, OpSum{});
      l[t] = x;
    }
    if (lane < PG) {  // row 0, lanes holding every head once
#pragma unroll
      for (int t = 0; t < NH; ++t) {
        sh.m[wave][lane * NH + t] = m[t];
        sh.l[wave][lane * NH + t] = l[t];
      }
    }
    constexpr int NA = G * V;  // accumulators per lane: (head, element) at g*V + e
    float a[NA];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < V; ++e) a[g * V + e] = acc[g][e];
    // rows {0,1} against {2,3}: lanes below 32 keep the first half of the values
#pragma unroll
    for (int i = 0; i < NA / 2; ++i) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a[i]),
                                                      __float_as_uint(a[i + NA / 2]), false, false);
      a[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    // rows 0 against 1 and 2 against 3: lanes with bit 4 clear keep the first half
#pragma unroll
    for (int i = 0; i < NA / 4; ++i) {
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a[i]),
                                                      __float_as_uint(a[i + NA / 4]), false, false);
      a[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    const int base = ((lane & 32) ? NA / 2 : 0) + ((lane & 16) ? NA / 4 : 0);
#pragma unroll
    for (int i = 0; i < NA / 4; ++i) {
      const int f = base + i, g = f / V, e = f % V;
      sh.o[wave][g][li * V + e] = a[i];
    }
  }
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));

// Per-wave online-softmax attention of the G <= 16 heads of a group with matrix cores (bf16,
// D = 128), chunks of 32 tokens. v_mfma_f32_16x16x32_bf16 takes, in lane l = 16j + c (j = l/16),
// row c of A and column c of B with the k-run of lane group j, and leaves D rows 4j..4j+3 of
// column c. Scores: A = 16 tokens of K (row c = token, dims 32s + 8j .. +8 at k-step s), B = Q^T
// (column c = head, the same dims; zero for heads >= G), so lane (j, c) gets tokens 4j+i of the
// tile for head c. Over the chunk's two tiles a lane thus holds head c's scores of the 8 tokens
// tok(j, e) = 16*(e/4) + 4j + e%4, and the weights P of those tokens are already the A operand of
// P V (row = head c, k-run = its 8 tokens). The B operand of P V needs V[tok(j, e)][d] for one
// column d: lane (j, c) loads the 16-byte rows V[tok(j, e)][8c .. 8c+8) and transposes them in
// registers, so column c of output tile t is dim 8c + t and lane (j, c) ends with heads 4j..4j+3
// of dims 8c .. 8c+8. P enters the product rounded to bf16; scores, weights and sums stay fp32.
template <int G, int NW = kAttWaves>
struct MfmaWave {
  static constexpr int D = 128;
  static_assert(G >= 1 && G <= 16, "heads of a group");
  bf16x8_t qb[4];  // B operand of the scores, k-steps s = 0..3
  f32x4_t o[8];    // o[t][i]: head 4j+i, dim 8c+t (unnormalised)
  float m, l;      // head c: running max (log2 units) and this lane's part of the sum
  float sc2;

  // The B operand of the scores, as loaded (init(scale2) then starts a slice).
  __device__ __forceinline__ void load_q(const bf16_t* __restrict__ q_bh) {
    const int lane = threadIdx.x & (kWave - 1), j = lane >> 4, c = lane & 15;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 raw = c < G ? load16(q_bh + (size_t)c * D + 32 * s + 8 * j) : make_uint4(0, 0, 0, 0);
      qb[s] = __builtin_bit_cast(bf16x8_t, raw);
    }
  }

  __device__ __forceinline__ void init(const bf16_t* __restrict__ q_bh, float scale2) {
    load_q(q_bh);
    init(scale2);
  }

  __device__ __forceinline__ void init(float scale2) {
    sc2 = scale2;
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  template <int DD>
  __device__ __forceinline__ void run(const bf16_t* __restrict__ kc_bh,
                                      const bf16_t* __restrict__ vc_bh, const int* pages,
                                      int ntok, int ps, int P, int Lc,
                                      const int32_t* __restrict__ rows, int row_hi,
                                      AttendShared<DD, G, NW>& sh) {
    run(kc_bh, vc_bh, pages, ntok, ps, P, Lc, rows, row_hi, sh.rowbuf[threadIdx.x / kWave]);
  }

  // Tokens [0, ntok) of the page list `pages` (LDS); this wave takes chunks wave, wave + NW, ...
  // rows (may be null): slot t of the view is row rows[t] of kc_bh / vc_bh, clamped into
  // [0, row_hi]. rowbuf: this wave's 32 LDS words.
  __device__ __forceinline__ void run(const bf16_t* __restrict__ kc_bh,
                                      const bf16_t* __restrict__ vc_bh, const int* pages,
                                      int ntok, int ps, int P, int Lc,
                                      const int32_t* __restrict__ rows, int row_hi,
                                      int (&rowbuf)[32]) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int j = lane >> 4, c = lane & 15;
    for (int c0 = wave * 32; c0 < ntok; c0 += NW * 32) {
      if (lane < 32) {
        const int ti = c0 + lane;
        int row = -1;
        if (ti < ntok) {
          const int page = pages[ti / ps];
          const int t = page * ps + ti % ps;
          if (page >= 0 && page < P && t < Lc) row = rows != nullptr ? min(max(rows[t], 0), row_hi) : t;
        }
        rowbuf[lane] = row;
      }
      __builtin_amdgcn_wave_barrier();
      // K rows of tokens c and 16 + c; V rows of tokens tok(j, e)
      const int rk0 = rowbuf[c], rk1 = rowbuf[16 + c];
      const int4 rv0 = *reinterpret_cast<const int4*>(&rowbuf[4 * j]);
      const int4 rv1 = *reinterpret_cast<const int4*>(&rowbuf[16 + 4 * j]);
      const int rv[8] = {rv0.x, rv0.y, rv0.z, rv0.w, rv1.x, rv1.y, rv1.z, rv1.w};
      uint4 kq[2][4], vv[8];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        kq[0][s] = load16_stream(kc_bh + (size_t)max(rk0, 0) * D + 32 * s + 8 * j);
        kq[1][s] = load16_stream(kc_bh + (size_t)max(rk1, 0) * D + 32 * s + 8 * j);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) vv[e] = load16_stream(vc_bh + (size_t)max(rv[e], 0) * D + 8 * c);
      __builtin_amdgcn_wave_barrier();
      // scores of head c for tokens tok(j, e), e = 4*tile + i
      f32x4_t st[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        st[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
          st[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kq[t][s]),
                                                          qb[s], st[t], 0, 0, 0);
      }
      float sv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) sv[e] = rv[e] >= 0 ? st[e >> 2][e & 3] * sc2 : -INFINITY;
      float mx = sv[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
      mx = xor16_step(mx, OpMax{});
      mx = xor32_step(mx, OpMax{});
      const float mn = fmaxf(m, mx);
      const float f = mn == -INFINITY ? 1.f : exp2_hw(m - mn);
      const float mu = mn == -INFINITY ? 0.f : mn;
      f32x8_t pv;
      float ps_sum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = exp2_hw(sv[e] - mu);
        pv[e] = pe;
        ps_sum += pe;
      }
      l = l * f + ps_sum;
      m = mn;
      // rescale the outputs of heads 4j+i by their factors (held by lanes 4j+i); skipped when no
      // head's max moved
      if (__builtin_amdgcn_ballot_w64(f != 1.f) != 0ull) {
        float fo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          fo[i] = __int_as_float(__builtin_amdgcn_ds_bpermute((4 * j + i) * 4, __float_as_int(f)));
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[t][i] *= fo[i];
      }
      const bf16x8_t pa = __builtin_convertvector(pv, bf16x8_t);
      // B operand of tile t: element t of each of the 8 V rows (dims 8c + t)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
        uint32_t w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t* a = reinterpret_cast<const uint32_t*>(&vv[2 * u]);
          const uint32_t* b = reinterpret_cast<const uint32_t*>(&vv[2 * u + 1]);
          w[u] = __builtin_amdgcn_perm(b[t >> 1], a[t >> 1], sel);
        }
        const uint4 vb = make_uint4(w[0], w[1], w[2], w[3]);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, __builtin_bit_cast(bf16x8_t, vb), o[t],
                                                       0, 0, 0);
      }
    }
  }

  // (m, l, o) of this wave into sh, in the layout of WaveState::publish.
  template <int DD>
  __device__ __forceinline__ void publish(AttendShared<DD, G, NW>& sh) {
    static_assert(DD == D, "head dim");
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int j = lane >> 4, c = lane & 15;
    float x = l;
    x = xor16_step(x, OpSum{});
    x = xor32_step(x, OpSum{});
    if (j == 0 && c < G) {
      sh.m[wave][c] = m;
      sh.l[wave][c] = x;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = 4 * j + i;
      if (g < G) {
#pragma unroll
        for (int t = 0; t < 8; ++t) sh.o[wave][g][8 * c + t] = o[t][i];
      }
    }
  }
};

// bf16 rows of 128 elements take the matrix-core wave; other shapes the VALU wave.
template <typename T, int D, int G, int NW, int SLOTS>
struct AttendWaveOf {
  using type = WaveState<T, D, G, NW, SLOTS>;
};
template <int G, int NW, int SLOTS>
struct AttendWaveOf<bf16_t, 128, G, NW, SLOTS> {
  using type = MfmaWave<G, NW>;
};
template <typename T, int D, int G, int NW = kAttWaves, int SLOTS = kAttSlots>
using AttendWave = typename AttendWaveOf<T, D, G, NW, SLOTS>::type;

// Combines the NW waves' (m, l, o) for output element idx = g*D + c.
template <int D, int G, int NW = kAttWaves>
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

}  // namespace rkv
