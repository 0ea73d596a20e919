// SnapKV++ permanent eviction at prefill (RocketKV rebuttal, "Measurement of Exact-TopK":
// one-time top-k filtering of the prompt; "SCBench Results": scored by the queries at the end of
// the prompt; summary page and rebuttal "Novelty of SnapKV++": attention summed over the GQA
// group; "Potential Sensitivity to Kernel Size in SnapKV++": 1D pooling with a chosen kernel).
//
// Pipeline per (b, KV head):
//   pass 1  window logits Q_win K^T (causal for window keys) -> per-chunk row (max, sum of exp)
//   merge   per-row log-sum-exp (log2 domain)
//   pass 2  logits again for prefix keys, exp(s - lse) summed over the group's G*W rows -> colsum
//   pool    zero-padded same-size box average (or max) of colsum
//   top-k   keep-W prefix positions (shared radix select), then the W window positions
//   gather  compressed K/V rows
// bf16 logits use MFMA (v_mfma_f32_32x32x16_bf16): the window rows stay in LDS, every wave
// streams 64 keys into registers and multiplies them against all row tiles. The dot product's
// head dimension runs in the operands' natural order (lane half h takes channels 16s + 8h .. +8
// at k-step s): the two lanes of a key then read 32 adjacent bytes per load, which streams K
// faster than one contiguous half row per lane.
// fp32 logits use plain FMAs (the small-workload path).
#include <math.h>

#include <algorithm>

#include "rkv_common.hpp"
#include "rkv_launch.hpp"

namespace rkv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kKeysPerSub = 256;  // 4 waves x 64 keys
constexpr int kPassBlocks = 512;  // blocks per window-pass launch: two per CU, all resident

inline int round32(int x) { return (x + 31) & ~31; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct EvictLayout {
  int GW, GWp, nchunk1, nsub1, nchunk2, nsub2, nprefix;
  int mt1, parts1;  // bf16 passes: row tiles per block (4 or 8) and parts the window rows split into
  int parts2;       // parts of the column sums (1 on the fp32 path, whose passes do not split)
  size_t off_stats, off_lse, off_colsum, off_pooled, off_topk, total;
};

EvictLayout layout_for(int B, int Hq, int Hkv, int L, int W, int keep, int dtype) {
  EvictLayout lo{};
  const int BH = B * Hkv;
  lo.GW = (Hq / Hkv) * W;
  lo.GWp = round32(lo.GW);
  lo.nprefix = L - W;
  lo.mt1 = lo.GWp <= 128 ? 4 : 8;
  lo.parts1 = (lo.GWp + 32 * lo.mt1 - 1) / (32 * lo.mt1);
  lo.parts2 = dtype == 0 ? 1 : lo.parts1;
  auto split = [&](int nkeys, int parts, int& nchunk, int& nsub) {
    const int subs = (nkeys + kKeysPerSub - 1) / kKeysPerSub;
    int want = (kPassBlocks + BH * parts - 1) / (BH * parts);
    if (want > subs) want = subs;
    if (want < 1) want = 1;
    nsub = (subs + want - 1) / want;
    nchunk = (subs + nsub - 1) / nsub;
    if (nchunk < 1) nchunk = 1;
  };
  split(L, lo.parts1, lo.nchunk1, lo.nsub1);
  if (dtype == 0) {  // the fp32 pass 1 takes one 256-key chunk per block
    lo.nchunk1 = (L + kThreads - 1) / kThreads;
    lo.nsub1 = 1;
  }
  split(lo.nprefix > 0 ? lo.nprefix : 1, lo.parts2, lo.nchunk2, lo.nsub2);
  size_t off = 0;
  lo.off_stats = off;
  off = align256(off + (size_t)BH * lo.nchunk1 * lo.GWp * sizeof(float2));
  lo.off_lse = off;
  off = align256(off + (size_t)BH * lo.GWp * sizeof(float));
  lo.off_colsum = off;
  off = align256(off + (size_t)lo.parts2 * BH * (lo.nprefix > 0 ? lo.nprefix : 1) *
                           sizeof(float));
  lo.off_pooled = off;
  off = align256(off + (size_t)BH * (lo.nprefix > 0 ? lo.nprefix : 1) * sizeof(float));
  lo.off_topk = off;
  off = align256(off + topk_ws_bytes(BH, lo.nprefix > 0 ? lo.nprefix : 1, keep - W));
  lo.total = off;
  return lo;
}

// ---------------------------------------------------------------------------- MFMA (bf16) passes

// K rows of one wave's 64 keys (two 32-key tiles) as MFMA operands: at k-step s, lane (half hf,
// row n) holds channels 16s + 8hf .. +8 of key key0 + kt*32 + n.
template <int D>
__device__ __forceinline__ void load_key_tiles(const bf16_t* __restrict__ k_bh, int key0,
                                               int last, int hf, int n,
                                               bf16x8 (&kf)[2][D / 16]) {
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int key = min(key0 + kt * 32 + n, last);
    const bf16_t* kr = k_bh + (size_t)key * D + hf * 8;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) kf[kt][s] = *reinterpret_cast<const bf16x8*>(kr + s * 16);
  }
}

// Window rows of one head into LDS (row pitch D + 8, rows GW..GWp-1 zero), eight 16-byte loads
// per thread in flight at a time.
template <int D>
__device__ __forceinline__ void stage_window_rows(uint16_t* smem, const bf16_t* __restrict__ qg,
                                                  int GW, int GWp, int tid) {
  constexpr int QS = D + 8, kBatch = 8;
  const int n16 = GWp * (D / 8);
  for (int base = 0; base < n16; base += kBatch * kThreads) {
    uint4 val[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int idx = base + j * kThreads + tid, row = idx / (D / 8), c8 = idx % (D / 8);
      val[j] = make_uint4(0, 0, 0, 0);
      if (row < GW) val[j] = load16(qg + (size_t)row * D + c8 * 8);
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int idx = base + j * kThreads + tid, row = idx / (D / 8), c8 = idx % (D / 8);
      if (idx < n16) *reinterpret_cast<uint4*>(smem + (size_t)row * QS + c8 * 8) = val[j];
    }
  }
}

// Pass 1: per window row, the running (max, sum of exp2) of its scaled logits over this block's
// keys, in log2 units. Each lane keeps the running pair of its row in every 32-row tile across
// all of the block's key groups; the pairs of the lane halves and the four waves merge once at
// the end. A block takes at most MT 32-row tiles (their running pairs stay in registers): the
// window rows split into parts of 32 * MT rows, part p of chunk c being block x = p * nchunk + c,
// so that the rows of a part fit two blocks per CU in LDS.
template <int D, int MT>
__global__ __launch_bounds__(kThreads) void k_win_stats_mfma(const bf16_t* __restrict__ q_win,
                                                             const bf16_t* __restrict__ k, int L,
                                                             int W, int GW, int nsub, int nchunk,
                                                             float scale2,
                                                             float2* __restrict__ stats) {
  constexpr int KS = D / 16;
  constexpr int QS = D + 8;
  constexpr int kMaxTiles = MT;
  extern __shared__ __align__(16) uint16_t smem[];
  const int GWp = (GW + 31) & ~31;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hf = lane >> 5, n = lane & 31;
  const int bh = blockIdx.y, part = blockIdx.x / nchunk, chunk = blockIdx.x % nchunk;
  const int row0 = part * 32 * MT;                 // this block's first window row
  const int GWl = min(GW - row0, 32 * MT);         // and its row count
  const int GWlp = (GWl + 31) & ~31, NRT = GWlp / 32;
  float2* wst = reinterpret_cast<float2*>(smem + (size_t)GWlp * QS);  // [4][GWlp]

  // Key groups are interleaved over the chunks (group j of chunk c starts at key
  // (j * nchunk + c) * 256), so the blocks of a head sweep its keys as one front. Key registers
  // are double-buffered: the next group's loads are in flight while the current one is
  // multiplied. The first group's loads go out before the window rows are staged.
  const bf16_t* k_bh = k + (size_t)bh * L * D;
  auto key_of = [&](int t) { return (t * nchunk + chunk) * kKeysPerSub + wave * 64; };
  bf16x8 kf0[2][KS], kf1[2][KS];
  load_key_tiles<D>(k_bh, key_of(0), L - 1, hf, n, kf0);

  stage_window_rows<D>(smem, q_win + ((size_t)bh * GW + row0) * D, GWl, GWlp, tid);
  __syncthreads();

  float m[kMaxTiles], l[kMaxTiles];
#pragma unroll
  for (int rt = 0; rt < kMaxTiles; ++rt) {
    m[rt] = -INFINITY;
    l[rt] = 0.f;
  }
  auto group_stats = [&](const bf16x8(&kf)[2][KS], int key0) {
    // keys below L-W are visible to every window row: only groups reaching it need the mask
    const bool masked = key0 + 63 >= L - W;
#pragma unroll
    for (int rt = 0; rt < kMaxTiles; ++rt) {
      if (rt >= NRT) break;
      f32x16 acc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[kt][i] = 0.f;
      const uint16_t* qrow = smem + (size_t)(rt * 32 + n) * QS + hf * 8;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 qf = *reinterpret_cast<const bf16x8*>(qrow + s * 16);
        acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[0][s], qf, acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[1][s], qf, acc[1], 0, 0, 0);
      }
      // lane holds window row rt*32+n against keys key0 + kt*32 + 8*(i/4) + 4*hf + i%4
      if (masked) {
        const int row = row0 + rt * 32 + n;               // the window row, in the whole group
        const int lim = row < GW ? L - W + (row % W) : -1;  // last visible key
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + kt * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
            acc[kt][i] = (key < L && key <= lim) ? acc[kt][i] : -INFINITY;
          }
      }
      float tmax = acc[0][0];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, acc[kt][i]);
      const float mn = fmaxf(m[rt], tmax * scale2);  // scale2 > 0: the scaled max
      if (mn != -INFINITY) {
        float sm = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) sm += exp2_hw(fmaf(acc[kt][i], scale2, -mn));
        l[rt] = l[rt] * exp2_hw(m[rt] - mn) + sm;
        m[rt] = mn;
      }
    }
  };
  // The next group's loads always go out (past the chunk's last group they re-read the current
  // rows, from cache): issued on some paths only, the compiler's wait for the current group
  // would also cover them.
  for (int t = 0; t < nsub; t += 2) {
    const int key0 = key_of(t), key1 = t + 1 < nsub ? key_of(t + 1) : key0;
    load_key_tiles<D>(k_bh, key1, L - 1, hf, n, kf1);
    group_stats(kf0, key0);
    if (t + 1 >= nsub) break;
    load_key_tiles<D>(k_bh, t + 2 < nsub ? key_of(t + 2) : key1, L - 1, hf, n, kf0);
    group_stats(kf1, key1);
  }
  // merge the two lane halves (same rows, other keys), then the waves through LDS
#pragma unroll
  for (int rt = 0; rt < kMaxTiles; ++rt) {
    if (rt >= NRT) break;
    const float mo = __shfl_xor(m[rt], 32, 64), lo = __shfl_xor(l[rt], 32, 64);
    const float mx = fmaxf(m[rt], mo);
    const float lx = mx == -INFINITY ? 0.f : l[rt] * exp2_hw(m[rt] - mx) + lo * exp2_hw(mo - mx);
    if (hf == 0) wst[wave * GWlp + rt * 32 + n] = make_float2(mx, lx);
  }
  __syncthreads();
  for (int r = tid; r < GWl; r += kThreads) {
    float mm = -INFINITY, ll = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float2 x = wst[w * GWlp + r];
      const float M = fmaxf(mm, x.x);
      if (M != -INFINITY) {
        ll = ll * exp2_hw(mm - M) + x.y * exp2_hw(x.x - M);
        mm = M;
      }
    }
    stats[((size_t)bh * nchunk + chunk) * GWp + row0 + r] = make_float2(mm, ll);
  }
}

// Pass 2: for each prefix key, the sum over the group's window rows of exp2(scaled logit - row
// log-sum-exp), i.e. its softmax probabilities summed over the G*W rows. Prefix keys are visible
// to every row, so no mask is needed. The rows split into parts of 32 * MT as in pass 1 (block x
// = p * nchunk + c); part p writes its partial sums to colsum + p * (rows of heads) * prefix, and
// the pooling adds the parts in order.
template <int D, int MT>
__global__ __launch_bounds__(kThreads) void k_win_colsum_mfma(const bf16_t* __restrict__ q_win,
                                                              const bf16_t* __restrict__ k,
                                                              const float* __restrict__ lse,
                                                              int L, int W, int GW, int nsub,
                                                              int nchunk, float scale2,
                                                              float* __restrict__ colsum) {
  constexpr int KS = D / 16;
  constexpr int QS = D + 8;
  extern __shared__ __align__(16) uint16_t smem[];
  const int GWp = (GW + 31) & ~31;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hf = lane >> 5, n = lane & 31;
  const int bh = blockIdx.y, part = blockIdx.x / nchunk, chunk = blockIdx.x % nchunk;
  const int row0 = part * 32 * MT, GWl = min(GW - row0, 32 * MT);
  const int GWlp = (GWl + 31) & ~31, NRT = GWlp / 32;
  const int nprefix = L - W;
  float* s_lse = reinterpret_cast<float*>(smem + (size_t)GWlp * QS);
  float* csp = colsum + (size_t)part * gridDim.y * nprefix;  // this part's partial sums

  // Key groups interleaved over the chunks and double-buffered as in pass 1, but visited in the
  // reverse of pass 1's order: the groups pass 1 read last are the likeliest to still be held by
  // the Infinity Cache. Keys past the prefix are loaded clamped (the prefix is never empty when
  // the passes run, as keep < L and W <= keep) and never written.
  const bf16_t* k_bh = k + (size_t)bh * L * D;
  auto key_of = [&](int t) { return ((nsub - 1 - t) * nchunk + chunk) * kKeysPerSub + wave * 64; };
  bf16x8 kf0[2][KS], kf1[2][KS];
  load_key_tiles<D>(k_bh, key_of(0), nprefix - 1, hf, n, kf0);

  stage_window_rows<D>(smem, q_win + ((size_t)bh * GW + row0) * D, GWl, GWlp, tid);
  for (int r = tid; r < GWlp; r += kThreads) {
    const float x = lse[(size_t)bh * GWp + row0 + min(r, GWl - 1)];
    s_lse[r] = r < GWl ? x : INFINITY;  // padded rows add exp2(-inf) = 0
  }
  __syncthreads();

  auto group_colsum = [&](const bf16x8(&kf)[2][KS], int key0) {
    float cs[2] = {0.f, 0.f};
    for (int rt = 0; rt < NRT; ++rt) {
      f32x16 acc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[kt][i] = 0.f;
      const uint16_t* qrow = smem + (size_t)(rt * 32 + n) * QS + hf * 8;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 qf = *reinterpret_cast<const bf16x8*>(qrow + s * 16);
        acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf, kf[0][s], acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf, kf[1][s], acc[1], 0, 0, 0);
      }
      // lane holds key key0 + kt*32 + n against rows rt*32 + 8*(i/4) + 4*hf + i%4
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float ls = s_lse[rt * 32 + 8 * (i >> 2) + 4 * hf + (i & 3)];
        cs[0] += exp2_hw(fmaf(acc[0][i], scale2, -ls));
        cs[1] += exp2_hw(fmaf(acc[1][i], scale2, -ls));
      }
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const float tot = cs[kt] + __shfl_xor(cs[kt], 32, 64);
      const int key = key0 + kt * 32 + n;
      if (hf == 0 && key < nprefix) csp[(size_t)bh * nprefix + key] = tot;
    }
  };
  for (int t = 0; t < nsub; t += 2) {  // the next group's loads always go out, as in pass 1
    const int key0 = key_of(t), key1 = t + 1 < nsub ? key_of(t + 1) : key0;
    load_key_tiles<D>(k_bh, key1, nprefix - 1, hf, n, kf1);
    group_colsum(kf0, key0);
    if (t + 1 >= nsub) break;
    load_key_tiles<D>(k_bh, t + 2 < nsub ? key_of(t + 2) : key1, nprefix - 1, hf, n, kf0);
    group_colsum(kf1, key1);
  }
}

// ---------------------------------------------------------------------------- fp32 passes

template <int D>
__global__ __launch_bounds__(kThreads) void k_win_stats_f32(const float* __restrict__ q_win,
                                                            const float* __restrict__ k, int L,
                                                            int W, int GW, int nchunk,
                                                            float scale2,
                                                            float2* __restrict__ stats) {
  extern __shared__ __align__(16) uint16_t smem[];
  float2* wst = reinterpret_cast<float2*>(smem);  // [4][GW]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bh = blockIdx.y, chunk = blockIdx.x;
  const int GWp = (GW + 31) & ~31;
  const int key = chunk * kThreads + tid;
  const float* kr = k + ((size_t)bh * L + min(key, L - 1)) * D;
  float kv[D];
#pragma unroll
  for (int c = 0; c < D; c += 4) {
    float x[4];
    unpack16<float>(load16(kr + c), x);
#pragma unroll
    for (int e = 0; e < 4; ++e) kv[c + e] = x[e];
  }
  const float* qg = q_win + (size_t)bh * GW * D;
  for (int row = 0; row < GW; ++row) {
    const float* qr = qg + (size_t)row * D;
    float d = 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) d = fmaf(qr[c], kv[c], d);
    const bool valid = key < L && key <= L - W + (row % W);
    const float v = valid ? d * scale2 : -INFINITY;
    const float m = group_max<64>(v);
    float sm = m != -INFINITY ? exp2_hw(v - m) : 0.f;
    sm = group_sum<64>(sm);
    if (lane == 0) wst[wave * GW + row] = make_float2(m, sm);
  }
  __syncthreads();
  for (int r = tid; r < GW; r += kThreads) {
    float m = -INFINITY, l = 0.f;
    for (int w = 0; w < 4; ++w) {
      const float2 x = wst[w * GW + r];
      const float M = fmaxf(m, x.x);
      if (M != -INFINITY) {
        l = l * exp2_hw(m - M) + x.y * exp2_hw(x.x - M);
        m = M;
      }
    }
    stats[((size_t)bh * nchunk + chunk) * GWp + r] = make_float2(m, l);
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void k_win_colsum_f32(const float* __restrict__ q_win,
                                                             const float* __restrict__ k,
                                                             const float* __restrict__ lse, int L,
                                                             int W, int GW, float scale2,
                                                             float* __restrict__ colsum) {
  const int bh = blockIdx.y;
  const int key = blockIdx.x * kThreads + threadIdx.x;
  const int nprefix = L - W;
  if (key >= nprefix) return;
  const int GWp = (GW + 31) & ~31;
  const float* kr = k + ((size_t)bh * L + key) * D;
  float kv[D];
#pragma unroll
  for (int c = 0; c < D; c += 4) {
    float x[4];
    unpack16<float>(load16(kr + c), x);
#pragma unroll
    for (int e = 0; e < 4; ++e) kv[c + e] = x[e];
  }
  const float* qg = q_win + (size_t)bh * GW * D;
  const float* lb = lse + (size_t)bh * GWp;
  float cs = 0.f;
  for (int row = 0; row < GW; ++row) {
    const float* qr = qg + (size_t)row * D;
    float d = 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) d = fmaf(qr[c], kv[c], d);
    cs += exp2_hw(d * scale2 - lb[row]);
  }
  colsum[(size_t)bh * nprefix + key] = cs;
}

// ---------------------------------------------------------------------------- shared stages

// Per window row, the log2-sum-exp of its scaled logits from the pass-1 chunk pairs: one wave per
// row, lanes over chunks (online merge per lane), then a wave-wide merge. The grid also clears
// the nzero words at zero (the kept-set top-k's digit histograms).
__global__ __launch_bounds__(kThreads) void k_win_lse(const float2* __restrict__ stats, int nchunk,
                                                      int GW, float* __restrict__ lse,
                                                      uint32_t* __restrict__ zero, size_t nzero) {
  {
    const size_t nthr = (size_t)gridDim.x * gridDim.y * kThreads;
    const size_t t0 = ((size_t)blockIdx.y * gridDim.x + blockIdx.x) * kThreads + threadIdx.x;
    for (size_t i = t0; i < nzero; i += nthr) zero[i] = 0u;
  }
  const int bh = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int r = blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
  const int GWp = (GW + 31) & ~31;
  if (r >= GW) return;  // whole waves leave together; no barrier follows
  float m = -INFINITY, l = 0.f;
  for (int c = lane; c < nchunk; c += kWave) {
    const float2 x = stats[((size_t)bh * nchunk + c) * GWp + r];
    const float M = fmaxf(m, x.x);
    if (M != -INFINITY) {
      l = l * exp2_hw(m - M) + x.y * exp2_hw(x.x - M);
      m = M;
    }
  }
  const float M = group_max<kWave>(m);
  const float part = M == -INFINITY ? 0.f : l * exp2_hw(m - M);
  const float tot = group_sum<kWave>(part);
  if (lane == 0) lse[(size_t)bh * GWp + r] = M + log2f(tot);
}

// Zero-padded same-size pooling of each row (KIND 0: box average, 1: box maximum); the tile and
// its halo are staged in LDS.
template <int KIND>
__global__ __launch_bounds__(kThreads) void k_pool(const float* __restrict__ colsum, int n,
                                                   int parts, int kernel,
                                                   float* __restrict__ pooled) {
  __shared__ float tile[kThreads + 128];
  const int bh = blockIdx.y;
  const int h = kernel / 2;
  const int j0 = blockIdx.x * kThreads;
  const float* src = colsum + (size_t)bh * n;
  const size_t pstride = (size_t)gridDim.y * n;  // between the window-row parts' partial sums
  for (int i = threadIdx.x; i < kThreads + 2 * h; i += kThreads) {
    const int j = j0 - h + i;
    const int jc = min(max(j, 0), n - 1);  // every address inside the row
    float x = src[jc];
    for (int p = 1; p < parts; ++p) x += src[p * pstride + jc];
    tile[i] = (j >= 0 && j < n) ? x : 0.f;
  }
  __syncthreads();
  const int j = j0 + threadIdx.x;
  if (j >= n) return;
  // four interleaved partial results keep the dependent chains short
  const float* t = tile + threadIdx.x;
  float a[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) a[e] = KIND == 0 ? 0.f : t[0];
  int u = 0;
  for (; u + 4 <= kernel; u += 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = KIND == 0 ? a[e] + t[u + e] : fmaxf(a[e], t[u + e]);
  }
  for (; u < kernel; ++u) a[0] = KIND == 0 ? a[0] + t[u] : fmaxf(a[0], t[u]);
  const float acc = KIND == 0 ? (a[0] + a[1]) + (a[2] + a[3])
                              : fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3]));
  pooled[(size_t)bh * n + j] = KIND == 0 ? acc / (float)kernel : acc;
}

// Box-average pooling fused with the first digit level of the multi-block kept-set top-k: a block
// pools kPoolSpan consecutive positions of one row, thread t the kPoolPer positions from
// kPoolPer * t by a sliding window (the first window summed in order, then one value in and one
// out per step), and counts each output's top key bits into the row's first-level histogram
// (already cleared), so the top-k skips that pass. The values differ from k_pool's direct box
// sums only in rounding.
constexpr int kPoolThreads = 1024;
constexpr int kPoolPer = 4;
constexpr int kPoolSpan = kPoolPer * kPoolThreads;

__global__ __launch_bounds__(kPoolThreads) void k_pool_count(const float* __restrict__ colsum, int n,
                                                         int parts, int kernel,
                                                         float* __restrict__ pooled,
                                                         uint32_t* __restrict__ hist0) {
  __shared__ float tile[kPoolSpan + 128];
  __shared__ uint32_t lh[kTopkLevel0Bins];
  const int bh = blockIdx.y, tid = threadIdx.x;
  const int h = kernel / 2;
  const int j0 = blockIdx.x * kPoolSpan;
  const float* src = colsum + (size_t)bh * n;
  const size_t pstride = (size_t)gridDim.y * n;  // between the window-row parts' partial sums
  for (int i = tid; i < kTopkLevel0Bins; i += kPoolThreads) lh[i] = 0u;
  for (int i = tid; i < kPoolSpan + 2 * h; i += kPoolThreads) {
    const int j = j0 - h + i;
    const int jc = min(max(j, 0), n - 1);  // every address inside the row
    float x = src[jc];
    for (int p = 1; p < parts; ++p) x += src[p * pstride + jc];
    tile[i] = (j >= 0 && j < n) ? x : 0.f;
  }
  __syncthreads();
  const int jb = kPoolPer * tid;  // this thread's first position in the block
  const float inv = 1.f / (float)kernel;
  float sum = 0.f;
  for (int u = 0; u < kernel; ++u) sum += tile[jb + u];
  float v[kPoolPer];
#pragma unroll
  for (int m = 0; m < kPoolPer; ++m) {
    v[m] = sum * inv;
    sum += tile[jb + m + kernel] - tile[jb + m];
  }
  const int nv = min(kPoolPer, n - (j0 + jb));  // may be <= 0 past the row's end
  float* out = pooled + (size_t)bh * n + j0 + jb;
  if (nv == kPoolPer && (reinterpret_cast<uintptr_t>(out) & 15) == 0) {
#pragma unroll
    for (int m = 0; m < kPoolPer; m += 4)
      *reinterpret_cast<float4*>(out + m) = make_float4(v[m], v[m + 1], v[m + 2], v[m + 3]);
  } else {
    for (int m = 0; m < nv; ++m) out[m] = v[m];
  }
  // a thread's outputs are consecutive box averages, mostly in one top-bit bin: runs of equal
  // bins are counted before one LDS addition each
  if (nv > 0) {
    uint32_t cur = order_key(v[0]) >> kTopkLevel0Shift, cnt = 1u;
#pragma unroll
    for (int m = 1; m < kPoolPer; ++m) {
      if (m >= nv) break;
      const uint32_t b = order_key(v[m]) >> kTopkLevel0Shift;
      if (b != cur) {
        atomicAdd(&lh[cur], cnt);
        cur = b;
        cnt = 0u;
      }
      ++cnt;
    }
    atomicAdd(&lh[cur], cnt);
  }
  __syncthreads();
  uint32_t* hr = hist0 + (size_t)bh * kTopkHistRowWords;
  for (int i = tid; i < kTopkLevel0Bins; i += kPoolThreads)
    if (lh[i] != 0u) atomicAdd(&hr[i], lh[i]);
}

// Completes kept_idx (window positions, or the identity when nothing is evicted) and gathers
// the compressed K/V rows, 16 bytes per lane.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void k_gather(const T* __restrict__ k,
                                                     const T* __restrict__ v, int L, int W, int Lc,
                                                     int identity, int32_t* __restrict__ kept,
                                                     T* __restrict__ k_out, T* __restrict__ v_out) {
  constexpr int V = vec16<T>::n;
  constexpr int LPT = D / V;
  constexpr int TPB = kThreads / LPT;  // tokens per block
  const int bh = blockIdx.y;
  const int t = blockIdx.x * TPB + threadIdx.x / LPT;
  const int li = threadIdx.x % LPT;
  if (t >= Lc) return;
  const int nsel = Lc - W;
  int src;
  if (identity) {
    src = t;
  } else if (t >= nsel) {
    src = L - W + (t - nsel);
  } else {
    // the kept-set top-k writes every slot below nsel with a prefix position; clamped all the
    // same, so that no index read here can address outside the head's rows
    src = min(max(kept[(size_t)bh * Lc + t], 0), L - W - 1);
  }
  if (li == 0 && (identity || t >= nsel)) kept[(size_t)bh * Lc + t] = src;
  if (k_out == nullptr) return;
  const size_t si = ((size_t)bh * L + src) * D + li * V;
  const size_t di = ((size_t)bh * Lc + t) * D + li * V;
  store16_stream(k_out + di, load16(k + si));
  store16_stream(v_out + di, load16(v + si));
}

template <typename T, int D>
hipError_t gather(const void* k, const void* v, int BH, int L, int W, int Lc, int identity,
                  int32_t* kept, void* k_out, void* v_out, hipStream_t stream) {
  constexpr int TPB = kThreads / (D / vec16<T>::n);
  dim3 grid((Lc + TPB - 1) / TPB, BH);
  hipLaunchKernelGGL((k_gather<T, D>), grid, dim3(kThreads), 0, stream,
                     static_cast<const T*>(k), static_cast<const T*>(v), L, W, Lc, identity, kept,
                     static_cast<T*>(k_out), static_cast<T*>(v_out));
  return hipGetLastError();
}

hipError_t gather_any(int dtype, int D, const void* k, const void* v, int BH, int L, int W, int Lc,
                      int identity, int32_t* kept, void* k_out, void* v_out, hipStream_t stream) {
  if (dtype == 0)
    return D == 64 ? gather<float, 64>(k, v, BH, L, W, Lc, identity, kept, k_out, v_out, stream)
                   : gather<float, 128>(k, v, BH, L, W, Lc, identity, kept, k_out, v_out, stream);
  return D == 64 ? gather<bf16_t, 64>(k, v, BH, L, W, Lc, identity, kept, k_out, v_out, stream)
                 : gather<bf16_t, 128>(k, v, BH, L, W, Lc, identity, kept, k_out, v_out, stream);
}

template <int D, int MT>
hipError_t scores_bf16(const void* q_win, const void* k, int BH, int L, int W,
                       const EvictLayout& lo, float scale2, char* ws, uint32_t* zero, size_t nzero,
                       hipStream_t stream) {
  constexpr int QS = D + 8;
  float2* stats = reinterpret_cast<float2*>(ws + lo.off_stats);
  float* lse = reinterpret_cast<float*>(ws + lo.off_lse);
  float* colsum = reinterpret_cast<float*>(ws + lo.off_colsum);
  const int rows = std::min(lo.GWp, 32 * MT);  // window rows per block of either pass
  const size_t lds1 = (size_t)rows * QS * 2 + (size_t)rows * sizeof(float2) * 4;
  const size_t lds2 = (size_t)rows * QS * 2 + (size_t)rows * sizeof(float);
  hipError_t e = hipSuccess;
  if (lds1 > 64 * 1024 &&
      (e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_win_stats_mfma<D, MT>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds1)) != hipSuccess)
    return e;
  if (lds2 > 64 * 1024 &&
      (e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_win_colsum_mfma<D, MT>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds2)) != hipSuccess)
    return e;
  hipLaunchKernelGGL((k_win_stats_mfma<D, MT>), dim3(lo.nchunk1 * lo.parts1, BH), dim3(kThreads),
                     lds1, stream, static_cast<const bf16_t*>(q_win),
                     static_cast<const bf16_t*>(k), L, W, lo.GW, lo.nsub1, lo.nchunk1, scale2,
                     stats);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_win_lse, dim3((lo.GW + 3) / 4, BH), dim3(kThreads), 0, stream, stats,
                     lo.nchunk1, lo.GW, lse, zero, nzero);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((k_win_colsum_mfma<D, MT>), dim3(lo.nchunk2 * lo.parts2, BH),
                     dim3(kThreads), lds2, stream, static_cast<const bf16_t*>(q_win),
                     static_cast<const bf16_t*>(k), lse, L, W, lo.GW, lo.nsub2, lo.nchunk2, scale2,
                     colsum);
  return hipGetLastError();
}

template <int D>
hipError_t scores_bf16_any(const void* q_win, const void* k, int BH, int L, int W,
                           const EvictLayout& lo, float scale2, char* ws, uint32_t* zero,
                           size_t nzero, hipStream_t stream) {
  return lo.mt1 == 4
             ? scores_bf16<D, 4>(q_win, k, BH, L, W, lo, scale2, ws, zero, nzero, stream)
             : scores_bf16<D, 8>(q_win, k, BH, L, W, lo, scale2, ws, zero, nzero, stream);
}

template <int D>
hipError_t scores_f32(const void* q_win, const void* k, int BH, int L, int W,
                      const EvictLayout& lo, float scale2, char* ws, uint32_t* zero, size_t nzero,
                      hipStream_t stream) {
  float2* stats = reinterpret_cast<float2*>(ws + lo.off_stats);
  float* lse = reinterpret_cast<float*>(ws + lo.off_lse);
  float* colsum = reinterpret_cast<float*>(ws + lo.off_colsum);
  const int nchunk = lo.nchunk1;
  hipLaunchKernelGGL(k_win_stats_f32<D>, dim3(nchunk, BH), dim3(kThreads),
                     (size_t)4 * lo.GW * sizeof(float2), stream, static_cast<const float*>(q_win),
                     static_cast<const float*>(k), L, W, lo.GW, nchunk, scale2, stats);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_win_lse, dim3((lo.GW + 3) / 4, BH), dim3(kThreads), 0, stream, stats,
                     nchunk, lo.GW, lse, zero, nzero);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_win_colsum_f32<D>, dim3((lo.nprefix + kThreads - 1) / kThreads, BH),
                     dim3(kThreads), 0, stream, static_cast<const float*>(q_win),
                     static_cast<const float*>(k), lse, L, W, lo.GW, scale2, colsum);
  return hipGetLastError();
}

}  // namespace

size_t evict_ws_bytes(int B, int Hq, int Hkv, int L, int D, int W, int keep, int dtype) {
  if (keep >= L) return 0;
  (void)D;
  return layout_for(B, Hq, Hkv, L, W, keep, dtype).total;
}

hipError_t launch_evict(const void* q_win, const void* k, const void* v, int B, int Hq, int Hkv,
                        int L, int D, int W, int keep, int pool_kernel, int pool_type, float scale,
                        int dtype, int32_t* kept_idx, void* k_out, void* v_out, float* pooled_out,
                        void* ws, hipStream_t stream) {
  const int BH = B * Hkv;
  if (keep >= L)
    return gather_any(dtype, D, k, v, BH, L, W, L, 1, kept_idx, k_out, v_out, stream);
  const EvictLayout lo = layout_for(B, Hq, Hkv, L, W, keep, dtype);
  char* w = static_cast<char*>(ws);
  const float scale2 = scale * kLog2e;
  const int n = lo.nprefix;
  // Rows the top-k spreads over blocks have their digit histograms (at the start of the top-k
  // workspace) cleared by the log-sum-exp launch, which saves the top-k its clearing launch.
  const bool cleared = topk_multiblock(n, keep - W);
  uint32_t* hist = cleared ? reinterpret_cast<uint32_t*>(w + lo.off_topk) : nullptr;
  const size_t nhist = cleared ? topk_hist_words(BH) : 0;
  hipError_t e;
  if (dtype == 0)
    e = D == 64 ? scores_f32<64>(q_win, k, BH, L, W, lo, scale2, w, hist, nhist, stream)
                : scores_f32<128>(q_win, k, BH, L, W, lo, scale2, w, hist, nhist, stream);
  else
    e = D == 64 ? scores_bf16_any<64>(q_win, k, BH, L, W, lo, scale2, w, hist, nhist, stream)
                : scores_bf16_any<128>(q_win, k, BH, L, W, lo, scale2, w, hist, nhist, stream);
  if (e != hipSuccess) return e;
  float* colsum = reinterpret_cast<float*>(w + lo.off_colsum);
  float* pooled = pooled_out != nullptr ? pooled_out : reinterpret_cast<float*>(w + lo.off_pooled);
  // average pooling ahead of the multi-block top-k also counts its first digit level
  const bool counted = cleared && pool_type == 0;
  if (counted)
    hipLaunchKernelGGL(k_pool_count, dim3((n + kPoolSpan - 1) / kPoolSpan, BH), dim3(kPoolThreads),
                       0, stream, colsum, n, lo.parts2, pool_kernel, pooled, hist);
  else if (pool_type == 0)
    hipLaunchKernelGGL(k_pool<0>, dim3((n + kThreads - 1) / kThreads, BH), dim3(kThreads), 0,
                       stream, colsum, n, lo.parts2, pool_kernel, pooled);
  else
    hipLaunchKernelGGL(k_pool<1>, dim3((n + kThreads - 1) / kThreads, BH), dim3(kThreads), 0,
                       stream, colsum, n, lo.parts2, pool_kernel, pooled);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  e = cleared ? launch_topk_cleared(pooled, BH, n, keep - W, kept_idx, keep, w + lo.off_topk,
                                    counted, stream)
              : launch_topk(pooled, BH, n, keep - W, kept_idx, keep, w + lo.off_topk, stream);
  if (e != hipSuccess) return e;
  return gather_any(dtype, D, k, v, BH, L, W, keep, 0, kept_idx, k_out, v_out, stream);
}

}  // namespace rkv
