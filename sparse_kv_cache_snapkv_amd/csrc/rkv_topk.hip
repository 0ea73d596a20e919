// Exact per-row top-k by radix select on order-preserving 32-bit keys (RocketKV rebuttal,
// "Explanation of Calculating Approximate Attention Scores": select the pages with higher
// scores; "Measurement of Exact-TopK": SnapKV's one-time top-k filter of the prompt).
//
// Rows of up to 8192 elements (page scores of a decode step): one block per row holds the row in
// registers and runs the block select of rkv_select.hpp. Longer rows (prompt token scores) are
// spread over blocks of 4096 elements each, in five short launches: clear the row histograms;
// three digit levels (bits 31..21, 20..10, 9..0 of the keys), each block counting the digits of
// its keys that match the prefix found so far into the row's global histogram (every block of
// the next launch re-derives that prefix from it), the last level also leaving each block's own
// counts under the prefix; and the ordered write, where each block fixes the threshold and
// offsets its block-level compaction by the counts of the blocks before it.
#include <algorithm>

#include "rkv_common.hpp"
#include "rkv_launch.hpp"
#include "rkv_select.hpp"

namespace rkv {

namespace {

constexpr int kBlockThreads = 256;

// One block per row, E keys per thread; rows of up to 4096 keys take 256 threads, longer ones
// (up to 8192) 512, which halves the keys each thread ranks and compacts.
template <int THREADS, int E>
__global__ __launch_bounds__(THREADS) void k_topk_block(const float* __restrict__ scores, int n,
                                                       int k, int32_t* __restrict__ out,
                                                       int out_stride) {
  __shared__ SelectShared<THREADS> sh;
  const float* row = scores + (size_t)blockIdx.x * n;
  int32_t* o = out + (size_t)blockIdx.x * out_stride;
  if (k >= n) {
    for (int i = threadIdx.x; i < n; i += THREADS) o[i] = i;
    return;
  }
  if (k <= 0) return;
  uint32_t key[E];
  const int i0 = threadIdx.x * E;
  const int nv = load_keys<E>(row, n, i0, key);
  uint32_t T, need_eq;
  block_threshold<THREADS, E>(key, nv, (uint32_t)k, T, need_eq, sh);
  block_compact<THREADS, E>(key, nv, T, need_eq, i0, 0u, (uint32_t)k, sh,
                            [&](uint32_t pos, int idx, bool take) {
                              if (take && pos < (uint32_t)k) o[pos] = idx;
                            });
}

// ------------------------------------------------------------------------------ long rows

constexpr int kLongPer = 16;                          // keys per thread
constexpr int kLongChunk = kBlockThreads * kLongPer;  // keys per block
constexpr int kLevels = 3;         // digit levels: key bits 31..21, 20..10, 9..0
constexpr int kHistStride = 2048;  // words per level and row
__host__ __device__ constexpr int level_shift(int lev) { return lev == 0 ? 21 : (lev == 1 ? 10 : 0); }
__host__ __device__ constexpr int level_bits(int lev) { return lev == 2 ? 10 : 11; }
__host__ __device__ constexpr int level_bins(int lev) { return 1 << level_bits(lev); }

static_assert(kLevels * kHistStride == kTopkHistRowWords && level_shift(0) == kTopkLevel0Shift &&
                  level_bins(0) == kTopkLevel0Bins,
              "the first digit level as declared to producers that count it");

// Per block of the last digit level: the suffix sums S[d] (its keys under the row's prefix with
// a last digit >= d, d < 1024) and, in word 1024, its keys above the prefix.
constexpr int kLastBins = level_bins(kLevels - 1);
constexpr int kStateWords = kLastBins + 1;

struct LongLayout {
  int nblk;
  size_t off_hist, off_state, total;
};

LongLayout long_layout(int rows, int n) {
  LongLayout lo{};
  lo.nblk = (n + kLongChunk - 1) / kLongChunk;
  lo.off_hist = 0;
  lo.off_state = lo.off_hist + (size_t)rows * kLevels * kHistStride * sizeof(uint32_t);
  lo.off_state = (lo.off_state + 255) & ~(size_t)255;
  lo.total = lo.off_state + (size_t)rows * lo.nblk * kStateWords * sizeof(uint32_t);
  lo.total = (lo.total + 255) & ~(size_t)255;
  return lo;
}

bool long_path(int n, int k) { return n > 32 * kBlockThreads && k > 0 && k < n; }

__global__ void k_long_zero(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// This thread's bins of one level's histogram (a row's, finished by an earlier launch), 8 or 4
// digits descending from nbins-1-bpt*tid; entries past the level's bins are 0.
__device__ __forceinline__ void load_bins(const uint32_t* __restrict__ hist, int nbins,
                                          uint32_t (&c)[8]) {
  const int bpt = nbins / kBlockThreads;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int bin = nbins - 1 - ((int)threadIdx.x * bpt + j);  // negative only when j >= bpt
    const uint32_t x = hist[bin < 0 ? 0 : bin];
    c[j] = j < bpt ? x : 0u;
  }
}

// The digit of a level (nbins digits, this thread's bins in c as load_bins leaves them) holding
// the krem-th largest key of the keys it counts, and how many counted keys lie in higher digits.
// Every thread must call it; two barriers.
__device__ __forceinline__ void find_digit(const uint32_t (&c)[8], int nbins, uint32_t krem,
                                           uint32_t& digit, uint32_t& above,
                                           SelectShared<kBlockThreads>& sh) {
  const int tid = threadIdx.x;
  const int bpt = nbins / kBlockThreads;
  uint32_t local = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) local += c[j];
  uint32_t excl, unused, tot, unused2;
  block_scan2<kBlockThreads>(local, 0u, excl, unused, tot, unused2, sh, 0);
  if (excl < krem && krem <= excl + local) {
    uint32_t run = excl;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < bpt && run < krem && krem <= run + c[j]) {
        sh.digit = (uint32_t)(nbins - 1 - (tid * bpt + j));
        sh.above = run;
      }
      run += c[j];
    }
  }
  __syncthreads();
  digit = sh.digit;
  above = sh.above;
  __syncthreads();  // sh.digit / the scan partials are rewritten by the next call
}

// Re-derives the prefix (the key bits above level `upto`) and the rank still to place within it.
// The histograms of all the levels it walks are loaded together before the first digit is found.
template <int UPTO>
__device__ __forceinline__ void long_prefix(const uint32_t* __restrict__ hist_row, uint32_t k,
                                            uint32_t& prefix, uint32_t& krem,
                                            SelectShared<kBlockThreads>& sh) {
  prefix = 0u;
  krem = k;
  if constexpr (UPTO > 0) {
    uint32_t c[UPTO][8];
#pragma unroll
    for (int lev = 0; lev < UPTO; ++lev) load_bins(hist_row + lev * kHistStride, level_bins(lev), c[lev]);
#pragma unroll
    for (int lev = 0; lev < UPTO; ++lev) {
      uint32_t d, above;
      find_digit(c[lev], level_bins(lev), krem, d, above, sh);
      prefix |= d << level_shift(lev);
      krem -= above;
    }
  }
}

// The row's histogram of digit level LEVEL over the keys under the prefix the earlier levels
// fixed. The last level also leaves each block's own counts (suffix sums of its digit histogram
// and its keys above the prefix) in `state`, from which the write launch places every block's
// keys without a counting pass of its own.
template <int LEVEL>
__global__ __launch_bounds__(kBlockThreads) void k_long_hist(const float* __restrict__ scores,
                                                            int n, int k,
                                                            uint32_t* __restrict__ hist,
                                                            uint32_t* __restrict__ state) {
  __shared__ SelectShared<kBlockThreads> sh;
  __shared__ uint32_t lh[kHistStride];
  const int tid = threadIdx.x, row = blockIdx.y;
  uint32_t* hist_row = hist + (size_t)row * kLevels * kHistStride;
  uint32_t prefix, krem;
  long_prefix<LEVEL>(hist_row, (uint32_t)k, prefix, krem, sh);
  constexpr int shift = level_shift(LEVEL), nbins = level_bins(LEVEL);
  constexpr int top = shift + level_bits(LEVEL);  // the digit's highest bit + 1
  for (int i = tid; i < nbins; i += kBlockThreads) lh[i] = 0u;
  __syncthreads();
  const float* s = scores + (size_t)row * n + (size_t)blockIdx.x * kLongChunk;
  const int nv = min(kLongChunk, n - (int)blockIdx.x * kLongChunk);
  float v[kLongPer];
#pragma unroll
  for (int j = 0; j < kLongPer; ++j) {
    v[j] = 0.f;
    if (j * kBlockThreads + tid < nv) v[j] = s[j * kBlockThreads + tid];
  }
  uint32_t above = 0;  // keys above the prefix (counted on the last level only)
#pragma unroll
  for (int j = 0; j < kLongPer; ++j) {
    const uint32_t key = order_key(v[j]);
    const bool valid = j * kBlockThreads + tid < nv;
    const bool match = valid && (top >= 32 || (key >> top) == (prefix >> top));
    if (match) atomicAdd(&lh[(key >> shift) & (uint32_t)(nbins - 1)], 1u);
    if constexpr (LEVEL == kLevels - 1) above += (valid && (key >> top) > (prefix >> top)) ? 1u : 0u;
  }
  __syncthreads();
  uint32_t* hl = hist_row + LEVEL * kHistStride;
  for (int i = tid; i < nbins; i += kBlockThreads)
    if (lh[i] != 0u) atomicAdd(&hl[i], lh[i]);
  if constexpr (LEVEL == kLevels - 1) {
    // thread t holds digits nbins-1-4t down to nbins-4-4t; the exclusive scan over the threads
    // gives the keys in the digits above them
    constexpr int bpt = nbins / kBlockThreads;
    uint32_t c[bpt], local = 0;
#pragma unroll
    for (int j = 0; j < bpt; ++j) {
      c[j] = lh[nbins - 1 - (tid * bpt + j)];
      local += c[j];
    }
    uint32_t excl, unused, tot, above_tot;
    block_scan2<kBlockThreads>(local, above, excl, unused, tot, above_tot, sh, 1);
    uint32_t* st = state + ((size_t)row * gridDim.x + blockIdx.x) * kStateWords;
    uint32_t run = excl;
#pragma unroll
    for (int j = 0; j < bpt; ++j) {
      run += c[j];
      st[nbins - 1 - (tid * bpt + j)] = run;
    }
    if (tid == 0) st[kLastBins] = above_tot;
  }
}

// Threshold key T (from the three histograms) and the number of keys equal to T to take; the
// keys above and equal to T in the blocks before this one come from their last-level counts;
// then the block writes its selected positions in order.
__global__ __launch_bounds__(kBlockThreads) void k_long_write(const float* __restrict__ scores,
                                                             int n, int k,
                                                             const uint32_t* __restrict__ hist,
                                                             const uint32_t* __restrict__ state,
                                                             int32_t* __restrict__ out,
                                                             int out_stride) {
  __shared__ SelectShared<kBlockThreads> sh;
  const int tid = threadIdx.x, row = blockIdx.y, blk = blockIdx.x, nblk = gridDim.x;
  uint32_t T, need;
  long_prefix<kLevels>(hist + (size_t)row * kLevels * kHistStride, (uint32_t)k, T, need, sh);
  const uint32_t d = T & (uint32_t)(kLastBins - 1);  // T's last digit
  uint32_t bgt = 0, beq = 0;
  for (int b = tid; b < blk; b += kBlockThreads) {
    const uint32_t* st = state + ((size_t)row * nblk + b) * kStateWords;
    const uint32_t sd = st[d], sd1 = d + 1 < (uint32_t)kLastBins ? st[d + 1] : 0u;
    bgt += st[kLastBins] + sd1;
    beq += sd - sd1;
  }
  uint32_t e0, e1, gt_base, eq_base;
  block_scan2<kBlockThreads>(bgt, beq, e0, e1, gt_base, eq_base, sh, 0);
  const int base = blk * kLongChunk;
  const float* s = scores + (size_t)row * n + base;
  const int nv_blk = min(kLongChunk, n - base);
  uint32_t key[kLongPer];
  const int i0 = tid * kLongPer;
  const int nv = load_keys<kLongPer>(s, nv_blk, i0, key);
  int32_t* o = out + (size_t)row * out_stride;
  block_compact<kBlockThreads, kLongPer>(
      key, nv, T, need, base + i0, 0u, (uint32_t)k, sh,
      [&](uint32_t pos, int idx, bool take) {
        if (take && pos < (uint32_t)k) o[pos] = idx;
      },
      gt_base, eq_base);
}

__global__ void k_fill_identity(int32_t* out, int n, int out_stride) {
  int32_t* o = out + (size_t)blockIdx.y * out_stride;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) o[i] = i;
}

}  // namespace

size_t topk_ws_bytes(int rows, int n, int k) {
  return long_path(n, k) ? long_layout(rows, n).total : 0;
}

bool topk_multiblock(int n, int k) { return long_path(n, k); }
size_t topk_hist_words(int rows) { return (size_t)rows * kLevels * kHistStride; }

namespace {

// The launches of the multi-block path; the clearing launch only where the histograms are not
// already zero.
hipError_t long_launches(const float* scores, int rows, int n, int k, int32_t* out,
                         int out_stride, void* ws, bool cleared, bool level0_counted,
                         hipStream_t stream) {
  const LongLayout lo = long_layout(rows, n);
  char* w = static_cast<char*>(ws);
  uint32_t* hist = reinterpret_cast<uint32_t*>(w + lo.off_hist);
  uint32_t* state = reinterpret_cast<uint32_t*>(w + lo.off_state);
  const dim3 lgrid(lo.nblk, rows);
  hipError_t e;
  if (!cleared) {
    const size_t nhist = topk_hist_words(rows);
    hipLaunchKernelGGL(k_long_zero, dim3((unsigned)std::min<size_t>((nhist + 255) / 256, 1024)),
                       dim3(256), 0, stream, hist, nhist);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (!level0_counted) {
    hipLaunchKernelGGL(k_long_hist<0>, lgrid, dim3(kBlockThreads), 0, stream, scores, n, k, hist,
                       state);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_long_hist<1>, lgrid, dim3(kBlockThreads), 0, stream, scores, n, k, hist,
                     state);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_long_hist<2>, lgrid, dim3(kBlockThreads), 0, stream, scores, n, k, hist,
                     state);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_long_write, lgrid, dim3(kBlockThreads), 0, stream, scores, n, k, hist,
                     state, out, out_stride);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk_cleared(const float* scores, int rows, int n, int k, int32_t* out,
                               int out_stride, void* ws, bool level0_counted, hipStream_t stream) {
  return long_launches(scores, rows, n, k, out, out_stride, ws, true, level0_counted, stream);
}

hipError_t launch_topk(const float* scores, int rows, int n, int k, int32_t* out, int out_stride,
                       void* ws, hipStream_t stream) {
  dim3 grid(rows);
  if (n <= 16 * kBlockThreads) {
    hipLaunchKernelGGL((k_topk_block<kBlockThreads, 16>), grid, dim3(kBlockThreads), 0, stream,
                       scores, n, k, out, out_stride);
    return hipGetLastError();
  }
  if (n <= 32 * kBlockThreads) {
    hipLaunchKernelGGL((k_topk_block<2 * kBlockThreads, 16>), grid, dim3(2 * kBlockThreads), 0,
                       stream, scores, n, k, out, out_stride);
    return hipGetLastError();
  }
  if (k <= 0) return hipSuccess;
  if (k >= n) {
    hipLaunchKernelGGL(k_fill_identity, dim3((n + kBlockThreads - 1) / kBlockThreads, rows),
                       dim3(kBlockThreads), 0, stream, out, n, out_stride);
    return hipGetLastError();
  }
  return long_launches(scores, rows, n, k, out, out_stride, ws, false, false, stream);
}

}  // namespace rkv
