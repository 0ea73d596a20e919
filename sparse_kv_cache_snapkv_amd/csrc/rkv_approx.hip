// Hybrid approximate page scores: head-dim reduction to the top-|q| channels of the GQA group
// and sign-selected Kmin/Kmax page bounds (RocketKV rebuttal, "Explanation of Calculating
// Approximate Attention Scores"; "Novelty": reduction along sequence and head dims).
//
// Block = (page range, b*Hkv+h): the block ranks the group's channels (a few hundred bytes of q,
// cache resident); then each row of 16 lanes scores one 16-byte vector of consecutive pages, each
// lane summing a sixteenth of the chosen channels with all of its loads in flight, and only the
// Kmin or the Kmax row of each channel is read. The fused decode step uses the same device
// functions, so both produce identical scores.
#include <algorithm>

#include "rkv_approx.hpp"
#include "rkv_common.hpp"
#include "rkv_launch.hpp"

namespace rkv {

namespace {

constexpr int kThreads = 256;
// A launch of many heads spans several passes of pages per block (up to kMaxSpan), keeping about
// kGridTarget blocks: each block then ranks its group's channels once for more pages.
constexpr int kMaxSpan = 8;
constexpr int kGridTarget = 4096;

template <typename T, int G>
__global__ __launch_bounds__(kThreads) void k_approx_scores(
    const T* __restrict__ q, const T* __restrict__ kmin_t, const T* __restrict__ kmax_t, int Hkv,
    int D, int P, int pitch, int r, int vec, int per_block, int32_t* __restrict__ chan_idx,
    float* __restrict__ scores) {
  __shared__ ChannelShared ch;
  const int bh = blockIdx.y, b = bh / Hkv, h = bh % Hkv;
  select_channels_block<T, G>(q, b, h, Hkv, D, r, ch);
  if (chan_idx != nullptr && blockIdx.x == 0)
    for (int j = threadIdx.x; j < r; j += kThreads) chan_idx[(size_t)bh * r + j] = ch.chan[j];
  const int p0 = blockIdx.x * per_block;
  float* srow = scores + (size_t)bh * P;
  auto sink = [&](int p, float v) { srow[p] = v; };
  const T* kmin_bh = kmin_t + (size_t)bh * D * pitch;
  const T* kmax_bh = kmax_t + (size_t)bh * D * pitch;
  if (vec)
    score_page_range<T, true>(kmin_bh, kmax_bh, D, pitch, r, p0, min(P, p0 + per_block), ch, sink);
  else
    score_page_range<T, false>(kmin_bh, kmax_bh, D, pitch, r, p0, min(P, p0 + per_block), ch,
                               sink);
}

template <typename T, int G>
hipError_t launch_g(const void* q, const void* kmin_t, const void* kmax_t, int B, int Hkv, int D,
                    int P, int pitch, int r, int32_t* chan_idx, float* scores, hipStream_t stream) {
  // vectors of pages need whole vectors inside every summary row
  const int vec = pitch % vec16<T>::n == 0;
  const int pass = (kThreads / kScoreGroups) * (vec ? vec16<T>::n : 1);
  const long BH = (long)B * Hkv;
  const long per_head = (P + pass - 1) / pass;
  const int span = (int)std::max(1L, std::min((long)kMaxSpan, BH * per_head / kGridTarget));
  const int per_block = pass * span;
  dim3 grid((P + per_block - 1) / per_block, (unsigned)BH);
  hipLaunchKernelGGL((k_approx_scores<T, G>), grid, dim3(kThreads), 0, stream,
                     static_cast<const T*>(q), static_cast<const T*>(kmin_t),
                     static_cast<const T*>(kmax_t), Hkv, D, P, pitch, r, vec, per_block, chan_idx,
                     scores);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const void* q, const void* kmin_t, const void* kmax_t, int B, int Hq, int Hkv,
                    int D, int P, int pitch, int r, int32_t* chan_idx, float* scores,
                    hipStream_t s) {
  switch (Hq / Hkv) {
    case 1: return launch_g<T, 1>(q, kmin_t, kmax_t, B, Hkv, D, P, pitch, r, chan_idx, scores, s);
    case 2: return launch_g<T, 2>(q, kmin_t, kmax_t, B, Hkv, D, P, pitch, r, chan_idx, scores, s);
    case 3: return launch_g<T, 3>(q, kmin_t, kmax_t, B, Hkv, D, P, pitch, r, chan_idx, scores, s);
    case 4: return launch_g<T, 4>(q, kmin_t, kmax_t, B, Hkv, D, P, pitch, r, chan_idx, scores, s);
    case 5: return launch_g<T, 5>(q, kmin_t, kmax_t, B, Hkv, D, P, pitch, r, chan_idx, scores, s);
    case 6: return launch_g<T, 6>(q, kmin_t, kmax_t, B, Hkv, D, P, pitch, r, chan_idx, scores, s);
    case 7: return launch_g<T, 7>(q, kmin_t, kmax_t, B, Hkv, D, P, pitch, r, chan_idx, scores, s);
    case 8: return launch_g<T, 8>(q, kmin_t, kmax_t, B, Hkv, D, P, pitch, r, chan_idx, scores, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_approx_scores_pitched(const void* q, const void* kmin_t, const void* kmax_t,
                                        int B, int Hq, int Hkv, int D, int P, int pitch, int r,
                                        int dtype, int32_t* chan_idx, float* page_scores,
                                        hipStream_t stream) {
  if (dtype == 0)
    return launch_t<float>(q, kmin_t, kmax_t, B, Hq, Hkv, D, P, pitch, r, chan_idx, page_scores,
                           stream);
  return launch_t<bf16_t>(q, kmin_t, kmax_t, B, Hq, Hkv, D, P, pitch, r, chan_idx, page_scores,
                          stream);
}

hipError_t launch_approx_scores(const void* q, const void* kmin_t, const void* kmax_t, int B,
                                int Hq, int Hkv, int D, int P, int r, int dtype,
                                int32_t* chan_idx, float* page_scores, hipStream_t stream) {
  return launch_approx_scores_pitched(q, kmin_t, kmax_t, B, Hq, Hkv, D, P, P, r, dtype, chan_idx,
                                      page_scores, stream);
}

}  // namespace rkv
