// Host side of the fused decode step (rkv_step.hpp): plan, workspace layout, launch, and the
// workspace's initialisation and status word.
#include <stdlib.h>

#include <algorithm>
#include <mutex>

#include "rkv_launch.hpp"
#include "rkv_step.hpp"

namespace rkv {

namespace {

// A waiting block does the missing work itself after this many microseconds; the environment
// variable RKV_STEAL_US overrides it (0: after one look; negative: every waiting block redoes all
// the work it waits for, which tests use to run the stealing paths on every call).
constexpr int kStealMicroseconds = 20;
constexpr int kWaitMicroseconds = 1000;  // bound of a wait for words already on their way

__global__ void k_zero_u32(unsigned* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// Steady-counter ticks per microsecond on the current device (the counter's rate is a device
// attribute, in kHz).
long long ticks_per_us() {
  static long long cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cache[dev] == 0) {
    int khz = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz < 1)
      khz = 100000;  // 100 MHz
    cache[dev] = std::max<long long>(1, khz / 1000);
  }
  return cache[dev];
}

}  // namespace

size_t decode_ws_bytes(int B, int Hq, int Hkv, int Lc, int D, int page_size, int, int) {
  const int P = (Lc + page_size - 1) / page_size;
  return step::layout(B, Hq, Hkv, D, P).total;
}

hipError_t launch_decode_ws_init(void* ws, size_t bytes, hipStream_t stream) {
  const size_t n = bytes / sizeof(unsigned);
  const int blocks = (int)std::min<size_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(k_zero_u32, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, stream,
                     static_cast<unsigned*>(ws), n);
  return hipGetLastError();
}

hipError_t read_decode_status(void* ws, int clear, uint32_t* status, hipStream_t stream) {
  hipError_t e = hipMemcpyAsync(status, ws, sizeof(uint32_t), hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return e;
  if (clear) {
    hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(64), 0, stream, static_cast<unsigned*>(ws),
                       (size_t)1);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipStreamSynchronize(stream);
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
  const step::Layout lo = step::layout(B, Hq, Hkv, D, Pcap);
  char* w = static_cast<char*>(ws);
  if (lo.pipe) {
    float* sc = page_scores != nullptr ? page_scores : reinterpret_cast<float*>(w + lo.off_pscores);
    int32_t* pg = page_idx != nullptr ? page_idx : reinterpret_cast<int32_t*>(w + lo.off_ppages);
    if (attend_ws_bytes(B, Hq, Hkv, D, page_size, n_pages, dtype) > lo.total - lo.off_ppart)
      return hipErrorInvalidValue;  // cannot happen: the layout holds the largest split
    hipError_t e = launch_approx_scores_pitched(q, kmin_t, kmax_t, B, Hq, Hkv, D, P, Pcap, r,
                                                dtype, chan_idx, sc, stream);
    if (e != hipSuccess) return e;
    e = launch_topk(sc, BH, P, n_pages, pg, n_pages, nullptr, stream);
    if (e != hipSuccess) return e;
    return launch_sparse_attend_view(q, k_c, v_c, rows, pg, B, Hq, Hkv, Lc, kv_pitch, D,
                                     page_size, n_pages, scale, dtype, out, w + lo.off_ppart,
                                     stream);
  }
  const int vmax = dtype == 0 ? vec16<float>::n : vec16<bf16_t>::n;
  const step::Plan pl = step::plan(BH, P, page_size, n_pages, device_cus(), vmax);
  if (pl.nb > 1 && (pl.ns > step::kMaxScorers || pl.na > lo.cap_a))
    return hipErrorInvalidValue;  // cannot happen: the layout holds the largest plan
  step::Args a{};
  a.q = q;
  a.kmin_t = kmin_t;
  a.kmax_t = kmax_t;
  a.k_c = k_c;
  a.v_c = v_c;
  a.BH = BH;
  a.Hkv = Hkv;
  a.Lc = Lc;
  a.ps = page_size;
  a.n_pages = n_pages;
  a.P = P;
  a.r = r;
  a.ns = pl.ns;
  a.na = pl.na;
  a.nb = pl.nb;
  a.ppb1 = pl.ppb1;
  a.pps = pl.pps;
  a.vec = Pcap % vmax == 0;
  a.cap_a = lo.cap_a;
  a.kv_pitch = kv_pitch;
  a.rows = rows;
  a.s_pitch = Pcap;
  // blocks y * BH + x of head x share an XCD exactly when BH is a multiple of the XCD count
  a.xcd_local = BH % step::kXcds == 0 ? 1 : 0;
  // Blocks that only score touch their share's best pages ahead of the attention where the budget
  // is small (its first loads are then on the critical path) and the lines land in the L2 that
  // the attenders read.
  a.pf = pl.nb > 1 && a.xcd_local && n_pages < P && n_pages * page_size <= step::kPrefetchTokens &&
                 pl.ppb1 <= step::kPrefetchShare
             ? std::min(step::kPrefetchPages, 2 * ((n_pages + pl.ns - 1) / pl.ns))
             : 0;
  a.scale2 = scale * kLog2e;
  const char* steal_env = getenv("RKV_STEAL_US");
  const long long steal_us = steal_env != nullptr ? atol(steal_env) : kStealMicroseconds;
  a.steal_ticks = steal_us < 0 ? -1 : ticks_per_us() * steal_us;
  a.wait_ticks = ticks_per_us() * kWaitMicroseconds;
  a.chan_idx = chan_idx;
  a.page_scores = page_scores;
  a.page_idx = page_idx;
  a.xscores = reinterpret_cast<uint64_t*>(w + lo.off_xscores);
  a.xpart = reinterpret_cast<uint64_t*>(w + lo.off_xpart);
  a.sync = reinterpret_cast<unsigned*>(w + lo.off_sync);
  a.out = out;
  const int G = Hq / Hkv;
  return dtype == 0 ? step_launch_f32(D, G, a, stream) : step_launch_bf16(D, G, a, stream);
}

// ---------------------------------------------------------------------------------------------
// Allocation-free variant. The scratch below stands in for the workspace; each device holds its
// own copy from the library's load until the process ends. Host code never uses the array's name
// as an address: the device address comes from hipGetSymbolAddress, once per device.

namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// What fixes the workspace layout and the heads whose call counters advance together; a call
// whose key differs from the previous call's on the device starts from a cleared scratch.
struct ScratchKey {
  int BH = 0, G = 0, D = 0, Pcap = 0, dtype = -1;
  bool operator==(const ScratchKey& o) const {
    return BH == o.BH && G == o.G && D == o.D && Pcap == o.Pcap && dtype == o.dtype;
  }
};

struct ScratchSlot {
  void* ptr = nullptr;  // device address of this device's copy of `scratch`
  bool used = false;
  ScratchKey key;
};

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
ScratchSlot g_scratch[kMaxDevices];

__global__ void k_take_status(unsigned* word, uint32_t* status) {
  if (threadIdx.x == 0) {
    *status = *word;
    *word = 0u;
  }
}

}  // namespace

hipError_t launch_decode_step_noalloc(const void* q, const void* kmin_t, const void* kmax_t,
                                      const void* k_c, const void* v_c, int B, int Hq, int Hkv,
                                      int Lc, int D, int page_size, int r, int n_pages,
                                      float scale, int dtype, int32_t* chan_idx,
                                      float* page_scores, int32_t* page_idx, void* out,
                                      uint32_t* status, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  const int P = (Lc + page_size - 1) / page_size;
  const size_t need = step::layout(B, Hq, Hkv, D, P).total;
  if (need > kNoAllocScratchBytes) return hipErrorInvalidValue;  // the caller checks first
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchSlot& slot = g_scratch[dev];
  if (slot.ptr == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    slot.ptr = ptr;
  }
  const ScratchKey key{B * Hkv, Hq / Hkv, D, P, dtype};
  if (!slot.used || !(slot.key == key)) {
    // counters, status word and every tagged word start from zero for a new layout
    e = launch_decode_ws_init(slot.ptr, need, stream);
    if (e != hipSuccess) return e;
    slot.used = true;
    slot.key = key;
  }
  e = launch_decode_step(q, kmin_t, kmax_t, k_c, v_c, nullptr, B, Hq, Hkv, Lc, Lc, Lc, D,
                         page_size, r, n_pages, scale, dtype, chan_idx, page_scores, page_idx, out,
                         slot.ptr, stream);
  if (e != hipSuccess) return e;
  if (status != nullptr) {
    hipLaunchKernelGGL(k_take_status, dim3(1), dim3(64), 0, stream,
                       static_cast<unsigned*>(slot.ptr), status);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace rkv
