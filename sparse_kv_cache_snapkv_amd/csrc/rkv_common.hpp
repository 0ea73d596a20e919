// Device helpers shared by the RocketKV kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rkv {

constexpr int kWave = 64;

// bfloat16 is carried as its 16-bit pattern.
struct bf16_t {
  uint16_t bits;
};

template <typename T>
struct elem;
template <>
struct elem<float> {
  static constexpr int bytes = 4;
};
template <>
struct elem<bf16_t> {
  static constexpr int bytes = 2;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return bf16_to_f32(x.bits); }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) {
  return x;
}
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  return bf16_t{f32_to_bf16(x)};
}

// 16 bytes of elements, unpacked to float. VEC = 4 (float) or 8 (bf16).
template <typename T>
struct vec16 {
  static constexpr int n = 16 / elem<T>::bytes;
};

template <typename T>
__device__ __forceinline__ void unpack16(const uint4& raw, float (&out)[vec16<T>::n]);

template <>
__device__ __forceinline__ void unpack16<float>(const uint4& raw, float (&out)[4]) {
  out[0] = __uint_as_float(raw.x);
  out[1] = __uint_as_float(raw.y);
  out[2] = __uint_as_float(raw.z);
  out[3] = __uint_as_float(raw.w);
}

template <>
__device__ __forceinline__ void unpack16<bf16_t>(const uint4& raw, float (&out)[8]) {
  out[0] = __uint_as_float(raw.x << 16);
  out[1] = __uint_as_float(raw.x & 0xffff0000u);
  out[2] = __uint_as_float(raw.y << 16);
  out[3] = __uint_as_float(raw.y & 0xffff0000u);
  out[4] = __uint_as_float(raw.z << 16);
  out[5] = __uint_as_float(raw.z & 0xffff0000u);
  out[6] = __uint_as_float(raw.w << 16);
  out[7] = __uint_as_float(raw.w & 0xffff0000u);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Dot product of two 16-byte vectors of bf16 (8 elements) by the gfx950 packed bf16 dot
// instruction, pairs (x, y, z, w) in turn, accumulated in fp32; every bf16 product is exact in
// fp32.
__device__ __forceinline__ float dot8_bf16(const uint4& a, const uint4& b) {
  auto p = [](uint32_t u) { return __builtin_bit_cast(bf16x2_t, u); };
  float d = __builtin_amdgcn_fdot2_f32_bf16(p(a.x), p(b.x), 0.f, false);
  d = __builtin_amdgcn_fdot2_f32_bf16(p(a.y), p(b.y), d, false);
  d = __builtin_amdgcn_fdot2_f32_bf16(p(a.z), p(b.z), d, false);
  return __builtin_amdgcn_fdot2_f32_bf16(p(a.w), p(b.w), d, false);
}

__device__ __forceinline__ uint4 load16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Non-temporal 16-byte load for data read exactly once (K/V rows of the gathered pages).
__device__ __forceinline__ uint4 load16_stream(const void* p) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  uint4 r;
  r.x = __builtin_nontemporal_load(&q->x);
  r.y = __builtin_nontemporal_load(&q->y);
  r.z = __builtin_nontemporal_load(&q->z);
  r.w = __builtin_nontemporal_load(&q->w);
  return r;
}

// Non-temporal 16-byte store, for output written once and not read back by the same launch:
// the channel-major page summaries (their 64-byte row segments run about 22% faster streamed
// out) and the compacted K/V rows of the eviction.
__device__ __forceinline__ void store16_stream(void* p, uint4 v) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  v4u w;
  __builtin_memcpy(&w, &v, 16);
  __builtin_nontemporal_store(w, reinterpret_cast<v4u*>(p));
}

// DPP lane permutations inside a row of 16 lanes (VALU ops, no LDS round trip).
enum : int {
  kDppXor1 = 0xB1,         // quad_perm [1,0,3,2]
  kDppXor2 = 0x4E,         // quad_perm [2,3,0,1]
  kDppHalfMirror = 0x141,  // lane i <- 7-i within each 8 lanes
  kDppMirror = 0x140,      // lane i <- 15-i within each row
  kDppRor8 = 0x128,        // lane i <- (i+8) mod 16 within each row
};

template <int ctrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, false));
}
template <int ctrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, ctrl, 0xF, 0xF, false);
}

// gfx950 row swaps (VALU, no LDS round trip). swap16: every lane gets {v of lane l & ~16,
// v of lane l | 16}; swap32: {v of lane l & ~32, v of lane l | 32}. Both values arrive in the
// same order in every lane, so a reduction step built on them gives the same bits in all lanes.
struct LanePair {
  uint32_t lo, hi;
};
__device__ __forceinline__ LanePair swap16(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return {r[0], r[1]};
}
__device__ __forceinline__ LanePair swap32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return {r[0], r[1]};
}

struct OpSum {
  __device__ float operator()(float a, float b) const { return a + b; }
};
struct OpMax {
  __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct OpMinU {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a < b ? a : b; }
};
struct OpMaxU {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; }
};

template <typename Op>
__device__ __forceinline__ float xor16_step(float v, Op op) {
  const LanePair p = swap16(__float_as_uint(v));
  return op(__uint_as_float(p.lo), __uint_as_float(p.hi));
}
template <typename Op>
__device__ __forceinline__ float xor32_step(float v, Op op) {
  const LanePair p = swap32(__float_as_uint(v));
  return op(__uint_as_float(p.lo), __uint_as_float(p.hi));
}

// Reduction inside groups of `width` consecutive lanes (a power of two <= 64); every lane of the
// group ends with the result.
template <int width, typename Op>
__device__ __forceinline__ float group_reduce(float v, Op op) {
  if constexpr (width >= 2) v = op(v, dpp<kDppXor1>(v));
  if constexpr (width >= 4) v = op(v, dpp<kDppXor2>(v));
  if constexpr (width >= 8) v = op(v, dpp<kDppHalfMirror>(v));
  if constexpr (width >= 16) v = op(v, dpp<kDppMirror>(v));
  if constexpr (width >= 32) v = xor16_step(v, op);
  if constexpr (width >= 64) v = xor32_step(v, op);
  return v;
}
template <int width>
__device__ __forceinline__ float group_sum(float v) {
  return group_reduce<width>(v, OpSum{});
}

// group_sum of N values at once, one reduction level across all of them before the next, so
// that no DPP read waits on the write just before it.
template <int width, int N>
__device__ __forceinline__ void group_sum_n(float (&v)[N]) {
  static_assert(width <= 16, "row-local widths");
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp<kDppXor1>(v[i]);
  if constexpr (width >= 4) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += dpp<kDppXor2>(v[i]);
  }
  if constexpr (width >= 8) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += dpp<kDppHalfMirror>(v[i]);
  }
  if constexpr (width >= 16) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += dpp<kDppMirror>(v[i]);
  }
}
template <int width>
__device__ __forceinline__ float group_max(float v) {
  return group_reduce<width>(v, OpMax{});
}

// Reduction across the lane groups of a wave: lanes l, l+stride, l+2*stride, ... (stride 8, 16,
// 32 or 64) all end with the result.
template <int stride, typename Op>
__device__ __forceinline__ float across_reduce(float v, Op op) {
  static_assert(stride == 8 || stride == 16 || stride == 32 || stride == 64, "stride");
  if constexpr (stride == 8) v = op(v, dpp<kDppRor8>(v));
  if constexpr (stride <= 16) v = xor16_step(v, op);
  if constexpr (stride <= 32) v = xor32_step(v, op);
  return v;
}
template <int stride>
__device__ __forceinline__ float across_sum(float v) {
  return across_reduce<stride>(v, OpSum{});
}
template <int stride>
__device__ __forceinline__ float across_max(float v) {
  return across_reduce<stride>(v, OpMax{});
}

// Whole-wave reduction of a 32-bit unsigned value; every lane ends with the result.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, Op op) {
  v = op(v, dpp_u32<kDppXor1>(v));
  v = op(v, dpp_u32<kDppXor2>(v));
  v = op(v, dpp_u32<kDppHalfMirror>(v));
  v = op(v, dpp_u32<kDppMirror>(v));
  LanePair p = swap16(v);
  v = op(p.lo, p.hi);
  p = swap32(v);
  return op(p.lo, p.hi);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: row shifts build per-row (16 lane)
// sums, then row broadcasts carry row totals into the following rows.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// float -> uint32 key whose unsigned order is the float order; -0.0 maps like +0.0.
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of order_key (the -0.0 -> +0.0 canonicalisation aside).
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Block barrier that orders LDS only. __syncthreads() also waits until every global load and store
// the wave has issued is complete; where a block communicates only through LDS (cross-block data
// moves through tagged device-coherent words, which need no ordering), that wait would put the
// acknowledgement of every earlier global store on the critical path.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

constexpr float kLog2e = 1.4426950408889634f;

// 2^x by the hardware instruction alone (v_exp_f32): results below the smallest normal float
// come out as zero, which the softmax sums and rescaling factors here tolerate, and 2^-inf = 0.
// The library exp2f wraps the same instruction in a rescaling for such results, several times
// the instructions on every element.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace rkv
