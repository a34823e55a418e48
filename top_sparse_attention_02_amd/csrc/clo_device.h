// Device helpers shared by the kernel sources: element access, wave reductions,
// memory-counter waits and unit addressing.  Each kernel source includes this
// header once; everything here has internal linkage.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/clo.h"
#include "clo_internal.h"

namespace clo {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- element access
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ void load8(const uint16_t* p, float (&x)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  x[0] = bf_lo(u.x); x[1] = bf_hi(u.x); x[2] = bf_lo(u.y); x[3] = bf_hi(u.y);
  x[4] = bf_lo(u.z); x[5] = bf_hi(u.z); x[6] = bf_lo(u.w); x[7] = bf_hi(u.w);
}

__device__ __forceinline__ void load2(const float* p, float& a, float& b) {
  const float2 v = *reinterpret_cast<const float2*>(p);
  a = v.x; b = v.y;
}

__device__ __forceinline__ void load2(const uint16_t* p, float& a, float& b) {
  const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
  a = bf_lo(w); b = bf_hi(w);
}

// fp32 -> bf16, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ void store_out(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_out(uint16_t* p, float v) { *p = to_bf16(v); }

// Order-preserving map of an fp32 score to uint32 (larger score -> larger key);
// -0 is folded onto +0 so that equal scores give equal keys.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wait until every vector memory operation this wave issued (loads, stores,
// atomics) has been acknowledged: s_waitcnt vmcnt(0), other counters left at
// their maxima (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
__device__ __forceinline__ void wait_vm_acks() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until this wave's LDS operations have completed: s_waitcnt lgkmcnt(0),
// vmcnt and expcnt left at their maxima (63 and 7).
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Bounded wait of one thread until *flag >= value: at most limit polls with a
// short sleep between them; on time-out CLO_E_TIMEOUT goes to *error_word (when
// not NULL) and the wait ends.  The polls are relaxed device-scope loads (read
// where the writes of every XCD meet); one acquire fence follows the last, so
// that what the flag's writer released before raising it is visible to the
// caller's later reads.  An acquire load per poll would add a cache
// invalidation to every poll of a wait that can last milliseconds beside other
// kernels.
__device__ __forceinline__ void poll_flag(const uint32_t* flag, uint32_t value, uint32_t limit,
                                          uint32_t* error_word) {
  uint32_t n = 0;
  while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < value) {
    if (++n >= limit) {
      if (error_word) __hip_atomic_store(error_word, (uint32_t)CLO_E_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(8);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Sum over the 16 lanes of a row group; the xor butterfly leaves the same
// bits in every lane of the group.
__device__ __forceinline__ float sum16(float x) {
  x += __shfl_xor(x, 8, 16);
  x += __shfl_xor(x, 4, 16);
  x += __shfl_xor(x, 2, 16);
  x += __shfl_xor(x, 1, 16);
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

// A selected index outside [0, N) -- a corrupt caller selection -- is read as
// the nearest row in range (no access leaves the unit's rows) and reported
// once in the caller's error word, the first error staying.
__device__ __forceinline__ int64_t checked_row(int64_t r, int64_t N, uint32_t* err) {
  if (r >= 0 && r < N) return r;
  if (err) atomicCAS(err, 0u, (uint32_t)CLO_E_INDEX);
  return r < 0 ? 0 : N - 1;
}

// Rank of KV head h among the heads of its kind (persistent or not), in head order.
__device__ __forceinline__ int head_slot(uint64_t pmask, int h) {
  const uint64_t below = pmask & ((1ull << h) - 1ull);
  return ((pmask >> h) & 1ull) ? __popcll(below) : h - __popcll(below);
}

template <typename T>
__device__ __forceinline__ const T* unit_keys(const LayerArgs& a, int b, int h) {
  const bool pers = (a.pmask >> h) & 1ull;
  const T* base = static_cast<const T*>(pers ? a.k_hbm : a.k_score);
  const int64_t heads = pers ? a.P : a.H;
  return base + ((int64_t)b * heads + head_slot(a.pmask, h)) * a.C * kHeadDim;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename F>
hipError_t dispatch_group(int G, F&& f) {
  switch (G) {
    case 1: return f(std::integral_constant<int, 1>{});
    case 2: return f(std::integral_constant<int, 2>{});
    case 3: return f(std::integral_constant<int, 3>{});
    case 4: return f(std::integral_constant<int, 4>{});
    case 5: return f(std::integral_constant<int, 5>{});
    case 6: return f(std::integral_constant<int, 6>{});
    case 7: return f(std::integral_constant<int, 7>{});
    case 8: return f(std::integral_constant<int, 8>{});
    default: return hipErrorInvalidValue;
  }
}

inline int grid_cap(int64_t items, int64_t cap) { return (int)(items < cap ? (items > 0 ? items : 1) : cap); }

}  // namespace
}  // namespace clo
