// HIP kernels of the gather (gfx950), A4: the selected K/V rows of offloaded
// heads read by the GPU straight from pinned host memory into the HBM cache,
// per layer or for many layers in one resident launch (CLO abstract, features
// (2) and (3); "CLO (2511.14510) -- L3 Per-Paper Synthesis", section 2.1 item 3).
#include <math.h>

#include <type_traits>

#include "../../include/clo.h"
#include "clo_device.h"
#include "clo_internal.h"

namespace clo {
namespace {

// ---------------------------------------------------------------- A4 gather
// Without a unit list (the standalone gather) every block first lists the units
// it serves -- offloaded heads that miss, ascending -- in LDS, so that the work
// counter runs over their items only instead of handing out (and skipping) the
// items of reuse and persistent units one claim at a time.  Layers of more than
// kGatherListCap units keep the skipping scheme.
constexpr int kGatherListCap = 2048;

__device__ __forceinline__ int list_gather_units(const LayerArgs& a, const uint8_t* __restrict__ reuse, int U,
                                                 int32_t* s_units, uint32_t* s_wcnt) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int total = 0;
  for (int base = 0; base < U; base += 256) {
    const int u = base + (int)threadIdx.x;
    bool f = false;
    if (u < U) f = !((a.pmask >> (u % a.Hkv)) & 1ull) && !(reuse && reuse[u]);
    const uint64_t m = __ballot(f);
    if (lane == 0) s_wcnt[wave] = (uint32_t)__popcll(m);
    __syncthreads();
    int off = total;
    for (int w = 0; w < wave; ++w) off += (int)s_wcnt[w];
    if (f) s_units[off + __popcll(m & ((1ull << lane) - 1ull))] = u;
    total += (int)(s_wcnt[0] + s_wcnt[1] + s_wcnt[2] + s_wcnt[3]);
    __syncthreads();
  }
  return total;
}

// The standalone gather's own wait: thread 0 of every block polls the flag
// (bounded, acquire once it is up), the block waits at a barrier.
__device__ __forceinline__ void gather_wait(const GatherSync& gs) {
  if (!gs.wait_flag) return;
  if (threadIdx.x == 0) poll_flag(gs.wait_flag, gs.wait_value, gs.limit, gs.error_word);
  __syncthreads();
}

// End of a standalone gather: each wave releases its cache rows at agent scope
// (written back past its XCD's L2), then the block counts itself done; the last
// block clears the work counters for the next launch on the workspace and, with
// a signal flag, publishes the layer with a release store.
__device__ __forceinline__ void gather_finish(const GatherSync& gs, uint32_t* counter) {
  if (!gs.done) return;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(gs.done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == gridDim.x - 1) {
      __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(gs.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (gs.signal_flag)
        __hip_atomic_store(gs.signal_flag, gs.signal_value, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Rows of d elements are moved as 16-byte pieces: LPR lanes per row.  The
// loads from pinned host memory are issued UNR rows deep per lane before any
// store; grid x UNR sets the bytes in flight on the host link.
template <typename T>
__device__ __forceinline__ void gather_native_rows(const LayerArgs& a, const uint8_t* __restrict__ reuse, Span sp,
                                                   uint32_t* __restrict__ counter, uint32_t* err) {
  constexpr int RB = kHeadDim * (int)sizeof(T);  // row bytes
  constexpr int LPR = RB / 16;
  constexpr int RPI = 256 / LPR;
  constexpr int UNR = kGatherUnroll;
  static_assert(kGatherChunk == 256, "one index per thread");
  __shared__ uint32_t s_item;
  __shared__ int32_t s_src[kGatherChunk];  // the item's source rows (checked_row)
  __shared__ int32_t s_units[kGatherListCap];
  __shared__ uint32_t s_wcnt[4];
  const int nch = (int)((a.k + kGatherChunk - 1) / kGatherChunk);
  const int lo = sp.list ? *sp.lo : 0;
  const int U = a.B * a.Hkv;
  const bool listed = !sp.list && U <= kGatherListCap;
  const int64_t n_units = sp.list ? (int64_t)(*sp.hi - lo)
                                  : (listed ? (int64_t)list_gather_units(a, reuse, U, s_units, s_wcnt) : (int64_t)U);
  const int64_t items = n_units * nch;
  const int sub = threadIdx.x % LPR, rl = threadIdx.x / LPR;
  for (;;) {
    if (threadIdx.x == 0) s_item = atomicAdd(counter, 1u);
    __syncthreads();
    const int64_t it = s_item;
    __syncthreads();
    if (it >= items) break;  // uniform per block
    const int u = sp.list ? sp.list[lo + it / nch] : (listed ? s_units[it / nch] : (int)(it / nch));
    const int c = (int)(it % nch);
    const int b = u / a.Hkv, h = u % a.Hkv;
    if (!sp.list && !listed && (((a.pmask >> h) & 1ull) || (reuse && reuse[u]))) continue;
    const int64_t slot = (int64_t)b * a.H + head_slot(a.pmask, h);
    const char* ks = static_cast<const char*>(a.k_host) + slot * a.C * RB;
    const char* vs = static_cast<const char*>(a.v_host) + slot * a.C * RB;
    char* kd = static_cast<char*>(a.k_cache) + slot * a.k * RB;
    char* vd = static_cast<char*>(a.v_cache) + slot * a.k * RB;
    const int32_t* ix = a.idx + (int64_t)u * a.k;
    const int64_t r0 = (int64_t)c * kGatherChunk;
    const int64_t r_end = (r0 + kGatherChunk < a.k) ? r0 + kGatherChunk : a.k;
    // the item's indices in one coalesced load, so that the host reads below
    // do not wait on an index load each time
    if (r0 + threadIdx.x < r_end) s_src[threadIdx.x] = (int32_t)checked_row(ix[r0 + threadIdx.x], a.N, err);
    __syncthreads();
    for (int64_t rb = r0; rb < r_end; rb += RPI * UNR) {
      // rows past the end re-read the last row (in bounds) and are not stored
      u32x4 kx[UNR], vx[UNR];
#pragma unroll
      for (int j = 0; j < UNR; ++j) {
        int64_t row = rb + j * RPI + rl;
        row = row < r_end ? row : r_end - 1;
        const int64_t src = s_src[row - r0];
        kx[j] = *reinterpret_cast<const u32x4*>(ks + src * RB + sub * 16);
        vx[j] = *reinterpret_cast<const u32x4*>(vs + src * RB + sub * 16);
      }
#pragma unroll
      for (int j = 0; j < UNR; ++j) {
        const int64_t row = rb + j * RPI + rl;
        if (row < r_end) {
          *reinterpret_cast<u32x4*>(kd + row * RB + sub * 16) = kx[j];
          *reinterpret_cast<u32x4*>(vd + row * RB + sub * 16) = vx[j];
        }
      }
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void gather_kernel(LayerArgs a, const uint8_t* __restrict__ reuse, Span sp,
                                                     uint32_t* __restrict__ counter, GatherSync gs) {
  gather_wait(gs);
  gather_native_rows<T>(a, reuse, sp, counter, a.err);
  gather_finish(gs, counter);
}

// Quantized host rows (CLO_HOST_INT8: 128 bytes per row; CLO_HOST_INT4: 64),
// read as 16-byte pieces of 16 or 32 values; the row's exponent e (device
// memory) turns q into q * 2^e, exact in T.  The rest is the native kernel's
// scheme: items of 256 rows from a counter, the item's source rows and
// exponents preloaded into LDS, several rows of K and V deep per lane.
__device__ __forceinline__ float pow2f(int e) { return __int_as_float((e + 127) << 23); }  // -126 <= e <= 127

// q of element n of a 16-byte piece: a signed byte (8-bit) or a signed nibble,
// value 2j in the low half of byte j (4-bit)
template <int BITS>
__device__ __forceinline__ float quant_at(const u32x4& w, int n) {
  const uint32_t x = w[n * BITS / 32];
  const int sh = (n * BITS) % 32;
  return (float)(((int32_t)(x << (32 - BITS - sh))) >> (32 - BITS));
}

// 16 * 8 / BITS values of one piece, times 2^e, stored as T; the products have at
// most 7 significant bits, so the bf16 pattern is the fp32 one's upper half
template <typename T, int BITS>
__device__ __forceinline__ void store_deq(T* dst, const u32x4& w, float scale) {
  constexpr int NV = 128 / BITS;  // values per piece
  if constexpr (std::is_same<T, uint16_t>::value) {
#pragma unroll
    for (int o = 0; o < NV / 8; ++o) {
      u32x4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float f0 = quant_at<BITS>(w, o * 8 + 2 * i) * scale, f1 = quant_at<BITS>(w, o * 8 + 2 * i + 1) * scale;
        r[i] = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xFFFF0000u);
      }
      reinterpret_cast<u32x4*>(dst)[o] = r;
    }
  } else {
#pragma unroll
    for (int o = 0; o < NV / 4; ++o) {
      u32x4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(quant_at<BITS>(w, o * 4 + i) * scale);
      reinterpret_cast<u32x4*>(dst)[o] = r;
    }
  }
}

template <typename T, int BITS>
__device__ __forceinline__ void gather_quant_rows(const LayerArgs& a, const uint8_t* __restrict__ reuse, Span sp,
                                                  uint32_t* __restrict__ counter, uint32_t* err) {
  // one record per token (K values, then V values): the first half of a row
  // group's lanes read its K values, the second half its V values, in a
  // single load of 16 (8-bit) or 8 (4-bit) lanes
  constexpr int kRec = 2 * kHeadDim * BITS / 8;  // record bytes
  constexpr int LPR = kRec / 16;                 // lanes per token
  constexpr int LPH = LPR / 2;                   // lanes per row
  constexpr int NV = 128 / BITS;                 // values per lane
  constexpr int RPI = 256 / LPR;
  constexpr int UNR = 2 * kGatherUnroll;  // 16-byte loads in flight per lane
  __shared__ uint32_t s_item;
  __shared__ int32_t s_src[kGatherChunk];
  __shared__ float s_sc[2][kGatherChunk];  // 2^e of the item's K and V rows
  __shared__ int32_t s_units[kGatherListCap];
  __shared__ uint32_t s_wcnt[4];
  const int nch = (int)((a.k + kGatherChunk - 1) / kGatherChunk);
  const int lo = sp.list ? *sp.lo : 0;
  const int U = a.B * a.Hkv;
  const bool listed = !sp.list && U <= kGatherListCap;
  const int64_t n_units = sp.list ? (int64_t)(*sp.hi - lo)
                                  : (listed ? (int64_t)list_gather_units(a, reuse, U, s_units, s_wcnt) : (int64_t)U);
  const int64_t items = n_units * nch;
  const int sub = threadIdx.x % LPR, rl = threadIdx.x / LPR;
  const int half = sub / LPH, piece = sub % LPH;  // 0 = K, 1 = V; piece of the row
  for (;;) {
    if (threadIdx.x == 0) s_item = atomicAdd(counter, 1u);
    __syncthreads();
    const int64_t it = s_item;
    __syncthreads();
    if (it >= items) break;  // uniform per block
    const int u = sp.list ? sp.list[lo + it / nch] : (listed ? s_units[it / nch] : (int)(it / nch));
    const int c = (int)(it % nch);
    const int b = u / a.Hkv, h = u % a.Hkv;
    if (!sp.list && !listed && (((a.pmask >> h) & 1ull) || (reuse && reuse[u]))) continue;
    const int64_t slot = (int64_t)b * a.H + head_slot(a.pmask, h);
    const char* rec = static_cast<const char*>(a.k_host) + slot * a.C * kRec;
    T* dst = static_cast<T*>(half ? a.v_cache : a.k_cache) + slot * a.k * kHeadDim;
    const int32_t* ix = a.idx + (int64_t)u * a.k;
    const int64_t r0 = (int64_t)c * kGatherChunk;
    const int64_t r_end = (r0 + kGatherChunk < a.k) ? r0 + kGatherChunk : a.k;
    if (r0 + threadIdx.x < r_end) {
      const int32_t src = (int32_t)checked_row(ix[r0 + threadIdx.x], a.N, err);
      s_src[threadIdx.x] = src;
      s_sc[0][threadIdx.x] = pow2f(a.k_exp[slot * a.C + src]);
      s_sc[1][threadIdx.x] = pow2f(a.v_exp[slot * a.C + src]);
    }
    __syncthreads();
    for (int64_t rb = r0; rb < r_end; rb += RPI * UNR) {
      u32x4 x[UNR];
#pragma unroll
      for (int j = 0; j < UNR; ++j) {
        int64_t row = rb + j * RPI + rl;
        row = row < r_end ? row : r_end - 1;
        x[j] = *reinterpret_cast<const u32x4*>(rec + (int64_t)s_src[row - r0] * kRec + sub * 16);
      }
#pragma unroll
      for (int j = 0; j < UNR; ++j) {
        const int64_t row = rb + j * RPI + rl;
        if (row < r_end) store_deq<T, BITS>(dst + row * kHeadDim + piece * NV, x[j], s_sc[half][row - r0]);
      }
    }
  }
}

template <typename T, int BITS>
__global__ __launch_bounds__(256) void gather_quant_kernel(LayerArgs a, const uint8_t* __restrict__ reuse, Span sp,
                                                           uint32_t* __restrict__ counter, GatherSync gs) {
  gather_wait(gs);
  gather_quant_rows<T, BITS>(a, reuse, sp, counter, a.err);
  gather_finish(gs, counter);
}

// One layer's rows in the layer's host format and dtype.
__device__ __forceinline__ void gather_rows_any(const LayerArgs& a, const uint8_t* __restrict__ reuse,
                                                uint32_t* __restrict__ counter, uint32_t* err) {
  const Span all{nullptr, nullptr, nullptr};
  const bool f32 = a.dtype == CLO_F32;
  if (a.host_fmt == CLO_HOST_INT8) {
    if (f32)
      gather_quant_rows<float, 8>(a, reuse, all, counter, err);
    else
      gather_quant_rows<uint16_t, 8>(a, reuse, all, counter, err);
  } else if (a.host_fmt == CLO_HOST_INT4) {
    if (f32)
      gather_quant_rows<float, 4>(a, reuse, all, counter, err);
    else
      gather_quant_rows<uint16_t, 4>(a, reuse, all, counter, err);
  } else if (f32) {
    gather_native_rows<float>(a, reuse, all, counter, err);
  } else {
    gather_native_rows<uint16_t>(a, reuse, all, counter, err);
  }
}

// The gathers of many layers in one launch (a resident kernel).  Layer by
// layer the blocks wait for the layer's selection flag, take its items from the
// layer's work counter, and count themselves done; the last block of a layer
// clears its counters and publishes the layer.  A block that runs out of a
// layer's items goes straight on to the next layer, so the layers' tails
// overlap and no launch separates them.
__global__ __launch_bounds__(256) void gather_layers_kernel(const GatherPlanLayer* __restrict__ plan, int n_layers,
                                                            uint32_t wait_value, uint32_t signal_value,
                                                            uint32_t limit, uint32_t* err) {
  for (int l = 0; l < n_layers; ++l) {
    const GatherPlanLayer& g = plan[l];
    const GatherSync gs{g.wait_flag, wait_value, limit, err, g.signal_flag, signal_value, g.done};
    gather_wait(gs);
    gather_rows_any(g.a, g.reuse, g.counter, err);
    gather_finish(gs, g.counter);
    __syncthreads();  // the next layer reuses the block's LDS
  }
}

// The host gathers of one decode step's unit ranges in one resident launch
// (BITS = 0: native rows).  Range by range the blocks wait until the range's
// top-k is done, take the range's items from its work counter and count
// themselves done; the last block of a range publishes it for attention.  A
// block that runs out of a range's items goes straight on to the next range,
// so that no launch gap or tail of one range leaves the host link idle.
template <typename T, int BITS>
__global__ __launch_bounds__(256) void gather_ranges_kernel(LayerArgs a, int32_t* __restrict__ meta,
                                                            const int32_t* __restrict__ list_host, int R,
                                                            uint32_t limit) {
  uint32_t* m = reinterpret_cast<uint32_t*>(meta);
  for (int r = 0; r < R; ++r) {
    const GatherSync gs{m + kMetaSelFlag + r, 1u, limit, a.err, m + kMetaGatherFlag + r, 1u, m + kMetaRangeDone + r};
    gather_wait(gs);
    const Span sp{list_host, meta + kMetaOffHost + r, meta + kMetaOffHost + r + 1};
    if constexpr (BITS == 0)
      gather_native_rows<T>(a, nullptr, sp, m + kMetaGather + r, a.err);
    else
      gather_quant_rows<T, BITS>(a, nullptr, sp, m + kMetaGather + r, a.err);
    gather_finish(gs, m + kMetaGather + r);
    __syncthreads();  // the next range reuses the block's LDS
  }
}

}  // namespace

hipError_t launch_gather_ranges(const LayerArgs& a, const Workspace& w, int ranges, int blocks, uint32_t limit,
                                hipStream_t s) {
  const bool f32 = a.dtype == CLO_F32;
  if (a.host_fmt == CLO_HOST_INT8) {
    if (f32)
      gather_ranges_kernel<float, 8><<<blocks, 256, 0, s>>>(a, w.meta, w.list_host, ranges, limit);
    else
      gather_ranges_kernel<uint16_t, 8><<<blocks, 256, 0, s>>>(a, w.meta, w.list_host, ranges, limit);
  } else if (a.host_fmt == CLO_HOST_INT4) {
    if (f32)
      gather_ranges_kernel<float, 4><<<blocks, 256, 0, s>>>(a, w.meta, w.list_host, ranges, limit);
    else
      gather_ranges_kernel<uint16_t, 4><<<blocks, 256, 0, s>>>(a, w.meta, w.list_host, ranges, limit);
  } else if (f32) {
    gather_ranges_kernel<float, 0><<<blocks, 256, 0, s>>>(a, w.meta, w.list_host, ranges, limit);
  } else {
    gather_ranges_kernel<uint16_t, 0><<<blocks, 256, 0, s>>>(a, w.meta, w.list_host, ranges, limit);
  }
  return hipGetLastError();
}

hipError_t launch_gather(const LayerArgs& a, const uint8_t* reuse, Span sp, int64_t max_units, int max_blocks,
                         uint32_t* counter, hipStream_t s, const GatherSync* gsp) {
  const int64_t nch = (a.k + kGatherChunk - 1) / kGatherChunk;
  // with its own wait the grid is fixed (every block arrives at the done count);
  // otherwise it shrinks to the work when that is smaller
  const int grid = gsp && gsp->wait_flag ? max_blocks : grid_cap(max_units * nch, (int64_t)max_blocks);
  GatherSync gs{};
  if (gsp) gs = *gsp;
  if (a.host_fmt == CLO_HOST_INT8) {
    if (a.dtype == CLO_F32)
      gather_quant_kernel<float, 8><<<grid, 256, 0, s>>>(a, reuse, sp, counter, gs);
    else
      gather_quant_kernel<uint16_t, 8><<<grid, 256, 0, s>>>(a, reuse, sp, counter, gs);
  } else if (a.host_fmt == CLO_HOST_INT4) {
    if (a.dtype == CLO_F32)
      gather_quant_kernel<float, 4><<<grid, 256, 0, s>>>(a, reuse, sp, counter, gs);
    else
      gather_quant_kernel<uint16_t, 4><<<grid, 256, 0, s>>>(a, reuse, sp, counter, gs);
  } else if (a.dtype == CLO_F32) {
    gather_kernel<float><<<grid, 256, 0, s>>>(a, reuse, sp, counter, gs);
  } else {
    gather_kernel<uint16_t><<<grid, 256, 0, s>>>(a, reuse, sp, counter, gs);
  }
  return hipGetLastError();
}

hipError_t launch_gather_layers(const GatherPlanLayer* plan, int n_layers, int blocks, uint32_t wait_value,
                                uint32_t signal_value, uint32_t limit, uint32_t* error_word, hipStream_t s) {
  gather_layers_kernel<<<blocks, 256, 0, s>>>(plan, n_layers, wait_value, signal_value, limit, error_word);
  return hipGetLastError();
}

}  // namespace clo
