// HIP kernels of the CLO decode step for gfx950 (MI355X) outside the five steps'
// own sources: quantization of rows for the quantized host copies, appending a decoded
// token (growing context), reference queries, the device-side wait and signal
// kernels that order work between streams, the HBM read probe, and the static
// scratch of clo_decode_step_static.  The steps themselves: clo_select.hip (A1
// reuse test, A2 scoring, A3 top-k), clo_gather.hip (A4), clo_attn.hip (A5).
//
// Element types: float (fp32) and uint16_t holding bf16 bit patterns.  All
// arithmetic is fp32.
#include <math.h>

#include <mutex>
#include <type_traits>

#include "../../include/clo.h"
#include "clo_device.h"
#include "clo_internal.h"

namespace clo {

// Workspace of clo_decode_step_static, for callers that cannot allocate.  In
// host code this name stands for the array and is no device address: the host
// side uses only the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

namespace {

// ---------------------------------------------------------------- quantization
// Row quantization of the quantized host formats by one wave: lane l holds
// elements 2l and 2l+1.  With M = 127 (8-bit values) or 7 (4-bit): m = max|x|;
// e = the smallest integer with m <= M * 2^e (0 for a zero row), at least
// kQuantMinExp; q = x * 2^-e rounded to nearest even.
template <int BITS>
__device__ __forceinline__ int quant_exponent(float m) {
  constexpr float M = BITS == 8 ? 127.f : 7.f;
  constexpr int F = BITS == 8 ? 6 : 2;  // 2^F <= M < 2^(F+1)
  if (m == 0.f) return 0;
  int E;
  frexpf(m, &E);  // m = f * 2^E, 0.5 <= f < 1
  int e = E - 1 - F;
  if (m > ldexpf(M, e)) e += 1;
  return e < kQuantMinExp ? kQuantMinExp : e;
}

__device__ __forceinline__ void quant_pair(float x0, float x1, int e, int& q0, int& q1) {
  const float inv = ldexpf(1.f, -e);  // exact power of two
  q0 = (int)rintf(x0 * inv);
  q1 = (int)rintf(x1 * inv);
}

template <typename T>
__device__ __forceinline__ void load_pair(const T* row, int lane, float& x0, float& x1);
template <>
__device__ __forceinline__ void load_pair<uint16_t>(const uint16_t* row, int lane, float& x0, float& x1) {
  const uint32_t w = reinterpret_cast<const uint32_t*>(row)[lane];
  x0 = bf_lo(w);
  x1 = bf_hi(w);
}
template <>
__device__ __forceinline__ void load_pair<float>(const float* row, int lane, float& x0, float& x1) {
  const float2 v = reinterpret_cast<const float2*>(row)[lane];
  x0 = v.x;
  x1 = v.y;
}

// Quantizes one row held by a wave and stores its values (8-bit: 2 bytes per
// lane; 4-bit: 1 byte, value 2l in the low half) plus the exponent.
template <typename T, int BITS>
__device__ __forceinline__ void quantize_row_wave(const T* row, uint8_t* dst, int8_t* dst_exp) {
  const int lane = threadIdx.x & 63;
  float x0, x1;
  load_pair<T>(row, lane, x0, x1);
  const float m = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
  const int e = quant_exponent<BITS>(m);
  int q0, q1;
  quant_pair(x0, x1, e, q0, q1);
  if (BITS == 8)
    reinterpret_cast<uint16_t*>(dst)[lane] = (uint16_t)((uint32_t)(q0 & 0xFF) | ((uint32_t)(q1 & 0xFF) << 8));
  else
    dst[lane] = (uint8_t)((q0 & 0xF) | ((q1 & 0xF) << 4));
  if (lane == 0) *dst_exp = (int8_t)e;
}

template <typename T, int BITS>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const T* __restrict__ src, int64_t n_rows, uint8_t* dst,
                                                            int64_t stride, int8_t* __restrict__ dst_exp) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n_rows) return;  // whole wave
  quantize_row_wave<T, BITS>(src + row * kHeadDim, dst + row * stride, dst_exp + row);
}

__global__ void zero_kernel(uint32_t* word, uint32_t* word2) {
  if (threadIdx.x == 0) {
    *word = 0u;
    if (word2) *word2 = 0u;
  }
}

// ---------------------------------------------------------------- growing context
// Row `position` of every (sequence, KV head) from k_new / v_new [B, Hkv, d]:
// one 64-lane wave per unit, 16-byte pieces (bf16: 16 lanes per row; fp32: 32).
// Offloaded heads' rows are stored by the GPU straight into pinned host memory
// and into the HBM score copy.
template <typename T>
__global__ __launch_bounds__(64) void append_kernel(LayerArgs a, const T* __restrict__ k_new,
                                                   const T* __restrict__ v_new, int64_t position, T* k_hbm,
                                                   T* v_hbm, T* k_host, T* v_host, T* k_score) {
  constexpr int kPieces = kHeadDim * (int)sizeof(T) / 16;  // 16-byte pieces per row
  const int u = blockIdx.x;
  const int b = u / a.Hkv, h = u % a.Hkv;
  const bool pers = (a.pmask >> h) & 1ull;
  const int64_t rows = pers ? a.P : a.H;
  const int64_t dst = (((int64_t)b * rows + head_slot(a.pmask, h)) * a.C + position) * kHeadDim;
  const int64_t src = (int64_t)u * kHeadDim;
  if (!pers && a.host_fmt != CLO_HOST_NATIVE) {
    // the quantized host copy gets the quantized row, the score copy the exact one
    const int64_t er = dst / kHeadDim;  // the token's row index
    const int64_t rb = quant_row_bytes(a.host_fmt);
    uint8_t* record = reinterpret_cast<uint8_t*>(k_host) + er * 2 * rb;  // K values, then V values
    int8_t* ke = const_cast<int8_t*>(a.k_exp) + er;
    int8_t* ve = const_cast<int8_t*>(a.v_exp) + er;
    if (a.host_fmt == CLO_HOST_INT8) {
      quantize_row_wave<T, 8>(k_new + src, record, ke);
      quantize_row_wave<T, 8>(v_new + src, record + rb, ve);
    } else {
      quantize_row_wave<T, 4>(k_new + src, record, ke);
      quantize_row_wave<T, 4>(v_new + src, record + rb, ve);
    }
    for (int i = threadIdx.x; i < kPieces; i += 64)
      reinterpret_cast<u32x4*>(k_score + dst)[i] = reinterpret_cast<const u32x4*>(k_new + src)[i];
    return;
  }
  for (int i = threadIdx.x; i < kPieces; i += 64) {
    const u32x4 kv = reinterpret_cast<const u32x4*>(k_new + src)[i];
    const u32x4 vv = reinterpret_cast<const u32x4*>(v_new + src)[i];
    if (pers) {
      reinterpret_cast<u32x4*>(k_hbm + dst)[i] = kv;
      reinterpret_cast<u32x4*>(v_hbm + dst)[i] = vv;
    } else {
      reinterpret_cast<u32x4*>(k_host + dst)[i] = kv;
      reinterpret_cast<u32x4*>(v_host + dst)[i] = vv;
      reinterpret_cast<u32x4*>(k_score + dst)[i] = kv;
    }
  }
}

// q_ref[unit] = q[unit] for every miss unit (the unit's g heads, contiguous).
template <typename T>
__global__ __launch_bounds__(64) void update_reference_kernel(const T* __restrict__ q,
                                                              const uint8_t* __restrict__ reuse, T* q_ref,
                                                              int G) {
  const int u = blockIdx.x;
  if (reuse && reuse[u]) return;
  const int64_t n = (int64_t)G * kHeadDim * (int)sizeof(T) / 16;  // 16-byte pieces of the unit
  const u32x4* src = reinterpret_cast<const u32x4*>(q + (int64_t)u * G * kHeadDim);
  u32x4* dst = reinterpret_cast<u32x4*>(q_ref + (int64_t)u * G * kHeadDim);
  for (int64_t i = threadIdx.x; i < n; i += 64) dst[i] = src[i];
}

// ---------------------------------------------------------------- device-side flags
// zero_word (may be NULL): a work counter of the kernel that follows on the
// stream, cleared here so that the wait and the reset take one launch
__global__ __launch_bounds__(64) void wait_kernel(const uint32_t* flag, uint32_t value, uint32_t limit,
                                                  uint32_t* error_word, uint32_t* zero_word) {
  if (threadIdx.x != 0) return;
  poll_flag(flag, value, limit, error_word);
  if (zero_word) *zero_word = 0u;
}

// flag[0 .. n) = value (release), one lane per flag (n <= 64)
__global__ __launch_bounds__(64) void signal_kernel(uint32_t* flag, uint32_t value, int n) {
  if ((int)threadIdx.x < n) __hip_atomic_store(flag + threadIdx.x, value, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}


// ---------------------------------------------------------------- measurement
// Streaming read of n16 16-byte words: the HBM read ceiling that the scoring
// and attention kernels are compared with.  Each thread keeps 8 loads in
// flight; the xor of everything read is stored only if it equals `never`, so
// the loads cannot be dropped and almost nothing is written.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, int64_t n16, uint32_t never,
                                                          uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t x = 0;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = p[i + j * stride];
#pragma unroll
    for (int j = 0; j < 8; ++j) x ^= w[j][0] ^ w[j][1] ^ w[j][2] ^ w[j][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 w = p[i];
    x ^= w[0] ^ w[1] ^ w[2] ^ w[3];
  }
  if (x == never) sink[0] = x;
}

}  // namespace

hipError_t launch_quantize_rows(const void* src, int64_t n_rows, int32_t dtype, int32_t host_fmt, uint8_t* dst,
                                int64_t stride, int8_t* dst_exp, hipStream_t s) {
  const int64_t blocks = (n_rows + 3) / 4;
  if (blocks <= 0) return hipSuccess;
  const unsigned grid = (unsigned)blocks;
  const float* sf = static_cast<const float*>(src);
  const uint16_t* sb = static_cast<const uint16_t*>(src);
  if (host_fmt == CLO_HOST_INT8) {
    if (dtype == CLO_F32)
      quantize_rows_kernel<float, 8><<<grid, 256, 0, s>>>(sf, n_rows, dst, stride, dst_exp);
    else
      quantize_rows_kernel<uint16_t, 8><<<grid, 256, 0, s>>>(sb, n_rows, dst, stride, dst_exp);
  } else {
    if (dtype == CLO_F32)
      quantize_rows_kernel<float, 4><<<grid, 256, 0, s>>>(sf, n_rows, dst, stride, dst_exp);
    else
      quantize_rows_kernel<uint16_t, 4><<<grid, 256, 0, s>>>(sb, n_rows, dst, stride, dst_exp);
  }
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, int64_t n16, int blocks, uint32_t* sink, hipStream_t s) {
  stream_read_kernel<<<blocks, 256, 0, s>>>(static_cast<const u32x4*>(src), n16, 0x9E3779B9u, sink);
  return hipGetLastError();
}

hipError_t launch_zero(uint32_t* word, hipStream_t s, uint32_t* word2) {
  zero_kernel<<<1, 64, 0, s>>>(word, word2);
  return hipGetLastError();
}

hipError_t launch_append(const LayerArgs& a, const void* k_new, const void* v_new, int64_t position,
                         void* k_hbm, void* v_hbm, void* k_host, void* v_host, void* k_score, hipStream_t s) {
  const unsigned grid = (unsigned)((int64_t)a.B * a.Hkv);
  if (a.dtype == CLO_F32)
    append_kernel<float><<<grid, 64, 0, s>>>(a, static_cast<const float*>(k_new), static_cast<const float*>(v_new),
                                             position, static_cast<float*>(k_hbm), static_cast<float*>(v_hbm),
                                             static_cast<float*>(k_host), static_cast<float*>(v_host),
                                             static_cast<float*>(k_score));
  else
    append_kernel<uint16_t><<<grid, 64, 0, s>>>(
        a, static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), position,
        static_cast<uint16_t*>(k_hbm), static_cast<uint16_t*>(v_hbm), static_cast<uint16_t*>(k_host),
        static_cast<uint16_t*>(v_host), static_cast<uint16_t*>(k_score));
  return hipGetLastError();
}

hipError_t launch_update_reference(const LayerArgs& a, const void* q, const uint8_t* reuse, void* q_ref,
                                   hipStream_t s) {
  const unsigned grid = (unsigned)((int64_t)a.B * a.Hkv);
  if (a.dtype == CLO_F32)
    update_reference_kernel<float><<<grid, 64, 0, s>>>(static_cast<const float*>(q), reuse,
                                                       static_cast<float*>(q_ref), a.G);
  else
    update_reference_kernel<uint16_t><<<grid, 64, 0, s>>>(static_cast<const uint16_t*>(q), reuse,
                                                          static_cast<uint16_t*>(q_ref), a.G);
  return hipGetLastError();
}

hipError_t launch_wait(const uint32_t* flag, uint32_t value, uint32_t spin_limit, uint32_t* error_word,
                       uint32_t* zero_word, hipStream_t s) {
  wait_kernel<<<1, 64, 0, s>>>(flag, value, spin_limit, error_word, zero_word);
  return hipGetLastError();
}

hipError_t launch_signal(uint32_t* flag, uint32_t value, hipStream_t s, int n) {
  signal_kernel<<<1, 64, 0, s>>>(flag, value, n);
  return hipGetLastError();
}

}  // namespace clo
