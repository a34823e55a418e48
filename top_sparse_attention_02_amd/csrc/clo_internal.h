// Internal launch interface between the C ABI (clo_api.cpp) and the HIP kernels (clo_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace clo {

constexpr int kHeadDim = 128;
constexpr int kMaxGroup = 8;      // query heads per KV head handled by one unit
constexpr int kMaxKvHeads = 64;   // width of the persistent mask

// Work decomposition (rows / keys per work item).
constexpr int kScoreChunk = 2048;   // keys scored by one work item
constexpr int kGatherChunk = 512;   // rows gathered by one work item
constexpr int kAttnChunk = 256;     // selected rows attended by one work item
constexpr int kPartStride = kHeadDim + 2;  // floats per (chunk, head) partial: o[d], m, l

// Everything a kernel needs to address one layer's buffers.
struct LayerArgs {
  int32_t B, Hq, Hkv, G, P, H;
  int64_t N, k, Np;  // Np: padded key-row stride of the score workspace
  float tau;
  int32_t dtype;
  uint64_t pmask;
  const void* k_hbm;
  const void* v_hbm;
  const void* k_host;
  const void* v_host;
  const void* k_score;
  void* k_cache;
  void* v_cache;
  int32_t* idx;
};

struct Workspace {
  int32_t* counts;     // [0] miss units, [1] miss units of non-persistent heads
  int32_t* list_all;   // [U] miss units, ascending
  int32_t* list_host;  // [U] miss units of non-persistent heads, ascending
  uint32_t* keys;      // [U][Np] order-preserving score keys
  float* part;         // [U][nch][G][kPartStride] attention partials
};

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Launchers: enqueue on `s`; return the HIP error of the launch.
hipError_t launch_reuse(const LayerArgs& a, const void* q, const void* q_prev, uint8_t* reuse, float* cos,
                        hipStream_t s);
hipError_t launch_compact(const LayerArgs& a, const uint8_t* reuse, const Workspace& w, hipStream_t s);
hipError_t launch_score(const LayerArgs& a, const void* q, const Workspace& w, int num_cu, hipStream_t s);
hipError_t launch_topk(const LayerArgs& a, const Workspace& w, int num_cu, hipStream_t s);
hipError_t launch_gather(const LayerArgs& a, const uint8_t* reuse, int num_cu, hipStream_t s);
hipError_t launch_attention(const LayerArgs& a, const void* q, void* out, const Workspace& w, hipStream_t s);
hipError_t launch_wait(const uint32_t* flag, uint32_t value, uint32_t spin_limit, uint32_t* error_word,
                       hipStream_t s);
hipError_t launch_signal(uint32_t* flag, uint32_t value, hipStream_t s);

}  // namespace clo
