// HIP kernels of the selection (gfx950): A1 reuse test and device-side unit
// lists, A2 scoring (s_j = max_h q_h . K_j, stored as order-preserving uint32
// keys), A3 exact top-k (radix select; one-launch and multi-launch paths) and
// its block-granular variant.  CLO abstract, feature (1); "CLO (2511.14510) --
// L3 Per-Paper Synthesis", sections 2.1 item 2, 2.2 and the 2.3 table.
#include <math.h>

#include <type_traits>

#include "../../include/clo.h"
#include "clo_device.h"
#include "clo_internal.h"

namespace clo {
namespace {

// ---------------------------------------------------------------- A1 reuse test
struct HeadTau {
  float t[kMaxKvHeads];
};

// Cosine of unit u's concatenated query group against the previous step's,
// by one wave (fp32 dot and norms); valid in every lane.
template <typename T>
__device__ __forceinline__ float group_cosine(const T* __restrict__ q, const T* __restrict__ qp, int u, int Hkv,
                                              int Hq, int G) {
  const int lane = threadIdx.x & 63;
  const int b = u / Hkv, h = u % Hkv;
  const int64_t off = ((int64_t)b * Hq + (int64_t)h * G) * kHeadDim;  // the group is contiguous
  const int n8 = G * kHeadDim / 8;
  float dot = 0.f, na = 0.f, nb = 0.f;
  for (int i = lane; i < n8; i += 64) {
    float x[8], y[8];
    load8(q + off + i * 8, x);
    load8(qp + off + i * 8, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      dot = fmaf(x[e], y[e], dot);
      na = fmaf(x[e], x[e], na);
      nb = fmaf(y[e], y[e], nb);
    }
  }
  dot = wave_sum(dot);
  na = wave_sum(na);
  nb = wave_sum(nb);
  return (na == 0.f || nb == 0.f) ? 0.f : dot / (sqrtf(na) * sqrtf(nb));
}

template <typename T>
__global__ __launch_bounds__(64) void reuse_kernel(const T* __restrict__ q, const T* __restrict__ qp,
                                                   uint8_t* __restrict__ reuse, float* __restrict__ cosv,
                                                   int Hkv, int Hq, int G, HeadTau tau) {
  const int u = blockIdx.x;
  const float c = group_cosine(q, qp, u, Hkv, Hq, G);
  if (threadIdx.x == 0) {
    if (cosv) cosv[u] = c;
    reuse[u] = (c >= tau.t[u % Hkv]) ? 1 : 0;
  }
}

// ---------------------------------------------------------------- unit lists
// One block scans the reuse flags in unit order into three ascending lists
// (miss units, miss units of non-persistent heads, reuse units) and the first
// list position of each of the R unit ranges; nothing is read back by the host.
template <typename MissF>
__device__ void compact_units(MissF is_miss, int U, int Hkv, uint64_t pmask, int R, const RangeBounds& rb,
                              int32_t* __restrict__ meta, int32_t* __restrict__ list_all,
                              int32_t* __restrict__ list_host, int32_t* __restrict__ list_hit,
                              uint32_t* __restrict__ h0, uint32_t* __restrict__ h0b) {
  __shared__ int wsum[3][16];
  __shared__ int base[3];
  __shared__ int rcount[2][kMaxRanges];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid < 3) base[tid] = 0;
  if (tid < 2 * kMaxRanges) (&rcount[0][0])[tid] = 0;
  __syncthreads();
  for (int t0 = 0; t0 < U; t0 += 1024) {
    const int u = t0 + tid;
    const bool valid = u < U;
    const bool miss = valid && is_miss(u);
    const bool host = miss && !((pmask >> (u % Hkv)) & 1ull);
    const bool hit = valid && !miss;
    if (miss) {
      int r = 0;
      while (r + 1 < R && u >= rb.first[r + 1]) ++r;
      atomicAdd(&rcount[0][r], 1);
      if (host) atomicAdd(&rcount[1][r], 1);
    }
    const uint64_t bm = __ballot(miss), bh = __ballot(host), bt = __ballot(hit);
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    if (lane == 0) {
      wsum[0][w] = __popcll(bm);
      wsum[1][w] = __popcll(bh);
      wsum[2][w] = __popcll(bt);
    }
    __syncthreads();
    int om = base[0] + __popcll(bm & below), oh = base[1] + __popcll(bh & below);
    int ot = base[2] + __popcll(bt & below);
    for (int i = 0; i < w; ++i) {
      om += wsum[0][i];
      oh += wsum[1][i];
      ot += wsum[2][i];
    }
    if (miss) {
      list_all[om] = u;
      // digit-1 histogram of the unit's top-k, filled by the scoring kernel
      u32x4* hz = reinterpret_cast<u32x4*>(h0 + (int64_t)u * 256);
      for (int i = 0; i < 64; ++i) hz[i] = u32x4{0u, 0u, 0u, 0u};
      if (h0b) {
        hz = reinterpret_cast<u32x4*>(h0b + (int64_t)u * 256);
        for (int i = 0; i < 64; ++i) hz[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (host) list_host[oh] = u;
    if (hit) list_hit[ot] = u;
    __syncthreads();
    if (tid == 0) {
      for (int i = 0; i < 16; ++i) {
        base[0] += wsum[0][i];
        base[1] += wsum[1][i];
        base[2] += wsum[2][i];
      }
    }
    __syncthreads();
  }
  if (tid < kMaxRanges) {
    meta[kMetaGather + tid] = 0;
    meta[kMetaScore + tid] = 0;
    meta[kMetaSelFlag + tid] = 0;
    meta[kMetaGatherFlag + tid] = 0;
    meta[kMetaRangeDone + tid] = 0;
  }
  if (tid == 0) meta[kMetaGatherDone] = 0;
  if (tid == 0) {
    meta[kMetaCountAll] = base[0];
    meta[kMetaCountHost] = base[1];
    meta[kMetaCountHit] = base[2];
    meta[kMetaZero] = 0;
    int oa = 0, oh = 0;
    for (int r = 0; r < R; ++r) {
      meta[kMetaOffAll + r] = oa;
      meta[kMetaOffHost + r] = oh;
      oa += rcount[0][r];
      oh += rcount[1][r];
    }
    meta[kMetaOffAll + R] = oa;
    meta[kMetaOffHost + R] = oh;
  }
}


__global__ __launch_bounds__(1024) void compact_kernel(const uint8_t* __restrict__ reuse, int U, int Hkv,
                                                       uint64_t pmask, int R, RangeBounds rb,
                                                       int32_t* __restrict__ meta,
                                                       int32_t* __restrict__ list_all,
                                                       int32_t* __restrict__ list_host,
                                                       int32_t* __restrict__ list_hit, uint32_t* __restrict__ h0,
                                                       uint32_t* __restrict__ h0b) {
  compact_units([&](int u) { return reuse == nullptr || reuse[u] == 0; }, U, Hkv, pmask, R, rb, meta, list_all,
                list_host, list_hit, h0, h0b);
}

// Reuse test and unit lists of a layer of at most kFusedReuseUnits units in one
// block: after an optional bounded wait on a device flag (as wait_kernel), the
// 16 waves compute the units' cosines, keep the decisions in LDS and compact
// them.  Three launches of a few microseconds each become one, which matters
// on a select stream whose every launch waits behind other streams' memory
// traffic.
template <typename T>
__device__ __forceinline__ void reuse_compact_body(const T* __restrict__ q, const T* __restrict__ qp,
                                                   uint8_t* __restrict__ reuse, float* __restrict__ cosv, int Hkv,
                                                   int Hq, int G, const float* tau_h, int U, uint64_t pmask,
                                                   int32_t* __restrict__ meta, int32_t* __restrict__ list_all,
                                                   int32_t* __restrict__ list_host, int32_t* __restrict__ list_hit,
                                                   uint32_t* __restrict__ h0, uint32_t* __restrict__ h0b,
                                                   const uint32_t* wait_flag, uint32_t wait_value, uint32_t limit,
                                                   uint32_t* error_word) {
  __shared__ uint8_t s_reuse[kFusedReuseUnits];
  static_assert(kFusedReuseUnits <= 1024, "one unit per thread in the compaction");
  if (wait_flag && threadIdx.x == 0) poll_flag(wait_flag, wait_value, limit, error_word);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int u = wave; u < U; u += 16) {
    const float c = group_cosine(q, qp, u, Hkv, Hq, G);
    if (lane == 0) {
      const uint8_t r = (c >= tau_h[u % Hkv]) ? 1 : 0;
      if (cosv) cosv[u] = c;
      reuse[u] = r;
      s_reuse[u] = r;
    }
  }
  __syncthreads();
  RangeBounds rb{};
  rb.first[1] = U;
  compact_units([&](int u) { return s_reuse[u] == 0; }, U, Hkv, pmask, 1, rb, meta, list_all, list_host, list_hit,
                h0, h0b);
}

template <typename T>
__global__ __launch_bounds__(1024) void reuse_compact_kernel(const T* __restrict__ q, const T* __restrict__ qp,
                                                             uint8_t* __restrict__ reuse, float* __restrict__ cosv,
                                                             int Hkv, int Hq, int G, HeadTau tau, int U,
                                                             uint64_t pmask, int32_t* __restrict__ meta,
                                                             int32_t* __restrict__ list_all,
                                                             int32_t* __restrict__ list_host,
                                                             int32_t* __restrict__ list_hit,
                                                             uint32_t* __restrict__ h0, uint32_t* __restrict__ h0b,
                                                             const uint32_t* wait_flag, uint32_t wait_value,
                                                             uint32_t limit, uint32_t* error_word) {
  reuse_compact_body<T>(q, qp, reuse, cosv, Hkv, Hq, G, tau.t, U, pmask, meta, list_all, list_host, list_hit, h0,
                        h0b, wait_flag, wait_value, limit, error_word);
}

// The same for the layers of a multi-layer selection, one block per layer (each
// after its own wait); block 0 also clears the scoring's work counter.
template <typename T>
__global__ __launch_bounds__(1024) void reuse_compact_layers_kernel(const SelectPlanLayer* __restrict__ plan,
                                                                    SelectPlanHeader* __restrict__ hdr, int first,
                                                                    uint32_t wait_value, uint32_t limit,
                                                                    uint32_t* error_word) {
  if ((uint32_t)first + gridDim.x > hdr->n_layers) {  // layers the plan does not hold: refused
    if (error_word && blockIdx.x == 0 && threadIdx.x == 0) atomicCAS(error_word, 0u, (uint32_t)CLO_E_ARG);
    return;
  }
  const SelectPlanLayer& L = plan[first + (int)blockIdx.x];
  if (blockIdx.x == 0 && threadIdx.x == 0) hdr->score_counter = 0u;
  reuse_compact_body<T>(static_cast<const T*>(L.q), static_cast<const T*>(L.q_prev), L.reuse, L.cos, L.a.Hkv, L.a.Hq,
                        L.a.G, L.a.tau_h, L.a.B * L.a.Hkv, L.a.pmask, L.w.meta, L.w.list_all, L.w.list_host,
                        L.w.list_hit, L.w.h0, nullptr, L.wait_flag, wait_value, limit, error_word);
}

// Miss units of the layers first .. first + count - 1 of a plan before each
// layer (pref[j]) and in all (pref[count]), from the counts the unit lists
// left in each layer's workspace; every thread of the block reads them after
// the barrier.
__device__ __forceinline__ void load_miss_prefix(const SelectPlanLayer* __restrict__ plan,
                                                 const SelectPlanHeader* __restrict__ hdr, int first, int count,
                                                 int32_t* pref) {
  if (threadIdx.x == 0) {
    // a launch past the plan's layers does no work (the reuse launch reported it)
    const bool held = (uint32_t)(first + count) <= hdr->n_layers;
    int32_t acc = 0;
    pref[0] = 0;
    for (int j = 0; j < count; ++j) {
      if (held) acc += plan[first + j].w.meta[kMetaCountAll];
      pref[j + 1] = acc;
    }
  }
  __syncthreads();
}

// The layer j (0 .. count - 1) whose miss units hold unit gu of the batch.
__device__ __forceinline__ int layer_of(const int32_t* pref, int gu) {
  int j = 0;
  while (pref[j + 1] <= gu) ++j;
  return j;
}

// End of a multi-layer selection: one wave stores signal_value to every layer's
// signal flag (release).  It runs as a launch of its own after the top-k: the
// kernel boundary makes the top-k's writes visible to every XCD with one L2
// write-back, where an agent-scope release in each top-k block would write back
// its XCD's whole L2 once per block (that made a 48-layer step 1.5-7% slower
// when tried on the attention combine).
__global__ __launch_bounds__(64) void signal_layers_kernel(const SelectPlanLayer* __restrict__ plan,
                                                           const SelectPlanHeader* __restrict__ hdr, int first,
                                                           int count, uint32_t signal_value) {
  const int j = (int)threadIdx.x;
  if (j >= count || (uint32_t)(first + count) > hdr->n_layers) return;
  uint32_t* f = plan[first + j].signal_flag;
  if (f) __hip_atomic_store(f, signal_value, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- A2 scoring
// Both scoring kernels also count digit 1 (the top 8 bits) of every key they
// produce in per-wave LDS histograms, which score_item_done adds to the unit's
// global histogram H0 at the end of each work item; the block that takes a
// unit's first item also clears the unit's H1 and resets its radix state
// (nothing reads either before the top-k kernels that follow).
// Body without barriers: the caller brackets it so that every wave has finished
// the item before it and no wave counts into s_h again until after it.
// The one-launch top-k's per-unit exchange words (pass histograms and arrival
// counts), cleared by 256 threads together with the unit's other radix state.
__device__ __forceinline__ void clear_fused_sync(uint32_t* __restrict__ fs, int u) {
  uint32_t* f = fs + (int64_t)u * kFusedSyncWords;
  for (int i = threadIdx.x; i < kFusedSyncWords; i += 256) f[i] = 0u;
}

template <int W>
__device__ __forceinline__ void flush_score_hist(uint32_t (*s_h)[W], int u, int c, int64_t k,
                                                 uint32_t* __restrict__ h0, uint32_t* __restrict__ h1,
                                                 TopkState* __restrict__ st, uint32_t* __restrict__ fs) {
  const int t = threadIdx.x;  // 256 threads, one bin each
  const uint32_t sum = s_h[0][t] + s_h[1][t] + s_h[2][t] + s_h[3][t];
  s_h[0][t] = 0u;
  s_h[1][t] = 0u;
  s_h[2][t] = 0u;
  s_h[3][t] = 0u;
  if (sum) atomicAdd(h0 + (int64_t)u * 256 + t, sum);
  if (c == 0) {
    h1[(int64_t)u * 256 + t] = 0u;
    if (t == 0) st[u] = TopkState{0u, 0u, (uint32_t)k, 0u};
    clear_fused_sync(fs, u);
  }
}

template <int W>
__device__ __forceinline__ void score_item_done(uint32_t (*s_h)[W], int u, int c, int64_t k,
                                                uint32_t* __restrict__ h0, uint32_t* __restrict__ h1,
                                                TopkState* __restrict__ st, uint32_t* __restrict__ fs) {
  __syncthreads();
  flush_score_hist(s_h, u, c, k, h0, h1, st, fs);
  __syncthreads();
}

template <int W>
__device__ __forceinline__ void clear_score_hist(uint32_t (*s_h)[W]) {
  for (int i = threadIdx.x; i < 4 * W; i += 256) (&s_h[0][0])[i] = 0u;
  __syncthreads();
}

// 16 lanes per key row (8 elements each), 4 rows per wave instruction.
template <typename T, int G>
__global__ __launch_bounds__(256) void score_kernel(LayerArgs a, const T* __restrict__ q, Span sp,
                                                    uint32_t* __restrict__ keys, uint32_t* __restrict__ h0,
                                                    uint32_t* __restrict__ h1, TopkState* __restrict__ st,
                                                    uint32_t* __restrict__ fs) {
  constexpr int UNR = 8;
  __shared__ uint32_t s_h[4][256];
  clear_score_hist(s_h);
  constexpr int kRowsPerWave = kScoreChunk / 4;
  const int nch = (int)((a.N + kScoreChunk - 1) / kScoreChunk);
  const int lo = *sp.lo;
  const int64_t items = (int64_t)(*sp.hi - lo) * nch;
  const int32_t* list = sp.list + lo;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane & 15, rg = lane >> 4;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int u = list[it / nch];
    const int c = (int)(it % nch);
    const int b = u / a.Hkv, h = u % a.Hkv;
    const T* kb = unit_keys<T>(a, b, h);
    float qv[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) load8(q + ((int64_t)b * a.Hq + (int64_t)h * G + g) * kHeadDim + sub * 8, qv[g]);
    uint32_t* kout = keys + (int64_t)u * a.Np;
    const int64_t r_begin = (int64_t)c * kScoreChunk + (int64_t)wave * kRowsPerWave;
    for (int r = 0; r < kRowsPerWave; r += 4 * UNR) {
      float kx[UNR][8];
      int64_t row[UNR];
#pragma unroll
      for (int j = 0; j < UNR; ++j) {
        row[j] = r_begin + r + j * 4 + rg;
        const int64_t rr = row[j] < a.N ? row[j] : a.N - 1;
        load8(kb + rr * kHeadDim + sub * 8, kx[j]);
      }
#pragma unroll
      for (int j = 0; j < UNR; ++j) {
        float best = kNegInf;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float s = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) s = fmaf(qv[g][e], kx[j][e], s);
          best = fmaxf(best, sum16(s));
        }
        if (sub == 0 && row[j] < a.N) {
          const uint32_t sk = score_key(best);
          kout[row[j]] = sk;
          atomicAdd(&s_h[wave][sk >> 24], 1u);
        }
      }
    }
    score_item_done(s_h, u, c, a.k, h0, h1, st, fs);
  }
}

// bf16 scoring on the matrix cores: per wave, S[16 x 16] = Qpad[16 x 128] . K^T[128 x 16]
// with v_mfma_f32_16x16x32_bf16 (four k-steps of 32).  Rows of Qpad are the
// unit's g query heads (zero rows past g); columns are 16 consecutive keys.
// Lane l supplies row/column l % 16 and the k-slice (l / 16) of each k-step for
// both operands, so every key row is read straight from HBM as 16-byte pieces;
// the dot product only needs A and B to share that k-slice mapping.  The
// result S[i][j] lands in lane j + 16 * (i / 4), register i % 4: lanes 0-15
// hold heads 0-3 of key j, lanes 16-31 heads 4-7.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Blocks are persistent and take items of kScoreItem keys (kScoreItem / 4 per
// wave) from a device counter, so that the last round of work is short and no
// block idles behind a slow one; the query operand is reloaded only when the
// unit changes.
constexpr int kScoreItem = 1024;

// The grid holds two blocks per CU, i.e. two waves per SIMD; telling the
// compiler so lets it keep all of an iteration's 16-byte key loads in flight
// instead of rationing registers for a higher occupancy (632 vs 650 us for
// 3.4 GB on MI355X).
// One work item of the MFMA scoring: keys c * kScoreItem .. of unit u, scored
// into keys[u], their digit 1 counted into s_h.  Thread 0 takes the next item
// from *counter once the item's last key loads are issued and leaves it in
// *s_item.
template <int G>
__device__ __forceinline__ void score_mfma_item(const LayerArgs& a, const uint16_t* __restrict__ q,
                                                uint32_t* __restrict__ keys, int u, int c,
                                                uint32_t* __restrict__ counter, uint32_t (*s_h)[257],
                                                uint32_t* s_item) {
  constexpr int TILES = 8;                         // 16-key tiles per wave iteration (128 keys)
  constexpr int kKeysPerWave = kScoreItem / 4;     // 256
  static_assert(G <= 8, "group of at most 8 query heads");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, ks = lane >> 4;       // tile column / k-slice of this lane
  bf16x8 qa[4];
  const int b = u / a.Hkv, h = u % a.Hkv;
  const uint16_t* kb = unit_keys<uint16_t>(a, b, h);
  {
    // the query operand of the item's unit (64 bytes per lane, an L2 hit after
    // the first item of the unit), loaded without a branch so that the item's
    // key loads are not held behind it
    const int head = col;  // row of Qpad
    const uint16_t* qh = q + ((int64_t)b * a.Hq + (int64_t)h * G + (head < G ? head : 0)) * kHeadDim;
    const uint32_t keep = head < G ? ~0u : 0u;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(qh + s * 32 + ks * 8);
      qa[s] = __builtin_bit_cast(bf16x8, w & keep);
    }
  }
  uint32_t* kout = keys + (int64_t)u * a.Np;
  const int64_t w_begin = (int64_t)c * kScoreItem + (int64_t)wave * kKeysPerWave;
  // digit-1 bins of the previous iteration's keys, counted only after this
  // iteration's loads are issued: an LDS atomic placed before them keeps the
  // compiler from issuing them early
  uint32_t pend[TILES / 4];
  bool have_pend = false;
  // the next item is claimed once the last key loads of this one are issued:
  // the counter's round trip then overlaps the item's tail, while a claim at
  // the item's start would hold work back from blocks that run out earlier
  uint32_t next_item = 0;
  bool claimed = false;
#pragma unroll
  for (int t0 = 0; t0 < kKeysPerWave; t0 += 16 * TILES) {
    if (w_begin + t0 >= a.N) break;  // uniform per wave
    u32x4 kbuf[TILES][4];
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      int64_t row = w_begin + t0 + t * 16 + col;
      row = row < a.N ? row : a.N - 1;
      const uint16_t* kr = kb + row * kHeadDim + ks * 8;
#pragma unroll
      for (int s = 0; s < 4; ++s) kbuf[t][s] = *reinterpret_cast<const u32x4*>(kr + s * 32);
    }
    if (t0 + 16 * TILES >= kKeysPerWave && threadIdx.x == 0) {
      next_item = atomicAdd(counter, 1u);
      claimed = true;
    }
    if (have_pend) {
#pragma unroll
      for (int i = 0; i < TILES / 4; ++i) atomicAdd(&s_h[wave][pend[i]], 1u);
    }
    float mt[TILES];  // tile maxima, valid in lanes 0..15 (lane = key within the tile)
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], __builtin_bit_cast(bf16x8, kbuf[t][s]), acc, 0, 0, 0);
      // max over the unit's heads: rows 0..min(G,4)-1 here, rows 4..G-1 in lane + 16
      float m = acc[0];
      if (G > 1) m = fmaxf(m, acc[1]);
      if (G > 2) m = fmaxf(m, acc[2]);
      if (G > 3) m = fmaxf(m, acc[3]);
      if (G > 4) {
        float m2 = acc[0];
        if (G > 5) m2 = fmaxf(m2, acc[1]);
        if (G > 6) m2 = fmaxf(m2, acc[2]);
        if (G > 7) m2 = fmaxf(m2, acc[3]);
        m = fmaxf(m, __shfl_down(m2, 16, 64));
      }
      mt[t] = m;
    }
    // lane L of the wave takes key L of each 4-tile group: one 256-byte store
    // per group instead of four 64-byte ones
#pragma unroll
    for (int t4 = 0; t4 < TILES; t4 += 4) {
      float v = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float x = __shfl(mt[t4 + t], col, 64);
        if (ks == t) v = x;
      }
      const int64_t key = w_begin + t0 + t4 * 16 + lane;
      const uint32_t sk = score_key(v);
      if (key < a.N) kout[key] = sk;
      pend[t4 / 4] = key < a.N ? sk >> 24 : 256u;
    }
    have_pend = true;
  }
  if (have_pend) {
#pragma unroll
    for (int i = 0; i < TILES / 4; ++i) atomicAdd(&s_h[wave][pend[i]], 1u);
  }
  // read at the top of the next iteration, after the barrier there; every
  // wave read the current value before the barrier that follows the flush
  if (threadIdx.x == 0) *s_item = claimed ? next_item : atomicAdd(counter, 1u);
  // the LDS writes of this item (s_item, the digit counts) complete before the
  // barrier at the loop top: hipcc (ROCm 7.2, gfx950) emits that barrier on
  // this back edge without the LDS wait its fence implies, and other waves
  // then read the previous item number
  wait_lds();
}

// The grid holds two blocks per CU, i.e. two waves per SIMD; telling the
// compiler so lets it keep all of an iteration's 16-byte key loads in flight
// instead of rationing registers for a higher occupancy (632 vs 650 us for
// 3.4 GB on MI355X).
template <int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void score_mfma_kernel(
    LayerArgs a, const uint16_t* __restrict__ q, Span sp, uint32_t* __restrict__ keys,
    uint32_t* __restrict__ counter, uint32_t* __restrict__ h0, uint32_t* __restrict__ h1,
    TopkState* __restrict__ st, uint32_t* __restrict__ fs) {
  __shared__ uint32_t s_item;
  __shared__ uint32_t s_h[4][257];  // bin 256 takes keys past the end (not flushed)
  clear_score_hist(s_h);
  const int nch = (int)((a.N + kScoreItem - 1) / kScoreItem);
  const int lo = *sp.lo;
  const int64_t items = (int64_t)(*sp.hi - lo) * nch;
  const int32_t* list = sp.list + lo;
  int cur_u = -1, prev_c = 0;
  if (threadIdx.x == 0) s_item = atomicAdd(counter, 1u);
  for (;;) {
    __syncthreads();
    const int64_t it = s_item;
    // every wave is past the previous item: add its histogram to the unit's
    if (cur_u >= 0) flush_score_hist(s_h, cur_u, prev_c, a.k, h0, h1, st, fs);
    __syncthreads();
    if (it >= items) break;  // uniform per block
    const int u = list[it / nch];
    const int c = (int)(it % nch);
    prev_c = c;
    cur_u = u;
    score_mfma_item<G>(a, q, keys, u, c, counter, s_h, &s_item);
  }
}

// The scoring of a multi-layer selection: the same persistent blocks take items
// from one counter over the miss units of all the batch's layers, layer after
// layer, so that the short scorings of small layers share one launch and one
// ramp-up and tail.
template <int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void score_mfma_layers_kernel(
    const SelectPlanLayer* __restrict__ plan, SelectPlanHeader* __restrict__ hdr, int first, int count,
    uint32_t* err) {
  __shared__ uint32_t s_item;
  __shared__ uint32_t s_h[4][257];
  __shared__ int32_t s_pref[kMaxSelectBatch + 1];
  clear_score_hist(s_h);
  load_miss_prefix(plan, hdr, first, count, s_pref);
  const int64_t nch = (plan[first].a.N + kScoreItem - 1) / kScoreItem;
  const int64_t items = (int64_t)s_pref[count] * nch;
  uint32_t* counter = &hdr->score_counter;
  int cur_u = -1, prev_c = 0, cur_j = 0;
  if (threadIdx.x == 0) s_item = atomicAdd(counter, 1u);
  for (;;) {
    __syncthreads();
    const int64_t it = s_item;
    if (cur_u >= 0) {
      const SelectPlanLayer& P = plan[first + cur_j];
      flush_score_hist(s_h, cur_u, prev_c, P.a.k, P.w.h0, P.w.h1, P.w.tstate, P.w.fsync);
    }
    __syncthreads();
    if (it >= items) break;  // uniform per block
    const int gu = (int)(it / nch);
    const int j = layer_of(s_pref, gu);
    const SelectPlanLayer& L = plan[first + j];
    if (L.a.G != G || L.a.N != plan[first].a.N) {  // a layer the launch was not shaped for: reported, skipped
      if (threadIdx.x == 0) {
        if (err) atomicCAS(err, 0u, (uint32_t)CLO_E_ARG);
        s_item = atomicAdd(counter, 1u);
      }
      cur_u = -1;
      wait_lds();  // s_item is in LDS before the loop-top barrier (see score_mfma_item)
      continue;
    }
    const int u = L.w.list_all[gu - s_pref[j]];
    const int c = (int)(it % nch);
    prev_c = c;
    cur_u = u;
    cur_j = j;
    score_mfma_item<G>(L.a, static_cast<const uint16_t*>(L.q), L.w.keys, u, c, counter, s_h, &s_item);
  }
}

// ---------------------------------------------------------------- A3 top-k
// Exact radix select over each miss unit's order-preserving score keys, four
// 8-bit digits from the most significant one.  For a digit position, a
// histogram of the keys that match the digits fixed so far gives the digit of
// the k-th largest key (pick_digit); after four digits, T = the k-th largest key
// and `rem` = how many keys equal to T are taken (the first rem by index, the
// tie rule).  The winners (keys > T, then those rem keys == T) are written in
// ascending index order.
//
//   scoring          digit 1 histogram of every miss unit (H0), built in LDS
//                    while the keys are produced and added per work item
//   single block     contexts of fewer than kTopkMultiMin chunks: one 1024-
//   (topk_unit)      thread block per unit takes digit 1 from H0 and runs
//                    digits 2-4 and the write itself
//   multi block      one 256-thread block per chunk of kTopkChunk keys:
//   (topk_pass x3)   digit 2 (every block takes digit 1 from H0 first), digit 3,
//                    digit 4; each block adds its LDS histogram to the unit's
//                    global one, and the last block of the unit to finish (an
//                    atomic done count) picks the digit.  The digit-4 pass also
//                    stores each chunk's own histogram and count of keys above
//                    the 24-bit prefix, from which every chunk's output offset
//                    follows once T is known.
//   (topk_write)     per chunk: offset from the earlier chunks' histograms,
//                    then a block scan writes the winners.
// H0 is cleared by the compaction kernel; H1 and the per-unit state by the
// scoring block that takes a unit's first work item.
constexpr int kTopkThreads = 256;
// Contexts of at least this many chunks (N >= 131072) take the multi-block
// path; shorter ones a single block per unit (fewer launches, and the many
// units of short-context batches already fill the GPU).  Measured on MI355X:
// 102 units at N = 131072 select in 0.81 ms (multi-block, with scoring) vs
// 0.84 ms; 128 units at N = 32768 in 0.29 ms (single block) vs 0.31 ms.
constexpr int kTopkMultiMin = 8;
constexpr int kTopkUnroll = 4;     // 16-byte key loads in flight per thread (single-block kernel)
// the multi-block digit passes issue all of a chunk's loads at once (16 per
// thread): beside the host gather every round trip to memory is slow
constexpr int kTopkPassUnroll = kTopkChunk / (kTopkThreads * 4);

// One full wave: the digit d whose bin holds the rem-th largest of the counted
// keys (bins scanned from 255 down) and `above` = the count in bins above d.
// Lane l reads bins 4l..4l+3 of h (LDS); every lane returns the same values.
// If fewer than rem keys were counted, d = 0 (cannot happen for valid counts).
__device__ __forceinline__ void pick_digit(const uint32_t* h, uint32_t rem, uint32_t& digit, uint32_t& above) {
  const int lane = threadIdx.x & 63;
  const uint32_t b0 = h[4 * lane], b1 = h[4 * lane + 1], b2 = h[4 * lane + 2], b3 = h[4 * lane + 3];
  const uint32_t s = b0 + b1 + b2 + b3;
  uint32_t S = s;  // keys in bins >= 4 lane
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_down(S, off, 64);
    if (lane + off < 64) S += y;
  }
  // S does not increase with the lane, so the lanes with S >= rem are 0..L
  const uint64_t m = __ballot(S >= rem);
  const int L = m ? 63 - __builtin_clzll(m) : 0;
  uint32_t acc = __shfl(S - s, L, 64);
  const uint32_t c3 = __shfl(b3, L, 64), c2 = __shfl(b2, L, 64), c1 = __shfl(b1, L, 64);
  uint32_t d = 4u * (uint32_t)L;
  if (acc + c3 >= rem) {
    d += 3;
  } else if ((acc += c3) + c2 >= rem) {
    d += 2;
  } else if ((acc += c2) + c1 >= rem) {
    d += 1;
  } else {
    acc += c1;
  }
  digit = d;
  above = acc;
}

struct UnitChunk {
  int u, c;
  bool valid;
};

__device__ __forceinline__ UnitChunk unit_chunk(const Span& sp, int cmax) {
  const int lo = *sp.lo;
  const int64_t n = (int64_t)(*sp.hi - lo) * cmax;
  UnitChunk r{0, 0, false};
  if ((int64_t)blockIdx.x >= n) return r;
  r.u = sp.list[lo + blockIdx.x / cmax];
  r.c = blockIdx.x % cmax;
  r.valid = true;
  return r;
}

// Block-wide sums of two per-thread counts (256 threads); every thread gets both.
__device__ __forceinline__ void block_sum2(uint32_t x, uint32_t y, uint32_t* s_x, uint32_t* s_y, uint32_t& tx,
                                           uint32_t& ty) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    x += __shfl_xor(x, off, 64);
    y += __shfl_xor(y, off, 64);
  }
  if (lane == 0) {
    s_x[wave] = x;
    s_y[wave] = y;
  }
  __syncthreads();
  tx = 0;
  ty = 0;
#pragma unroll
  for (int w = 0; w < kTopkThreads / 64; ++w) {
    tx += s_x[w];
    ty += s_y[w];
  }
  __syncthreads();
}

// Digit pass over one chunk of one unit (shift 16, 8 or 0).  Histograms: digit 2
// and digit 4 accumulate in H1, digit 3 in H0 (which the digit-2 pass clears
// once every block has read digit 1 from it).
__global__ __launch_bounds__(kTopkThreads) void topk_pass_kernel(LayerArgs a, Span sp,
                                                                 const uint32_t* __restrict__ keys,
                                                                 uint32_t* __restrict__ h0, uint32_t* __restrict__ h1,
                                                                 TopkState* __restrict__ st,
                                                                 uint32_t* __restrict__ chist, int cmax, int shift) {
  __shared__ uint32_t hist[kTopkThreads / 64][256];
  __shared__ uint32_t tot[256];
  __shared__ uint32_t s_prefix, s_mask, s_rem, s_x[4], s_y[4];
  __shared__ int s_last;
  const UnitChunk uc = unit_chunk(sp, cmax);
  if (!uc.valid) return;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int64_t N = a.N;
  const int64_t c0 = (int64_t)uc.c * kTopkChunk;
  const int64_t c1 = (c0 + kTopkChunk < N) ? c0 + kTopkChunk : N;
  const uint32_t* kk = keys + (int64_t)uc.u * a.Np;
  uint32_t* h0u = h0 + (int64_t)uc.u * 256;
  uint32_t* h1u = h1 + (int64_t)uc.u * 256;
  uint32_t* acc_h = shift == 8 ? h0u : h1u;
  if (shift == 16) {
    // digit 1 from the scoring histogram
    tot[tid] = h0u[tid];
    __syncthreads();
    if (wave == 0) {
      uint32_t d, above;
      pick_digit(tot, (uint32_t)a.k, d, above);
      if (tid == 0) {
        s_prefix = d << 24;
        s_mask = 0xFF000000u;
        s_rem = (uint32_t)a.k - above;
      }
    }
  } else if (tid == 0) {
    s_prefix = st[uc.u].prefix;
    s_mask = st[uc.u].mask;
    s_rem = st[uc.u].rem;
  }
  for (int i = tid; i < (kTopkThreads / 64) * 256; i += kTopkThreads) (&hist[0][0])[i] = 0u;
  __syncthreads();
  const uint32_t prefix = s_prefix, mask = s_mask;
  uint32_t gt = 0;  // digit-4 pass: keys whose fixed 24 bits exceed the prefix
  constexpr int kStep = kTopkThreads * 4;
  for (int64_t base = c0 + (int64_t)tid * 4; base < c1; base += (int64_t)kStep * kTopkPassUnroll) {
    u32x4 v[kTopkPassUnroll];
#pragma unroll
    for (int j = 0; j < kTopkPassUnroll; ++j) {
      const int64_t i = base + (int64_t)j * kStep;
      v[j] = i < c1 ? *reinterpret_cast<const u32x4*>(kk + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < kTopkPassUnroll; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t kv = v[j][e];
        const bool valid = base + (int64_t)j * kStep + e < c1;
        if (valid && (kv & mask) == prefix) atomicAdd(&hist[wave][(kv >> shift) & 255u], 1u);
        gt += valid && (kv & mask) > prefix;
      }
  }
  __syncthreads();
  {
    const uint32_t sum = hist[0][tid] + hist[1][tid] + hist[2][tid] + hist[3][tid];
    if (sum) atomicAdd(&acc_h[tid], sum);
    if (shift == 0) chist[((int64_t)uc.u * cmax + uc.c) * kChunkHist + tid] = sum;
  }
  if (shift == 0) {
    uint32_t g, unused;
    block_sum2(gt, 0u, s_x, s_y, g, unused);
    if (tid == 0) chist[((int64_t)uc.u * cmax + uc.c) * kChunkHist + 256] = g;
  }
  // Device-scope atomics are performed at the device's point of coherence; once
  // this thread's adds are acknowledged they are visible to every block, so
  // waiting for the acknowledgements before the done count suffices.  (A
  // __threadfence here would write back and invalidate the whole L2 of this
  // XCD in every block.)
  wait_vm_acks();
  __syncthreads();
  if (tid == 0) {
    const int nchunks = (int)((N + kTopkChunk - 1) / kTopkChunk);
    s_last = atomicAdd(&st[uc.u].done, 1u) == (uint32_t)(nchunks - 1);
  }
  __syncthreads();
  if (!s_last) return;
  // last block of this unit: every other block's adds were acknowledged before
  // its done increment; the totals are read with device-scope atomic loads
  tot[tid] = __hip_atomic_load(acc_h + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  acc_h[tid] = 0u;
  if (shift == 16) h0u[tid] = 0u;  // every block has read digit 1 from it
  __syncthreads();
  if (wave == 0) {
    uint32_t d, above;
    pick_digit(tot, s_rem, d, above);
    if (tid == 0)
      st[uc.u] = TopkState{prefix | (d << shift), mask | (255u << shift), s_rem - above, 0u};
  }
}

// Short contexts: one 1024-thread block per miss unit takes digit 1 from H0
// and runs digits 2-4 and the compaction itself (one launch; many units keep
// many CUs busy).
constexpr int kUnitThreads = 1024;
constexpr int kUnitPerThread = 16;

__device__ __forceinline__ void topk_unit_one(const LayerArgs& a, int u, const uint32_t* __restrict__ keys,
                                              const uint32_t* __restrict__ h0) {
  __shared__ uint32_t hist[16][256];
  __shared__ uint32_t tot[256];
  __shared__ uint32_t s_prefix, s_mask, s_rem, s_base_gt, s_base_eq;
  __shared__ uint32_t s_wgt[16], s_weq[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t N = a.N;
  const uint32_t* kk = keys + (int64_t)u * a.Np;
  int32_t* out = a.idx + (int64_t)u * a.k;
  if (tid < 256) tot[tid] = h0[(int64_t)u * 256 + tid];
  __syncthreads();
  if (wave == 0) {
    uint32_t d, above;
    pick_digit(tot, (uint32_t)a.k, d, above);
    if (tid == 0) {
      s_prefix = d << 24;
      s_mask = 0xFF000000u;
      s_rem = (uint32_t)a.k - above;
    }
  }
  for (int shift = 16; shift >= 0; shift -= 8) {
    for (int i = tid; i < 16 * 256; i += kUnitThreads) (&hist[0][0])[i] = 0u;
    __syncthreads();
    const uint32_t prefix = s_prefix, mask = s_mask;
    constexpr int kStep = kUnitThreads * 4;
    for (int64_t base = (int64_t)tid * 4; base < N; base += (int64_t)kStep * kTopkUnroll) {
      u32x4 v[kTopkUnroll];
#pragma unroll
      for (int j = 0; j < kTopkUnroll; ++j) {
        const int64_t i = base + (int64_t)j * kStep;
        v[j] = i < N ? *reinterpret_cast<const u32x4*>(kk + i) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int j = 0; j < kTopkUnroll; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t kv = v[j][e];
          if (base + (int64_t)j * kStep + e < N && (kv & mask) == prefix)
            atomicAdd(&hist[wave][(kv >> shift) & 255u], 1u);
        }
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t sum = 0;
      for (int w = 0; w < 16; ++w) sum += hist[w][tid];
      tot[tid] = sum;
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t d, above;
      pick_digit(tot, s_rem, d, above);
      if (tid == 0) {
        s_rem -= above;
        s_prefix = prefix | (d << shift);
        s_mask = mask | (255u << shift);
      }
    }
    __syncthreads();
  }
  const uint32_t T = s_prefix, need = s_rem;
  if (tid == 0) {
    s_base_gt = 0u;
    s_base_eq = 0u;
  }
  __syncthreads();
  constexpr int kTile = kUnitThreads * kUnitPerThread;
  for (int64_t t0 = 0; t0 < N; t0 += kTile) {
    const int64_t i0 = t0 + (int64_t)tid * kUnitPerThread;
    u32x4 v[kUnitPerThread / 4];
#pragma unroll
    for (int j = 0; j < kUnitPerThread / 4; ++j)
      v[j] = (i0 + 4 * j < N) ? *reinterpret_cast<const u32x4*>(kk + i0 + 4 * j) : u32x4{0u, 0u, 0u, 0u};
    uint32_t cg = 0, ce = 0;
#pragma unroll
    for (int j = 0; j < kUnitPerThread / 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool valid = i0 + 4 * j + e < N;
        cg += (valid && v[j][e] > T);
        ce += (valid && v[j][e] == T);
      }
    uint32_t xg = cg, xe = ce;
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t yg = __shfl_up(xg, off, 64), ye = __shfl_up(xe, off, 64);
      if (lane >= off) {
        xg += yg;
        xe += ye;
      }
    }
    if (lane == 63) {
      s_wgt[wave] = xg;
      s_weq[wave] = xe;
    }
    __syncthreads();
    uint32_t pg = s_base_gt + xg - cg, pe = s_base_eq + xe - ce;
    for (int w = 0; w < wave; ++w) {
      pg += s_wgt[w];
      pe += s_weq[w];
    }
#pragma unroll
    for (int j = 0; j < kUnitPerThread / 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t i = i0 + 4 * j + e;
        if (i >= N) continue;
        const uint32_t kv = v[j][e];
        if (kv > T) {
          const uint32_t pos = pg + (pe < need ? pe : need);
          if (pos < (uint32_t)a.k) out[pos] = (int32_t)i;
          ++pg;
        } else if (kv == T) {
          if (pe < need && pg + pe < (uint32_t)a.k) out[pg + pe] = (int32_t)i;
          ++pe;
        }
      }
    __syncthreads();
    if (tid == 0) {
      for (int w = 0; w < 16; ++w) {
        s_base_gt += s_wgt[w];
        s_base_eq += s_weq[w];
      }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kUnitThreads) void topk_unit_kernel(LayerArgs a, Span sp,
                                                                 const uint32_t* __restrict__ keys,
                                                                 const uint32_t* __restrict__ h0) {
  const int lo = *sp.lo;
  const int n_units = *sp.hi - lo;
  const int32_t* list = sp.list + lo;
  for (int it = blockIdx.x; it < n_units; it += gridDim.x) topk_unit_one(a, list[it], keys, h0);
}

// The single-block top-k of a multi-layer selection: the blocks take the miss
// units of all the batch's layers.
__global__ __launch_bounds__(kUnitThreads) void topk_unit_layers_kernel(const SelectPlanLayer* __restrict__ plan,
                                                                        const SelectPlanHeader* __restrict__ hdr,
                                                                        int first, int count) {
  __shared__ int32_t s_pref[kMaxSelectBatch + 1];
  load_miss_prefix(plan, hdr, first, count, s_pref);
  const int total = s_pref[count];
  for (int gu = blockIdx.x; gu < total; gu += gridDim.x) {
    const int j = layer_of(s_pref, gu);
    const SelectPlanLayer& L = plan[first + j];
    topk_unit_one(L.a, L.w.list_all[gu - s_pref[j]], L.w.keys, L.w.h0);
  }
}

// Block-wide exclusive scan of two counts (keys > T, keys == T) of each thread.
__device__ __forceinline__ void scan2(uint32_t cg, uint32_t ce, uint32_t* s_wg, uint32_t* s_we, uint32_t& eg,
                                      uint32_t& ee, uint32_t& tg, uint32_t& te) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t xg = cg, xe = ce;
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t yg = __shfl_up(xg, off, 64), ye = __shfl_up(xe, off, 64);
    if (lane >= off) {
      xg += yg;
      xe += ye;
    }
  }
  if (lane == 63) {
    s_wg[wave] = xg;
    s_we[wave] = xe;
  }
  __syncthreads();
  eg = xg - cg;
  ee = xe - ce;
  tg = 0;
  te = 0;
  for (int w = 0; w < kTopkThreads / 64; ++w) {
    if (w < wave) {
      eg += s_wg[w];
      ee += s_we[w];
    }
    tg += s_wg[w];
    te += s_we[w];
  }
  __syncthreads();
}

constexpr int kTopkPerThread = 16;  // consecutive keys per thread per tile in the write

__global__ __launch_bounds__(kTopkThreads) void topk_write_kernel(LayerArgs a, Span sp,
                                                                  const uint32_t* __restrict__ keys,
                                                                  const TopkState* __restrict__ st,
                                                                  const uint32_t* __restrict__ chist, int cmax) {
  __shared__ uint32_t s_wg[kTopkThreads / 64], s_we[kTopkThreads / 64];
  const UnitChunk uc = unit_chunk(sp, cmax);
  if (!uc.valid) return;
  const int tid = threadIdx.x;
  const int64_t N = a.N;
  const int64_t c0 = (int64_t)uc.c * kTopkChunk;
  const int64_t c1 = (c0 + kTopkChunk < N) ? c0 + kTopkChunk : N;
  const uint32_t* kk = keys + (int64_t)uc.u * a.Np;
  int32_t* out = a.idx + (int64_t)uc.u * a.k;
  const uint32_t T = st[uc.u].prefix, need = st[uc.u].rem;
  const uint32_t D = T & 255u;
  // the chunk's keys are requested first (16 loads per thread), then the
  // earlier chunks' histograms 8 chunks at a time: beside the host gather
  // every round trip to memory is slow, and this kernel used to make one per
  // earlier chunk and one per tile
  constexpr int kTile = kTopkThreads * kTopkPerThread;
  constexpr int kTiles = kTopkChunk / kTile;
  static_assert(kTopkChunk % kTile == 0, "whole tiles per chunk");
  u32x4 v[kTiles][kTopkPerThread / 4];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    const int64_t i0 = c0 + (int64_t)t * kTile + (int64_t)tid * kTopkPerThread;
#pragma unroll
    for (int j = 0; j < kTopkPerThread / 4; ++j)
      v[t][j] = (i0 + 4 * j < c1) ? *reinterpret_cast<const u32x4*>(kk + i0 + 4 * j) : u32x4{0u, 0u, 0u, 0u};
  }
  // winners before this chunk: each earlier chunk's keys above the 24-bit
  // prefix of T, plus its digit-4 bins above D (> T) and at D (== T)
  uint32_t base_g, base_e;
  {
    uint32_t sg = 0, se = 0;
    const uint32_t* ch = chist + (int64_t)uc.u * cmax * kChunkHist;
    constexpr int kBatch = 8;
    for (int cb = 0; cb < uc.c; cb += kBatch) {
      uint32_t x[kBatch], y[kBatch];
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const int c = cb + q < uc.c ? cb + q : uc.c - 1;  // in range; counted below only if cb + q < uc.c
        x[q] = ch[(int64_t)c * kChunkHist + tid];
        y[q] = tid == 0 ? ch[(int64_t)c * kChunkHist + 256] : 0u;
      }
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        if (cb + q < uc.c) {
          sg += ((uint32_t)tid > D ? x[q] : 0u) + y[q];
          se += (uint32_t)tid == D ? x[q] : 0u;
        }
      }
    }
    block_sum2(sg, se, s_wg, s_we, base_g, base_e);
  }
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    const int64_t t0 = c0 + (int64_t)t * kTile;
    if (t0 >= c1) break;  // uniform per block
    const int64_t i0 = t0 + (int64_t)tid * kTopkPerThread;
    uint32_t cg = 0, ce = 0;
#pragma unroll
    for (int j = 0; j < kTopkPerThread / 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool valid = i0 + 4 * j + e < c1;
        cg += valid && v[t][j][e] > T;
        ce += valid && v[t][j][e] == T;
      }
    uint32_t eg, ee, tg, te;
    scan2(cg, ce, s_wg, s_we, eg, ee, tg, te);
    uint32_t pg = base_g + eg, pe = base_e + ee;
#pragma unroll
    for (int j = 0; j < kTopkPerThread / 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t i = i0 + 4 * j + e;
        if (i >= c1) continue;
        const uint32_t kv = v[t][j][e];
        if (kv > T) {
          const uint32_t pos = pg + (pe < need ? pe : need);
          if (pos < (uint32_t)a.k) out[pos] = (int32_t)i;
          ++pg;
        } else if (kv == T) {
          if (pe < need && pg + pe < (uint32_t)a.k) out[pg + pe] = (int32_t)i;
          ++pe;
        }
      }
    base_g += tg;
    base_e += te;
  }
}

// ---------------------------------------------------------------- A3 top-k in one launch
// The same exact select with the chunk blocks of a unit cooperating inside one
// launch.  Each block reads its chunk of keys from global memory once, into
// LDS (16384 keys = 64 KiB of gfx950's 160 KiB per CU), and keeps it there for
// digits 2-4 and the write.  For each digit the blocks add their LDS histograms
// into the unit's histogram of that digit (device-scope atomics, performed at
// the device's point of coherence), wait until every chunk block of the unit
// has arrived, read the unit's histogram back and all pick the same digit.
// After digit 4 each block publishes its counts of keys above and equal to the
// k-th key; after one more arrival every block knows where its winners go.  A
// launch beside the host gather costs each memory round trip many times over;
// this path has one launch and one read of the keys per unit, where the
// multi-launch path has four of each.
//
// Every chunk block of a unit waits for the others, so all blocks of a launch
// must be resident at once: a launch has at most kFusedMaxBlocks blocks, in
// groups of cmax consecutive blocks (one per chunk), and each group takes the
// span's units g, g + groups, g + 2 groups, ... one after another.  Two blocks
// fit a CU (66 KiB of LDS each), so four such launches running side by side
// still fit the GPU.  The waits are bounded all the same (the error word gets
// CLO_E_TIMEOUT, and every block still runs to its end).  kFusedMaxBlocks is
// in clo_internal.h.

// Block-wide arrival at one of a unit's exchange counts: the block's device-scope
// atomics are acknowledged first, then thread 0 arrives and polls until all n
// chunk blocks have arrived.
__device__ __forceinline__ void unit_arrive_wait(uint32_t* arrive, uint32_t n, uint32_t limit, uint32_t* err) {
  wait_vm_acks();
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t spins = 0;
    while (__hip_atomic_load(arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < n) {
      if (++spins >= limit) {
        if (err) atomicCAS(err, 0u, (uint32_t)CLO_E_TIMEOUT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

// One unit's select by the chunk block c of the unit's group (the block's
// chunk of keys into LDS, digits 2-4 with the other chunk blocks, the write).
__device__ __forceinline__ void topk_fused_unit(const LayerArgs& a, int u, int c, int cmax,
                                                const uint32_t* __restrict__ keys, const uint32_t* __restrict__ h0,
                                                uint32_t* __restrict__ fsync, uint32_t* __restrict__ ccnt,
                                                uint32_t limit, uint32_t* err) {
  constexpr int kLoads = kTopkChunk / (kTopkThreads * 4);  // 16-byte loads per thread
  __shared__ u32x4 s_keys[kTopkChunk / 4];
  __shared__ uint32_t s_hist[256];
  __shared__ uint32_t s_prefix, s_mask, s_rem, s_x[4], s_y[4];
  const int tid = threadIdx.x;
  const int64_t N = a.N;
  const int64_t c0 = (int64_t)c * kTopkChunk;
  const int nk = (int)((c0 + kTopkChunk < N) ? kTopkChunk : N - c0);
  const uint32_t* kk = keys + (int64_t)u * a.Np + c0;
  uint32_t* fs = fsync + (int64_t)u * kFusedSyncWords;
  // the chunk's keys into LDS: all loads issued first (the row stride is a
  // multiple of 64 keys, so a 16-byte load that starts below nk stays in the row)
  {
    u32x4 v[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int i = (j * kTopkThreads + tid) * 4;
      v[j] = i < nk ? *reinterpret_cast<const u32x4*>(kk + i) : u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();  // the previous unit's write has read s_keys
#pragma unroll
    for (int j = 0; j < kLoads; ++j) s_keys[j * kTopkThreads + tid] = v[j];
  }
  // digit 1 from the scoring histogram
  s_hist[tid] = h0[(int64_t)u * 256 + tid];
  __syncthreads();
  if (tid < 64) {
    uint32_t d, above;
    pick_digit(s_hist, (uint32_t)a.k, d, above);
    if (tid == 0) {
      s_prefix = d << 24;
      s_mask = 0xFF000000u;
      s_rem = (uint32_t)a.k - above;
    }
  }
  __syncthreads();
  for (int p = 0; p < 3; ++p) {
    const int shift = 16 - 8 * p;
    const uint32_t prefix = s_prefix, mask = s_mask, rem = s_rem;
    s_hist[tid] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int i = (j * kTopkThreads + tid) * 4;
      const u32x4 w = s_keys[j * kTopkThreads + tid];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (i + e < nk && (w[e] & mask) == prefix) atomicAdd(&s_hist[(w[e] >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (s_hist[tid]) atomicAdd(fs + p * 256 + tid, s_hist[tid]);
    unit_arrive_wait(fs + 768 + p, (uint32_t)cmax, limit, err);
    s_hist[tid] = __hip_atomic_load(fs + p * 256 + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (tid < 64) {
      uint32_t d, above;
      pick_digit(s_hist, rem, d, above);
      if (tid == 0) {
        s_prefix = prefix | (d << shift);
        s_mask = mask | (255u << shift);
        s_rem = rem - above;
      }
    }
    __syncthreads();
  }
  // T = the k-th largest key; `need` of the keys equal to T are taken, the first by index
  const uint32_t T = s_prefix, need = s_rem;
  uint32_t cg = 0, ce = 0;
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int i = (j * kTopkThreads + tid) * 4;
    const u32x4 w = s_keys[j * kTopkThreads + tid];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      cg += (i + e < nk) && w[e] > T;
      ce += (i + e < nk) && w[e] == T;
    }
  }
  uint32_t tg, te;
  block_sum2(cg, ce, s_x, s_y, tg, te);
  uint32_t* cc = ccnt + (int64_t)u * cmax * kChunkHist;
  if (tid == 0) {
    __hip_atomic_store(cc + (int64_t)c * kChunkHist, tg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(cc + (int64_t)c * kChunkHist + 1, te, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  unit_arrive_wait(fs + 768 + 3, (uint32_t)cmax, limit, err);
  // winners in the earlier chunks
  uint32_t base_g, base_e;
  {
    uint32_t g = 0, e = 0;
    if (tid < c) {
      g = __hip_atomic_load(cc + (int64_t)tid * kChunkHist, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      e = __hip_atomic_load(cc + (int64_t)tid * kChunkHist + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    block_sum2(g, e, s_x, s_y, base_g, base_e);
  }
  // the winners of this chunk in ascending index order: tiles of kTopkThreads x
  // kTopkPerThread consecutive keys, a block-wide scan per tile
  int32_t* out = a.idx + (int64_t)u * a.k;
  constexpr int kTile = kTopkThreads * kTopkPerThread;
  for (int t0 = 0; t0 < nk; t0 += kTile) {  // uniform per block
    const int i0 = t0 + tid * kTopkPerThread;
    u32x4 v[kTopkPerThread / 4];
#pragma unroll
    for (int j = 0; j < kTopkPerThread / 4; ++j) v[j] = s_keys[(i0 >> 2) + j];
    uint32_t xg = 0, xe = 0;
#pragma unroll
    for (int j = 0; j < kTopkPerThread / 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool valid = i0 + 4 * j + e < nk;
        xg += valid && v[j][e] > T;
        xe += valid && v[j][e] == T;
      }
    uint32_t eg, ee, sg, se;
    scan2(xg, xe, s_x, s_y, eg, ee, sg, se);
    uint32_t pg = base_g + eg, pe = base_e + ee;
#pragma unroll
    for (int j = 0; j < kTopkPerThread / 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + 4 * j + e;
        if (i >= nk) continue;
        const uint32_t kv = v[j][e];
        if (kv > T) {
          const uint32_t pos = pg + (pe < need ? pe : need);
          if (pos < (uint32_t)a.k) out[pos] = (int32_t)(c0 + i);
          ++pg;
        } else if (kv == T) {
          if (pe < need && pg + pe < (uint32_t)a.k) out[pg + pe] = (int32_t)(c0 + i);
          ++pe;
        }
      }
    base_g += sg;
    base_e += se;
  }
}

__global__ __launch_bounds__(kTopkThreads) void topk_fused_kernel(LayerArgs a, Span sp,
                                                                  const uint32_t* __restrict__ keys,
                                                                  const uint32_t* __restrict__ h0,
                                                                  uint32_t* __restrict__ fsync,
                                                                  uint32_t* __restrict__ ccnt, int cmax,
                                                                  uint32_t limit) {
  const int lo = *sp.lo;
  const int n_units = *sp.hi - lo;
  const int groups = (int)(gridDim.x / cmax);
  const int c = (int)(blockIdx.x % cmax);
  for (int ui = (int)(blockIdx.x / cmax); ui < n_units; ui += groups)  // the same units for a group's blocks
    topk_fused_unit(a, sp.list[lo + ui], c, cmax, keys, h0, fsync, ccnt, limit, a.err);
}

// The one-launch top-k of a multi-layer selection: the groups take the miss
// units of all the batch's layers in turn.
__global__ __launch_bounds__(kTopkThreads) void topk_fused_layers_kernel(const SelectPlanLayer* __restrict__ plan,
                                                                         const SelectPlanHeader* __restrict__ hdr,
                                                                         int first, int count, int cmax,
                                                                         uint32_t limit, uint32_t* err) {
  __shared__ int32_t s_pref[kMaxSelectBatch + 1];
  load_miss_prefix(plan, hdr, first, count, s_pref);
  const int total = s_pref[count];
  const int groups = (int)(gridDim.x / cmax);
  const int c = (int)(blockIdx.x % cmax);
  for (int gu = (int)(blockIdx.x / cmax); gu < total; gu += groups) {
    const int j = layer_of(s_pref, gu);
    const SelectPlanLayer& L = plan[first + j];
    if ((L.a.N + kTopkChunk - 1) / kTopkChunk != cmax) {  // not the launch's chunk count: reported, skipped
      if (err && threadIdx.x == 0) atomicCAS(err, 0u, (uint32_t)CLO_E_ARG);
      continue;
    }
    topk_fused_unit(L.a, L.w.list_all[gu - s_pref[j]], c, cmax, L.w.keys, L.w.h0, L.w.fsync, L.w.chist, limit,
                    err);
  }
}

// ---------------------------------------------------------------- A3 top-k over token blocks
// Block b of a unit covers tokens b*bs .. b*bs+bs-1 (full blocks only); its key is
// the largest of its tokens' keys (= the key of its best score).  Each CTA takes
// kBlockKeysPerCta blocks of one unit, writes their keys, counts their digit 1
// into the unit's block histogram (h0b, cleared by the compact kernel), and the
// CTA with the unit's first chunk clears h1 and resets the radix state: the top-k
// kernels then select among the block keys as they do among token keys.
constexpr int kBlockKeysPerCta = 4096;

__global__ __launch_bounds__(256) void block_keys_kernel(LayerArgs a, Span sp, const uint32_t* __restrict__ keys,
                                                         uint32_t* __restrict__ bkeys, int64_t nb, int64_t npb,
                                                         int cmaxb, uint32_t* __restrict__ h0b,
                                                         uint32_t* __restrict__ h1, TopkState* __restrict__ st,
                                                         int64_t kb, uint32_t* __restrict__ fs) {
  __shared__ uint32_t s_h[4][256];
  const UnitChunk uc = unit_chunk(sp, cmaxb);
  if (!uc.valid) return;
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int i = tid; i < 4 * 256; i += 256) (&s_h[0][0])[i] = 0u;
  __syncthreads();
  const uint32_t* kk = keys + (int64_t)uc.u * a.Np;
  uint32_t* bo = bkeys + (int64_t)uc.u * npb;
  const int64_t j0 = (int64_t)uc.c * kBlockKeysPerCta;
  const int64_t j1 = (j0 + kBlockKeysPerCta < nb) ? j0 + kBlockKeysPerCta : nb;
  for (int64_t j = j0 + tid; j < j1; j += 256) {
    const uint32_t* t = kk + j * a.bs;
    uint32_t m = 0u;
    if ((a.bs & 3) == 0) {
      for (int i = 0; i < a.bs; i += 4) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(t + i);
        m = max(max(m, max(v[0], v[1])), max(v[2], v[3]));
      }
    } else {
      for (int i = 0; i < a.bs; ++i) m = max(m, t[i]);
    }
    bo[j] = m;
    atomicAdd(&s_h[wave][m >> 24], 1u);
  }
  __syncthreads();
  const uint32_t sum = s_h[0][tid] + s_h[1][tid] + s_h[2][tid] + s_h[3][tid];
  if (sum) atomicAdd(h0b + (int64_t)uc.u * 256 + tid, sum);
  if (uc.c == 0) {
    h1[(int64_t)uc.u * 256 + tid] = 0u;
    if (tid == 0) st[uc.u] = TopkState{0u, 0u, (uint32_t)kb, 0u};
    clear_fused_sync(fs, uc.u);
  }
}

// idx[u][i] = the i-th token of the unit's selected blocks (blocks ascending).
__global__ __launch_bounds__(256) void expand_blocks_kernel(LayerArgs a, Span sp, const int32_t* __restrict__ bidx,
                                                            int64_t kb, int cmaxe) {
  const UnitChunk uc = unit_chunk(sp, cmaxe);
  if (!uc.valid) return;
  const int64_t i0 = (int64_t)uc.c * 1024;
  const int64_t i1 = (i0 + 1024 < a.k) ? i0 + 1024 : a.k;
  for (int64_t i = i0 + threadIdx.x; i < i1; i += 256)
    a.idx[(int64_t)uc.u * a.k + i] = bidx[(int64_t)uc.u * kb + i / a.bs] * a.bs + (int32_t)(i % a.bs);
}

}  // namespace

hipError_t launch_reuse(const LayerArgs& a, const void* q, const void* q_prev, uint8_t* reuse, float* cos,
                        hipStream_t s) {
  const int U = a.B * a.Hkv;
  HeadTau th;
  for (int h = 0; h < kMaxKvHeads; ++h) th.t[h] = a.tau_h[h];
  if (a.dtype == CLO_F32)
    reuse_kernel<float><<<U, 64, 0, s>>>(static_cast<const float*>(q), static_cast<const float*>(q_prev), reuse,
                                         cos, a.Hkv, a.Hq, a.G, th);
  else
    reuse_kernel<uint16_t><<<U, 64, 0, s>>>(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(q_prev),
                                            reuse, cos, a.Hkv, a.Hq, a.G, th);
  return hipGetLastError();
}

hipError_t launch_reuse_compact(const LayerArgs& a, const void* q, const void* q_prev, uint8_t* reuse, float* cos,
                                const Workspace& w, const uint32_t* wait_flag, uint32_t wait_value, uint32_t limit,
                                uint32_t* error_word, hipStream_t s) {
  const int U = a.B * a.Hkv;
  if (U > kFusedReuseUnits) return hipErrorInvalidValue;
  HeadTau th;
  for (int h = 0; h < kMaxKvHeads; ++h) th.t[h] = a.tau_h[h];
  uint32_t* h0b = a.bs > 1 ? w.h0b : nullptr;
  if (a.dtype == CLO_F32)
    reuse_compact_kernel<float><<<1, 1024, 0, s>>>(static_cast<const float*>(q), static_cast<const float*>(q_prev),
                                                   reuse, cos, a.Hkv, a.Hq, a.G, th, U, a.pmask, w.meta, w.list_all,
                                                   w.list_host, w.list_hit, w.h0, h0b, wait_flag, wait_value, limit,
                                                   error_word);
  else
    reuse_compact_kernel<uint16_t><<<1, 1024, 0, s>>>(static_cast<const uint16_t*>(q),
                                                      static_cast<const uint16_t*>(q_prev), reuse, cos, a.Hkv, a.Hq,
                                                      a.G, th, U, a.pmask, w.meta, w.list_all, w.list_host,
                                                      w.list_hit, w.h0, h0b, wait_flag, wait_value, limit,
                                                      error_word);
  return hipGetLastError();
}

hipError_t launch_compact(const LayerArgs& a, const uint8_t* reuse, const Workspace& w, int ranges,
                          const RangeBounds& bounds, hipStream_t s) {
  compact_kernel<<<1, 1024, 0, s>>>(reuse, a.B * a.Hkv, a.Hkv, a.pmask, ranges, bounds, w.meta, w.list_all,
                                    w.list_host, w.list_hit, w.h0, a.bs > 1 ? w.h0b : nullptr);
  return hipGetLastError();
}

hipError_t launch_score(const LayerArgs& a, const void* q, Span sp, int64_t max_units, const Workspace& w,
                        uint32_t* counter, int num_cu, hipStream_t s) {
  uint32_t* keys = w.keys;
  return dispatch_group(a.G, [&](auto gc) {
    constexpr int G = decltype(gc)::value;
    if (a.dtype == CLO_F32) {
      const int64_t nch = (a.N + kScoreChunk - 1) / kScoreChunk;
      const int grid = grid_cap(max_units * nch, (int64_t)num_cu * 32);
      score_kernel<float, G><<<grid, 256, 0, s>>>(a, static_cast<const float*>(q), sp, keys, w.h0, w.h1, w.tstate,
                                                  w.fsync);
    } else {
      // persistent: two blocks (eight waves) per CU keep enough 16-byte loads in
      // flight to stream K; more blocks only add contention
      const int64_t nch = (a.N + kScoreItem - 1) / kScoreItem;
      const int grid = grid_cap(max_units * nch, (int64_t)num_cu * 2);
      score_mfma_kernel<G><<<grid, 256, 0, s>>>(a, static_cast<const uint16_t*>(q), sp, keys, counter, w.h0, w.h1,
                                                 w.tstate, w.fsync);
    }
    return hipGetLastError();
  });
}

hipError_t launch_topk(const LayerArgs& a, Span sp, int64_t max_units, const uint32_t* keys, const Workspace& w,
                       hipStream_t s) {
  const int cmax = w.cmax;
  if (cmax < kTopkMultiMin) {
    const int grid = grid_cap(max_units, 4096);
    topk_unit_kernel<<<grid, kUnitThreads, 0, s>>>(a, sp, keys, w.h0);
    return hipGetLastError();
  }
  if (cmax <= kFusedMaxBlocks) {
    // one launch: groups of cmax blocks, as many groups as the units need and
    // kFusedMaxBlocks allows
    const int64_t units = max_units > 0 ? max_units : 1;
    const int64_t groups = units < kFusedMaxBlocks / cmax ? units : kFusedMaxBlocks / cmax;
    topk_fused_kernel<<<(unsigned)(groups * cmax), kTopkThreads, 0, s>>>(a, sp, keys, w.h0, w.fsync, w.chist, cmax,
                                                                        1u << 20);
    return hipGetLastError();
  }
  const int64_t grid = max_units * cmax;
  const unsigned cg = (unsigned)(grid > 0 ? grid : 1);
  for (int shift = 16; shift >= 0; shift -= 8)
    topk_pass_kernel<<<cg, kTopkThreads, 0, s>>>(a, sp, keys, w.h0, w.h1, w.tstate, w.chist, cmax, shift);
  topk_write_kernel<<<cg, kTopkThreads, 0, s>>>(a, sp, keys, w.tstate, w.chist, cmax);
  return hipGetLastError();
}

hipError_t launch_select_layers(const SelectPlanLayer* plan, SelectPlanHeader* hdr, int first, int count,
                                const LayerArgs& a, int cmax, uint32_t wait_value, uint32_t signal_value,
                                uint32_t limit, uint32_t* error_word, int num_cu, hipStream_t s) {
  if (count < 1 || count > kMaxSelectBatch || a.dtype != CLO_BF16 || a.B * a.Hkv > kFusedReuseUnits ||
      cmax > kFusedMaxBlocks)
    return hipErrorInvalidValue;
  const int64_t U = (int64_t)a.B * a.Hkv;
  reuse_compact_layers_kernel<uint16_t><<<(unsigned)count, 1024, 0, s>>>(plan, hdr, first, wait_value, limit,
                                                                         error_word);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = dispatch_group(a.G, [&](auto gc) {
    constexpr int G = decltype(gc)::value;
    const int64_t nch = (a.N + kScoreItem - 1) / kScoreItem;
    const int grid = grid_cap(count * U * nch, (int64_t)num_cu * 2);
    score_mfma_layers_kernel<G><<<grid, 256, 0, s>>>(plan, hdr, first, count, error_word);
    return hipGetLastError();
  });
  if (e != hipSuccess) return e;
  if (cmax < kTopkMultiMin) {
    const int grid = grid_cap(count * U, 4096);
    topk_unit_layers_kernel<<<grid, kUnitThreads, 0, s>>>(plan, hdr, first, count);
  } else {
    const int64_t units = count * U;
    const int64_t groups = units < kFusedMaxBlocks / cmax ? units : kFusedMaxBlocks / cmax;
    topk_fused_layers_kernel<<<(unsigned)(groups * cmax), kTopkThreads, 0, s>>>(plan, hdr, first, count, cmax,
                                                                               1u << 20, error_word);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  signal_layers_kernel<<<1, 64, 0, s>>>(plan, hdr, first, count, signal_value);
  return hipGetLastError();
}

hipError_t launch_select(const LayerArgs& a, Span sp, int64_t max_units, const Workspace& w, hipStream_t s) {
  if (a.bs <= 1) return launch_topk(a, sp, max_units, w.keys, w, s);
  const int64_t nb = a.N / a.bs, kb = a.k / a.bs;
  LayerArgs ab = a;  // the blocks as the "tokens" of a top-k
  ab.N = nb;
  ab.k = kb;
  ab.Np = w.npb;
  ab.idx = w.bidx;
  ab.bs = 1;
  Workspace wb = w;
  wb.h0 = w.h0b;
  wb.keys = w.bkeys;
  wb.cmax = (int32_t)((nb + kTopkChunk - 1) / kTopkChunk);
  const int cmaxb = (int)((nb + kBlockKeysPerCta - 1) / kBlockKeysPerCta);
  const unsigned g1 = (unsigned)(max_units * cmaxb > 0 ? max_units * cmaxb : 1);
  block_keys_kernel<<<g1, 256, 0, s>>>(a, sp, w.keys, w.bkeys, nb, w.npb, cmaxb, w.h0b, w.h1, w.tstate, kb,
                                       w.fsync);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = launch_topk(ab, sp, max_units, w.bkeys, wb, s)) != hipSuccess) return e;
  const int cmaxe = (int)((a.k + 1023) / 1024);
  const unsigned g2 = (unsigned)(max_units * cmaxe > 0 ? max_units * cmaxe : 1);
  expand_blocks_kernel<<<g2, 256, 0, s>>>(a, sp, w.bidx, kb, cmaxe);
  return hipGetLastError();
}

}  // namespace clo
