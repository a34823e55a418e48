// HIP kernels of the sparse attention (gfx950), A5: softmax attention over the
// selected rows, split over chunks of rows and merged with the usual max/sum
// rescale ("CLO (2511.14510) -- L3 Per-Paper Synthesis", section 2.3 table).
#include <math.h>

#include <type_traits>

#include "../../include/clo.h"
#include "clo_device.h"
#include "clo_internal.h"

namespace clo {
namespace {

// ---------------------------------------------------------------- A5 attention
// Work item = (unit, chunk of kAttnChunk selected rows).  Phase 1: logits of
// every (head, row) into LDS; phase 2: per-head max and exp-sum; phase 3:
// p-weighted V sum.  In phases 1 and 3 a row is read by 16 lanes, 16 bytes
// each (bf16: 8 elements; fp32: 8 elements = two 16-byte pieces), 4 rows per
// wave instruction, and each lane issues kAttnBatch rows' loads before it
// uses any of them.  The partial (o, m, l) of each chunk is merged by
// attn_combine_kernel.
constexpr int kAttnBatch = 8;

template <typename T>
struct Row8;  // raw 8 elements of a row as loaded
template <>
struct Row8<uint16_t> {
  u32x4 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ void unpack(float (&x)[8]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf_lo(w[i]);
      x[2 * i + 1] = bf_hi(w[i]);
    }
  }
};
template <>
struct Row8<float> {
  u32x4 w0, w1;
  __device__ __forceinline__ void load(const float* p) {
    w0 = *reinterpret_cast<const u32x4*>(p);
    w1 = *reinterpret_cast<const u32x4*>(p + 4);
  }
  __device__ __forceinline__ void unpack(float (&x)[8]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = __uint_as_float(w0[i]);
      x[4 + i] = __uint_as_float(w1[i]);
    }
  }
};

// The partial of unit u's chunk c, by one 256-thread block (an index out of
// range is reported in *err).
template <typename T, int G>
__device__ __forceinline__ void attn_partial_item(const LayerArgs& a, const T* __restrict__ q,
                                                  float* __restrict__ part, int nch, int u, int c, uint32_t* err) {
  __shared__ float lg[G][kAttnChunk];
  __shared__ float red[4][G][kHeadDim];
  __shared__ float sm[G], sl[G];
  const int b = u / a.Hkv, h = u % a.Hkv;
  const bool pers = (a.pmask >> h) & 1ull;
  const int64_t r0 = (int64_t)c * kAttnChunk;
  const int nrows = (int)((a.k - r0) < kAttnChunk ? (a.k - r0) : kAttnChunk);
  const int32_t* ix = a.idx + (int64_t)u * a.k + r0;
  const T* kbase;
  const T* vbase;
  if (pers) {
    const int64_t s = ((int64_t)b * a.P + head_slot(a.pmask, h)) * a.C * kHeadDim;
    kbase = static_cast<const T*>(a.k_hbm) + s;
    vbase = static_cast<const T*>(a.v_hbm) + s;
  } else {
    const int64_t s = (((int64_t)b * a.H + head_slot(a.pmask, h)) * a.k + r0) * kHeadDim;
    kbase = static_cast<const T*>(a.k_cache) + s;
    vbase = static_cast<const T*>(a.v_cache) + s;
  }
  // row of the source tensor holding selected row i (< nrows) of this chunk
  auto row_of = [&](int i) -> int64_t { return pers ? checked_row(ix[i], a.N, err) : (int64_t)i; };
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane & 15, rg = lane >> 4;
  const float scale = 0.08838834764831845f;  // 1 / sqrt(128)
  // this lane's rows: wave w owns rows [64 w, 64 w + 64); row group rg takes every 4th
  const int row_base = wave * 64 + rg;

  // phase 1: logits
  if constexpr (sizeof(T) == 2) {
    // bf16: on the matrix cores, as in scoring.  Wave w takes its 64 rows as four
    // 16-row tiles: D[head][row] = sum over 128 dims of Q[head] K[row], A = the
    // unit's G query heads padded to 16 rows, B = 16 rows x 32 dims per k-step,
    // each lane loading 16-byte pieces of its row straight into B registers.
    // D leaves heads 4 (lane / 16) .. + 3 of row (lane % 16) in each lane.
    const int col = lane & 15, ks = lane >> 4;
    bf16x8 qa[4];
    {
      const uint16_t* qh = reinterpret_cast<const uint16_t*>(q) +
                           ((int64_t)b * a.Hq + (int64_t)h * G + (col < G ? col : 0)) * kHeadDim;
      const uint32_t keep = col < G ? ~0u : 0u;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(qh + s4 * 32 + ks * 8);
        qa[s4] = __builtin_bit_cast(bf16x8, w & keep);
      }
    }
    const T* kb16 = kbase;
#pragma unroll
    for (int t0 = 0; t0 < 4; t0 += 2) {
      u32x4 kt[2][4];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int i = wave * 64 + (t0 + t) * 16 + col;
        const T* kr = kb16 + row_of(i < nrows ? i : nrows - 1) * kHeadDim + ks * 8;
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) kt[t][s4] = *reinterpret_cast<const u32x4*>(kr + s4 * 32);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s4], __builtin_bit_cast(bf16x8, kt[t][s4]), acc, 0, 0, 0);
        const int i = wave * 64 + (t0 + t) * 16 + col;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int g = ks * 4 + r;
          if (g < G) lg[g][i] = (i < nrows) ? acc[r] * scale : kNegInf;
        }
      }
    }
  } else {
    float qv[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) load8(q + ((int64_t)b * a.Hq + (int64_t)h * G + g) * kHeadDim + sub * 8, qv[g]);
#pragma unroll
    for (int j0 = 0; j0 < 16; j0 += kAttnBatch) {
      Row8<T> kr[kAttnBatch];
#pragma unroll
      for (int j = 0; j < kAttnBatch; ++j) {
        const int i = row_base + 4 * (j0 + j);
        kr[j].load(kbase + row_of(i < nrows ? i : nrows - 1) * kHeadDim + sub * 8);
      }
#pragma unroll
      for (int j = 0; j < kAttnBatch; ++j) {
        const int i = row_base + 4 * (j0 + j);
        float kx[8];
        kr[j].unpack(kx);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float s = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) s = fmaf(qv[g][e], kx[e], s);
          s = sum16(s);
          if (sub == 0) lg[g][i] = (i < nrows) ? s * scale : kNegInf;
        }
      }
    }
  }
  // the first batch of V rows is requested now, so that its loads are in flight
  // across the softmax phase
  Row8<T> vpre[kAttnBatch];
#pragma unroll
  for (int j = 0; j < kAttnBatch; ++j) {
    const int i = row_base + 4 * j;
    vpre[j].load(vbase + row_of(i < nrows ? i : nrows - 1) * kHeadDim + sub * 8);
  }
  __syncthreads();
  // phase 2: softmax statistics per head
  for (int g = wave; g < G; g += 4) {
    float m = kNegInf;
    for (int i = lane; i < kAttnChunk; i += 64) m = fmaxf(m, lg[g][i]);
    m = wave_max(m);
    float s = 0.f;
    for (int i = lane; i < kAttnChunk; i += 64) {
      const float p = (i < nrows) ? expf(lg[g][i] - m) : 0.f;
      lg[g][i] = p;
      s += p;
    }
    s = wave_sum(s);
    if (lane == 0) {
      sm[g] = m;
      sl[g] = s;
    }
  }
  __syncthreads();
  // phase 3: p-weighted sum of V rows, columns 8 sub .. 8 sub + 7 in this lane
  {
    float acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
#pragma unroll
    for (int j0 = 0; j0 < 16; j0 += kAttnBatch) {
      Row8<T> vr[kAttnBatch];
#pragma unroll
      for (int j = 0; j < kAttnBatch; ++j) {
        const int i = row_base + 4 * (j0 + j);
        if (j0 == 0)
          vr[j] = vpre[j];
        else
          vr[j].load(vbase + row_of(i < nrows ? i : nrows - 1) * kHeadDim + sub * 8);
      }
#pragma unroll
      for (int j = 0; j < kAttnBatch; ++j) {
        const int i = row_base + 4 * (j0 + j);
        float vx[8];
        vr[j].unpack(vx);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float p = lg[g][i];  // 0 past the last valid row
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(p, vx[e], acc[g][e]);
        }
      }
    }
    // sum the four row groups of the wave (lanes sub, sub + 16, sub + 32, sub + 48)
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = acc[g][e];
        x += __shfl_xor(x, 16, 64);
        x += __shfl_xor(x, 32, 64);
        acc[g][e] = x;
      }
    if (rg == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) red[wave][g][sub * 8 + e] = acc[g][e];
    }
  }
  __syncthreads();
  float* dst = part + ((int64_t)u * nch + c) * G * kPartStride;
  for (int t = tid; t < G * kHeadDim; t += 256) {
    const int g = t / kHeadDim, col = t % kHeadDim;
    dst[g * kPartStride + col] = (red[0][g][col] + red[1][g][col]) + (red[2][g][col] + red[3][g][col]);
  }
  if (tid < G) {
    dst[tid * kPartStride + kHeadDim] = sm[tid];
    dst[tid * kPartStride + kHeadDim + 1] = sl[tid];
  }
}

template <typename T, int G>
__global__ __launch_bounds__(256) void attn_partial_kernel(LayerArgs a, const T* __restrict__ q,
                                                           float* __restrict__ part, int nch, Span sp) {
  int u;
  if (sp.list) {
    const int lo = *sp.lo;
    if ((int64_t)blockIdx.x >= (int64_t)(*sp.hi - lo) * nch) return;  // whole block
    u = sp.list[lo + blockIdx.x / nch];
  } else {
    u = blockIdx.x / nch;
  }
  attn_partial_item<T, G>(a, q, part, nch, u, (int)(blockIdx.x % nch), a.err);
}

// Merge the chunk partials of one (unit, head) with the usual max/sum
// rescaling.  S groups of 128 threads (one per output column) each merge a
// contiguous run of the chunks, kAttnBatch chunks' partials loaded before any is
// used; group 0 then merges the S group results from LDS.  Long selections
// (many chunks, few units) take S up to 8, so that no single thread walks
// hundreds of chunks one load latency after another.
template <typename T, int S>
__device__ __forceinline__ void attn_combine_item(const LayerArgs& a, const float* __restrict__ part, int nch,
                                                  T* __restrict__ out, int u, int g) {
  __shared__ float sM[S], sL[S], sO[S][kHeadDim];
  const int G = a.G;
  const int b = u / a.Hkv, h = u % a.Hkv;
  const int grp = threadIdx.x / kHeadDim, col = threadIdx.x % kHeadDim;
  const int per = (nch + S - 1) / S;
  const int cb = grp * per, ce = (cb + per < nch) ? cb + per : nch;
  const float* p = part + ((int64_t)u * nch * G + g) * kPartStride;
  const int64_t cstride = (int64_t)G * kPartStride;
  float M = kNegInf, L = 0.f, O = 0.f;
  for (int c0 = cb; c0 < ce; c0 += kAttnBatch) {
    float m[kAttnBatch], l[kAttnBatch], o[kAttnBatch];
#pragma unroll
    for (int j = 0; j < kAttnBatch; ++j) {
      const int c = c0 + j < ce ? c0 + j : ce - 1;
      m[j] = p[c * cstride + kHeadDim];
      l[j] = p[c * cstride + kHeadDim + 1];
      o[j] = p[c * cstride + col];
    }
#pragma unroll
    for (int j = 0; j < kAttnBatch; ++j) {
      if (c0 + j >= ce) break;
      const float Mn = fmaxf(M, m[j]);
      const float sa = expf(M - Mn), sb = expf(m[j] - Mn);
      L = L * sa + l[j] * sb;
      O = O * sa + o[j] * sb;
      M = Mn;
    }
  }
  if (S == 1) {
    store_out(out + ((int64_t)b * a.Hq + (int64_t)h * G + g) * kHeadDim + col, O / L);
    return;
  }
  if (col == 0) {
    sM[grp] = M;
    sL[grp] = L;
  }
  sO[grp][col] = O;
  __syncthreads();
  if (grp != 0) return;
  // group 0 holds at least one chunk, so Mx is finite; empty groups (M = -inf) weigh 0
  float Mx = sM[0];
#pragma unroll
  for (int i = 1; i < S; ++i) Mx = fmaxf(Mx, sM[i]);
  float Lt = 0.f, Ot = 0.f;
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const float w = expf(sM[i] - Mx);
    Lt += sL[i] * w;
    Ot += sO[i][col] * w;
  }
  store_out(out + ((int64_t)b * a.Hq + (int64_t)h * G + g) * kHeadDim + col, Ot / Lt);
}

template <typename T, int S>
__global__ __launch_bounds__(128 * S) void attn_combine_kernel(LayerArgs a, const float* __restrict__ part, int nch,
                                                               Span sp, T* __restrict__ out) {
  const int i = blockIdx.x / a.G, g = blockIdx.x % a.G;
  int u = i;
  if (sp.list) {
    const int lo = *sp.lo;
    if (i >= *sp.hi - lo) return;  // uniform per block
    u = sp.list[lo + i];
  }
  attn_combine_item<T, S>(a, part, nch, out, u, g);
}

// ---------------------------------------------------------------- many layers
// The attention of plan layers first .. first + count - 1 (every unit of each)
// in four launches: a one-wave wait for every layer's rows (lane j polls layer
// j's flag), the partials of all the layers' (unit, chunk) items, their
// combines, and a one-wave launch storing the signal value to every layer's
// flag.  The per-item bodies are the single-layer kernels'.  A launch past the
// plan's layers, or a layer whose shape is not the launch's, is reported
// (CLO_E_ARG) and does nothing.
__device__ __forceinline__ bool attend_layer_ok(const AttendPlanLayer& L, const AttendPlanHeader* hdr, int first,
                                                int count, const LayerArgs& shape, uint32_t* err) {
  const bool ok = (uint32_t)(first + count) <= hdr->n_layers && L.a.B == shape.B && L.a.Hq == shape.Hq &&
                  L.a.Hkv == shape.Hkv && L.a.k == shape.k && L.a.dtype == shape.dtype;
  if (!ok && threadIdx.x == 0 && err) atomicCAS(err, 0u, (uint32_t)CLO_E_ARG);
  return ok;
}

__global__ __launch_bounds__(64) void attend_wait_layers_kernel(const AttendPlanLayer* __restrict__ plan,
                                                                const AttendPlanHeader* __restrict__ hdr, int first,
                                                                int count, uint32_t wait_value, uint32_t limit,
                                                                uint32_t* err) {
  const int j = (int)threadIdx.x;
  if (j >= count || (uint32_t)(first + count) > hdr->n_layers) return;
  const uint32_t* f = plan[first + j].wait_flag;
  if (f) poll_flag(f, wait_value, limit, err);
}

template <typename T, int G>
__global__ __launch_bounds__(256) void attn_partial_layers_kernel(const AttendPlanLayer* __restrict__ plan,
                                                                  const AttendPlanHeader* __restrict__ hdr,
                                                                  int first, int count, LayerArgs shape, int nch,
                                                                  uint32_t* err) {
  const int64_t per = (int64_t)shape.B * shape.Hkv * nch;  // items of one layer
  const int j = (int)(blockIdx.x / per);
  const int it = (int)(blockIdx.x % per);
  const AttendPlanLayer& L = plan[first + j];
  if (!attend_layer_ok(L, hdr, first, count, shape, err)) return;
  attn_partial_item<T, G>(L.a, static_cast<const T*>(L.q), L.part, nch, it / nch, it % nch, err);
}

template <typename T, int S>
__global__ __launch_bounds__(128 * S) void attn_combine_layers_kernel(const AttendPlanLayer* __restrict__ plan,
                                                                      const AttendPlanHeader* __restrict__ hdr,
                                                                      int first, int count, LayerArgs shape, int nch,
                                                                      uint32_t* err) {
  const int64_t per = (int64_t)shape.B * shape.Hkv * shape.G;  // (unit, head) pairs of one layer
  const int j = (int)(blockIdx.x / per);
  const int it = (int)(blockIdx.x % per);
  const AttendPlanLayer& L = plan[first + j];
  if (!attend_layer_ok(L, hdr, first, count, shape, err)) return;
  attn_combine_item<T, S>(L.a, L.part, nch, static_cast<T*>(L.out), it / shape.G, it % shape.G);
}

__global__ __launch_bounds__(64) void attend_signal_layers_kernel(const AttendPlanLayer* __restrict__ plan,
                                                                  const AttendPlanHeader* __restrict__ hdr,
                                                                  int first, int count, uint32_t signal_value) {
  const int j = (int)threadIdx.x;
  if (j >= count || (uint32_t)(first + count) > hdr->n_layers) return;
  uint32_t* f = plan[first + j].signal_flag;
  if (f) __hip_atomic_store(f, signal_value, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// chunk groups of the combine: about 16 or more chunks each
int combine_groups(int nch) { return nch > 64 ? 8 : nch > 32 ? 4 : nch > 16 ? 2 : 1; }

}  // namespace

hipError_t launch_attn_partial(const LayerArgs& a, const void* q, float* part, Span sp, int64_t max_units,
                               hipStream_t s) {
  const int nch = (int)((a.k + kAttnChunk - 1) / kAttnChunk);
  const unsigned grid = (unsigned)(max_units > 0 ? max_units * nch : 1);
  return dispatch_group(a.G, [&](auto gc) {
    constexpr int G = decltype(gc)::value;
    if (a.dtype == CLO_F32)
      attn_partial_kernel<float, G><<<grid, 256, 0, s>>>(a, static_cast<const float*>(q), part, nch, sp);
    else
      attn_partial_kernel<uint16_t, G><<<grid, 256, 0, s>>>(a, static_cast<const uint16_t*>(q), part, nch, sp);
    return hipGetLastError();
  });
}

hipError_t launch_attn_combine(const LayerArgs& a, const float* part, void* out, Span sp, int64_t max_units,
                               hipStream_t s) {
  const int nch = (int)((a.k + kAttnChunk - 1) / kAttnChunk);
  const int64_t units = sp.list ? max_units : (int64_t)a.B * a.Hkv;
  if (units <= 0) return hipSuccess;
  const unsigned grid = (unsigned)(units * a.G);
  const int S = combine_groups(nch);
  auto go = [&](auto sc) {
    constexpr int SG = decltype(sc)::value;
    if (a.dtype == CLO_F32)
      attn_combine_kernel<float, SG><<<grid, 128 * SG, 0, s>>>(a, part, nch, sp, static_cast<float*>(out));
    else
      attn_combine_kernel<uint16_t, SG><<<grid, 128 * SG, 0, s>>>(a, part, nch, sp, static_cast<uint16_t*>(out));
  };
  switch (S) {
    case 1: go(std::integral_constant<int, 1>{}); break;
    case 2: go(std::integral_constant<int, 2>{}); break;
    case 4: go(std::integral_constant<int, 4>{}); break;
    default: go(std::integral_constant<int, 8>{}); break;
  }
  return hipGetLastError();
}

hipError_t launch_attend_layers(const AttendPlanLayer* plan, const AttendPlanHeader* hdr, int first, int count,
                                const LayerArgs& shape, uint32_t wait_value, uint32_t signal_value, uint32_t limit,
                                uint32_t* err, hipStream_t s) {
  const int nch = (int)((shape.k + kAttnChunk - 1) / kAttnChunk);
  const int64_t U = (int64_t)shape.B * shape.Hkv;
  attend_wait_layers_kernel<<<1, 64, 0, s>>>(plan, hdr, first, count, wait_value, limit, err);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned pgrid = (unsigned)(count * U * nch);
  e = dispatch_group(shape.G, [&](auto gc) {
    constexpr int G = decltype(gc)::value;
    if (shape.dtype == CLO_F32)
      attn_partial_layers_kernel<float, G><<<pgrid, 256, 0, s>>>(plan, hdr, first, count, shape, nch, err);
    else
      attn_partial_layers_kernel<uint16_t, G><<<pgrid, 256, 0, s>>>(plan, hdr, first, count, shape, nch, err);
    return hipGetLastError();
  });
  if (e != hipSuccess) return e;
  const unsigned cgrid = (unsigned)(count * U * shape.G);
  auto go = [&](auto sc) {
    constexpr int SG = decltype(sc)::value;
    if (shape.dtype == CLO_F32)
      attn_combine_layers_kernel<float, SG><<<cgrid, 128 * SG, 0, s>>>(plan, hdr, first, count, shape, nch, err);
    else
      attn_combine_layers_kernel<uint16_t, SG><<<cgrid, 128 * SG, 0, s>>>(plan, hdr, first, count, shape, nch, err);
  };
  switch (combine_groups(nch)) {
    case 1: go(std::integral_constant<int, 1>{}); break;
    case 2: go(std::integral_constant<int, 2>{}); break;
    case 4: go(std::integral_constant<int, 4>{}); break;
    default: go(std::integral_constant<int, 8>{}); break;
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  attend_signal_layers_kernel<<<1, 64, 0, s>>>(plan, hdr, first, count, signal_value);
  return hipGetLastError();
}

}  // namespace clo
