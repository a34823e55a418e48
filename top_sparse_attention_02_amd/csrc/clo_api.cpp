#include <algorithm>
#include <vector>
// C ABI of the CLO decode-step library: host-side validation, workspace
// layout and the launch sequence of each entry point.  Declarations and the
// contract of every call are in include/clo.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstddef>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <cstdlib>
#include <mutex>

#include "../../include/clo.h"
#include "clo_internal.h"

using namespace clo;

namespace {

thread_local clo_status g_last_status = CLO_OK;
thread_local char g_last_msg[512] = "";

clo_status fail(clo_status st, const char* fmt, ...) {
  g_last_status = st;
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_msg, sizeof g_last_msg, fmt, ap);
  va_end(ap);
  return st;
}

clo_status ok() {
  return CLO_OK;
}

int num_cus() {
  static thread_local int dev = -1, n = 0;
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess) {
    (void)hipGetLastError();
    return 256;
  }
  if (d != dev) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      n = 256;
    }
    dev = d;
  }
  return n;
}

size_t esize(int32_t dtype) { return dtype == CLO_F32 ? 4 : 2; }

clo_status check_shape(const clo_shape* s) {
  if (!s) return fail(CLO_E_ARG, "shape is NULL");
  if (s->dtype != CLO_F32 && s->dtype != CLO_BF16) return fail(CLO_E_UNSUPPORTED, "dtype %d is not fp32 or bf16", s->dtype);
  if (s->head_dim != kHeadDim) return fail(CLO_E_UNSUPPORTED, "head_dim %d (only 128 is supported)", s->head_dim);
  if (s->batch < 0) return fail(CLO_E_ARG, "batch %d < 0", s->batch);
  if (s->n_kv_heads < 1 || s->n_kv_heads > kMaxKvHeads)
    return fail(CLO_E_ARG, "n_kv_heads %d outside 1..%d", s->n_kv_heads, kMaxKvHeads);
  if (s->n_q_heads < 1 || s->n_q_heads % s->n_kv_heads)
    return fail(CLO_E_ARG, "n_q_heads %d is not a positive multiple of n_kv_heads %d", s->n_q_heads, s->n_kv_heads);
  if (s->n_q_heads / s->n_kv_heads > kMaxGroup)
    return fail(CLO_E_UNSUPPORTED, "group size %d > %d", s->n_q_heads / s->n_kv_heads, kMaxGroup);
  if (s->context < 1 || s->context > (int64_t)INT32_MAX) return fail(CLO_E_ARG, "context %lld out of range", (long long)s->context);
  if (s->topk < 1 || s->topk > s->context)
    return fail(CLO_E_ARG, "topk %lld outside 1..context (%lld)", (long long)s->topk, (long long)s->context);
  if (s->block_size < 0 || s->block_size > 65536) return fail(CLO_E_ARG, "block_size %d outside 0..65536", s->block_size);
  if (s->block_size > 1) {
    if (s->topk % s->block_size)
      return fail(CLO_E_ARG, "topk %lld is not a multiple of block_size %d", (long long)s->topk, s->block_size);
    if (s->topk > s->context / s->block_size * s->block_size)
      return fail(CLO_E_ARG, "topk %lld exceeds the %lld tokens of the full blocks", (long long)s->topk,
                  (long long)(s->context / s->block_size * s->block_size));
  }
  if (s->capacity != 0 && (s->capacity < s->context || s->capacity > (int64_t)INT32_MAX))
    return fail(CLO_E_ARG, "capacity %lld outside context (%lld)..2^31-1", (long long)s->capacity,
                (long long)s->context);
  return ok();
}

// Device memory of this process (torch allocations, hipMalloc, managed).
clo_status check_device(const void* p, size_t bytes, const char* name, uintptr_t align = 16) {
  if (!p) return fail(CLO_E_ARG, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) & (align - 1))
    return fail(CLO_E_ARG, "%s is not %zu-byte aligned", name, (size_t)align);
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return fail(CLO_E_ARG, "%s is not memory known to HIP", name);
  }
  if (at.type != hipMemoryTypeDevice && at.type != hipMemoryTypeManaged && at.type != hipMemoryTypeUnified)
    return fail(CLO_E_ARG, "%s is not device memory (memory type %d)", name, (int)at.type);
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, const_cast<void*>(p)) == hipSuccess) {
    if (static_cast<const char*>(p) + bytes > static_cast<const char*>(base) + size)
      return fail(CLO_E_ARG, "%s: %zu bytes needed but the allocation ends %zu bytes after it", name, bytes,
                  (size_t)(static_cast<const char*>(base) + size - static_cast<const char*>(p)));
  } else {
    (void)hipGetLastError();
  }
  return ok();
}

// Pinned host memory the device can address; returns its device address.
clo_status check_host(const void* p, size_t bytes, const char* name, const void** dev) {
  if (!p) return fail(CLO_E_ARG, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) & 15u) return fail(CLO_E_ARG, "%s is not 16-byte aligned", name);
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return fail(CLO_E_ARG, "%s is not pinned host memory (pageable memory cannot be read by the GPU)", name);
  }
  if (at.type == hipMemoryTypeDevice) {
    *dev = p;  // device-resident copy: allowed, the gather then reads HBM
    return check_device(p, bytes, name);
  }
  if (at.type != hipMemoryTypeHost && at.type != hipMemoryTypeManaged && at.type != hipMemoryTypeUnified)
    return fail(CLO_E_ARG, "%s is not pinned host memory (memory type %d)", name, (int)at.type);
  if (!at.devicePointer) return fail(CLO_E_ARG, "%s is not mapped for device access", name);
  *dev = static_cast<const char*>(at.devicePointer) +
         (static_cast<const char*>(p) - static_cast<const char*>(at.hostPointer ? at.hostPointer : p));
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, const_cast<void*>(*dev)) == hipSuccess) {
    if (static_cast<const char*>(*dev) + bytes > static_cast<const char*>(base) + size)
      return fail(CLO_E_ARG, "%s: %zu bytes needed but the allocation is shorter", name, bytes);
  } else {
    (void)hipGetLastError();
  }
  return ok();
}

struct Plan {
  LayerArgs a;
  size_t e;     // element bytes
  int64_t U;    // units per layer
  int nch_attn;
};

clo_status make_plan(const clo_shape* s, uint64_t pmask, Plan* p) {
  clo_status st = check_shape(s);
  if (st) return st;
  if (s->n_kv_heads < 64 && (pmask >> s->n_kv_heads))
    return fail(CLO_E_ARG, "persistent_mask has bits at or above n_kv_heads (%d)", s->n_kv_heads);
  LayerArgs& a = p->a;
  memset(&a, 0, sizeof a);
  a.B = s->batch;
  a.Hq = s->n_q_heads;
  a.Hkv = s->n_kv_heads;
  a.G = s->n_q_heads / s->n_kv_heads;
  a.N = s->context;
  a.C = s->capacity ? s->capacity : s->context;
  a.bs = s->block_size > 1 ? s->block_size : 1;
  a.k = s->topk;
  a.Np = round_up(s->context, 64);
  a.tau = s->tau;
  for (int h = 0; h < kMaxKvHeads; ++h) a.tau_h[h] = (s->tau_heads && h < s->n_kv_heads) ? s->tau_heads[h] : s->tau;
  a.dtype = s->dtype;
  a.pmask = pmask;
  a.P = __builtin_popcountll(pmask);
  a.H = a.Hkv - a.P;
  p->e = esize(s->dtype);
  p->U = (int64_t)a.B * a.Hkv;
  p->nch_attn = (int)((a.k + kAttnChunk - 1) / kAttnChunk);
  // every grid and work-item count (at most units x 256-key chunks) fits in 31 bits
  if (p->U * ((a.N + 255) / 256) > (int64_t)INT32_MAX)
    return fail(CLO_E_ARG, "batch x n_kv_heads x context/256 = %lld exceeds 2^31-1",
                (long long)(p->U * ((a.N + 255) / 256)));
  return ok();
}

// Workspace layout: meta | list_all | list_host | list_hit | h0 | h1 | tstate | chist | keys | part,
// each 256-byte aligned.
struct WsLayout {
  size_t meta, list_all, list_host, list_hit, h0, h1, tstate, chist, keys, part, bkeys, h0b, bidx, fsync, total;
  int64_t npb;
  int cmax;
};

WsLayout ws_layout(const Plan& p) {
  WsLayout w;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (size_t)round_up((int64_t)bytes, 256);
    return at;
  };
  w.meta = take(kMetaInts * 4);
  w.list_all = take((size_t)p.U * 4);
  w.list_host = take((size_t)p.U * 4);
  w.list_hit = take((size_t)p.U * 4);
  w.cmax = (int)((p.a.N + kTopkChunk - 1) / kTopkChunk);
  w.h0 = take((size_t)p.U * 256 * 4);
  w.h1 = take((size_t)p.U * 256 * 4);
  w.tstate = take((size_t)p.U * sizeof(TopkState));
  w.fsync = take((size_t)p.U * kFusedSyncWords * 4);
  w.chist = take((size_t)p.U * (size_t)w.cmax * kChunkHist * 4);
  w.keys = take((size_t)p.U * (size_t)p.a.Np * 4);
  w.part = take((size_t)p.U * (size_t)p.nch_attn * (size_t)p.a.G * kPartStride * 4);
  w.bkeys = w.h0b = w.bidx = 0;
  w.npb = 0;
  if (p.a.bs > 1) {  // block selection
    w.npb = round_up(p.a.N / p.a.bs, 64);
    w.bkeys = take((size_t)p.U * (size_t)w.npb * 4);
    w.h0b = take((size_t)p.U * 256 * 4);
    w.bidx = take((size_t)p.U * (size_t)(p.a.k / p.a.bs) * 4);
  }
  w.total = off;
  return w;
}

// Carves the workspace into its parts.  trusted: ws is the library's own
// static scratch, whose extent is known, so the runtime is not asked about it.
clo_status bind_ws(const Plan& p, void* ws, size_t ws_bytes, Workspace* w, bool trusted = false) {
  const WsLayout L = ws_layout(p);
  if (!ws) return fail(CLO_E_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) & 255u) return fail(CLO_E_WORKSPACE, "workspace is not 256-byte aligned");
  if (ws_bytes < L.total) return fail(CLO_E_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, L.total);
  if (!trusted && check_device(ws, L.total, "workspace")) {
    char why[sizeof g_last_msg];
    memcpy(why, g_last_msg, sizeof why);
    return fail(CLO_E_WORKSPACE, "%s", why);
  }
  char* b = static_cast<char*>(ws);
  w->meta = reinterpret_cast<int32_t*>(b + L.meta);
  w->list_all = reinterpret_cast<int32_t*>(b + L.list_all);
  w->list_host = reinterpret_cast<int32_t*>(b + L.list_host);
  w->list_hit = reinterpret_cast<int32_t*>(b + L.list_hit);
  w->h0 = reinterpret_cast<uint32_t*>(b + L.h0);
  w->h1 = reinterpret_cast<uint32_t*>(b + L.h1);
  w->tstate = reinterpret_cast<TopkState*>(b + L.tstate);
  w->fsync = reinterpret_cast<uint32_t*>(b + L.fsync);
  w->chist = reinterpret_cast<uint32_t*>(b + L.chist);
  w->cmax = L.cmax;
  w->keys = reinterpret_cast<uint32_t*>(b + L.keys);
  w->part = reinterpret_cast<float*>(b + L.part);
  w->bkeys = p.a.bs > 1 ? reinterpret_cast<uint32_t*>(b + L.bkeys) : nullptr;
  w->h0b = p.a.bs > 1 ? reinterpret_cast<uint32_t*>(b + L.h0b) : nullptr;
  w->bidx = p.a.bs > 1 ? reinterpret_cast<int32_t*>(b + L.bidx) : nullptr;
  w->npb = L.npb;
  return ok();
}

Span span_all_misses(const Workspace& w) { return Span{w.list_all, w.meta + kMetaZero, w.meta + kMetaCountAll}; }
Span span_hits(const Workspace& w) { return Span{w.list_hit, w.meta + kMetaZero, w.meta + kMetaCountHit}; }
Span span_range(const Workspace& w, int r) {
  return Span{w.list_all, w.meta + kMetaOffAll + r, w.meta + kMetaOffAll + r + 1};
}
Span span_host_range(const Workspace& w, int r) {
  return Span{w.list_host, w.meta + kMetaOffHost + r, w.meta + kMetaOffHost + r + 1};
}
constexpr Span kAllUnits{nullptr, nullptr, nullptr};

RangeBounds one_range(const Plan& p) {
  RangeBounds rb{};
  rb.first[1] = (int32_t)p.U;
  return rb;
}
uint32_t* score_counter(const Workspace& w, int r) { return reinterpret_cast<uint32_t*>(w.meta + kMetaScore + r); }

// CUs the scoring of the ranges (or batches of layers) from `first` on is
// spread over (two persistent blocks each).  The first range's scoring runs
// alone and takes every CU; the later ones run beside the gather and the
// attention of earlier ranges, whose blocks find no registers left on a CU
// holding two scoring blocks.  At half the CUs, steps/s: B=16, N=32768
// 332.3-332.5 -> 333.2 (int4 rows 837-838 -> 862-865); B=64, N=131072
// unchanged at 81.9 (int4 rows 226-227 -> 229-230); the 48-layer loop at B=1,
// N=524288 unchanged at 56.0 (int8 rows 104.6-104.7 -> 105.2, int4 140.8-140.9
// -> 141.3-141.4).
int score_cus(int first, int cu) { return first == 0 ? cu : std::max(1, cu / 2); }

// Per-device helper streams and events of the overlapped decode step, created
// on first use and kept for the life of the process.  They hold no user data.
struct DeviceQueues {
  std::mutex mu;  // one decode step enqueues at a time per device
  bool ready = false;
  hipStream_t gather = nullptr;   // the gathers of the even unit ranges, or the resident gather
  hipStream_t gather2 = nullptr;  // the gathers of the odd unit ranges
  hipStream_t attend = nullptr;   // attention: reuse units first, then each range's misses
  hipEvent_t ev_lists = nullptr;     // unit lists and range flags ready (resident gather)
  hipEvent_t ev_gathered = nullptr;  // the resident gather ended
  hipEvent_t ev_attn = nullptr;      // the attention stream's work ended
  hipEvent_t ev_topk[kMaxRanges] = {}, ev_gather[kMaxRanges] = {};
  // timing events around the last overlapped step's gather launches (start; end
  // on each gather stream) and how many end events that step recorded
  hipEvent_t ev_g_start = nullptr, ev_g_end[2] = {};
  int g_ends = 0;
};

DeviceQueues g_queues[64];
std::mutex g_queues_init;

clo_status device_queues(DeviceQueues** out) {
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= 64) {
    (void)hipGetLastError();
    return fail(CLO_E_HIP, "no current HIP device");
  }
  DeviceQueues& q = g_queues[d];
  std::lock_guard<std::mutex> lk(g_queues_init);
  if (!q.ready) {
    hipError_t e = hipStreamCreateWithFlags(&q.gather, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&q.gather2, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&q.attend, hipStreamNonBlocking);
    for (hipEvent_t* ev : {&q.ev_lists, &q.ev_gathered, &q.ev_attn})
      if (e == hipSuccess) e = hipEventCreateWithFlags(ev, hipEventDisableTiming);
    for (int r = 0; r < kMaxRanges && e == hipSuccess; ++r) {
      e = hipEventCreateWithFlags(&q.ev_topk[r], hipEventDisableTiming);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&q.ev_gather[r], hipEventDisableTiming);
    }
    for (hipEvent_t* ev : {&q.ev_g_start, &q.ev_g_end[0], &q.ev_g_end[1]})
      if (e == hipSuccess) e = hipEventCreateWithFlags(ev, hipEventDefault);
    if (e != hipSuccess) return fail(CLO_E_HIP, "creating helper streams/events: %s", hipGetErrorString(e));
    q.ready = true;
  }
  *out = &q;
  return ok();
}

// Buffer sizes in bytes.
size_t q_bytes(const Plan& p) { return (size_t)p.a.B * p.a.Hq * kHeadDim * p.e; }
size_t full_bytes(const Plan& p, int heads) { return (size_t)p.a.B * heads * (size_t)p.a.C * kHeadDim * p.e; }
size_t cache_bytes(const Plan& p) { return (size_t)p.a.B * p.a.H * (size_t)p.a.k * kHeadDim * p.e; }
size_t idx_bytes(const Plan& p) { return (size_t)p.U * (size_t)p.a.k * 4; }

// Which layer buffers a call reads or writes.
enum Need : unsigned { NEED_SCORE = 1, NEED_HOST = 2, NEED_CACHE = 4, NEED_HBM_KV = 8, NEED_HBM_K = 16, NEED_IDX = 32 };

clo_status check_layer(const clo_layer* l, Plan* p, unsigned need) {
  if (!l) return fail(CLO_E_ARG, "layer is NULL");
  clo_status st;
  LayerArgs& a = p->a;
  if (need & NEED_IDX) {
    if ((st = check_device(l->idx, idx_bytes(*p), "layer.idx"))) return st;
    a.idx = l->idx;
  }
  if (a.P > 0 && (need & (NEED_HBM_KV | NEED_HBM_K))) {
    if ((st = check_device(l->k_hbm, full_bytes(*p, a.P), "layer.k_hbm"))) return st;
    a.k_hbm = l->k_hbm;
    if (need & NEED_HBM_KV) {
      if ((st = check_device(l->v_hbm, full_bytes(*p, a.P), "layer.v_hbm"))) return st;
      a.v_hbm = l->v_hbm;
    }
  }
  if (a.H > 0) {
    if (need & NEED_SCORE) {
      if ((st = check_device(l->k_score, full_bytes(*p, a.H), "layer.k_score"))) return st;
      a.k_score = l->k_score;
    }
    if (need & NEED_HOST) {
      const void* dk = nullptr;
      const void* dv = nullptr;
      if (l->host_format != CLO_HOST_NATIVE && l->host_format != CLO_HOST_INT8 && l->host_format != CLO_HOST_INT4)
        return fail(CLO_E_ARG, "layer.host_format %d is not a clo_host_format", l->host_format);
      a.host_fmt = l->host_format;
      const size_t rows = (size_t)a.B * a.H * (size_t)a.C;
      const bool quant = a.host_fmt != CLO_HOST_NATIVE;
      if (quant) {
        // one record (K values, then V values) per token; v_host unused
        if ((st = check_host(l->k_host, rows * 2 * quant_row_bytes(a.host_fmt), "layer.k_host", &dk))) return st;
      } else {
        if ((st = check_host(l->k_host, full_bytes(*p, a.H), "layer.k_host", &dk))) return st;
        if ((st = check_host(l->v_host, full_bytes(*p, a.H), "layer.v_host", &dv))) return st;
      }
      a.k_host = dk;
      a.v_host = dv;
      if (quant) {
        if ((st = check_device(l->k_host_exp, rows, "layer.k_host_exp", 1))) return st;
        if ((st = check_device(l->v_host_exp, rows, "layer.v_host_exp", 1))) return st;
        a.k_exp = l->k_host_exp;
        a.v_exp = l->v_host_exp;
      }
    }
    if (need & NEED_CACHE) {
      if ((st = check_device(l->k_cache, cache_bytes(*p), "layer.k_cache"))) return st;
      if ((st = check_device(l->v_cache, cache_bytes(*p), "layer.v_cache"))) return st;
      a.k_cache = l->k_cache;
      a.v_cache = l->v_cache;
    }
  }
  return ok();
}

// Flags and the error word are single 32-bit words (often slices of one
// tensor), so they need only 4-byte alignment.
clo_status check_flag_ptr(const void* p, const char* name) {
  if (!p) return ok();
  if (reinterpret_cast<uintptr_t>(p) & 3u) return fail(CLO_E_ARG, "%s is not 4-byte aligned", name);
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return fail(CLO_E_ARG, "%s is not memory known to HIP", name);
  }
  if (at.type != hipMemoryTypeDevice && at.type != hipMemoryTypeManaged && at.type != hipMemoryTypeUnified)
    return fail(CLO_E_ARG, "%s is not device memory", name);
  return ok();
}

clo_status check_sync_flags(const clo_sync* sy) {
  if (!sy) return ok();
  clo_status st;
  if ((st = check_flag_ptr(sy->wait_flag, "sync.wait_flag"))) return st;
  if ((st = check_flag_ptr(sy->signal_flag, "sync.signal_flag"))) return st;
  if ((st = check_flag_ptr(sy->error_word, "sync.error_word"))) return st;
  return ok();
}

clo_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return CLO_OK;
  return fail(CLO_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// zero_word (may be NULL): a work counter the next kernel needs at zero; it is
// cleared by the wait kernel, or by a launch of its own when there is no wait
clo_status pre_wait(const clo_sync* sy, hipStream_t s, uint32_t* zero_word = nullptr) {
  if (!sy || !sy->wait_flag)
    return zero_word ? hip_status(launch_zero(zero_word, s), "counter reset launch") : CLO_OK;
  const uint32_t limit = sy->spin_limit ? sy->spin_limit : kDefaultSpinLimit;
  return hip_status(launch_wait(sy->wait_flag, sy->wait_value, limit, sy->error_word, zero_word, s), "wait launch");
}

clo_status post_signal(const clo_sync* sy, hipStream_t s) {
  if (!sy || !sy->signal_flag) return CLO_OK;
  return hip_status(launch_signal(sy->signal_flag, sy->signal_value, s), "signal launch");
}

}  // namespace

extern "C" {

size_t clo_workspace_size(const clo_shape* shape) {
  Plan p;
  if (make_plan(shape, 0, &p)) return 0;
  return ws_layout(p).total;
}

clo_status clo_reuse_test(const clo_shape* shape, const void* q, const void* q_prev, uint8_t* reuse, float* cos,
                          const clo_sync* sync, void* stream) {
  Plan p;
  clo_status st;
  if ((st = make_plan(shape, 0, &p))) return st;
  if ((st = check_sync_flags(sync))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.U == 0) {
    if ((st = pre_wait(sync, s))) return st;
    return post_signal(sync, s);
  }
  if ((st = check_device(q, q_bytes(p), "q"))) return st;
  if ((st = check_device(q_prev, q_bytes(p), "q_prev"))) return st;
  if ((st = check_device(reuse, (size_t)p.U, "reuse"))) return st;
  if (cos && (st = check_device(cos, (size_t)p.U * 4, "cos"))) return st;
  if ((st = pre_wait(sync, s))) return st;
  if ((st = hip_status(launch_reuse(p.a, q, q_prev, reuse, cos, s), "reuse launch"))) return st;
  return post_signal(sync, s);
}

clo_status clo_topk_select(const clo_shape* shape, const clo_layer* layer, const void* q, const uint8_t* reuse,
                           void* ws, size_t ws_bytes, const clo_sync* sync, void* stream) {
  Plan p;
  clo_status st;
  if ((st = make_plan(shape, layer ? layer->persistent_mask : 0, &p))) return st;
  if ((st = check_sync_flags(sync))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.U == 0) {
    if ((st = pre_wait(sync, s))) return st;
    return post_signal(sync, s);
  }
  Workspace w;
  if ((st = check_layer(layer, &p, NEED_IDX | NEED_SCORE | NEED_HBM_K))) return st;
  p.a.err = sync ? sync->error_word : nullptr;
  if ((st = check_device(q, q_bytes(p), "q"))) return st;
  if (reuse && (st = check_device(reuse, (size_t)p.U, "reuse"))) return st;
  if ((st = bind_ws(p, ws, ws_bytes, &w))) return st;
  const int cu = num_cus();
  if ((st = pre_wait(sync, s))) return st;
  if ((st = hip_status(launch_compact(p.a, reuse, w, 1, one_range(p), s), "compact launch"))) return st;
  if ((st = hip_status(launch_score(p.a, q, span_all_misses(w), p.U, w, score_counter(w, 0), cu, s), "score launch"))) return st;
  if ((st = hip_status(launch_select(p.a, span_all_misses(w), p.U, w, s), "top-k launch"))) return st;
  return post_signal(sync, s);
}

clo_status clo_reuse_select(const clo_shape* shape, const clo_layer* layer, const void* q, const void* q_prev,
                            uint8_t* reuse, float* cos, void* ws, size_t ws_bytes, const clo_sync* sync,
                            void* stream) {
  Plan p;
  clo_status st;
  if ((st = make_plan(shape, layer ? layer->persistent_mask : 0, &p))) return st;
  if ((st = check_sync_flags(sync))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.U == 0) {
    if ((st = pre_wait(sync, s))) return st;
    return post_signal(sync, s);
  }
  Workspace w;
  if ((st = check_layer(layer, &p, NEED_IDX | NEED_SCORE | NEED_HBM_K))) return st;
  p.a.err = sync ? sync->error_word : nullptr;
  if ((st = check_device(q, q_bytes(p), "q"))) return st;
  if ((st = check_device(q_prev, q_bytes(p), "q_prev"))) return st;
  if ((st = check_device(reuse, (size_t)p.U, "reuse"))) return st;
  if (cos && (st = check_device(cos, (size_t)p.U * 4, "cos"))) return st;
  if ((st = bind_ws(p, ws, ws_bytes, &w))) return st;
  const int cu = num_cus();
  if (p.U <= kFusedReuseUnits) {
    const bool wait = sync && sync->wait_flag;
    const uint32_t limit = wait && sync->spin_limit ? sync->spin_limit : kDefaultSpinLimit;
    if ((st = hip_status(launch_reuse_compact(p.a, q, q_prev, reuse, cos, w, wait ? sync->wait_flag : nullptr,
                                              wait ? sync->wait_value : 0u, limit,
                                              wait ? sync->error_word : nullptr, s),
                         "reuse test launch")))
      return st;
  } else {
    if ((st = pre_wait(sync, s))) return st;
    if ((st = hip_status(launch_reuse(p.a, q, q_prev, reuse, cos, s), "reuse launch"))) return st;
    if ((st = hip_status(launch_compact(p.a, reuse, w, 1, one_range(p), s), "compact launch"))) return st;
  }
  if ((st = hip_status(launch_score(p.a, q, span_all_misses(w), p.U, w, score_counter(w, 0), cu, s), "score launch"))) return st;
  if ((st = hip_status(launch_select(p.a, span_all_misses(w), p.U, w, s), "top-k launch"))) return st;
  return post_signal(sync, s);
}

clo_status clo_gather_kv(const clo_shape* shape, const clo_layer* layer, const uint8_t* reuse, void* ws,
                         size_t ws_bytes, const clo_sync* sync, void* stream) {
  Plan p;
  clo_status st;
  if ((st = make_plan(shape, layer ? layer->persistent_mask : 0, &p))) return st;
  if ((st = check_sync_flags(sync))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.U == 0 || p.a.H == 0) {
    if ((st = pre_wait(sync, s))) return st;
    return post_signal(sync, s);
  }
  Workspace w;
  if ((st = check_layer(layer, &p, NEED_IDX | NEED_HOST | NEED_CACHE))) return st;
  p.a.err = sync ? sync->error_word : nullptr;
  if (reuse && (st = check_device(reuse, (size_t)p.U, "reuse"))) return st;
  if ((st = bind_ws(p, ws, ws_bytes, &w))) return st;
  uint32_t* counter = reinterpret_cast<uint32_t*>(w.meta + kMetaGather);
  uint32_t* done = reinterpret_cast<uint32_t*>(w.meta + kMetaGatherDone);
  const int blocks = alone_gather_blocks(p.U, p.a.host_fmt);
  if (sync && sync->wait_flag) {
    // one launch: the gather's blocks wait for the flag themselves, and the last
    // one to finish signals; the work counters are zero (every call on the
    // workspace leaves them so, and every selection call sets them)
    const GatherSync gs{sync->wait_flag, sync->wait_value, sync->spin_limit ? sync->spin_limit : kDefaultSpinLimit,
                        sync->error_word, sync->signal_flag, sync->signal_value, done};
    return hip_status(launch_gather(p.a, reuse, kAllUnits, p.U, blocks, counter, s, &gs), "gather launch");
  }
  // the counters are cleared before (a fresh workspace) and by the kernel's last block
  const GatherSync gs{nullptr, 0u, 0u, nullptr, nullptr, 0u, done};
  if ((st = hip_status(launch_zero(counter, s, done), "counter reset launch"))) return st;
  if ((st = hip_status(launch_gather(p.a, reuse, kAllUnits, p.U, blocks, counter, s, &gs), "gather launch"))) return st;
  return post_signal(sync, s);
}

size_t clo_gather_plan_size(int32_t n_layers) {
  if (n_layers < 1 || n_layers > 4096) return 0;
  return (size_t)round_up((int64_t)n_layers * (int64_t)sizeof(GatherPlanLayer), 256);
}

clo_status clo_gather_plan(const clo_gather_layer* layers, int32_t n_layers, void* plan, size_t plan_bytes,
                           int32_t* blocks) {
  if (!layers || !blocks) return fail(CLO_E_ARG, "layers or blocks is NULL");
  const size_t need = clo_gather_plan_size(n_layers);
  if (!need) return fail(CLO_E_ARG, "n_layers %d outside 1..4096", n_layers);
  if (plan_bytes < need) return fail(CLO_E_ARG, "plan has %zu bytes, %zu needed", plan_bytes, need);
  clo_status st;
  if ((st = check_device(plan, need, "plan"))) return st;
  std::vector<GatherPlanLayer> host((size_t)n_layers);
  int grid = kGatherBlocksAlone;
  for (int32_t l = 0; l < n_layers; ++l) {
    const clo_gather_layer& g = layers[l];
    Plan p;
    if ((st = make_plan(g.shape, g.layer ? g.layer->persistent_mask : 0, &p))) return st;
    GatherPlanLayer& d = host[(size_t)l];
    memset(&d, 0, sizeof d);
    if ((st = check_flag_ptr(g.wait_flag, "wait_flag")) || (st = check_flag_ptr(g.signal_flag, "signal_flag")))
      return st;
    if (!g.wait_flag) return fail(CLO_E_ARG, "layer %d: wait_flag is NULL", l);
    d.wait_flag = g.wait_flag;
    d.signal_flag = g.signal_flag;
    if (p.U > 0 && p.a.H > 0) {
      Workspace w;
      if ((st = check_layer(g.layer, &p, NEED_IDX | NEED_HOST | NEED_CACHE))) return st;
      if (g.reuse && (st = check_device(g.reuse, (size_t)p.U, "reuse"))) return st;
      if ((st = bind_ws(p, g.ws, g.ws_bytes, &w))) return st;
      d.a = p.a;
      d.reuse = g.reuse;
      d.counter = reinterpret_cast<uint32_t*>(w.meta + kMetaGather);
      d.done = reinterpret_cast<uint32_t*>(w.meta + kMetaGatherDone);
      const uint32_t zero = 0;
      hipError_t e = hipMemcpy(d.counter, &zero, 4, hipMemcpyHostToDevice);
      if (e == hipSuccess) e = hipMemcpy(d.done, &zero, 4, hipMemcpyHostToDevice);
      if ((st = hip_status(e, "clearing the gather counters"))) return st;
      grid = std::max(grid, alone_gather_blocks(p.U, p.a.host_fmt));
    } else {
      // nothing to gather: the layer's items are none, its counters live in the plan
      d.a = p.a;
      d.a.B = 0;
      d.counter = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(plan) + (size_t)l * sizeof(GatherPlanLayer) +
                                              offsetof(GatherPlanLayer, zero_words));
      d.done = d.counter + 1;
    }
  }
  if ((st = hip_status(hipMemcpy(plan, host.data(), host.size() * sizeof(GatherPlanLayer), hipMemcpyHostToDevice),
                       "writing the gather plan")))
    return st;
  *blocks = grid;
  return ok();
}

clo_status clo_gather_layers(const void* plan, int32_t n_layers, int32_t blocks, uint32_t wait_value,
                             uint32_t signal_value, uint32_t* error_word, uint32_t spin_limit, void* stream) {
  const size_t need = clo_gather_plan_size(n_layers);
  if (!need) return fail(CLO_E_ARG, "n_layers %d outside 1..4096", n_layers);
  if (blocks < 1 || blocks > 1024) return fail(CLO_E_ARG, "blocks %d outside 1..1024", blocks);
  clo_status st;
  if ((st = check_device(plan, need, "plan"))) return st;
  if ((st = check_flag_ptr(error_word, "error_word"))) return st;
  return hip_status(launch_gather_layers(static_cast<const GatherPlanLayer*>(plan), n_layers, blocks, wait_value,
                                         signal_value, spin_limit ? spin_limit : kDefaultSpinLimit, error_word,
                                         static_cast<hipStream_t>(stream)),
                    "gather launch");
}

size_t clo_select_plan_size(int32_t n_layers) {
  if (n_layers < 1 || n_layers > 4096) return 0;
  return (size_t)round_up((int64_t)sizeof(SelectPlanHeader) + (int64_t)n_layers * (int64_t)sizeof(SelectPlanLayer),
                          256);
}

namespace {

// What the multi-layer selection supports: bf16 layers of at most
// kFusedReuseUnits units, token top-k, and at most kFusedMaxBlocks chunks.
clo_status check_select_shape(const Plan& p, const char* what) {
  if (p.a.dtype != CLO_BF16) return fail(CLO_E_UNSUPPORTED, "%s: multi-layer selection takes bf16 layers", what);
  if (p.U < 1 || p.U > kFusedReuseUnits)
    return fail(CLO_E_UNSUPPORTED, "%s: batch * n_kv_heads = %lld outside 1..%d", what, (long long)p.U,
                kFusedReuseUnits);
  if (p.a.bs > 1) return fail(CLO_E_UNSUPPORTED, "%s: multi-layer selection takes token top-k (block_size <= 1)", what);
  if ((p.a.N + kTopkChunk - 1) / kTopkChunk > kFusedMaxBlocks)
    return fail(CLO_E_UNSUPPORTED, "%s: context %lld beyond %lld", what, (long long)p.a.N,
                (long long)kFusedMaxBlocks * kTopkChunk);
  return ok();
}

}  // namespace

clo_status clo_select_plan(const clo_select_layer* layers, int32_t n_layers, void* plan, size_t plan_bytes) {
  if (!layers) return fail(CLO_E_ARG, "layers is NULL");
  const size_t need = clo_select_plan_size(n_layers);
  if (!need) return fail(CLO_E_ARG, "n_layers %d outside 1..4096", n_layers);
  if (plan_bytes < need) return fail(CLO_E_ARG, "plan has %zu bytes, %zu needed", plan_bytes, need);
  clo_status st;
  if ((st = check_device(plan, need, "plan"))) return st;
  std::vector<SelectPlanLayer> host((size_t)n_layers);
  Plan p0;
  for (int32_t l = 0; l < n_layers; ++l) {
    const clo_select_layer& g = layers[l];
    Plan p;
    if ((st = make_plan(g.shape, g.layer ? g.layer->persistent_mask : 0, &p))) return st;
    if ((st = check_select_shape(p, "layer"))) return st;
    if (l == 0) {
      p0 = p;
    } else if (p.a.B != p0.a.B || p.a.Hq != p0.a.Hq || p.a.Hkv != p0.a.Hkv || p.a.N != p0.a.N ||
               p.a.k != p0.a.k) {
      return fail(CLO_E_ARG, "layer %d: batch, heads, context and top-k must equal layer 0's", l);
    }
    if ((st = check_flag_ptr(g.wait_flag, "wait_flag")) || (st = check_flag_ptr(g.signal_flag, "signal_flag")))
      return st;
    if ((st = check_layer(g.layer, &p, NEED_IDX | NEED_SCORE | NEED_HBM_K))) return st;
    if ((st = check_device(g.q, q_bytes(p), "q"))) return st;
    if ((st = check_device(g.q_prev, q_bytes(p), "q_prev"))) return st;
    if ((st = check_device(g.reuse, (size_t)p.U, "reuse"))) return st;
    if (g.cos && (st = check_device(g.cos, (size_t)p.U * 4, "cos"))) return st;
    Workspace w;
    if ((st = bind_ws(p, g.ws, g.ws_bytes, &w))) return st;
    SelectPlanLayer& d = host[(size_t)l];
    memset(&d, 0, sizeof d);
    d.a = p.a;
    d.a.err = nullptr;
    d.q = g.q;
    d.q_prev = g.q_prev;
    d.reuse = g.reuse;
    d.cos = g.cos;
    d.w = w;
    d.wait_flag = g.wait_flag;
    d.signal_flag = g.signal_flag;
  }
  SelectPlanHeader hdr;
  memset(&hdr, 0, sizeof hdr);
  hdr.n_layers = (uint32_t)n_layers;
  hipError_t e = hipMemcpy(plan, &hdr, sizeof hdr, hipMemcpyHostToDevice);
  if (e == hipSuccess)
    e = hipMemcpy(static_cast<char*>(plan) + sizeof(SelectPlanHeader), host.data(),
                  host.size() * sizeof(SelectPlanLayer), hipMemcpyHostToDevice);
  return hip_status(e, "writing the selection plan");
}

clo_status clo_select_layers(const clo_shape* shape, const void* plan, int32_t first, int32_t count,
                             uint32_t wait_value, uint32_t signal_value, uint32_t* error_word, uint32_t spin_limit,
                             void* stream) {
  Plan p;
  clo_status st;
  if ((st = make_plan(shape, 0, &p))) return st;
  if ((st = check_select_shape(p, "shape"))) return st;
  if (count < 1 || count > kMaxSelectBatch) return fail(CLO_E_ARG, "count %d outside 1..%d", count, kMaxSelectBatch);
  if (first < 0 || first > 4096 - count) return fail(CLO_E_ARG, "first %d outside the plan's 4096 layers", first);
  const size_t need = clo_select_plan_size(first + count);
  if ((st = check_device(plan, need, "plan"))) return st;
  if ((st = check_flag_ptr(error_word, "error_word"))) return st;
  auto* hdr = static_cast<SelectPlanHeader*>(const_cast<void*>(plan));
  auto* entries = reinterpret_cast<const SelectPlanLayer*>(static_cast<const char*>(plan) + sizeof(SelectPlanHeader));
  const int cmax = (int)((p.a.N + kTopkChunk - 1) / kTopkChunk);
  return hip_status(launch_select_layers(entries, hdr, first, count, p.a, cmax, wait_value, signal_value,
                                         spin_limit ? spin_limit : kDefaultSpinLimit, error_word,
                                         score_cus(first, num_cus()), static_cast<hipStream_t>(stream)),
                    "selection launch");
}

size_t clo_attend_plan_size(int32_t n_layers) {
  if (n_layers < 1 || n_layers > 4096) return 0;
  return (size_t)round_up((int64_t)sizeof(AttendPlanHeader) + (int64_t)n_layers * (int64_t)sizeof(AttendPlanLayer),
                          256);
}

clo_status clo_attend_plan(const clo_attend_layer* layers, int32_t n_layers, void* plan, size_t plan_bytes) {
  if (!layers) return fail(CLO_E_ARG, "layers is NULL");
  const size_t need = clo_attend_plan_size(n_layers);
  if (!need) return fail(CLO_E_ARG, "n_layers %d outside 1..4096", n_layers);
  if (plan_bytes < need) return fail(CLO_E_ARG, "plan has %zu bytes, %zu needed", plan_bytes, need);
  clo_status st;
  if ((st = check_device(plan, need, "plan"))) return st;
  std::vector<AttendPlanLayer> host((size_t)n_layers);
  Plan p0;
  for (int32_t l = 0; l < n_layers; ++l) {
    const clo_attend_layer& g = layers[l];
    Plan p;
    if ((st = make_plan(g.shape, g.layer ? g.layer->persistent_mask : 0, &p))) return st;
    if (p.U < 1) return fail(CLO_E_ARG, "layer %d has no units", l);
    if (l == 0) {
      p0 = p;
    } else if (p.a.B != p0.a.B || p.a.Hq != p0.a.Hq || p.a.Hkv != p0.a.Hkv || p.a.k != p0.a.k ||
               p.a.dtype != p0.a.dtype) {
      return fail(CLO_E_ARG, "layer %d: batch, heads, top-k and dtype must equal layer 0's", l);
    }
    if ((st = check_flag_ptr(g.wait_flag, "wait_flag")) || (st = check_flag_ptr(g.signal_flag, "signal_flag")))
      return st;
    if ((st = check_layer(g.layer, &p, NEED_IDX | NEED_CACHE | NEED_HBM_KV))) return st;
    if ((st = check_device(g.q, q_bytes(p), "q"))) return st;
    if ((st = check_device(g.out, q_bytes(p), "out"))) return st;
    Workspace w;
    if ((st = bind_ws(p, g.ws, g.ws_bytes, &w))) return st;
    AttendPlanLayer& d = host[(size_t)l];
    memset(&d, 0, sizeof d);
    d.a = p.a;
    d.a.err = nullptr;
    d.q = g.q;
    d.part = w.part;
    d.out = g.out;
    d.wait_flag = g.wait_flag;
    d.signal_flag = g.signal_flag;
  }
  AttendPlanHeader hdr;
  memset(&hdr, 0, sizeof hdr);
  hdr.n_layers = (uint32_t)n_layers;
  hipError_t e = hipMemcpy(plan, &hdr, sizeof hdr, hipMemcpyHostToDevice);
  if (e == hipSuccess)
    e = hipMemcpy(static_cast<char*>(plan) + sizeof(AttendPlanHeader), host.data(),
                  host.size() * sizeof(AttendPlanLayer), hipMemcpyHostToDevice);
  return hip_status(e, "writing the attention plan");
}

clo_status clo_attend_layers(const clo_shape* shape, const void* plan, int32_t first, int32_t count,
                             uint32_t wait_value, uint32_t signal_value, uint32_t* error_word, uint32_t spin_limit,
                             void* stream) {
  Plan p;
  clo_status st;
  if ((st = make_plan(shape, 0, &p))) return st;
  if (p.U < 1) return fail(CLO_E_ARG, "shape has no units");
  if (count < 1 || count > kMaxAttendBatch) return fail(CLO_E_ARG, "count %d outside 1..%d", count, kMaxAttendBatch);
  if (first < 0 || first > 4096 - count) return fail(CLO_E_ARG, "first %d outside the plan's 4096 layers", first);
  const size_t need = clo_attend_plan_size(first + count);
  if ((st = check_device(plan, need, "plan"))) return st;
  if ((st = check_flag_ptr(error_word, "error_word"))) return st;
  const auto* hdr = static_cast<const AttendPlanHeader*>(plan);
  const auto* entries =
      reinterpret_cast<const AttendPlanLayer*>(static_cast<const char*>(plan) + sizeof(AttendPlanHeader));
  return hip_status(launch_attend_layers(entries, hdr, first, count, p.a, wait_value, signal_value,
                                         spin_limit ? spin_limit : kDefaultSpinLimit, error_word,
                                         static_cast<hipStream_t>(stream)),
                    "attention launch");
}

clo_status clo_sparse_attn(const clo_shape* shape, const clo_layer* layer, const void* q, void* out, void* ws,
                           size_t ws_bytes, const clo_sync* sync, void* stream) {
  Plan p;
  clo_status st;
  if ((st = make_plan(shape, layer ? layer->persistent_mask : 0, &p))) return st;
  if ((st = check_sync_flags(sync))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.U == 0) {
    if ((st = pre_wait(sync, s))) return st;
    return post_signal(sync, s);
  }
  Workspace w;
  if ((st = check_layer(layer, &p, NEED_IDX | NEED_CACHE | NEED_HBM_KV))) return st;
  p.a.err = sync ? sync->error_word : nullptr;
  if ((st = check_device(q, q_bytes(p), "q"))) return st;
  if ((st = check_device(out, q_bytes(p), "out"))) return st;
  if ((st = bind_ws(p, ws, ws_bytes, &w))) return st;
  if ((st = pre_wait(sync, s))) return st;
  if ((st = hip_status(launch_attn_partial(p.a, q, w.part, kAllUnits, p.U, s), "attention launch"))) return st;
  if ((st = hip_status(launch_attn_combine(p.a, w.part, out, kAllUnits, p.U, s), "attention combine launch"))) return st;
  return post_signal(sync, s);
}

namespace {

// Decode step with every kernel in order on the caller's stream: layers without
// offloaded heads (nothing to overlap), layers of fewer than kOverlapUnits units
// (a range per unit would leave most ranges empty and make the call's ~70
// launches and stream waits cost more host time than the overlap saves), steps
// enqueued under graph capture, and clo_decode_step_static, which creates no
// helper streams.  The gather of
// offloaded heads follows the top-k.
clo_status step_in_order(const Plan& p, const Workspace& w, const void* q, const void* q_prev, void* out,
                         uint8_t* reuse, float* cos, hipStream_t s) {
  clo_status st;
  const int cu = num_cus();
  if (p.U <= kFusedReuseUnits) {
    if ((st = hip_status(launch_reuse_compact(p.a, q, q_prev, reuse, cos, w, nullptr, 0u, 0u, nullptr, s),
                         "reuse test launch")))
      return st;
  } else {
    if ((st = hip_status(launch_reuse(p.a, q, q_prev, reuse, cos, s), "reuse launch"))) return st;
    if ((st = hip_status(launch_compact(p.a, reuse, w, 1, one_range(p), s), "compact launch"))) return st;
  }
  if ((st = hip_status(launch_score(p.a, q, span_all_misses(w), p.U, w, score_counter(w, 0), cu, s), "score launch"))) return st;
  if ((st = hip_status(launch_select(p.a, span_all_misses(w), p.U, w, s), "top-k launch"))) return st;
  if (p.a.H > 0) {
    // the unit lists hold one range; its offloaded misses, and the work counter
    // the list kernel cleared
    if ((st = hip_status(launch_gather(p.a, reuse, span_host_range(w, 0), p.U,
                                       alone_gather_blocks(p.U, p.a.host_fmt),
                                       reinterpret_cast<uint32_t*>(w.meta + kMetaGather), s),
                         "gather launch")))
      return st;
  }
  if ((st = hip_status(launch_attn_partial(p.a, q, w.part, kAllUnits, p.U, s), "attention launch"))) return st;
  return hip_status(launch_attn_combine(p.a, w.part, out, kAllUnits, p.U, s), "attention combine launch");
}

// Decode step with offloaded heads, overlapped on the helper streams.  Units
// are split into R ranges of equal unit counts; the caller's stream scores and
// selects them in order, the gather reads each range's host rows once its
// top-k is done, and the attention stream first attends the reuse units (which
// need nothing new) and then each range's miss units once their rows have
// arrived, combining the chunk partials range by range so that only the last
// range's remain at the end.  Everything is ordered on the GPU (events and
// device flags); the host never waits.  The caller's stream finally waits for
// the helper streams, so the call is ordered like a single-stream call.
//
// Two schedules of the gather.  Layers of fewer than kResidentGatherUnits
// units launch a gather per range, on two gather streams in turn (so that one
// range's host reads start while the previous range's last items finish
// instead of after a launch gap), each behind an event after the range's
// top-k, and attention waits on events.  Larger layers keep one gather launch
// resident for the whole step: it reads range after range, each once the
// range's flag is up, and raises a flag per gathered range that attention
// waits for; their ranges are selected in groups of 1, 1, 2, 4 ranges, since
// beside the host reads every launch takes several times its time alone.
// Steps/s measured side by side on one box, streams / resident:
//   B=64, N=131072 (512 units)  native 80.9-81.1 / 81.8-81.9, int4 rows
//                               224-225 / 227-230, int4 16-token blocks 257 / 263-266
//   B=16, N=32768 (128 units)   native 330.6-332.4 / 328.7-330.4, int4 rows
//                               839-849 / 797-801
// (Up to 8 ranges.  At B=64, N=131072, ranges growing from 1/64 of the units so
// that the first gather starts sooner, and a small last range, lost 0.7%
// against equal ranges: the larger middle ranges are selected beside the
// gather, whose host reads slow the selection's latency-bound top-k kernels
// several times over.)
struct Ranges {
  int R;
  RangeBounds rb;
  int64_t per;  // the most units in one range: sizes the per-range grids
};

Ranges split_ranges(const Plan& p) {
  Ranges x{};
  x.R = (int)(p.U < 8 ? p.U : 8);
  for (int r = 0; r <= x.R; ++r) x.rb.first[r] = (int32_t)(p.U * r / x.R);
  x.per = 1;
  for (int r = 0; r < x.R; ++r) x.per = std::max<int64_t>(x.per, x.rb.first[r + 1] - x.rb.first[r]);
  return x;
}

#define CLO_TRY(expr, what) \
  if ((st = hip_status((expr), (what)))) return st

clo_status step_overlapped_streams(const Plan& p, const Workspace& w, const void* q, const void* q_prev, void* out,
                                   uint8_t* reuse, float* cos, DeviceQueues* dq, hipStream_t s) {
  clo_status st;
  const int cu = num_cus();
  const Ranges x = split_ranges(p);
  hipStream_t as = dq->attend;
  CLO_TRY(launch_reuse(p.a, q, q_prev, reuse, cos, s), "reuse launch");
  CLO_TRY(launch_compact(p.a, reuse, w, x.R, x.rb, s), "compact launch");
  for (int r = 0; r < x.R; ++r) {
    CLO_TRY(launch_score(p.a, q, span_range(w, r), x.per, w, score_counter(w, r), score_cus(r, cu), s),
            "score launch");
    CLO_TRY(launch_select(p.a, span_range(w, r), x.per, w, s), "top-k launch");
    CLO_TRY(hipEventRecord(dq->ev_topk[r], s), "event record");
    hipStream_t gsr = (r & 1) ? dq->gather2 : dq->gather;
    CLO_TRY(hipStreamWaitEvent(gsr, dq->ev_topk[r], 0), "stream wait");
    if (r == 0) CLO_TRY(hipEventRecord(dq->ev_g_start, gsr), "event record");
    CLO_TRY(launch_gather(p.a, reuse, span_host_range(w, r), x.per, kGatherBlocksOverlapped,
                          reinterpret_cast<uint32_t*>(w.meta + kMetaGather + r), gsr),
            "gather launch");
    CLO_TRY(hipEventRecord(dq->ev_gather[r], gsr), "event record");
  }
  CLO_TRY(hipEventRecord(dq->ev_g_end[0], dq->gather), "event record");
  dq->g_ends = 1;
  if (x.R > 1) {
    CLO_TRY(hipEventRecord(dq->ev_g_end[1], dq->gather2), "event record");
    dq->g_ends = 2;
  }
  // reuse units need no new rows; they are attended once the first range is
  // selected, so that their many short blocks do not delay the first top-k
  CLO_TRY(hipStreamWaitEvent(as, dq->ev_topk[0], 0), "stream wait");
  CLO_TRY(launch_attn_partial(p.a, q, w.part, span_hits(w), p.U, as), "attention launch");
  CLO_TRY(launch_attn_combine(p.a, w.part, out, span_hits(w), p.U, as), "attention combine launch");
  for (int r = 0; r < x.R; ++r) {
    CLO_TRY(hipStreamWaitEvent(as, dq->ev_gather[r], 0), "stream wait");
    CLO_TRY(launch_attn_partial(p.a, q, w.part, span_range(w, r), x.per, as), "attention launch");
    CLO_TRY(launch_attn_combine(p.a, w.part, out, span_range(w, r), x.per, as), "attention combine launch");
  }
  CLO_TRY(hipEventRecord(dq->ev_attn, as), "event record");
  CLO_TRY(hipStreamWaitEvent(s, dq->ev_attn, 0), "stream wait");
  return ok();
}

clo_status step_overlapped_resident(const Plan& p, const Workspace& w, const void* q, const void* q_prev,
                                    void* out, uint8_t* reuse, float* cos, uint32_t limit, DeviceQueues* dq,
                                    hipStream_t s) {
  clo_status st;
  const int cu = num_cus();
  const Ranges x = split_ranges(p);
  hipStream_t gs = dq->gather, as = dq->attend;
  uint32_t* meta = reinterpret_cast<uint32_t*>(w.meta);
  CLO_TRY(launch_reuse(p.a, q, q_prev, reuse, cos, s), "reuse launch");
  // the unit lists; the range flags, counters and done counts at zero
  CLO_TRY(launch_compact(p.a, reuse, w, x.R, x.rb, s), "compact launch");
  CLO_TRY(hipEventRecord(dq->ev_lists, s), "event record");
  // groups of 1, 1, 2, 4, ... ranges
  for (int r0 = 0, n = 1, g = 0; r0 < x.R; r0 += n, n = g >= 1 ? 2 * n : n, ++g) {
    n = std::min(n, x.R - r0);
    const Span sp{w.list_all, w.meta + kMetaOffAll + r0, w.meta + kMetaOffAll + r0 + n};
    CLO_TRY(launch_score(p.a, q, sp, x.per * n, w, score_counter(w, g), score_cus(r0, cu), s), "score launch");
    CLO_TRY(launch_select(p.a, sp, x.per * n, w, s), "top-k launch");
    // the kernel boundary makes the ranges' indices visible to the gather
    CLO_TRY(launch_signal(meta + kMetaSelFlag + r0, 1u, s, n), "signal launch");
    if (r0 == 0) CLO_TRY(hipEventRecord(dq->ev_topk[0], s), "event record");
  }
  // The gather polls every group's flag, so it is enqueued after the last
  // group's selection: streams beyond the device's hardware queues share one,
  // whose kernels start in the order they were enqueued, and a gather queued
  // ahead of a selection it polls for would wait out its bound.  It still
  // starts reading with the first group (the host has enqueued the whole step
  // long before that group's top-k ends), and a failed launch above leaves no
  // gather waiting.
  CLO_TRY(hipStreamWaitEvent(gs, dq->ev_lists, 0), "stream wait");
  CLO_TRY(hipEventRecord(dq->ev_g_start, gs), "event record");
  CLO_TRY(launch_gather_ranges(p.a, w, x.R, kGatherBlocksRanges, limit, gs), "gather launch");
  CLO_TRY(hipEventRecord(dq->ev_g_end[0], gs), "event record");
  dq->g_ends = 1;
  CLO_TRY(hipEventRecord(dq->ev_gathered, gs), "event record");
  CLO_TRY(hipStreamWaitEvent(as, dq->ev_topk[0], 0), "stream wait");
  CLO_TRY(launch_attn_partial(p.a, q, w.part, span_hits(w), p.U, as), "attention launch");
  CLO_TRY(launch_attn_combine(p.a, w.part, out, span_hits(w), p.U, as), "attention combine launch");
  for (int r = 0; r < x.R; ++r) {
    CLO_TRY(launch_wait(meta + kMetaGatherFlag + r, 1u, limit, p.a.err, nullptr, as), "wait launch");
    CLO_TRY(launch_attn_partial(p.a, q, w.part, span_range(w, r), x.per, as), "attention launch");
    CLO_TRY(launch_attn_combine(p.a, w.part, out, span_range(w, r), x.per, as), "attention combine launch");
  }
  CLO_TRY(hipEventRecord(dq->ev_attn, as), "event record");
  CLO_TRY(hipStreamWaitEvent(s, dq->ev_attn, 0), "stream wait");
  CLO_TRY(hipStreamWaitEvent(s, dq->ev_gathered, 0), "stream wait");
  return ok();
}

#undef CLO_TRY

// CLO_STEP_IN_ORDER=1 in the environment runs every decode step in order on the
// caller's stream, as under graph capture: for tools that run one kernel at a
// time (hardware counter collection), under which the overlapped step's
// gather and attention would wait for flags that kernels queued behind them
// raise, until their bounds.
bool step_in_order_forced() {
  static const bool forced = [] {
    const char* e = std::getenv("CLO_STEP_IN_ORDER");
    return e != nullptr && e[0] == '1';
  }();
  return forced;
}

// How clo_decode_step runs a layer (clo_decode_step_schedule reports it).
clo_step_mode step_mode(const Plan& p, bool capturing) {
  if (p.a.H == 0 || p.U < kOverlapUnits || capturing || step_in_order_forced()) return CLO_STEP_IN_ORDER;
  return p.U >= kResidentGatherUnits ? CLO_STEP_RESIDENT_GATHER : CLO_STEP_RANGE_GATHERS;
}

clo_status step_overlapped(const Plan& p, const Workspace& w, const void* q, const void* q_prev, void* out,
                           uint8_t* reuse, float* cos, uint32_t limit, clo_step_mode mode, hipStream_t s) {
  DeviceQueues* dq = nullptr;
  clo_status st;
  if ((st = device_queues(&dq))) return st;
  std::lock_guard<std::mutex> lk(dq->mu);
  dq->g_ends = 0;
  return mode == CLO_STEP_RESIDENT_GATHER
             ? step_overlapped_resident(p, w, q, q_prev, out, reuse, cos, limit, dq, s)
             : step_overlapped_streams(p, w, q, q_prev, out, reuse, cos, dq, s);
}

}  // namespace

clo_status clo_decode_step(const clo_shape* shape, const clo_layer* layer, const void* q, const void* q_prev,
                           void* out, uint8_t* reuse, float* cos, void* ws, size_t ws_bytes, const clo_sync* sync,
                           void* stream) {
  Plan p;
  clo_status st;
  if ((st = make_plan(shape, layer ? layer->persistent_mask : 0, &p))) return st;
  if ((st = check_sync_flags(sync))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.U == 0) {
    if ((st = pre_wait(sync, s))) return st;
    return post_signal(sync, s);
  }
  Workspace w;
  if ((st = check_layer(layer, &p, NEED_IDX | NEED_SCORE | NEED_HOST | NEED_CACHE | NEED_HBM_KV))) return st;
  p.a.err = sync ? sync->error_word : nullptr;
  if ((st = check_device(q, q_bytes(p), "q"))) return st;
  if ((st = check_device(q_prev, q_bytes(p), "q_prev"))) return st;
  if ((st = check_device(out, q_bytes(p), "out"))) return st;
  if ((st = check_device(reuse, (size_t)p.U, "reuse"))) return st;
  if (cos && (st = check_device(cos, (size_t)p.U * 4, "cos"))) return st;
  if ((st = bind_ws(p, ws, ws_bytes, &w))) return st;
  if ((st = pre_wait(sync, s))) return st;
  // Under stream capture the step runs in order on `stream`: a graph may run
  // independent branches one after another, and the overlapped step's gather
  // and attention poll flags that kernels on another branch raise.
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess) {
    (void)hipGetLastError();
    cap = hipStreamCaptureStatusActive;
  }
  // The overlapped step's own waits (its streams' hand-offs) are bounded by the
  // library's default, not by sync->spin_limit: a bound the caller chose for its
  // own flag could end them before the kernels they wait for have run.
  const clo_step_mode mode = step_mode(p, cap != hipStreamCaptureStatusNone);
  st = mode != CLO_STEP_IN_ORDER ? step_overlapped(p, w, q, q_prev, out, reuse, cos, kDefaultSpinLimit, mode, s)
                                 : step_in_order(p, w, q, q_prev, out, reuse, cos, s);
  if (st) return st;
  return post_signal(sync, s);
}

clo_status clo_decode_step_schedule(const clo_shape* shape, uint64_t persistent_mask, int32_t host_format,
                                    clo_step_schedule* out) {
  Plan p;
  clo_status st;
  if (!out) return fail(CLO_E_ARG, "out is NULL");
  if ((st = make_plan(shape, persistent_mask, &p))) return st;
  if (host_format != CLO_HOST_NATIVE && host_format != CLO_HOST_INT8 && host_format != CLO_HOST_INT4)
    return fail(CLO_E_ARG, "host_format %d is not a clo_host_format", host_format);
  p.a.host_fmt = host_format;
  clo_step_schedule x;
  memset(&x, 0, sizeof x);
  x.mode = step_mode(p, false);
  x.host_bytes_per_gather_block = kGatherBytesPerBlock;
  if (x.mode == CLO_STEP_IN_ORDER) {
    x.ranges = 1;
    x.gather_blocks = p.a.H > 0 && p.U > 0 ? alone_gather_blocks(p.U, p.a.host_fmt) : 0;
    x.gather_blocks_in_flight = x.gather_blocks;
  } else {
    x.ranges = split_ranges(p).R;
    const bool resident = x.mode == CLO_STEP_RESIDENT_GATHER;
    x.gather_blocks = resident ? kGatherBlocksRanges : kGatherBlocksOverlapped;
    x.gather_blocks_in_flight = resident ? kGatherBlocksRanges : 2 * kGatherBlocksOverlapped;  // two streams
  }
  x.host_bytes_in_flight = (int64_t)x.gather_blocks_in_flight * kGatherBytesPerBlock;
  *out = x;
  return ok();
}

clo_status clo_last_step_gather_ms(float* ms) {
  if (!ms) return fail(CLO_E_ARG, "ms is NULL");
  DeviceQueues* dq = nullptr;
  clo_status st;
  if ((st = device_queues(&dq))) return st;
  std::lock_guard<std::mutex> lk(dq->mu);
  if (dq->g_ends == 0) return fail(CLO_E_ARG, "no overlapped decode step has gathered on this device");
  float best = 0.f;
  for (int i = 0; i < dq->g_ends; ++i) {
    float t = 0.f;
    const hipError_t e = hipEventElapsedTime(&t, dq->ev_g_start, dq->ev_g_end[i]);
    if (e == hipErrorNotReady) {
      (void)hipGetLastError();
      return fail(CLO_E_ARG, "the last decode step has not finished");
    }
    if ((st = hip_status(e, "gather timing"))) return st;
    best = std::max(best, t);
  }
  *ms = best;
  return ok();
}

clo_status clo_decode_step_static(const clo_shape* shape, const clo_layer* layer, const void* q,
                                  const void* q_prev, void* out, uint8_t* reuse, float* cos, const clo_sync* sync,
                                  void* stream) {
  Plan p;
  clo_status st;
  if ((st = make_plan(shape, layer ? layer->persistent_mask : 0, &p))) return st;
  if ((st = check_sync_flags(sync))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.U == 0) {
    if ((st = pre_wait(sync, s))) return st;
    return post_signal(sync, s);
  }
  const size_t need = ws_layout(p).total;
  if (need > kStaticScratchBytes)
    return fail(CLO_E_WORKSPACE, "the step needs %zu bytes of scratch; the static scratch holds %zu (use clo_decode_step)",
                need, (size_t)kStaticScratchBytes);
  Workspace w;
  if ((st = check_layer(layer, &p, NEED_IDX | NEED_SCORE | NEED_HOST | NEED_CACHE | NEED_HBM_KV))) return st;
  p.a.err = sync ? sync->error_word : nullptr;
  if ((st = check_device(q, q_bytes(p), "q"))) return st;
  if ((st = check_device(q_prev, q_bytes(p), "q_prev"))) return st;
  if ((st = check_device(out, q_bytes(p), "out"))) return st;
  if ((st = check_device(reuse, (size_t)p.U, "reuse"))) return st;
  if (cos && (st = check_device(cos, (size_t)p.U * 4, "cos"))) return st;
  void* scratch = nullptr;
  if ((st = hip_status(static_scratch(&scratch), "static scratch lookup"))) return st;
  if ((st = bind_ws(p, scratch, kStaticScratchBytes, &w, true))) return st;
  if ((st = pre_wait(sync, s))) return st;
  if ((st = step_in_order(p, w, q, q_prev, out, reuse, cos, s))) return st;
  return post_signal(sync, s);
}

clo_status clo_append_kv(const clo_shape* shape, const clo_layer* layer, const void* k_new, const void* v_new,
                         int64_t position, const clo_sync* sync, void* stream) {
  Plan p;
  clo_status st;
  if ((st = make_plan(shape, layer ? layer->persistent_mask : 0, &p))) return st;
  if ((st = check_sync_flags(sync))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (position < 0 || position >= p.a.C)
    return fail(CLO_E_ARG, "position %lld outside 0..capacity-1 (%lld)", (long long)position, (long long)p.a.C);
  if (p.U == 0) {
    if ((st = pre_wait(sync, s))) return st;
    return post_signal(sync, s);
  }
  if ((st = check_layer(layer, &p, NEED_SCORE | NEED_HOST | NEED_HBM_KV))) return st;
  const size_t row_bytes = (size_t)p.U * kHeadDim * p.e;
  if ((st = check_device(k_new, row_bytes, "k_new"))) return st;
  if ((st = check_device(v_new, row_bytes, "v_new"))) return st;
  if ((st = pre_wait(sync, s))) return st;
  const LayerArgs& a = p.a;
  if ((st = hip_status(launch_append(a, k_new, v_new, position, const_cast<void*>(a.k_hbm), const_cast<void*>(a.v_hbm),
                                     const_cast<void*>(a.k_host), const_cast<void*>(a.v_host),
                                     const_cast<void*>(a.k_score), s),
                       "append launch")))
    return st;
  return post_signal(sync, s);
}

clo_status clo_update_reference(const clo_shape* shape, const void* q, const uint8_t* reuse, void* q_ref,
                                const clo_sync* sync, void* stream) {
  Plan p;
  clo_status st;
  if ((st = make_plan(shape, 0, &p))) return st;
  if ((st = check_sync_flags(sync))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.U == 0) {
    if ((st = pre_wait(sync, s))) return st;
    return post_signal(sync, s);
  }
  if ((st = check_device(q, q_bytes(p), "q"))) return st;
  if ((st = check_device(q_ref, q_bytes(p), "q_ref"))) return st;
  if (reuse && (st = check_device(reuse, (size_t)p.U, "reuse"))) return st;
  if ((st = pre_wait(sync, s))) return st;
  if ((st = hip_status(launch_update_reference(p.a, q, reuse, q_ref, s), "reference launch"))) return st;
  return post_signal(sync, s);
}

clo_status clo_plan_persistent(const float* s_hat, int32_t n_layers, int32_t n_kv_heads, int32_t n_persist,
                               uint64_t* masks) {
  if (!s_hat || !masks) return fail(CLO_E_ARG, "s_hat or masks is NULL");
  if (n_layers < 0) return fail(CLO_E_ARG, "n_layers %d < 0", n_layers);
  if (n_kv_heads < 1 || n_kv_heads > kMaxKvHeads)
    return fail(CLO_E_ARG, "n_kv_heads %d outside 1..%d", n_kv_heads, kMaxKvHeads);
  const int64_t slots = (int64_t)n_layers * n_kv_heads;
  if (n_persist < 0 || n_persist > slots)
    return fail(CLO_E_ARG, "n_persist %d outside 0..%lld", n_persist, (long long)slots);
  std::vector<int64_t> order((size_t)slots);
  for (int64_t i = 0; i < slots; ++i) {
    if (std::isnan(s_hat[i])) return fail(CLO_E_ARG, "s_hat[%lld] is NaN", (long long)i);
    order[(size_t)i] = i;
  }
  // lowest mean similarity first; equal values keep the lower slot index first
  std::stable_sort(order.begin(), order.end(), [&](int64_t x, int64_t y) { return s_hat[x] < s_hat[y]; });
  for (int l = 0; l < n_layers; ++l) masks[l] = 0;
  for (int i = 0; i < n_persist; ++i) {
    const int64_t slot = order[(size_t)i];
    masks[slot / n_kv_heads] |= 1ull << (slot % n_kv_heads);
  }
  return ok();
}

clo_status clo_stream_read(const void* src, size_t bytes, int32_t blocks, uint32_t* sink, void* stream) {
  if (bytes % 16) return fail(CLO_E_ARG, "bytes %zu is not a multiple of 16", bytes);
  if (blocks < 1 || blocks > (1 << 20)) return fail(CLO_E_ARG, "blocks %d is not in [1, 2^20]", (int)blocks);
  if (bytes == 0) return ok();
  clo_status st;
  if ((st = check_device(src, bytes, "src"))) return st;
  if ((st = check_device(sink, 4, "sink", 4))) return st;
  return hip_status(launch_stream_read(src, (int64_t)(bytes / 16), blocks, sink, static_cast<hipStream_t>(stream)),
                    "stream read launch");
}

clo_status clo_quantize_rows(const void* src, int64_t n_rows, int32_t dtype, int32_t host_format, void* dst,
                             int64_t dst_stride, int8_t* dst_exp, const clo_sync* sync, void* stream) {
  clo_status st;
  if (dtype != CLO_F32 && dtype != CLO_BF16) return fail(CLO_E_UNSUPPORTED, "dtype %d is not fp32 or bf16", dtype);
  if (host_format != CLO_HOST_INT8 && host_format != CLO_HOST_INT4)
    return fail(CLO_E_ARG, "host_format %d is not CLO_HOST_INT8 or CLO_HOST_INT4", host_format);
  if (n_rows < 0) return fail(CLO_E_ARG, "n_rows %lld < 0", (long long)n_rows);
  const int64_t row_bytes = quant_row_bytes(host_format);
  if (dst_stride < row_bytes || dst_stride % 16)
    return fail(CLO_E_ARG, "dst_stride %lld is not a multiple of 16 of at least %lld", (long long)dst_stride,
                (long long)row_bytes);
  if ((st = check_sync_flags(sync))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (n_rows == 0) {
    if ((st = pre_wait(sync, s))) return st;
    return post_signal(sync, s);
  }
  const size_t e = dtype == CLO_F32 ? 4 : 2;
  if ((st = check_device(src, (size_t)n_rows * kHeadDim * e, "src"))) return st;
  const void* d = nullptr;
  if ((st = check_host(dst, (size_t)(n_rows - 1) * dst_stride + row_bytes, "dst", &d))) return st;  // or device
  if ((st = check_device(dst_exp, (size_t)n_rows, "dst_exp", 1))) return st;
  if ((st = pre_wait(sync, s))) return st;
  if ((st = hip_status(launch_quantize_rows(src, n_rows, dtype, host_format,
                                            static_cast<uint8_t*>(const_cast<void*>(d)), dst_stride, dst_exp, s),
                       "quantize launch")))
    return st;
  return post_signal(sync, s);
}

const char* clo_status_string(clo_status status) {
  switch (status) {
    case CLO_OK: return "ok";
    case CLO_E_ARG: return "invalid argument";
    case CLO_E_UNSUPPORTED: return "unsupported shape or dtype";
    case CLO_E_WORKSPACE: return "workspace missing or too small";
    case CLO_E_HIP: return "HIP runtime error";
    case CLO_E_TIMEOUT: return "device-side wait timed out";
    case CLO_E_INDEX: return "selected index out of range";
  }
  return "unknown status";
}

clo_status clo_last_error(char* buf, size_t len) {
  if (buf && len) {
    strncpy(buf, g_last_msg, len - 1);
    buf[len - 1] = '\0';
  }
  return g_last_status;
}

}  // extern "C"
