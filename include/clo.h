/*
 * clo.h -- C ABI of the CLO decode-step library for AMD Instinct MI355X (gfx950).
 *
 * One decode step of CPU-light KV-cache offloading ("CLO: Efficient LLM
 * Inference System with CPU-Light KVCache Offloading via Algorithm-System
 * Co-Design", abstract; "CLO (2511.14510) -- L3 Per-Paper Synthesis",
 * sections 2.1-2.3) for every unit u = (sequence b, KV head kvh) of one layer:
 *
 *   A1 reuse test    cosine of the unit's current query group against the
 *                    previous step's (synthesis 2.1 item 2: adjacent-step
 *                    queries are highly similar, > 0.8, on most heads; abstract
 *                    feature (1): head-wise coarse-grained approximate caching).
 *   A2 scoring       s_j = max over the group's query heads of q_h . K_j.
 *   A3 top-k         the k highest-scoring tokens (synthesis 2.2: top-k = 10%).
 *   A4 gather        the selected K/V rows of non-persistent heads are read by
 *                    the GPU straight from pinned host memory into an HBM cache
 *                    (abstract feature (3): zero-copy transfer engine; feature
 *                    (2): persistent heads keep their whole KV on the GPU).
 *   A5 attention     softmax(q_h . K_sel / sqrt(d)) . V_sel per query head
 *                    (synthesis 2.3 table: top-k sparse attention).
 *
 * A unit whose cosine reaches tau (its head's tau_heads entry when given) reuses the previous step's selection and
 * cached rows; A2-A4 run for the other ("miss") units only.  Query head h
 * belongs to KV head h / g, g = n_q_heads / n_kv_heads.
 *
 * Conventions for every entry point:
 *  - All buffers are caller-owned.  The library allocates no memory, frees
 *    nothing and keeps no pointer after the call returns (the only state it
 *    keeps is clo_decode_step's helper streams and events, see there).
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  Buffers must stay alive until the stream work completes.
 *  - Arguments are validated on the host before anything is launched; a
 *    non-OK status from validation means nothing was enqueued.  CLO_E_HIP (a
 *    launch the runtime refused) can follow kernels of the same call that
 *    were already enqueued: the call's outputs are then undefined, and none of
 *    its enqueued kernels waits for a flag of the call that no enqueued kernel
 *    raises.  clo_last_error() gives the reason (thread-local).  No exception
 *    crosses the ABI and nothing aborts.
 *  - Device buffers must be device memory of the current device; host K/V
 *    buffers must be pinned host memory that the device can address (e.g.
 *    hipHostMalloc); pageable host memory is rejected with CLO_E_ARG.  Every
 *    tensor pointer must be 16-byte aligned (int8 exponent arrays: any byte).  Where the runtime reports an
 *    allocation's extent, a tensor that would run past it is rejected.
 *  - Inputs must be finite; results for NaN/Inf inputs are unspecified (no
 *    out-of-bounds access happens either way).
 *  - Calls on distinct buffers and streams may run concurrently, with two
 *    limits.  Concurrent clo_decode_step calls on one device share that
 *    device's helper streams: a lock serializes their enqueueing and their
 *    GPU work runs one after another.  The top-k of a layer of 8 or more
 *    chunks of 16384 keys runs as one launch of at most 128 blocks that wait
 *    for one another, so all of them must be resident at once: four such
 *    launches side by side fit an MI355X (two blocks per CU); beyond that a
 *    launch's waits can run out (CLO_E_TIMEOUT in the error word, every
 *    kernel still finishes) instead of hanging.
 *
 * Tensor layouts (row-major, element type = shape->dtype unless noted), with
 * P = number of persistent KV heads (bits set in persistent_mask), H = n_kv_heads - P,
 * C = shape->capacity (or N when 0), and "slot" = a head's rank among the
 * persistent (or non-persistent) heads in head order:
 *   q, q_prev, out   [B, Hq, d]
 *   k_hbm, v_hbm     [B, P, C, d]   device   full K/V of persistent heads (rows < N used)
 *   k_host, v_host   [B, H, C, d]   pinned   full K/V of non-persistent heads; with
 *                                            CLO_HOST_INT8: k_host [B, H, C, 2, d] int8
 *                                            (K row, V row per token), v_host unused;
 *                                            CLO_HOST_INT4: k_host [B, H, C, 2, d/2] uint8
 *                                            (4-bit K row, V row per token), v_host unused
 *   k_score          [B, H, C, d]   device   copy of k_host read by scoring
 *   k_cache, v_cache [B, H, k, d]   device   rows k_host[idx], v_host[idx]
 *   idx              [B, Hkv, k]    int32    selected token indices, ascending
 *   reuse            [B, Hkv]       uint8    1 = reuse (hit), 0 = miss
 *   cos              [B, Hkv]       float    group cosine
 */
#ifndef CLO_H
#define CLO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { CLO_F32 = 0, CLO_BF16 = 1 } clo_dtype;

/* Element format of the offloaded K/V in host memory (clo_layer.host_format).
 *   CLO_HOST_NATIVE  rows in the shape's dtype (the pages' format)
 *   CLO_HOST_INT8    quantized rows: 128 int8 values q_i per row and one scale
 *                    exponent e per row (int8, kept in device memory); the row's
 *                    values are q_i * 2^e.  A token's K and V rows are stored
 *                    together as one 256-byte record (K values, then V values)
 *                    in k_host, so that the GPU reads a selected token with one
 *                    256-byte request; v_host is not used.  A row x is quantized as: m = max|x_i|;
 *                    e = the smallest integer with m <= 127 * 2^e (e = 0 when m = 0),
 *                    raised to -120 if smaller; q_i = x_i * 2^-e rounded to the
 *                    nearest integer, ties to even.  q_i * 2^e is exact in bf16 and
 *                    fp32, so dequantized rows are exact.
 *   CLO_HOST_INT4    the same with 4-bit values: q_i in [-7, 7], e the smallest
 *                    integer with m <= 7 * 2^e (0 when m = 0), at least -120, q_i =
 *                    x_i * 2^-e rounded to nearest even.  A row is 64 bytes, value 2j
 *                    in the low 4 bits of byte j and value 2j+1 in the high 4 bits,
 *                    each as a 4-bit two's complement code; a token is one 128-byte
 *                    record (K row, then V row) in k_host; exponents as for
 *                    CLO_HOST_INT8.  The same article's quantized offloading
 *                    passage gives 2- and 3-bit schemes as examples; the format here
 *                    is this library's. */
typedef enum { CLO_HOST_NATIVE = 0, CLO_HOST_INT8 = 1, CLO_HOST_INT4 = 2 } clo_host_format;

typedef enum {
  CLO_OK = 0,
  CLO_E_ARG = 1,          /* invalid argument (null/misaligned pointer, bad shape, bad memory kind) */
  CLO_E_UNSUPPORTED = 2,  /* valid but unsupported: head_dim != 128, dtype, group size > 8 */
  CLO_E_WORKSPACE = 3,    /* workspace missing or smaller than clo_workspace_size() */
  CLO_E_HIP = 4,          /* the HIP runtime reported an error at launch */
  CLO_E_TIMEOUT = 5,      /* written to clo_sync.error_word when a device-side wait gives up */
  CLO_E_INDEX = 6         /* written to clo_sync.error_word when a kernel meets a selected index
                             outside 0..context-1 (the read is clamped into range) */
} clo_status;

/* Problem shape of one layer. */
typedef struct {
  int32_t batch;       /* B >= 0 (B == 0: nothing to do, returns CLO_OK) */
  int32_t n_q_heads;   /* Hq, a multiple of n_kv_heads, Hq / Hkv <= 8 */
  int32_t n_kv_heads;  /* Hkv, 1..64 */
  int32_t head_dim;    /* d, must be 128 */
  int64_t context;     /* N >= 1 tokens */
  int64_t topk;        /* k, 1 <= k <= N (the pages use k = ceil(N / 10)) */
  float tau;           /* reuse threshold: reuse when cos >= tau; +inf forces every unit to miss */
  int32_t dtype;       /* clo_dtype of q, q_prev, K, V, caches and out */
  int64_t capacity;    /* rows allocated per (sequence, head) in k_hbm, v_hbm, k_host, v_host and
                          k_score: the row stride of those tensors.  0 = context.  A context that
                          grows during decoding (clo_append_kv) keeps capacity fixed and raises
                          context; only rows 0..context-1 are read. */
  const float* tau_heads;  /* per-head thresholds (synthesis section 3.3, attack point 6, and
                              section 5.3: profiling sets a threshold per head): host array
                              of exactly n_kv_heads floats (the library reads that many; a
                              shorter array is read past its end), read during the call;
                              unit (b, h) reuses when cos >= tau_heads[h].  NULL = tau for
                              every head. */
  int32_t block_size;  /* selection granularity (KV-cache offloading article: pillar 2, PulseInfer
                          paragraph -- per-head selection fragments host transfers; pillar 3,
                          block-sparse recall -- whole blocks keep each recall one transfer).  0 or 1 =
                          tokens.  B > 1: the context is cut into floor(N / B) full blocks of B
                          consecutive tokens (a partial tail block is not selectable), a block
                          scores the max of its tokens' scores, the k / B best blocks are taken
                          (ties to the lower block) and idx lists their tokens ascending.  Needs
                          topk a multiple of B and at most floor(N / B) * B. */
} clo_shape;

/* Where one layer's keys, values, selections and cached rows live. */
typedef struct {
  uint64_t persistent_mask;  /* bit h set: KV head h keeps its full K/V in HBM (same for all sequences) */
  const void* k_hbm;         /* [B, P, C, d] device; may be NULL when P == 0 */
  const void* v_hbm;
  const void* k_host;        /* [B, H, C, d] pinned host (dtype, or int8); may be NULL when H == 0 */
  const void* v_host;
  const void* k_score;       /* [B, H, C, d] device copy of k_host, read by scoring */
  void* k_cache;             /* [B, H, k, d] device, written for miss units, read by attention */
  void* v_cache;
  int32_t* idx;              /* [B, Hkv, k] device, written for miss units, read for all units */
  int32_t host_format;       /* clo_host_format of k_host / v_host (0 = the shape's dtype) */
  const int8_t* k_host_exp;  /* CLO_HOST_INT8/INT4: [B, H, C] device, row scale exponents of k_host */
  const int8_t* v_host_exp;  /*                [B, H, C] device, of v_host */
} clo_layer;

/*
 * Device-side ordering between streams (the pages' GPU-centric
 * synchronization: abstract, feature (3); synthesis section 2.1 item 3, "UVA
 * polling" instead of coarse CPU-centric synchronization).  Every entry point
 * takes one (NULL = none).  All pointers are device memory and may be NULL
 * (then that half is skipped).  A producer's signal must be enqueued (in host
 * order) before the consumer's wait, as with events: streams beyond the
 * device's hardware queues (GPU_MAX_HW_QUEUES) share one, which starts kernels
 * in the order they were enqueued, so there a wait enqueued ahead of its
 * signal runs out its bound.
 *   wait_flag/wait_value      before its first kernel, the call waits on the
 *                             GPU until *wait_flag >= wait_value (acquire,
 *                             agent scope), polling at most spin_limit times
 *                             (0 = a default of about one second); on time-out
 *                             it writes CLO_E_TIMEOUT to *error_word (when not
 *                             NULL) and continues.
 *   signal_flag/signal_value  after its last kernel, the call stores
 *                             signal_value to *signal_flag (release, agent scope).
 *   error_word                asynchronous errors of the call's kernels: a
 *                             timed-out wait (CLO_E_TIMEOUT) or a selected index
 *                             outside 0..context-1 met by the gather or by
 *                             attention over persistent heads (CLO_E_INDEX; the
 *                             kernel reads the nearest row in range instead and
 *                             finishes normally).  Only a zero word is written,
 *                             so the first error stays; the caller clears it.
 *                             NULL = such errors are not reported.
 */
typedef struct {
  const uint32_t* wait_flag;
  uint32_t wait_value;
  uint32_t* signal_flag;
  uint32_t signal_value;
  uint32_t* error_word;
  uint32_t spin_limit;
} clo_sync;

/* Bytes of device workspace the calls below need for `shape` (0 for a bad shape). */
size_t clo_workspace_size(const clo_shape* shape);

/*
 * A1 -- reuse test (synthesis 2.1 item 2; abstract feature (1)).
 * For each unit: c = <q_g, q_prev_g> / (|q_g| |q_prev_g|) over the unit's g
 * query heads read as one g*d vector (c = 0 when a norm is 0), in fp32;
 * reuse[u] = (c >= tau).  cos and sync may be NULL.
 */
clo_status clo_reuse_test(const clo_shape* shape, const void* q, const void* q_prev,
                          uint8_t* reuse, float* cos, const clo_sync* sync, void* stream);

/*
 * A2 + A3 -- scoring and exact top-k (synthesis 2.2 and 2.3 table).
 * For every miss unit (reuse[u] == 0; all units when reuse is NULL): scores
 * s_j = max_h q_h . K_j accumulated in fp32 over the unit's keys (k_hbm for
 * persistent heads, k_score otherwise), then idx[u] = the k tokens with the
 * largest s_j (ties to the smaller index), ascending (with shape->block_size
 * > 1: the tokens of the k / block_size best blocks).  idx of hit units is
 * left untouched.  ws: device workspace of at least clo_workspace_size() bytes.
 * sync may be NULL.
 */
clo_status clo_topk_select(const clo_shape* shape, const clo_layer* layer, const void* q,
                           const uint8_t* reuse, void* ws, size_t ws_bytes, const clo_sync* sync,
                           void* stream);

/*
 * A1 + A2 + A3 in one call -- clo_reuse_test followed by clo_topk_select(reuse),
 * with the same arguments, outputs and errors as the two calls (reuse and cos
 * written for every unit, idx for the miss units).  For pipelines that gather
 * and attend on other streams (one-layer-ahead prefetch, synthesis 5.6): on
 * layers of at most 64 units (batch x KV heads) the reuse test, the unit lists
 * and the wait on sync->wait_flag take one launch instead of three.  sync may be NULL (its
 * wait precedes the reuse test, its signal follows the top-k).
 */
clo_status clo_reuse_select(const clo_shape* shape, const clo_layer* layer, const void* q,
                            const void* q_prev, uint8_t* reuse, float* cos, void* ws, size_t ws_bytes,
                            const clo_sync* sync, void* stream);

/*
 * A4 -- gather (abstract features (2) and (3); synthesis 2.1 item 3).
 * For every miss unit of a non-persistent head: k_cache[u][i] = k_host[u][idx[u][i]]
 * and v_cache[u][i] = v_host[u][idx[u][i]], read by the GPU directly from pinned
 * host memory (bit-exact copies; with CLO_HOST_INT8 the rows are dequantized
 * exactly, q_i * 2^e, on the way into the cache).  An idx entry outside
 * 0..context-1 (a corrupt caller selection) is reported as CLO_E_INDEX in
 * sync->error_word and the row nearest to it is copied.  Persistent heads need no transfer: attention
 * reads their rows in place.  reuse NULL = all units miss.  ws: device workspace
 * as for clo_topk_select (the gather's blocks take work from a counter in it;
 * calls that share one workspace must not overlap).  sync may be NULL.  With
 * sync->wait_flag the wait and the signal happen inside the gather kernel (its
 * blocks poll the flag, the last block to finish stores the signal), so the
 * call is one launch; it then needs the workspace's two gather counters at zero,
 * as every call on a workspace leaves them and every selection call
 * (clo_topk_select, clo_reuse_select, clo_decode_step) sets them: a workspace
 * whose first use is such a call must be zero-filled once.
 */
clo_status clo_gather_kv(const clo_shape* shape, const clo_layer* layer, const uint8_t* reuse,
                         void* ws, size_t ws_bytes, const clo_sync* sync, void* stream);

/*
 * A4 for many layers in one launch (a resident gather: the KV-cache offloading
 * article, pillar 3, on a long-running kernel that decides on the GPU when to
 * move data; synthesis section 5.6, one-layer-ahead prefetch; abstract feature
 * (3), GPU-centric synchronization).  Layer by layer, in plan order, the
 * kernel's blocks wait until the layer's wait_flag reaches the step's
 * wait_value (its selection is done), gather the layer exactly as
 * clo_gather_kv does, and the last block to finish stores the step's
 * signal_value to the layer's signal_flag (release, agent scope); a block
 * that runs out of a layer's work goes straight on to the next layer.
 *
 * clo_gather_plan validates every layer as clo_gather_kv would, writes their
 * descriptors into `plan` (device memory of clo_gather_plan_size(n_layers)
 * bytes, caller-owned) with a blocking copy, clears each layer's gather
 * counters in its workspace, and returns in *blocks the grid size to pass to
 * clo_gather_layers.  The plan stays valid while the layers' buffers, reuse
 * flags, workspaces and flags stay where they were.  Layers may differ in shape,
 * dtype and host format.  n_layers in 1..4096.
 *
 * clo_gather_layers enqueues one launch on `stream`.  Every layer's wait_flag
 * must be signalled by work enqueued (in host order) before this call.  Waits
 * are bounded by spin_limit polls per block and layer (0 = about a second); a
 * time-out or a selected index out of range is reported in error_word (device,
 * may be NULL) as for clo_sync.  A layer's workspace must not be used by
 * other calls while the launch runs.
 */
typedef struct {
  const clo_shape* shape;
  const clo_layer* layer;
  const uint8_t* reuse;       /* device [B, Hkv] reuse flags (NULL = every unit misses) */
  void* ws;                   /* the layer's workspace, as for clo_gather_kv */
  size_t ws_bytes;
  const uint32_t* wait_flag;  /* device: the layer's selection is done once *wait_flag >= wait_value */
  uint32_t* signal_flag;      /* device: set to signal_value once the layer's rows are in its cache */
} clo_gather_layer;

size_t clo_gather_plan_size(int32_t n_layers);
clo_status clo_gather_plan(const clo_gather_layer* layers, int32_t n_layers, void* plan, size_t plan_bytes,
                           int32_t* blocks);
clo_status clo_gather_layers(const void* plan, int32_t n_layers, int32_t blocks, uint32_t wait_value,
                             uint32_t signal_value, uint32_t* error_word, uint32_t spin_limit, void* stream);

/*
 * Selection of many layers in four launches -- for each layer what
 * clo_reuse_select does (A1 reuse test, then A2 scoring and A3 top-k of its
 * miss units), with the layers' launches merged: the reuse test and unit lists
 * of every layer in one launch (one block per layer, each after the layer's
 * own wait), the scoring of all the layers' miss units in one launch, their
 * top-k in one more, and a one-wave launch that signals every layer.  For
 * decode steps whose layers are small (a few sequences: each layer's own
 * scoring and top-k launches are short, their ramp-up, tail and launch gaps
 * cost more than their keys), with the selections running ahead of the
 * layers' attention as the pages' prefetch does (synthesis section 5.6;
 * abstract feature (3), GPU-centric synchronization).
 *
 * clo_select_plan writes, into `plan` (device, clo_select_plan_size bytes),
 * everything the launches need for each layer: its shape (thresholds
 * included), buffers, workspace, and flags.  All layers of a plan must have
 * the same batch, heads, context and top-k, bf16 data, batch * n_kv_heads <=
 * 64, token top-k (block_size <= 1) and a context of at most 128 chunks of
 * 16384 keys (CLO_E_UNSUPPORTED otherwise; the per-layer calls take the other
 * shapes).  A plan stays valid while its buffers, workspaces and flags stay
 * where they were; it is written once, with hipMemcpy (the call synchronizes).
 *
 * clo_select_layers enqueues the selection of plan layers first .. first +
 * count - 1 (count <= 64) on `stream`: each layer waits until *wait_flag >=
 * wait_value (bounded by spin_limit polls, 0 = about a second; a time-out
 * writes CLO_E_TIMEOUT to error_word and the layer goes on), and once every
 * layer of the call is selected, signal_value is stored to each layer's
 * signal_flag (release, agent scope).  `shape` is the shape the plan's layers
 * share (its tau and tau_heads are not used: each layer keeps its own); a
 * layer that does not match it is skipped and CLO_E_ARG written to
 * error_word.  Outputs are bit for bit those of clo_reuse_select on each layer.
 * Calls on one plan must not overlap (they share its counters).
 */
typedef struct {
  const clo_shape* shape;
  const clo_layer* layer;     /* persistent_mask, k_hbm, k_score and idx are used */
  const void* q;              /* [B, Hq, d] device: the query the layer selects with */
  const void* q_prev;         /* [B, Hq, d] device: the reuse test's reference */
  uint8_t* reuse;             /* [B, Hkv] device */
  float* cos;                 /* [B, Hkv] device, may be NULL */
  void* ws;                   /* the layer's workspace (clo_workspace_size) */
  size_t ws_bytes;
  const uint32_t* wait_flag;  /* device, may be NULL */
  uint32_t* signal_flag;      /* device, may be NULL */
} clo_select_layer;

size_t clo_select_plan_size(int32_t n_layers);
clo_status clo_select_plan(const clo_select_layer* layers, int32_t n_layers, void* plan, size_t plan_bytes);
clo_status clo_select_layers(const clo_shape* shape, const void* plan, int32_t first, int32_t count,
                             uint32_t wait_value, uint32_t signal_value, uint32_t* error_word, uint32_t spin_limit,
                             void* stream);

/*
 * A5 -- sparse attention over the selected rows, every unit (synthesis 2.3
 * table).  For query head h of unit u: l_i = q_h . K_sel_i / sqrt(d),
 * p = softmax(l), out_h = sum_i p_i V_sel_i, accumulated in fp32 and rounded
 * to dtype.  Rows come from k_cache/v_cache (non-persistent heads) or from
 * k_hbm/v_hbm at idx (persistent heads; an index outside 0..context-1 is
 * reported as CLO_E_INDEX in sync->error_word and the nearest row is read).
 * ws as for clo_topk_select.
 */
clo_status clo_sparse_attn(const clo_shape* shape, const clo_layer* layer, const void* q, void* out,
                           void* ws, size_t ws_bytes, const clo_sync* sync, void* stream);

/*
 * A5 over many layers -- the attention of a batch of layers in four launches
 * instead of four per layer (clo_sparse_attn with a wait and a signal), for a
 * layer loop whose attention stream follows a gather layer by layer (synthesis
 * section 5.6 prefetch; abstract feature (3), GPU-centric synchronization):
 * beside the host reads of a running gather every launch takes several times
 * its work alone.
 *
 * clo_attend_plan writes, into `plan` (device, clo_attend_plan_size bytes),
 * what the launches need for each layer: its shape, buffers (k_cache, v_cache,
 * k_hbm, v_hbm, idx and persistent_mask of `layer`), query, output, workspace
 * (whose chunk partials it uses) and flags.  All layers of a plan must have the
 * same batch, heads, top-k and dtype.  A plan stays valid while those buffers
 * stay where they were; it is written once, with hipMemcpy (the call
 * synchronizes).
 *
 * clo_attend_layers enqueues on `stream` the attention of plan layers first ..
 * first + count - 1 (count <= 64): a wait until every layer's *wait_flag >=
 * wait_value (bounded by spin_limit polls, 0 = about a second; a time-out
 * writes CLO_E_TIMEOUT to error_word and the attention goes on), the outputs
 * of every unit of every layer, bit for bit those of clo_sparse_attn on each
 * layer, and then signal_value stored to each layer's signal_flag (release,
 * agent scope).  `shape` is the shape the plan's layers share; a layer that
 * does not match it is skipped and CLO_E_ARG written to error_word, as is a
 * call reaching past the plan's layers (which then does nothing).  Selected
 * indices out of range on persistent heads are reported as CLO_E_INDEX in
 * error_word, as by clo_sparse_attn.  Calls whose layers share a workspace
 * must not overlap.
 */
typedef struct {
  const clo_shape* shape;
  const clo_layer* layer;
  const void* q;               /* [B, Hq, d] device: the query the layer attends with */
  void* out;                   /* [B, Hq, d] device */
  void* ws;                    /* the layer's workspace */
  size_t ws_bytes;
  const uint32_t* wait_flag;   /* device, may be NULL */
  uint32_t* signal_flag;       /* device, may be NULL */
} clo_attend_layer;

size_t clo_attend_plan_size(int32_t n_layers);
clo_status clo_attend_plan(const clo_attend_layer* layers, int32_t n_layers, void* plan, size_t plan_bytes);
clo_status clo_attend_layers(const clo_shape* shape, const void* plan, int32_t first, int32_t count,
                             uint32_t wait_value, uint32_t signal_value, uint32_t* error_word, uint32_t spin_limit,
                             void* stream);

/*
 * A1..A5 -- one whole decode step of one layer: reuse test, then scoring,
 * top-k and gather for the miss units, then attention for all units.  Same
 * buffers and semantics as the calls above; the reuse decisions never leave
 * the GPU.  cos may be NULL; reuse must not be NULL.
 *
 * When the layer has offloaded heads (and at least 16 units), `stream` is not
 * capturing a graph and the environment variable CLO_STEP_IN_ORDER is not "1"
 * (set it for tools that run one kernel at a time, such as hardware counter
 * collection), the step overlaps its HBM work with the host gather (otherwise
 * every kernel runs in order on `stream`): units are split into ranges;
 * `stream` scores and selects range after range, helper streams read each
 * range's host rows once its top-k is done (a gather launch per range on two
 * streams in turn, or, from 256 units on, one resident gather launch for all
 * ranges), and another helper stream attends the reuse units and then each
 * gathered range.
 * The helper streams (default priority, non-blocking) and their events are
 * created by the library on first use per device and kept until the process
 * ends; they hold no user data.  All ordering is done on the GPU, with events
 * and with flags in the workspace that the consumers poll (bounded at about a
 * second whatever sync->spin_limit says, which bounds the caller's own wait
 * only; a time-out writes CLO_E_TIMEOUT to sync->error_word and the consumer
 * goes on); the call is ordered after
 * earlier work on `stream`, and later work on `stream` is ordered after all of
 * the step.  Every kernel that polls a flag is enqueued after the kernels that
 * raise it, so the step also completes where its streams share hardware
 * queues (then its parts run partly or wholly one after another).  Concurrent
 * calls on one device share the helper streams (their work then runs one
 * after another).
 */
clo_status clo_decode_step(const clo_shape* shape, const clo_layer* layer, const void* q,
                           const void* q_prev, void* out, uint8_t* reuse, float* cos,
                           void* ws, size_t ws_bytes, const clo_sync* sync, void* stream);

/*
 * How clo_decode_step runs a layer of this shape (persistent_mask and
 * host_format as in clo_layer), on a stream that is not capturing a graph: every kernel in order
 * on the stream, a gather launch per unit range on two helper streams in turn,
 * or one resident gather launch for all ranges; the ranges, the gather's grid
 * and the host bytes its loads keep in flight (the quantity the gather grids
 * are sized by: a few hundred KiB saturate the host link, and more slows every
 * HBM kernel beside it).  Host-only; writes *out.
 */
typedef enum {
  CLO_STEP_IN_ORDER = 0,
  CLO_STEP_RANGE_GATHERS = 1,
  CLO_STEP_RESIDENT_GATHER = 2
} clo_step_mode;

typedef struct {
  int32_t mode;                         /* clo_step_mode */
  int32_t ranges;                       /* unit ranges (1 in order) */
  int32_t gather_blocks;                /* blocks of one gather launch (0: nothing to gather) */
  int32_t gather_blocks_in_flight;      /* gather blocks running at once at most */
  int64_t host_bytes_per_gather_block;  /* host reads one gather block keeps in flight */
  int64_t host_bytes_in_flight;         /* gather_blocks_in_flight x host_bytes_per_gather_block */
} clo_step_schedule;

clo_status clo_decode_step_schedule(const clo_shape* shape, uint64_t persistent_mask, int32_t host_format,
                                    clo_step_schedule* out);

/*
 * GPU time, in ms, of the gather inside the last overlapped clo_decode_step on
 * the current device (clo_step_mode 1 or 2): from the start of its first
 * gather launch to the end of its last, measured with events on the helper
 * streams the gathers run on.  For measurement: the caller's events cannot
 * bracket work on the library's streams.  Call once that step has completed
 * (CLO_E_ARG while it runs, or when no overlapped step has gathered on this
 * device).  The resident launch's time includes its wait for the first
 * range's selection.
 */
clo_status clo_last_step_gather_ms(float* ms);

/*
 * clo_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, semantics and outputs
 * as clo_decode_step, bit for bit.  Its workspace is the library's static
 * device scratch of CLO_STATIC_SCRATCH_BYTES per device (part of the library's
 * code object, held until the process ends); the call allocates, frees and
 * creates nothing, and runs every kernel in order on `stream` (no helper
 * streams, so the host gather does not overlap the scoring here).  A shape whose
 * clo_workspace_size() exceeds CLO_STATIC_SCRATCH_BYTES is rejected with
 * CLO_E_WORKSPACE before anything is launched.  Every call on one device uses
 * the same scratch, which keeps the last call's contents (the step clears what
 * must start at zero itself): calls that overlap on one device -- on different
 * streams, or from different threads -- race and must not be made.
 */
#define CLO_STATIC_SCRATCH_BYTES (32u << 20)
clo_status clo_decode_step_static(const clo_shape* shape, const clo_layer* layer, const void* q,
                                  const void* q_prev, void* out, uint8_t* reuse, float* cos, const clo_sync* sync,
                                  void* stream);

/*
 * Multi-step decoding with a growing context -- appending the decoded token
 * (synthesis section 5.7 on incremental offloading: new KV goes to host memory
 * as it is produced; abstract feature (3): the GPU moves KV without CPU work).
 * Writes k_new[b][h] and v_new[b][h] ([B, Hkv, d] device, dtype of the shape)
 * as row `position` of every (sequence, KV head): into k_hbm/v_hbm for
 * persistent heads; for the others into k_host/v_host, stored by the GPU
 * straight into pinned host memory (quantized first when the layer's
 * host_format is CLO_HOST_INT8 or CLO_HOST_INT4, its exponents into
 * k_host_exp/v_host_exp), and
 * into the k_score copy.  Requires
 * 0 <= position < capacity (CLO_E_ARG otherwise); shape->context is not used
 * beyond validation and the row is visible to later calls on the same stream
 * (a decode step with context = position + 1 reads it).  k_cache, v_cache and
 * idx are not touched.  sync may be NULL.
 */
clo_status clo_append_kv(const clo_shape* shape, const clo_layer* layer, const void* k_new, const void* v_new,
                         int64_t position, const clo_sync* sync, void* stream);

/*
 * Reference queries for the reuse test across many steps (synthesis section
 * 2.1 item 2; the pages leave open which earlier query a step is compared
 * with).  For every unit with reuse[u] == 0 (all units when reuse is NULL),
 * copies the unit's g query heads of q into q_ref ([B, Hq, d], device, dtype
 * of the shape); reuse units keep their reference.  Passing q_ref as q_prev to
 * the next step then compares each unit with the query of its last refresh
 * instead of the previous step's query.  sync may be NULL.
 */
clo_status clo_update_reference(const clo_shape* shape, const void* q, const uint8_t* reuse, void* q_ref,
                                const clo_sync* sync, void* stream);

/*
 * Profiling-based choice of persistent heads (synthesis section 3.3 attack
 * point 6 and section 5.3: offline profiling fixes each head's mean adjacent-
 * step query similarity and the number of persistent heads).  s_hat is a host
 * array [n_layers, n_kv_heads] of per-(layer, KV head) mean cosines; the
 * n_persist slots with the lowest s_hat (the heads that miss most, whose
 * transfers a persistent copy saves) become persistent, ties to the lower
 * (layer, head) index.  Writes masks[l] (bit h = KV head h persistent) for
 * every layer.  Host only: launches nothing.  CLO_E_ARG for NULL pointers,
 * n_kv_heads outside 1..64, n_persist outside 0..n_layers*n_kv_heads or a NaN
 * in s_hat.
 */
clo_status clo_plan_persistent(const float* s_hat, int32_t n_layers, int32_t n_kv_heads, int32_t n_persist,
                               uint64_t* masks);

/*
 * Quantize rows for a quantized host copy (CLO_HOST_INT8 or CLO_HOST_INT4;
 * quantized offloaded KV, KV-cache offloading article, pillar 3, quantized
 * offloading: fewer bytes cross the host link and the GPU dequantizes).
 * Reads n_rows rows of 128 elements of `dtype` from src (device), writes their
 * quantized values (host_format CLO_HOST_INT8: 128 bytes per row; CLO_HOST_INT4:
 * 64 bytes) to dst (device or pinned host memory; row r at dst + r * dst_stride
 * bytes, dst_stride at least the row's bytes and a multiple of 16: twice the
 * row's bytes fills the K or V half of the format's records) and their scale
 * exponents to dst_exp (device, [n_rows]), by the rules documented at
 * clo_host_format.  CLO_E_ARG for another host_format.  Finite inputs only.
 * sync may be NULL.
 */
clo_status clo_quantize_rows(const void* src, int64_t n_rows, int32_t dtype, int32_t host_format, void* dst,
                             int64_t dst_stride, int8_t* dst_exp, const clo_sync* sync, void* stream);

/*
 * Measurement helper (no step of the method): reads `bytes` (a multiple of 16)
 * of device memory at src (16-byte aligned) with `blocks` blocks of 256
 * threads, 16-byte loads, and leaves *sink (device, 4 bytes) unchanged except
 * with probability 2^-32.  Timed around its launch it gives the HBM read
 * ceiling against which the HBM-bound kernels (scoring, attention) are
 * reported, as the pinned->device copy gives the host link's.  Asynchronous
 * on `stream`; bytes == 0 launches nothing.  CLO_E_ARG for a size that is not
 * a multiple of 16, blocks outside 1..2^20, or a src / sink that is NULL,
 * misaligned, not device memory or shorter than the size.
 */
clo_status clo_stream_read(const void* src, size_t bytes, int32_t blocks, uint32_t* sink, void* stream);

/* Static text for a status code. */
const char* clo_status_string(clo_status status);

/* Copies the calling thread's message for its last non-OK status into buf
 * (NUL-terminated, truncated to len) and returns that status. */
clo_status clo_last_error(char* buf, size_t len);

#ifdef __cplusplus
}
#endif

#endif /* CLO_H */
