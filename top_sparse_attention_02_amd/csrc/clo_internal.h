// Internal launch interface between the C ABI (clo_api.cpp) and the HIP kernel
// sources (clo_select.hip, clo_gather.hip, clo_attn.hip, clo_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace clo {

constexpr int kHeadDim = 128;
constexpr int kMaxGroup = 8;      // query heads per KV head handled by one unit
constexpr int kMaxKvHeads = 64;   // width of the persistent mask

// Work decomposition (rows / keys per work item).
constexpr int kScoreChunk = 2048;   // keys scored by one work item
constexpr int kGatherChunk = 256;   // rows gathered by one work item
constexpr int kAttnChunk = 256;     // selected rows attended by one work item
constexpr int kPartStride = kHeadDim + 2;  // floats per (chunk, head) partial: o[d], m, l

// Gather grid and depth.  Each 4-wave block keeps kGatherUnroll rows x 2 (K, V)
// x 16 B per lane in flight.  The host link saturates with about 256-512 KiB of
// reads in flight; beyond that the extra slow host reads only fill the memory
// request queues and stall HBM kernels running beside the gather.  Measured on
// MI355X (1 M random 256-byte rows from pinned memory, with an HBM scoring
// kernel and a pointer chase on other streams):
//   in flight   gather alone   scoring beside it   pointer chase beside it
//   4096 KiB    56.1 GB/s      8-24x slower        18x slower
//    512 KiB    56.8 GB/s      1.3-1.5x            1.5x
//    384 KiB    56.7 GB/s      1.2-1.35x           1.3x   (24 blocks x 2 rows)
//    128 KiB    49.4 GB/s      1.1-1.3x            1.2x
// The overlapped single-layer step is bound by the gather alone.  Its unit
// ranges alternate between two gather streams of 20 blocks each (640 KiB in
// flight while both run).  ms per step, one stream of 32 / 24 blocks, two of
// 32 / 24 / 20 / 16: B=64, N=131072 12.41 / 13.19, 12.86 / 13.10 / 12.37 /
// 12.39; B=16, N=32768 3.13 / -, 3.26 / 3.28 / - / 3.03; B=64 with int8 host
// KV 6.65 / -, 6.98 / 7.28 / 6.48 / 6.60 (two streams of 24 fall off a cliff:
// more host reads in flight than the link needs slow every HBM kernel).  A
// standalone gather (one layer of the 48-layer loop, or a phase of its own)
// takes 24 blocks, or 40 for layers of 64 units or more.  Beside the gather,
// the select stream of the 48-layer loop is the longer one, and fewer host
// reads in flight slow its kernels less.  ms per 48-layer step with the
// standalone gather at 16 / 20 / 24 / 32 / 40 blocks:
//   B=1, N=524288 (8 units)    native 19.38 / 19.20 / 19.12 / 20.46 / 21.61
//                              int8   11.71 / 11.31 / 11.26 / 12.19 / 12.76
// and B=8, N=262144 (64 units) 77.9 with 24, 32 or 40 blocks.
// The int8 gather alone (512 x 13108 rows) reads 52.7 / 55.2 / 56.3 GB/s with
// 24 / 32 / 40 blocks: its items wait on index and exponent loads before any
// host read, and its rows carry half the host bytes.
constexpr int kGatherUnroll = 2;
constexpr int kGatherBlocksOverlapped = 20;  // per gather stream
constexpr int kGatherBlocksRanges = 40;      // the resident range gather of clo_decode_step
// host bytes one gather block keeps in flight: 256 lanes x 4 loads of 16 bytes
// (kGatherUnroll rows of K and of V, or 2 x kGatherUnroll quantized records)
constexpr int64_t kGatherBytesPerBlock = 256 * 2 * kGatherUnroll * 16;
constexpr int kGatherBlocksAlone = 24;
constexpr int kGatherBlocksAloneQuant = 32;  // int8 / int4 host rows
constexpr int kGatherBlocksAloneWide = 40;  // layers of at least kGatherWideUnits units
constexpr int kGatherWideUnits = 64;
// Grid of a gather that runs alone on its stream (clo_gather_kv, the in-order
// step, the resident multi-layer gather).  ms per 48-layer step at B=1,
// N=524288 (8 units per layer) with 24 / 32 / 40 blocks: native rows 17.84 /
// 17.91-17.98 / 18.00-18.02, int8 rows 9.84-9.85 / 9.55, int4 rows 7.27-7.34 /
// 7.02-7.08 / 7.41-7.43 (28 and 36: 7.07 and 7.17); at B=8, N=262144 (64
// units) flat within 0.2% over 24-40 (int4 rows 27.87 / 27.81 with 32 / 40,
// 28.45 with 48).  Quantized items wait on index and exponent loads before any
// host read, so they keep fewer bytes in flight per block.
inline int alone_gather_blocks(int64_t units, int32_t host_fmt) {
  if (units >= kGatherWideUnits) return kGatherBlocksAloneWide;
  return host_fmt == CLO_HOST_NATIVE ? kGatherBlocksAlone : kGatherBlocksAloneQuant;
}

// Everything a kernel needs to address one layer's buffers.
struct LayerArgs {
  int32_t B, Hq, Hkv, G, P, H;
  int64_t N, k, Np;  // Np: padded key-row stride of the score workspace
  int64_t C;         // rows allocated per (sequence, head) in the full K/V tensors (>= N)
  float tau;
  float tau_h[kMaxKvHeads];  // threshold of each KV head (tau when none are given)
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
  int32_t bs;            // selection block size (1 = tokens)
  int32_t host_fmt;      // CLO_HOST_NATIVE, CLO_HOST_INT8 or CLO_HOST_INT4
  const int8_t* k_exp;   // CLO_HOST_INT8/INT4: [B, H, C] row exponents of k_host / v_host
  const int8_t* v_exp;
  uint32_t* err;         // device error word for selected indices out of range (may be NULL)
};

constexpr int kQuantMinExp = -120;  // smallest row exponent of the quantized host formats
// bytes of one quantized row of kHeadDim values (a record holds a K and a V row)
constexpr int64_t quant_row_bytes(int32_t host_fmt) { return host_fmt == CLO_HOST_INT4 ? kHeadDim / 2 : kHeadDim; }

// Unit ranges of one decode step: units are split into R contiguous ranges
// [first[r], first[r + 1]) so that the gather of one range can run while the
// next range is scored.
// Layers of at most this many units take the reuse test and the unit lists in
// one single-block launch (16 waves, at most 4 units each; wider layers keep a
// wave per unit in a launch of its own).
constexpr int kFusedReuseUnits = 64;
// clo_decode_step overlaps selection, gather and attention over unit ranges on
// helper streams for layers of at least this many units, and runs smaller
// layers in order on the caller's stream
constexpr int kOverlapUnits = 16;
// ... and from this many units on, with one resident gather launch for all the
// ranges instead of a gather launch per range
constexpr int kResidentGatherUnits = 256;
constexpr int kMaxRanges = 16;
// polls of a device-side wait when the caller gives no bound (about a second:
// 1.35 s measured on an idle MI355X, 0.32 us per poll)
constexpr uint32_t kDefaultSpinLimit = 1u << 22;
struct RangeBounds {
  int32_t first[kMaxRanges + 1];  // first unit of each range; first[R] = U
};

// Layout of the int32 "meta" block at the start of the workspace.
constexpr int kMetaCountAll = 0;   // miss units
constexpr int kMetaCountHost = 1;  // miss units of non-persistent heads
constexpr int kMetaCountHit = 2;   // reuse units
constexpr int kMetaZero = 4;       // always 0
constexpr int kMetaOffAll = 16;    // [R + 1] first position of each range in list_all
constexpr int kMetaOffHost = 40;   // [R + 1] first position of each range in list_host
constexpr int kMetaGather = 64;    // [kMaxRanges] work counters of the range gathers
constexpr int kMetaScore = 80;     // [kMaxRanges] work counters of the range scorings
constexpr int kMetaGatherDone = 96;  // blocks of the standalone gather that have finished
// clo_decode_step's resident range gather (cleared by the compact kernel):
constexpr int kMetaSelFlag = 128;     // [kMaxRanges] 1 once the range's top-k is done
constexpr int kMetaGatherFlag = 144;  // [kMaxRanges] 1 once the range's host rows are in the cache
constexpr int kMetaRangeDone = 160;   // [kMaxRanges] blocks done with the range
constexpr int kMetaInts = 192;

// Multi-block top-k: each unit's keys are split into chunks of kTopkChunk keys,
// one 256-thread block per chunk.
constexpr int kTopkChunk = 16384;

// Per-unit radix-select state in the workspace.
struct TopkState {
  uint32_t prefix;  // digits of the k-th largest key found so far
  uint32_t mask;    // bits of prefix already fixed
  uint32_t rem;     // how many keys still to take among those matching prefix
  uint32_t done;    // chunk blocks finished in the current pass
};

// Per chunk of the digit-4 pass: 256 bins of the chunk's keys that match the
// 24-bit prefix, and the count of its keys above that prefix.  (The one-launch
// top-k keeps only each chunk's counts of keys above and equal to the k-th key
// in the first two words.)
constexpr int kChunkHist = 257;

// Per-unit exchange words of the one-launch top-k: the unit-wide histograms of
// digits 2, 3 and 4 (256 bins each) and four arrival counts.
constexpr int kFusedSyncWords = 3 * 256 + 16;

struct Workspace {
  int32_t* meta;       // counts and range offsets (layout above)
  uint32_t* h0;        // [U][256] per-unit radix histograms (digits 1 and 3)
  uint32_t* h1;        // [U][256] (digits 2 and 4)
  TopkState* tstate;   // [U]
  uint32_t* chist;     // [U][cmax][kChunkHist] per-chunk digit-4 histograms
  int32_t cmax;        // chunks per unit (ceil(N / kTopkChunk))
  int32_t* list_all;   // [U] miss units, ascending
  int32_t* list_host;  // [U] miss units of non-persistent heads, ascending
  int32_t* list_hit;   // [U] reuse units, ascending
  uint32_t* keys;      // [U][Np] order-preserving score keys
  uint32_t* bkeys;     // block selection: [U][Npb] block keys (max of their tokens' keys)
  uint32_t* h0b;       // block selection: [U][256] digit-1 histograms of the block keys
  int32_t* bidx;       // block selection: [U][k / bs] selected blocks, ascending
  int64_t npb;         // block selection: padded row stride of bkeys
  float* part;         // [U][nch][G][kPartStride] attention partials
  uint32_t* fsync;     // [U][kFusedSyncWords] one-launch top-k exchange words
};

// A device-side list of units: list[*lo .. *hi).  list == nullptr means "all
// units" (and, for the gather, "skip reuse units and persistent heads").
struct Span {
  const int32_t* list;
  const int32_t* lo;
  const int32_t* hi;
};

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Device scratch of clo_decode_step_static: a file-scope array in the kernels'
// code object (each device holds its own copy until the process ends).
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
// Device address of the current device's scratch array (looked up once per
// device with hipGetSymbolAddress and kept).
hipError_t static_scratch(void** ptr);

// Launchers: enqueue on `s`; return the HIP error of the launch.
hipError_t launch_reuse(const LayerArgs& a, const void* q, const void* q_prev, uint8_t* reuse, float* cos,
                        hipStream_t s);
// Reuse test + unit lists (one range) in one block, after an optional wait on
// a device flag; layers of at most kFusedReuseUnits units.
hipError_t launch_reuse_compact(const LayerArgs& a, const void* q, const void* q_prev, uint8_t* reuse, float* cos,
                                const Workspace& w, const uint32_t* wait_flag, uint32_t wait_value, uint32_t limit,
                                uint32_t* error_word, hipStream_t s);
// max_units: an upper bound on the span's length, used to size the grid.
hipError_t launch_compact(const LayerArgs& a, const uint8_t* reuse, const Workspace& w, int ranges,
                          const RangeBounds& bounds, hipStream_t s);
// counter: zero at launch (the compact kernel clears the range counters).
// Writes w.keys and the digit-1 histograms of the span's units (cleared by the
// compact kernel).
hipError_t launch_score(const LayerArgs& a, const void* q, Span sp, int64_t max_units, const Workspace& w,
                        uint32_t* counter, int num_cu, hipStream_t s);
hipError_t launch_topk(const LayerArgs& a, Span sp, int64_t max_units, const uint32_t* keys, const Workspace& w,
                       hipStream_t s);
// Top-k of tokens, or of token blocks when a.bs > 1, into a.idx (ascending tokens).
hipError_t launch_select(const LayerArgs& a, Span sp, int64_t max_units, const Workspace& w, hipStream_t s);
// max_blocks bounds the grid: the host link saturates with a few hundred
// waves in flight, and a smaller grid leaves the CUs to concurrent kernels.
// Blocks take work items from *counter (zero at launch) so that blocks that
// start late, behind other streams' work, simply take fewer items.
// Ordering done inside the standalone gather kernel: with wait_flag every block
// polls it before its first read; with done, the last block to finish (done
// counts them) clears *counter and *done for the next launch on the workspace
// and then, with signal_flag, stores signal_value there (release).
struct GatherSync {
  const uint32_t* wait_flag;
  uint32_t wait_value;
  uint32_t limit;
  uint32_t* error_word;
  uint32_t* signal_flag;
  uint32_t signal_value;
  uint32_t* done;
};
hipError_t launch_gather(const LayerArgs& a, const uint8_t* reuse, Span sp, int64_t max_units, int max_blocks,
                         uint32_t* counter, hipStream_t s, const GatherSync* gs = nullptr);
// One layer of a multi-layer gather plan (device memory, written by the host).
struct GatherPlanLayer {
  LayerArgs a;
  const uint8_t* reuse;        // NULL = every unit misses
  uint32_t* counter;           // the layer's gather work counter (in its workspace)
  uint32_t* done;              // blocks done with the layer (in its workspace)
  const uint32_t* wait_flag;   // the layer's rows may be read once *wait_flag >= wait_value
  uint32_t* signal_flag;       // set to signal_value once the layer's rows are in its cache
  uint32_t zero_words[2];      // counter and done of a layer with nothing to gather
};
// The host gathers of a decode step's R unit ranges in one resident launch of
// `blocks` blocks: range by range every block waits (bounded by limit; a
// time-out is written to a.err) until meta[kMetaSelFlag + r] is 1, takes the
// range's items of list_host from meta[kMetaGather + r], and the last block
// done with the range sets meta[kMetaGatherFlag + r] to 1 (release).
hipError_t launch_gather_ranges(const LayerArgs& a, const Workspace& w, int ranges, int blocks, uint32_t limit,
                                hipStream_t s);
hipError_t launch_gather_layers(const GatherPlanLayer* plan, int n_layers, int blocks, uint32_t wait_value,
                                uint32_t signal_value, uint32_t limit, uint32_t* error_word, hipStream_t s);
// One layer of a multi-layer selection plan (device memory, written by the host):
// what clo_reuse_select needs for the layer, its workspace views and its flags.
struct SelectPlanLayer {
  LayerArgs a;
  const void* q;
  const void* q_prev;
  uint8_t* reuse;
  float* cos;
  Workspace w;
  const uint32_t* wait_flag;   // the layer's selection starts once *wait_flag >= wait_value (may be NULL)
  uint32_t* signal_flag;       // set to signal_value once the layer's selection is done (may be NULL)
};
// Counters of a selection launch sequence, at the start of the plan.
struct SelectPlanHeader {
  uint32_t score_counter;  // scoring work items taken
  uint32_t n_layers;       // layers the plan holds (launches past them are refused on the GPU)
  uint32_t pad[62];
};
constexpr int kMaxSelectBatch = 64;  // layers per multi-layer selection
// One layer of a multi-layer attention plan (device memory, written by the host).
struct AttendPlanLayer {
  LayerArgs a;
  const void* q;               // the query the layer attends with
  float* part;                 // the layer's chunk partials (its workspace)
  void* out;
  const uint32_t* wait_flag;   // the layer's rows are ready once *wait_flag >= wait_value (may be NULL)
  uint32_t* signal_flag;       // set to signal_value once the layer's outputs are written (may be NULL)
};
struct AttendPlanHeader {
  uint32_t n_layers;  // layers the plan holds (launches past them are refused on the GPU)
  uint32_t pad[63];
};
constexpr int kMaxAttendBatch = 64;  // layers per multi-layer attention
// The attention of plan layers first .. first + count - 1 (shape: the layers'
// common shape) in four launches: a one-wave wait for every layer's flag
// (bounded by limit), the partials, the combines, and a one-wave launch
// storing signal_value to every layer's signal flag (release).
hipError_t launch_attend_layers(const AttendPlanLayer* plan, const AttendPlanHeader* hdr, int first, int count,
                                const LayerArgs& shape, uint32_t wait_value, uint32_t signal_value, uint32_t limit,
                                uint32_t* err, hipStream_t s);
// Blocks of a one-launch top-k, all resident at once (so chunks per unit at most).
constexpr int kFusedMaxBlocks = 128;
// Reuse test and unit lists (one block per layer, after the layer's wait),
// scoring and top-k of plan layers first .. first + count - 1, then a one-wave
// launch storing signal_value to every layer's signal flag.
hipError_t launch_select_layers(const SelectPlanLayer* plan, SelectPlanHeader* hdr, int first, int count,
                                const LayerArgs& shape, int cmax, uint32_t wait_value, uint32_t signal_value,
                                uint32_t limit, uint32_t* error_word, int num_cu, hipStream_t s);
hipError_t launch_zero(uint32_t* word, hipStream_t s, uint32_t* word2 = nullptr);
hipError_t launch_stream_read(const void* src, int64_t n16, int blocks, uint32_t* sink, hipStream_t s);
hipError_t launch_attn_partial(const LayerArgs& a, const void* q, float* part, Span sp, int64_t max_units,
                               hipStream_t s);
// Output rows of the span's units (all units when sp.list == nullptr).
hipError_t launch_attn_combine(const LayerArgs& a, const float* part, void* out, Span sp, int64_t max_units,
                               hipStream_t s);
hipError_t launch_append(const LayerArgs& a, const void* k_new, const void* v_new, int64_t position,
                         void* k_hbm, void* v_hbm, void* k_host, void* v_host, void* k_score, hipStream_t s);
hipError_t launch_update_reference(const LayerArgs& a, const void* q, const uint8_t* reuse, void* q_ref,
                                   hipStream_t s);
hipError_t launch_quantize_rows(const void* src, int64_t n_rows, int32_t dtype, int32_t host_fmt, uint8_t* dst,
                                int64_t stride, int8_t* dst_exp, hipStream_t s);
hipError_t launch_wait(const uint32_t* flag, uint32_t value, uint32_t spin_limit, uint32_t* error_word,
                       uint32_t* zero_word, hipStream_t s);
// flag[0 .. n) = value (release, agent scope), n <= 64
hipError_t launch_signal(uint32_t* flag, uint32_t value, hipStream_t s, int n = 1);

}  // namespace clo
