// Host-only exercise of the C ABI, built with AddressSanitizer and UBSan by
// tests/test_host_sanitizers.py: shape validation and workspace sizing over
// valid, edge and invalid shapes; the persistent-head planner on seeded
// inputs (checked against a brute-force selection); status strings; the
// last-error buffer at every length.  Nothing here reaches a kernel launch:
// invalid arguments are rejected before any HIP call, and the valid calls
// use an empty batch, which returns before touching the device.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "clo.h"

static int failures = 0;
#define CHECK(cond)                                                 \
  do {                                                              \
    if (!(cond)) {                                                  \
      std::fprintf(stderr, "CHECK failed line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                   \
    }                                                               \
  } while (0)

static clo_shape shape(int B, int Hq, int Hkv, int d, int64_t N, int64_t k, float tau, int dtype) {
  clo_shape s;
  std::memset(&s, 0, sizeof s);
  s.batch = B;
  s.n_q_heads = Hq;
  s.n_kv_heads = Hkv;
  s.head_dim = d;
  s.context = N;
  s.topk = k;
  s.tau = tau;
  s.dtype = (clo_dtype)dtype;
  return s;
}

static uint64_t lcg(uint64_t& x) {
  x = x * 6364136223846793005ull + 1442695040888963407ull;
  return x >> 11;
}

int main() {
  // workspace sizes: valid shapes give a size, invalid ones 0
  struct Case { clo_shape s; bool ok; };
  std::vector<Case> cases = {
      {shape(64, 32, 8, 128, 131072, 13108, 0.8f, CLO_BF16), true},
      {shape(1, 40, 8, 128, 524288, 52429, 0.8f, CLO_BF16), true},
      {shape(1, 32, 8, 128, 4096, 410, 0.8f, CLO_F32), true},
      {shape(3, 10, 2, 128, 1, 1, 0.8f, CLO_BF16), true},
      {shape(2, 8, 2, 128, 300000, 300000, INFINITY, CLO_F32), true},
      {shape(0, 8, 2, 128, 100, 10, 0.8f, CLO_BF16), true},
      {shape(1, 8, 2, 64, 100, 10, 0.8f, CLO_BF16), false},     // head_dim
      {shape(1, 9, 2, 128, 100, 10, 0.8f, CLO_BF16), false},    // Hq % Hkv
      {shape(1, 8, 2, 128, 100, 101, 0.8f, CLO_BF16), false},   // k > N
      {shape(1, 8, 2, 128, 100, 0, 0.8f, CLO_BF16), false},     // k = 0
      {shape(1, 130, 65, 128, 100, 10, 0.8f, CLO_BF16), false}, // Hkv > 64
      {shape(-1, 8, 2, 128, 100, 10, 0.8f, CLO_BF16), false},   // negative batch
      {shape(1, 8, 2, 128, 100, 10, 0.8f, 7), false},           // dtype
      {shape(1 << 20, 64, 64, 128, 1 << 30, 10, 0.8f, CLO_BF16), false},  // 31-bit grid bound
  };
  for (const Case& c : cases) {
    const size_t ws = clo_workspace_size(&c.s);
    CHECK((ws > 0) == c.ok);
  }
  CHECK(clo_workspace_size(nullptr) == 0);

  // entry points reject bad shapes and NULL pointers without touching the GPU
  char msg[256];
  for (const Case& c : cases) {
    if (c.ok) continue;
    clo_status st = clo_reuse_test(&c.s, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
    CHECK(st == CLO_E_ARG || st == CLO_E_UNSUPPORTED);
    CHECK(clo_last_error(msg, sizeof msg) == st && std::strlen(msg) > 0);
    clo_layer L;
    std::memset(&L, 0, sizeof L);
    st = clo_decode_step(&c.s, &L, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr, nullptr);
    CHECK(st == CLO_E_ARG || st == CLO_E_UNSUPPORTED);
    st = clo_reuse_select(&c.s, &L, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr, nullptr);
    CHECK(st == CLO_E_ARG || st == CLO_E_UNSUPPORTED);
  }
  {
    clo_shape s = shape(2, 8, 2, 128, 1000, 100, 0.8f, CLO_BF16);
    clo_layer L;
    std::memset(&L, 0, sizeof L);
    CHECK(clo_topk_select(&s, &L, nullptr, nullptr, nullptr, 0, nullptr, nullptr) == CLO_E_ARG);
    CHECK(clo_gather_kv(&s, &L, nullptr, nullptr, 0, nullptr, nullptr) == CLO_E_ARG);
    CHECK(clo_sparse_attn(&s, &L, nullptr, nullptr, nullptr, 0, nullptr, nullptr) == CLO_E_ARG);
    CHECK(clo_decode_step(&s, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr, nullptr) ==
          CLO_E_ARG);
    L.persistent_mask = 1ull << 5;  // bit above n_kv_heads
    CHECK(clo_reuse_select(&s, &L, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr, nullptr) == CLO_E_ARG);
    // an empty batch returns before any launch
    clo_shape e = shape(0, 8, 2, 128, 1000, 100, 0.8f, CLO_BF16);
    std::memset(&L, 0, sizeof L);
    CHECK(clo_reuse_select(&e, &L, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr, nullptr) == CLO_OK);
    CHECK(clo_stream_read(nullptr, 17, 1, nullptr, nullptr) == CLO_E_ARG);
    CHECK(clo_stream_read(nullptr, 16, 0, nullptr, nullptr) == CLO_E_ARG);
    CHECK(clo_stream_read(nullptr, 0, 1, nullptr, nullptr) == CLO_OK);
    CHECK(clo_quantize_rows(nullptr, 0, 5, CLO_HOST_INT8, nullptr, 128, nullptr, nullptr, nullptr) ==
          CLO_E_UNSUPPORTED);
    CHECK(clo_quantize_rows(nullptr, -1, CLO_BF16, CLO_HOST_INT8, nullptr, 128, nullptr, nullptr, nullptr) == CLO_E_ARG);
    CHECK(clo_quantize_rows(nullptr, 0, CLO_BF16, CLO_HOST_NATIVE, nullptr, 128, nullptr, nullptr, nullptr) ==
          CLO_E_ARG);
    CHECK(clo_quantize_rows(nullptr, 0, CLO_BF16, CLO_HOST_INT8, nullptr, 64, nullptr, nullptr, nullptr) == CLO_E_ARG);
    CHECK(clo_quantize_rows(nullptr, 0, CLO_BF16, CLO_HOST_INT4, nullptr, 64, nullptr, nullptr, nullptr) == CLO_OK);
    CHECK(clo_quantize_rows(nullptr, 0, CLO_BF16, CLO_HOST_INT4, nullptr, 56, nullptr, nullptr, nullptr) == CLO_E_ARG);
    // the gather and selection plans: sizes and argument checks made before any HIP call
    CHECK(clo_gather_plan_size(0) == 0 && clo_gather_plan_size(4097) == 0 && clo_gather_plan_size(48) > 0);
    CHECK(clo_select_plan_size(0) == 0 && clo_select_plan_size(4097) == 0);
    CHECK(clo_select_plan_size(48) >= 48 * 64 && clo_select_plan_size(48) % 256 == 0);
    CHECK(clo_select_plan(nullptr, 4, nullptr, 1 << 20) == CLO_E_ARG);
    clo_select_layer sl;
    std::memset(&sl, 0, sizeof sl);
    CHECK(clo_select_plan(&sl, 0, nullptr, 1 << 20) == CLO_E_ARG);
    CHECK(clo_select_plan(&sl, 1, nullptr, 16) == CLO_E_ARG);  // plan smaller than clo_select_plan_size(1)
    {
      clo_shape ok_shape = shape(1, 8, 2, 128, 524288, 52429, 0.8f, CLO_BF16);
      CHECK(clo_select_layers(&ok_shape, nullptr, 0, 0, 0, 1, nullptr, 0, nullptr) == CLO_E_ARG);
      CHECK(clo_select_layers(&ok_shape, nullptr, 0, 65, 0, 1, nullptr, 0, nullptr) == CLO_E_ARG);
      CHECK(clo_select_layers(&ok_shape, nullptr, -1, 4, 0, 1, nullptr, 0, nullptr) == CLO_E_ARG);
      clo_shape f32 = shape(1, 8, 2, 128, 524288, 52429, 0.8f, CLO_F32);
      CHECK(clo_select_layers(&f32, nullptr, 0, 4, 0, 1, nullptr, 0, nullptr) == CLO_E_UNSUPPORTED);
      clo_shape wide = shape(64, 32, 8, 128, 131072, 13108, 0.8f, CLO_BF16);  // 512 units per layer
      CHECK(clo_select_layers(&wide, nullptr, 0, 4, 0, 1, nullptr, 0, nullptr) == CLO_E_UNSUPPORTED);
      clo_shape blocks = shape(1, 8, 2, 128, 524288, 52432, 0.8f, CLO_BF16);
      blocks.block_size = 16;
      CHECK(clo_select_layers(&blocks, nullptr, 0, 4, 0, 1, nullptr, 0, nullptr) == CLO_E_UNSUPPORTED);
      clo_shape longer = shape(1, 8, 2, 128, 128 * 16384 + 1, 209716, 0.8f, CLO_BF16);  // 129 chunks
      CHECK(clo_select_layers(&longer, nullptr, 0, 4, 0, 1, nullptr, 0, nullptr) == CLO_E_UNSUPPORTED);
    }
    // the multi-layer attention plan
    CHECK(clo_attend_plan_size(0) == 0 && clo_attend_plan_size(4097) == 0);
    CHECK(clo_attend_plan_size(48) >= 48 * 64 && clo_attend_plan_size(48) % 256 == 0);
    CHECK(clo_attend_plan(nullptr, 4, nullptr, 1 << 20) == CLO_E_ARG);
    {
      clo_attend_layer al;
      std::memset(&al, 0, sizeof al);
      CHECK(clo_attend_plan(&al, 0, nullptr, 1 << 20) == CLO_E_ARG);
      CHECK(clo_attend_plan(&al, 1, nullptr, 16) == CLO_E_ARG);  // plan smaller than clo_attend_plan_size(1)
      clo_shape ok_shape = shape(1, 8, 2, 128, 524288, 52429, 0.8f, CLO_BF16);
      CHECK(clo_attend_layers(&ok_shape, nullptr, 0, 0, 0, 1, nullptr, 0, nullptr) == CLO_E_ARG);
      CHECK(clo_attend_layers(&ok_shape, nullptr, 0, 65, 0, 1, nullptr, 0, nullptr) == CLO_E_ARG);
      CHECK(clo_attend_layers(&ok_shape, nullptr, -1, 4, 0, 1, nullptr, 0, nullptr) == CLO_E_ARG);
      CHECK(clo_attend_layers(&ok_shape, nullptr, 4093, 4, 0, 1, nullptr, 0, nullptr) == CLO_E_ARG);
      clo_shape empty = shape(0, 8, 2, 128, 524288, 52429, 0.8f, CLO_BF16);
      CHECK(clo_attend_layers(&empty, nullptr, 0, 4, 0, 1, nullptr, 0, nullptr) == CLO_E_ARG);
    }
    // how a step runs (host-only) and the gather timer before any overlapped step
    {
      clo_shape b64 = shape(64, 32, 8, 128, 131072, 13108, 0.8f, CLO_BF16);
      clo_step_schedule sc;
      std::memset(&sc, 0xAB, sizeof sc);
      CHECK(clo_decode_step_schedule(nullptr, 0, CLO_HOST_NATIVE, &sc) == CLO_E_ARG);
      CHECK(clo_decode_step_schedule(&b64, 0, CLO_HOST_NATIVE, nullptr) == CLO_E_ARG);
      CHECK(clo_decode_step_schedule(&b64, 0, 7, &sc) == CLO_E_ARG);
      CHECK(clo_decode_step_schedule(&b64, 0, CLO_HOST_NATIVE, &sc) == CLO_OK);
      CHECK(sc.mode == CLO_STEP_RESIDENT_GATHER && sc.ranges == 8 && sc.gather_blocks > 0);
      CHECK(sc.host_bytes_in_flight == (int64_t)sc.gather_blocks_in_flight * sc.host_bytes_per_gather_block);
      CHECK(clo_decode_step_schedule(&b64, 0xFF, CLO_HOST_NATIVE, &sc) == CLO_OK);  // every head persistent
      CHECK(sc.mode == CLO_STEP_IN_ORDER && sc.gather_blocks == 0 && sc.host_bytes_in_flight == 0);
      float ms = -1.f;
      CHECK(clo_last_step_gather_ms(nullptr) == CLO_E_ARG);
      CHECK(clo_last_step_gather_ms(&ms) != CLO_OK && ms == -1.f);
    }
  }

  // the last-error buffer at every length, including 0 and 1
  {
    clo_shape s = shape(1, 8, 2, 64, 100, 10, 0.8f, CLO_BF16);
    clo_reuse_test(&s, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
    char full[512];
    const clo_status st = clo_last_error(full, sizeof full);
    const size_t n = std::strlen(full);
    for (size_t len = 0; len <= n + 2; ++len) {
      std::vector<char> b(len ? len : 1, 'x');
      CHECK(clo_last_error(len ? b.data() : nullptr, len) == st);
      if (len) CHECK(std::strlen(b.data()) == (len - 1 < n ? len - 1 : n));
    }
  }
  for (int c = 0; c < 8; ++c) CHECK(clo_status_string((clo_status)c) != nullptr);  // the enum's value range

  // persistent-head planner against a brute-force choice on seeded inputs
  uint64_t x = 0x5EED;
  for (int trial = 0; trial < 200; ++trial) {
    const int L = 1 + (int)(lcg(x) % 48), H = 1 + (int)(lcg(x) % 64);
    const int slots = L * H;
    const int np = (int)(lcg(x) % (slots + 1));
    std::vector<float> s_hat(slots);
    for (float& v : s_hat) v = (float)(lcg(x) % 16) / 16.0f;  // many ties
    std::vector<uint64_t> masks(L, ~0ull);
    CHECK(clo_plan_persistent(s_hat.data(), L, H, np, masks.data()) == CLO_OK);
    // brute force: the np smallest (value, slot index) pairs
    std::vector<char> want(slots, 0);
    for (int i = 0; i < np; ++i) {
      int best = -1;
      for (int j = 0; j < slots; ++j)
        if (!want[j] && (best < 0 || s_hat[j] < s_hat[best])) best = j;
      want[best] = 1;
    }
    for (int j = 0; j < slots; ++j) CHECK((((masks[j / H] >> (j % H)) & 1ull) != 0) == (want[j] != 0));
  }
  {
    float s[4] = {0.1f, NAN, 0.2f, 0.3f};
    uint64_t m[2];
    CHECK(clo_plan_persistent(s, 2, 2, 1, m) == CLO_E_ARG);
    CHECK(clo_plan_persistent(s, 2, 2, 5, m) == CLO_E_ARG);
    CHECK(clo_plan_persistent(s, 2, 65, 1, m) == CLO_E_ARG);
    CHECK(clo_plan_persistent(nullptr, 2, 2, 1, m) == CLO_E_ARG);
  }
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("host ABI checks passed\n");
  return 0;
}
