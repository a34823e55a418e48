/* A C11 caller of the library: the decode step called the way the README
 * shows.  tests/test_c_header.py compiles it with gcc (-pedantic, warnings as
 * errors), links it against libclo.so and runs main(), which makes no GPU call. */
#include <stddef.h>
#include <stdint.h>
#include "clo.h"

clo_status decode_one_layer(const void* q, const void* q_prev, void* out, uint8_t* reuse, float* cos,
                            const void* k_host, const void* v_host, const void* k_score, void* k_cache,
                            void* v_cache, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  clo_shape s = {0};
  s.batch = 64; s.n_q_heads = 32; s.n_kv_heads = 8; s.head_dim = 128;
  s.context = 131072; s.topk = 13108; s.tau = 0.8f; s.dtype = CLO_BF16;
  if (clo_workspace_size(&s) > ws_bytes) return CLO_E_WORKSPACE;
  clo_layer L = {0};
  L.k_host = k_host; L.v_host = v_host;
  L.k_score = k_score;
  L.k_cache = k_cache; L.v_cache = v_cache;
  L.idx = idx;
  clo_status st = clo_decode_step(&s, &L, q, q_prev, out, reuse, cos, ws, ws_bytes, NULL, stream);
  if (st != CLO_OK) {
    char why[256];
    clo_last_error(why, sizeof why);
  }
  return st;
}

int main(void) {
  /* no GPU call: the status strings are host-only */
  return clo_status_string(CLO_OK) == NULL;
}
