/*
 * Seeded synthetic-input generator (test and benchmark infrastructure).
 *
 * Counter-based: element e of a stream with 64-bit key `key` is a pure
 * function of (key, e), so any slice of any tensor can be produced on its
 * own, in any order and with any number of threads, with identical bits.
 *
 *   u64(key, i)  = SplitMix64 output i of the stream whose state starts at
 *                  `key` (Steele, Lea and Flood, "Fast splittable
 *                  pseudorandom number generators", OOPSLA 2014): the state
 *                  after i+1 increments by the golden-ratio gamma, passed
 *                  through the variant-13 finaliser.
 *   normal pair m = Box-Muller transform (Box and Muller, 1958) of the two
 *                  uniforms built from u64(key, 2m) and u64(key, 2m+1);
 *                  element 2m takes the cosine branch, 2m+1 the sine branch.
 *
 * Nothing here computes any part of the decode step itself.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <string.h>

#define SM64_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t sm64_at(uint64_t key, uint64_t i) {
  return sm64_mix(key + (i + 1) * SM64_GAMMA);
}

static inline void normal_pair(uint64_t key, uint64_t m, double* z0, double* z1) {
  const uint64_t a = sm64_at(key, 2 * m);
  const uint64_t b = sm64_at(key, 2 * m + 1);
  const double u1 = (double)((a >> 11) + 1) * 0x1.0p-53; /* (0, 1] */
  const double u2 = (double)(b >> 11) * 0x1.0p-53;       /* [0, 1) */
  const double r = sqrt(-2.0 * log(u1));
  const double t = 6.283185307179586476925286766559 * u2;
  *z0 = r * cos(t);
  *z1 = r * sin(t);
}

static inline double normal_at(uint64_t key, uint64_t e) {
  double z0, z1;
  normal_pair(key, e >> 1, &z0, &z1);
  return (e & 1) ? z1 : z0;
}

/* fp32 -> bf16 bit pattern, round to nearest even (inputs are finite). */
static inline uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

uint64_t gen_u64(uint64_t key, uint64_t i) { return sm64_at(key, i); }
uint64_t gen_mix(uint64_t z) { return sm64_mix(z); }

/* out[i] = u64(key, first + i) */
void gen_u64_fill(uint64_t* out, int64_t n, uint64_t key, int64_t first) {
  for (int64_t i = 0; i < n; ++i) out[i] = sm64_at(key, (uint64_t)(first + i));
}

/* out[i] = uniform [0,1) from u64(key, first + i) */
void gen_uniform_f64(double* out, int64_t n, uint64_t key, int64_t first) {
  for (int64_t i = 0; i < n; ++i)
    out[i] = (double)(sm64_at(key, (uint64_t)(first + i)) >> 11) * 0x1.0p-53;
}

/* out[i] = N(0,1) element (first + i) of stream key, in double. */
void gen_normal_f64(double* out, int64_t n, uint64_t key, int64_t first) {
  for (int64_t i = 0; i < n; ++i) out[i] = normal_at(key, (uint64_t)(first + i));
}

/* out[i * cols + c] = N(0,1) element (rows[i] * cols + c) of stream keys[i]:
 * row rows[i] of a [*, cols] block drawn from stream keys[i]. */
void gen_normal_rows(double* out, const uint64_t* keys, const int64_t* rows, int64_t n, int64_t cols) {
  for (int64_t i = 0; i < n; ++i)
    for (int64_t c = 0; c < cols; ++c)
      out[i * cols + c] = normal_at(keys[i], (uint64_t)(rows[i] * cols + c));
}

/*
 * Fill a [rows, cols] block: row r, column c takes normal element
 * (r * cols + c) of stream key, times row_scale[r] when row_scale is not
 * NULL, rounded to fp32 (dtype 0) or to a bf16 bit pattern (dtype 1).
 */
void gen_fill_rows(void* out, int64_t rows, int64_t cols, uint64_t key,
                   const float* row_scale, int dtype, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  const int64_t total = rows * cols;
  const int64_t npairs = (total + 1) / 2;
#pragma omp parallel for num_threads(nthreads) schedule(static, 65536)
  for (int64_t m = 0; m < npairs; ++m) {
    double z[2];
    normal_pair(key, (uint64_t)m, &z[0], &z[1]);
    for (int j = 0; j < 2; ++j) {
      const int64_t e = 2 * m + j;
      if (e >= total) break;
      double v = z[j];
      if (row_scale) v *= (double)row_scale[e / cols];
      if (dtype == 0)
        ((float*)out)[e] = (float)v;
      else
        ((uint16_t*)out)[e] = f32_to_bf16((float)v);
    }
  }
}

/* Round an fp64 array to fp32 (dtype 0) or bf16 bit patterns (dtype 1). */
void gen_round(void* out, const double* in, int64_t n, int dtype) {
  for (int64_t i = 0; i < n; ++i) {
    if (dtype == 0)
      ((float*)out)[i] = (float)in[i];
    else
      ((uint16_t*)out)[i] = f32_to_bf16((float)in[i]);
  }
}

/* Multi-threaded memcpy, for staging large generated blocks. */
void gen_copy(void* dst, const void* src, int64_t bytes, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  const int64_t chunk = 1 << 22;
  const int64_t nchunks = (bytes + chunk - 1) / chunk;
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t off = c * chunk;
    const int64_t len = (off + chunk <= bytes) ? chunk : bytes - off;
    memcpy((char*)dst + off, (const char*)src + off, (size_t)len);
  }
}
