/*
 * Seeded synthetic inputs for exact attention: i.i.d. N(0,1) values rounded to bf16,
 * and seeded row samples. This module holds no attention arithmetic; it only produces
 * the bytes that both the fp64 oracle and the GPU library consume.
 *
 * Definition (fixed so either side can regenerate any element on its own):
 *   sm64(x)   = first output of Vigna's splitmix64 generator whose state is x
 *               (state += 0x9E3779B97F4A7C15, then the two xor-shift-multiply rounds).
 *   key(t)    = sm64(seed ^ (t << 56)),  t = 1 Q, 2 K, 3 V, 4 dO, 5 row sample.
 *   x_n       = sm64(key(t) + n) for the flat row-major element index n.
 *   u1 = ((x_n >> 32) + 1) / 2^32  in (0, 1],   u2 = (x_n & 0xffffffff) / 2^32  in [0, 1).
 *   z  = sqrt(-2 ln u1) * cos(2 pi u2)   (Box-Muller, fp64), then fp64 -> fp32 -> bf16,
 *        each step round-to-nearest-even.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static inline uint64_t sm64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t seedgen_sm64(uint64_t x) { return sm64(x); }

uint64_t seedgen_stream_key(uint64_t seed, uint32_t tensor) {
  return sm64(seed ^ ((uint64_t)tensor << 56));
}

/* fp32 -> bf16 bit pattern, round to nearest, ties to even (inputs are finite). */
uint16_t seedgen_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

double seedgen_normal_f64(uint64_t key, uint64_t n) {
  uint64_t x = sm64(key + n);
  double u1 = ((double)(x >> 32) + 1.0) * (1.0 / 4294967296.0);
  double u2 = (double)(x & 0xFFFFFFFFull) * (1.0 / 4294967296.0);
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

typedef struct {
  uint64_t key, start, count;
  uint16_t* out;
} fill_job;

static void* fill_worker(void* p) {
  fill_job* j = (fill_job*)p;
  for (uint64_t i = 0; i < j->count; ++i)
    j->out[i] = seedgen_f32_to_bf16((float)seedgen_normal_f64(j->key, j->start + i));
  return NULL;
}

/* out[i] = bf16(z_{start+i}) for i in [0, count). Thread count only splits the range. */
int seedgen_normal_bf16(uint64_t seed, uint32_t tensor, uint64_t start, uint64_t count,
                        uint16_t* out, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (count < (uint64_t)nthreads * 65536) nthreads = 1;
  uint64_t key = seedgen_stream_key(seed, tensor);
  fill_job jobs[256];
  pthread_t th[256];
  uint64_t per = count / (uint64_t)nthreads, rem = count % (uint64_t)nthreads, off = 0;
  for (int t = 0; t < nthreads; ++t) {
    uint64_t c = per + ((uint64_t)t < rem ? 1 : 0);
    jobs[t].key = key; jobs[t].start = start + off; jobs[t].count = c; jobs[t].out = out + off;
    off += c;
  }
  if (nthreads == 1) { fill_worker(&jobs[0]); return 0; }
  int created[256];
  for (int t = 0; t < nthreads; ++t) {
    created[t] = pthread_create(&th[t], NULL, fill_worker, &jobs[t]) == 0;
    if (!created[t]) fill_worker(&jobs[t]);
  }
  for (int t = 0; t < nthreads; ++t)
    if (created[t]) pthread_join(th[t], NULL);
  return 0;
}

/*
 * fp64 -> OCP FP8 E4M3FN bit pattern: sign, 4 exponent bits with bias 7, 3 mantissa bits;
 * largest finite value 448, subnormals m/8 * 2^-6, no infinities (0x7F/0xFF are NaN). Round to
 * nearest, ties to even, then saturate to +-448 (inputs are finite).
 */
uint8_t seedgen_f64_to_e4m3(double x) {
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs(x);
  if (a < 0.015625) { /* below 2^-6: subnormal step 2^-9; code 8 is the smallest normal */
    double m = rint(a * 512.0);
    return (uint8_t)(sign | (uint8_t)m);
  }
  int E;
  double f = frexp(a, &E); /* a = f 2^E, f in [0.5, 1) */
  int e = E - 1 + 7;       /* biased exponent of a = (2f) 2^(E-1) */
  double m = rint((2.0 * f - 1.0) * 8.0);
  if (m >= 8.0) {
    m = 0.0;
    e += 1;
  }
  int code = (e << 3) | (int)m;
  if (code > 0x7E) code = 0x7E;
  return (uint8_t)(sign | code);
}

typedef struct {
  uint64_t key, start, count;
  double inv_scale;
  uint8_t* out;
} fill8_job;

static void* fill8_worker(void* p) {
  fill8_job* j = (fill8_job*)p;
  for (uint64_t i = 0; i < j->count; ++i)
    j->out[i] = seedgen_f64_to_e4m3(seedgen_normal_f64(j->key, j->start + i) * j->inv_scale);
  return NULL;
}

/* out[i] = e4m3(z_{start+i} * inv_scale): the same N(0,1) stream as seedgen_normal_bf16,
   quantised to FP8 E4M3FN at scale 1 / inv_scale. */
int seedgen_normal_e4m3(uint64_t seed, uint32_t tensor, uint64_t start, uint64_t count,
                        double inv_scale, uint8_t* out, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (count < (uint64_t)nthreads * 65536) nthreads = 1;
  uint64_t key = seedgen_stream_key(seed, tensor);
  fill8_job jobs[256];
  pthread_t th[256];
  uint64_t per = count / (uint64_t)nthreads, rem = count % (uint64_t)nthreads, off = 0;
  for (int t = 0; t < nthreads; ++t) {
    uint64_t c = per + ((uint64_t)t < rem ? 1 : 0);
    jobs[t].key = key; jobs[t].start = start + off; jobs[t].count = c;
    jobs[t].inv_scale = inv_scale; jobs[t].out = out + off;
    off += c;
  }
  if (nthreads == 1) { fill8_worker(&jobs[0]); return 0; }
  int created[256];
  for (int t = 0; t < nthreads; ++t) {
    created[t] = pthread_create(&th[t], NULL, fill8_worker, &jobs[t]) == 0;
    if (!created[t]) fill8_worker(&jobs[t]);
  }
  for (int t = 0; t < nthreads; ++t)
    if (created[t]) pthread_join(th[t], NULL);
  return 0;
}

static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/*
 * Seeded row sample for one (batch, head) slice: rows 0..min(16,N)-1, row N-1, and the
 * remaining count-17 rows drawn without replacement from [16, N-1) by a partial
 * Fisher-Yates shuffle driven by x = sm64(key(5) + (slice << 32) + step). Output sorted.
 * If count >= N every row is returned. Returns the number of rows written.
 */
int seedgen_sample_rows(uint64_t seed, uint64_t slice, int32_t N, int32_t count, int32_t* rows) {
  if (N <= 0 || count <= 0) return 0;
  if (count >= N) {
    for (int32_t i = 0; i < N; ++i) rows[i] = i;
    return N;
  }
  int32_t w = 0;
  int32_t head = N < 16 ? N : 16;
  for (int32_t i = 0; i < head && w < count; ++i) rows[w++] = i;
  if (N - 1 >= head && w < count) rows[w++] = N - 1;
  int32_t lo = head, hi = N - 1; /* candidates [lo, hi) */
  int32_t ncand = hi - lo;
  int32_t need = count - w;
  if (need > ncand) need = ncand;
  if (need > 0) {
    int32_t* cand = (int32_t*)malloc(sizeof(int32_t) * (size_t)ncand);
    for (int32_t i = 0; i < ncand; ++i) cand[i] = lo + i;
    uint64_t key = seedgen_stream_key(seed, 5) + (slice << 32);
    for (int32_t s = 0; s < need; ++s) {
      uint64_t x = sm64(key + (uint64_t)s);
      int32_t pick = s + (int32_t)(x % (uint64_t)(ncand - s));
      int32_t tmp = cand[s]; cand[s] = cand[pick]; cand[pick] = tmp;
      rows[w++] = cand[s];
    }
    free(cand);
  }
  qsort(rows, (size_t)w, sizeof(int32_t), cmp_i32);
  return w;
}
