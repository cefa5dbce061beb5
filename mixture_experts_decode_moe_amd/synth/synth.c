/*
 * Seeded synthetic inputs for the routed mixture-of-experts FFN layer.
 *
 * This module only draws random numbers and lays them out in the weight
 * formats the layer consumes; it holds none of the layer's arithmetic
 * (no dequantisation, no routing, no products).  Both the CPU oracle's
 * tests and the GPU path's tests and benchmark take their inputs from it.
 *
 * Generator: counter-based SplitMix64 (Steele, Lea and Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014).  Word i of the
 * stream (seed, stream) is mix64(key + (i + 1) * GAMMA) with
 * key = mix64(seed ^ mix64(stream + STREAM_SALT)), so any slice of a tensor
 * can be drawn independently of the rest and on any number of threads.
 *
 * Normals: Box-Muller in double precision from words 2i and 2i+1.
 * Bounded integers: multiply-shift of a 32-bit half word onto [lo, hi]
 * (bias below 2^-24, irrelevant for test data).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL
#define STREAM_SALT 0x632BE59BD9B4E019ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(seed ^ mix64(stream + STREAM_SALT));
}

static inline uint64_t word_at(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

/* u in (0, 1]: never zero, so log(u) is finite. */
static inline double unit_open0(uint64_t r) { return (double)((r >> 11) + 1) * 0x1.0p-53; }
static inline double unit_closed0(uint64_t r) { return (double)(r >> 11) * 0x1.0p-53; }

static inline double normal_at(uint64_t key, uint64_t i) {
  double u1 = unit_open0(word_at(key, 2 * i));
  double u2 = unit_closed0(word_at(key, 2 * i + 1));
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

static inline int64_t bounded(uint32_t r, int64_t lo, int64_t hi) {
  uint64_t span = (uint64_t)(hi - lo + 1);
  return lo + (int64_t)(((uint64_t)r * span) >> 32);
}

/* float32 -> bfloat16, round to nearest even (finite inputs only). */
static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

/* double -> IEEE binary16, round to nearest even, for finite values in the
 * normal or subnormal range (the scales drawn here are ~1e-3). */
static uint16_t f64_to_f16_rne(double v) {
  uint16_t sign = 0;
  if (v < 0) { sign = 0x8000; v = -v; }
  if (v == 0.0) return sign;
  int e2;
  frexp(v, &e2); /* v = m * 2^e2, m in [0.5, 1) */
  int e = e2 - 1; /* v in [2^e, 2^(e+1)) */
  if (e < -14) e = -14; /* subnormal spacing 2^-24 */
  double spacing = ldexp(1.0, e - 10);
  double q = nearbyint(v / spacing); /* default mode: ties to even */
  double r = q * spacing;
  if (r >= 65520.0) return sign | 0x7C00;
  /* encode the exactly representable r */
  if (r < ldexp(1.0, -14)) return sign | (uint16_t)q; /* subnormal */
  frexp(r, &e2);
  e = e2 - 1;
  uint32_t mant = (uint32_t)(ldexp(r, 10 - e) - 1024.0);
  return sign | (uint16_t)((e + 15) << 10) | (uint16_t)mant;
}

/* ---------------------------------------------------------------------- */
/* threading helper                                                        */

typedef void (*range_fn)(const void *ctx, uint64_t begin, uint64_t end);

typedef struct {
  range_fn fn;
  const void *ctx;
  uint64_t begin, end;
} job_t;

static void *job_run(void *p) {
  job_t *j = (job_t *)p;
  j->fn(j->ctx, j->begin, j->end);
  return NULL;
}

static void parallel_for(uint64_t n, int nthreads, range_fn fn, const void *ctx) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (n < (uint64_t)1 << 16 || nthreads == 1) {
    fn(ctx, 0, n);
    return;
  }
  pthread_t th[256];
  job_t jobs[256];
  uint64_t chunk = (n + nthreads - 1) / nthreads;
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    uint64_t b = (uint64_t)t * chunk, e = b + chunk;
    if (b >= n) break;
    if (e > n) e = n;
    jobs[t].fn = fn;
    jobs[t].ctx = ctx;
    jobs[t].begin = b;
    jobs[t].end = e;
    if (pthread_create(&th[t], NULL, job_run, &jobs[t]) != 0) {
      fn(ctx, b, e);
      jobs[t].fn = NULL;
    }
    started = t + 1;
  }
  for (int t = 0; t < started; ++t)
    if (jobs[t].fn) pthread_join(th[t], NULL);
}

/* ---------------------------------------------------------------------- */
/* exported fillers; `first` is the counter index of out[0]               */

typedef struct {
  uint64_t key, first;
  double mean, std;
  void *out;
} normal_ctx;

static void normal_bf16_range(const void *c, uint64_t b, uint64_t e) {
  const normal_ctx *x = (const normal_ctx *)c;
  uint16_t *o = (uint16_t *)x->out;
  for (uint64_t i = b; i < e; ++i)
    o[i] = f32_to_bf16_rne((float)(x->mean + x->std * normal_at(x->key, x->first + i)));
}

static void normal_f32_range(const void *c, uint64_t b, uint64_t e) {
  const normal_ctx *x = (const normal_ctx *)c;
  float *o = (float *)x->out;
  for (uint64_t i = b; i < e; ++i) o[i] = (float)(x->mean + x->std * normal_at(x->key, x->first + i));
}

static void normal_f64_range(const void *c, uint64_t b, uint64_t e) {
  const normal_ctx *x = (const normal_ctx *)c;
  double *o = (double *)x->out;
  for (uint64_t i = b; i < e; ++i) o[i] = x->mean + x->std * normal_at(x->key, x->first + i);
}

/* bf16(N(mean, std^2)) */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t first, double mean, double std,
                       uint16_t *out, uint64_t n, int nthreads) {
  normal_ctx c = {stream_key(seed, stream), first, mean, std, out};
  parallel_for(n, nthreads, normal_bf16_range, &c);
}

/* float32(N(mean, std^2)) */
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t first, double mean, double std,
                      float *out, uint64_t n, int nthreads) {
  normal_ctx c = {stream_key(seed, stream), first, mean, std, out};
  parallel_for(n, nthreads, normal_f32_range, &c);
}

/* N(mean, std^2) in double (used to perturb inputs before rounding) */
void synth_normal_f64(uint64_t seed, uint64_t stream, uint64_t first, double mean, double std,
                      double *out, uint64_t n, int nthreads) {
  normal_ctx c = {stream_key(seed, stream), first, mean, std, out};
  parallel_for(n, nthreads, normal_f64_range, &c);
}

typedef struct {
  uint64_t key, first;
  int64_t lo, hi;
  void *out;
} int_ctx;

static void int8_range(const void *c, uint64_t b, uint64_t e) {
  const int_ctx *x = (const int_ctx *)c;
  int8_t *o = (int8_t *)x->out;
  for (uint64_t i = b; i < e; ++i) {
    uint64_t r = word_at(x->key, x->first + i);
    o[i] = (int8_t)bounded((uint32_t)(r >> 32), x->lo, x->hi);
  }
}

/* int8 uniform on [lo, hi] inclusive, one counter word per element */
void synth_uniform_int8(uint64_t seed, uint64_t stream, uint64_t first, int lo, int hi, int8_t *out,
                        uint64_t n, int nthreads) {
  int_ctx c = {stream_key(seed, stream), first, lo, hi, out};
  parallel_for(n, nthreads, int8_range, &c);
}

static void nib_range(const void *c, uint64_t b, uint64_t e) {
  const int_ctx *x = (const int_ctx *)c;
  uint8_t *o = (uint8_t *)x->out;
  for (uint64_t i = b; i < e; ++i) {
    uint64_t r = word_at(x->key, x->first + i);
    /* element 2j in the low nibble, 2j+1 in the high one, each stored as q + 8 */
    uint8_t lo = (uint8_t)(bounded((uint32_t)(r >> 32), x->lo, x->hi) + 8);
    uint8_t hi = (uint8_t)(bounded((uint32_t)r, x->lo, x->hi) + 8);
    o[i] = (uint8_t)(lo | (hi << 4));
  }
}

/* Packed int4 bytes: two values q uniform on [lo, hi] (within [-7, 7]) per
 * byte, stored offset-binary (q + 8), low nibble = even element. */
void synth_packed_int4(uint64_t seed, uint64_t stream, uint64_t first, int lo, int hi, uint8_t *out,
                       uint64_t nbytes, int nthreads) {
  int_ctx c = {stream_key(seed, stream), first, lo, hi, out};
  parallel_for(nbytes, nthreads, nib_range, &c);
}

typedef struct {
  uint64_t key, first;
  double lo, hi, mult;
  void *out;
} scale_ctx;

static void scale_f16_range(const void *c, uint64_t b, uint64_t e) {
  const scale_ctx *x = (const scale_ctx *)c;
  uint16_t *o = (uint16_t *)x->out;
  for (uint64_t i = b; i < e; ++i) {
    double u = x->lo + (x->hi - x->lo) * unit_closed0(word_at(x->key, x->first + i));
    o[i] = f64_to_f16_rne(x->mult * u);
  }
}

static void scale_f32_range(const void *c, uint64_t b, uint64_t e) {
  const scale_ctx *x = (const scale_ctx *)c;
  float *o = (float *)x->out;
  for (uint64_t i = b; i < e; ++i) {
    double u = x->lo + (x->hi - x->lo) * unit_closed0(word_at(x->key, x->first + i));
    o[i] = (float)(x->mult * u);
  }
}

/* binary16(mult * u), u uniform on [lo, hi) */
void synth_scale_f16(uint64_t seed, uint64_t stream, uint64_t first, double lo, double hi, double mult,
                     uint16_t *out, uint64_t n, int nthreads) {
  scale_ctx c = {stream_key(seed, stream), first, lo, hi, mult, out};
  parallel_for(n, nthreads, scale_f16_range, &c);
}

/* float32(mult * u), u uniform on [lo, hi) */
void synth_scale_f32(uint64_t seed, uint64_t stream, uint64_t first, double lo, double hi, double mult,
                     float *out, uint64_t n, int nthreads) {
  scale_ctx c = {stream_key(seed, stream), first, lo, hi, mult, out};
  parallel_for(n, nthreads, scale_f32_range, &c);
}

/* Seeded permutation of 0..n-1 (Fisher-Yates driven by counter words). */
void synth_permutation(uint64_t seed, uint64_t stream, int32_t *out, int32_t n) {
  uint64_t key = stream_key(seed, stream);
  for (int32_t i = 0; i < n; ++i) out[i] = i;
  for (int32_t i = n - 1; i > 0; --i) {
    uint64_t r = word_at(key, (uint64_t)(n - 1 - i));
    int32_t j = (int32_t)bounded((uint32_t)(r >> 32), 0, i);
    int32_t t = out[i];
    out[i] = out[j];
    out[j] = t;
  }
}

/* float32 -> bfloat16 (round to nearest even) for arrays the recipes
 * perturb in double first. */
void synth_f64_to_bf16(const double *in, uint16_t *out, uint64_t n) {
  for (uint64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne((float)in[i]);
}

/* raw counter words, for tests of the generator itself */
void synth_words(uint64_t seed, uint64_t stream, uint64_t first, uint64_t *out, uint64_t n) {
  uint64_t key = stream_key(seed, stream);
  for (uint64_t i = 0; i < n; ++i) out[i] = word_at(key, first + i);
}

/* the SplitMix64 output function alone, for known-answer tests */
uint64_t synth_mix64(uint64_t z) { return mix64(z); }
