/*
 * Seeded synthetic inputs for the LM-head logits projection.
 *
 * This module only *draws* inputs. It holds none of the projection's
 * arithmetic: no dot product, no scaling, no output rounding. Both the CPU
 * oracle and the GPU path consume the same bytes produced here.
 *
 * Every element is a pure function of (seed, stream, index), so any slice of
 * a tensor can be regenerated alone and the bytes do not depend on the number
 * of threads.
 *
 * Definitions used:
 *   - SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable pseudorandom
 *     number generators", OOPSLA 2014; the variant popularised by S. Vigna):
 *     state_n = state_0 + n * 0x9E3779B97F4A7C15, output_n = mix(state_n).
 *     Here output(key, i) = mix(key + (i + 1) * golden).
 *   - Box-Muller (G. Box, M. Muller, Ann. Math. Statist. 1958): one normal
 *     per pair of uniforms, z = sqrt(-2 ln u1) * cos(2 pi u2).
 *   - bfloat16: the top 16 bits of an IEEE binary32, rounded to nearest even.
 *   - OCP FP8 E4M3 (OCP 8-bit Floating Point Specification, 2023): bias 7,
 *     3 mantissa bits, max 448, no infinities.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* The i-th output of a SplitMix64 sequence whose state starts at `key`. */
uint64_t synth_splitmix64_at(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * GOLDEN);
}

/* Key of the sequence for (seed, stream): the first output of a SplitMix64
 * sequence started at seed, xor-ed with the stream id spread by one more mix. */
uint64_t synth_key(uint64_t seed, uint64_t stream) {
  return synth_splitmix64_at(seed, 0) ^ mix64(stream * GOLDEN + 0x632BE59BD9B4E019ULL);
}

/* u in (0, 1]: 53 random bits, offset by one so that log(u) is finite. */
static inline double unit_open0(uint64_t x) { return (double)((x >> 11) + 1) * 0x1.0p-53; }
/* u in [0, 1). */
static inline double unit_closed0(uint64_t x) { return (double)(x >> 11) * 0x1.0p-53; }

static inline uint16_t f32_to_bf16_bits_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u); /* quiet NaN */
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Element i of a standard normal sequence: two uniforms from counters 2i, 2i+1. */
static inline double normal_at(uint64_t key, uint64_t i) {
  double u1 = unit_open0(synth_splitmix64_at(key, 2 * i));
  double u2 = unit_closed0(synth_splitmix64_at(key, 2 * i + 1));
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

/* fp32 -> OCP E4M3 bits, round to nearest even, saturating at +-448 (inputs
 * here are finite and in range). */
static uint8_t f32_to_e4m3_rne(float f) {
  uint8_t sign = signbit(f) ? 0x80 : 0x00;
  double a = fabs((double)f);
  if (a == 0.0) return sign;
  if (a >= 448.0) return sign | 0x7E;
  int e;
  frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) -> a in [2^(e-1), 2^e) */
  int ue = e - 1; /* unbiased exponent of a */
  if (ue < -6) ue = -6; /* subnormal range shares the 2^-6 quantum spacing */
  double q = ldexp(1.0, ue - 3); /* spacing of representable values */
  double n = a / q;              /* exact: power-of-two scaling */
  double r = nearbyint(n);       /* default rounding mode: nearest even */
  long ri = (long)r;
  /* ri in [0, 16]; 16 means carry into the next binade. */
  int be, man;
  if (ue == -6 && ri < 8) {
    be = 0;
    man = (int)ri;
  } else {
    if (ri >= 16) {
      ri = 8;
      ue += 1;
    }
    be = ue + 7;
    man = (int)ri - 8;
  }
  if (be > 15 || (be == 15 && man > 6)) return sign | 0x7E;
  return sign | (uint8_t)((be << 3) | man);
}

/* ---------------- threaded fill over [0, n) ---------------- */

typedef struct {
  int kind;
  uint64_t key, start, n;
  double a, b;
  void *out;
} job_t;

enum { K_NORMAL_BF16 = 0, K_INT_BF16 = 1, K_BYTES = 2, K_UNIFORM_E4M3 = 3, K_NORMAL_F32 = 4, K_INT_F32 = 5 };

static void run_range(const job_t *j, uint64_t lo, uint64_t hi) {
  switch (j->kind) {
    case K_NORMAL_BF16: {
      uint16_t *o = (uint16_t *)j->out;
      for (uint64_t i = lo; i < hi; ++i) {
        float f = (float)(j->a + j->b * normal_at(j->key, j->start + i));
        o[i] = f32_to_bf16_bits_rne(f);
      }
    } break;
    case K_NORMAL_F32: {
      float *o = (float *)j->out;
      for (uint64_t i = lo; i < hi; ++i) o[i] = (float)(j->a + j->b * normal_at(j->key, j->start + i));
    } break;
    case K_INT_BF16: { /* integers uniform in [a, b], exact in bf16 for |x| <= 256 */
      uint16_t *o = (uint16_t *)j->out;
      uint64_t span = (uint64_t)(j->b - j->a + 1.0);
      for (uint64_t i = lo; i < hi; ++i) {
        uint64_t x = synth_splitmix64_at(j->key, j->start + i);
        double v = j->a + (double)((x >> 32) % span);
        o[i] = f32_to_bf16_bits_rne((float)v);
      }
    } break;
    case K_INT_F32: { /* integers uniform in [a, b] as binary32 (exact for |x| <= 2^24) */
      float *o = (float *)j->out;
      uint64_t span = (uint64_t)(j->b - j->a + 1.0);
      for (uint64_t i = lo; i < hi; ++i) {
        uint64_t x = synth_splitmix64_at(j->key, j->start + i);
        o[i] = (float)(j->a + (double)((x >> 32) % span));
      }
    } break;
    case K_BYTES: { /* uniform bytes: every bit independent */
      uint8_t *o = (uint8_t *)j->out;
      for (uint64_t i = lo; i < hi; ++i) o[i] = (uint8_t)(synth_splitmix64_at(j->key, j->start + i) >> 56);
    } break;
    case K_UNIFORM_E4M3: {
      uint8_t *o = (uint8_t *)j->out;
      for (uint64_t i = lo; i < hi; ++i) {
        double u = unit_closed0(synth_splitmix64_at(j->key, j->start + i));
        o[i] = f32_to_e4m3_rne((float)(j->a + (j->b - j->a) * u));
      }
    } break;
  }
}

typedef struct {
  const job_t *j;
  uint64_t lo, hi;
} part_t;

static void *worker(void *p) {
  part_t *q = (part_t *)p;
  run_range(q->j, q->lo, q->hi);
  return NULL;
}

static void run(job_t *j, int threads) {
  if (threads < 1) threads = 1;
  if (threads > 64) threads = 64;
  if (j->n < (uint64_t)threads * 65536) threads = 1;
  if (threads == 1) {
    run_range(j, 0, j->n);
    return;
  }
  pthread_t tid[64];
  part_t parts[64];
  uint64_t chunk = (j->n + threads - 1) / threads;
  int started = 0;
  for (int t = 0; t < threads; ++t) {
    uint64_t lo = (uint64_t)t * chunk, hi = lo + chunk;
    if (lo >= j->n) break;
    if (hi > j->n) hi = j->n;
    parts[t].j = j;
    parts[t].lo = lo;
    parts[t].hi = hi;
    if (pthread_create(&tid[t], NULL, worker, &parts[t]) != 0) {
      run_range(j, lo, hi);
      parts[t].j = NULL;
    }
    started = t + 1;
  }
  for (int t = 0; t < started; ++t)
    if (parts[t].j) pthread_join(tid[t], NULL);
}

/* bf16 bits of (mean + std * N(0,1)), elements [start, start+n) of stream. */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t start, uint64_t n, double mean,
                       double std, uint16_t *out, int threads) {
  job_t j = {K_NORMAL_BF16, synth_key(seed, stream), start, n, mean, std, out};
  run(&j, threads);
}

/* fp32 of (mean + std * N(0,1)). */
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t start, uint64_t n, double mean,
                      double std, float *out, int threads) {
  job_t j = {K_NORMAL_F32, synth_key(seed, stream), start, n, mean, std, out};
  run(&j, threads);
}

/* bf16 bits of integers drawn uniformly from [lo, hi]. */
void synth_int_bf16(uint64_t seed, uint64_t stream, uint64_t start, uint64_t n, int lo, int hi,
                    uint16_t *out, int threads) {
  job_t j = {K_INT_BF16, synth_key(seed, stream), start, n, (double)lo, (double)hi, out};
  run(&j, threads);
}

/* binary32 integers drawn uniformly from [lo, hi]. */
void synth_int_f32(uint64_t seed, uint64_t stream, uint64_t start, uint64_t n, int lo, int hi,
                   float *out, int threads) {
  job_t j = {K_INT_F32, synth_key(seed, stream), start, n, (double)lo, (double)hi, out};
  run(&j, threads);
}

/* Uniform random bytes (two uniform 4-bit codes per byte). */
void synth_bytes(uint64_t seed, uint64_t stream, uint64_t start, uint64_t n, uint8_t *out, int threads) {
  job_t j = {K_BYTES, synth_key(seed, stream), start, n, 0, 0, out};
  run(&j, threads);
}

/* E4M3 bytes of fp32 uniforms in [lo, hi), rounded to nearest even. */
void synth_uniform_e4m3(uint64_t seed, uint64_t stream, uint64_t start, uint64_t n, double lo,
                        double hi, uint8_t *out, int threads) {
  job_t j = {K_UNIFORM_E4M3, synth_key(seed, stream), start, n, lo, hi, out};
  run(&j, threads);
}
