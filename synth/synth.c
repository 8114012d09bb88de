/*
 * Seeded synthetic input generators, shared by the oracle side and the GPU side.
 *
 * This file holds no step of the quantization method: it only draws the fp16
 * tensors that both sides consume.  Everything is counter based, so any thread
 * partition produces the same bits.
 *
 *   rand64(seed, c)  = splitmix64 output number c for initial state `seed`
 *                      (Steele, Lea and Flood, "Fast splittable pseudorandom
 *                      number generators", OOPSLA 2014; constants as published
 *                      with Vigna's reference splitmix64.c).
 *   normal(seed, i)  = Box-Muller in binary64 on rand64(seed, 2i), rand64(seed, 2i+1):
 *                      u1 = (r1 >> 11 + 1) * 2^-53 in (0, 1],
 *                      u2 = (r2 >> 11) * 2^-53 in [0, 1),
 *                      z  = sqrt(-2 ln u1) * cos(2 pi u2).
 *   fp16             = binary64 -> binary16, round to nearest even, overflow to inf.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_rand64(uint64_t seed, uint64_t c) {
  return mix64(seed + (c + 1) * 0x9E3779B97F4A7C15ULL);
}

static inline double normal_at(uint64_t seed, uint64_t i) {
  uint64_t r1 = synth_rand64(seed, 2 * i);
  uint64_t r2 = synth_rand64(seed, 2 * i + 1);
  double u1 = (double)((r1 >> 11) + 1) * 0x1.0p-53;
  double u2 = (double)(r2 >> 11) * 0x1.0p-53;
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

/* binary64 -> binary16 bits, round to nearest even (gradual underflow, inf on overflow). */
uint16_t synth_f64_to_f16(double v) {
  uint64_t b;
  memcpy(&b, &v, 8);
  uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  int e = (int)((b >> 52) & 0x7FF);
  uint64_t mant = b & 0xFFFFFFFFFFFFFULL;
  if (e == 0x7FF) return sign | (mant ? 0x7E00u : 0x7C00u);
  if (e == 0 && mant == 0) return sign;
  /* value = 1.mant * 2^(e-1023) (normal binary64); subnormal binary64 underflows to 0 */
  if (e == 0) return sign;
  int exp = e - 1023;
  uint64_t sig = mant | (1ULL << 52);          /* 53-bit significand */
  int shift;                                     /* bits of sig to drop */
  uint16_t out_exp;
  if (exp >= -14) {
    if (exp > 15) return sign | 0x7C00u;
    shift = 52 - 10;                             /* keep 11 bits */
    out_exp = (uint16_t)(exp + 15);
  } else {
    /* binary16 subnormal: value = m * 2^-24, m < 1024 */
    shift = 52 - 10 + (-14 - exp);
    out_exp = 0;
    if (shift > 63) return sign;
  }
  uint64_t kept = sig >> shift;
  uint64_t rem = sig & ((1ULL << shift) - 1);
  uint64_t half = 1ULL << (shift - 1);
  if (rem > half || (rem == half && (kept & 1))) kept += 1;
  uint32_t res;
  if (out_exp == 0) {
    res = (uint32_t)kept;                        /* may carry into the normal range: still correct */
  } else {
    if (kept == (1ULL << 11)) {                  /* mantissa carry */
      kept >>= 1;
      out_exp += 1;
      if (out_exp >= 31) return sign | 0x7C00u;
    }
    res = ((uint32_t)out_exp << 10) | (uint32_t)(kept & 0x3FF);
  }
  return sign | (uint16_t)res;
}

/* ---- bulk generation ---------------------------------------------------- */

typedef struct {
  uint64_t seed;
  double sigma;
  int64_t rows, cols;
  const uint8_t* col_outlier; /* NULL or [cols] flags */
  double outlier_scale;
  uint16_t* out;
  int64_t r0, r1;
} job_t;

static void* run_job(void* p) {
  job_t* j = (job_t*)p;
  for (int64_t r = j->r0; r < j->r1; ++r) {
    for (int64_t c = 0; c < j->cols; ++c) {
      uint64_t i = (uint64_t)(r * j->cols + c);
      double z = normal_at(j->seed, i) * j->sigma;
      if (j->col_outlier && j->col_outlier[c]) z *= j->outlier_scale;
      j->out[i] = synth_f64_to_f16(z);
    }
  }
  return NULL;
}

/* out[r][c] = fp16(sigma * normal(seed, r*cols + c) * (outlier_scale if col_outlier[c] else 1)).
   nthreads <= 1 runs on the calling thread. */
void synth_normal_f16(uint64_t seed, double sigma, int64_t rows, int64_t cols,
                      const uint8_t* col_outlier, double outlier_scale,
                      uint16_t* out, int nthreads) {
  if (rows <= 0 || cols <= 0) return;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  if (nthreads > rows) nthreads = (int)rows;
  job_t jobs[64];
  pthread_t th[64];
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = (job_t){seed, sigma, rows, cols, col_outlier, outlier_scale, out,
                      rows * t / nthreads, rows * (t + 1) / nthreads};
  }
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, run_job, &jobs[t]);
  run_job(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
}
