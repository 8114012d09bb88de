/*
 * flexq_oracle.c -- plain CPU oracle for the FlexQ W6A6 / W6A8 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg; never by the product path.  It shares no code,
 * header, table or helper with the GPU library.
 *
 * What each function follows is cited in flexq_oracle.h and at the function.
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math (no FMA contraction,
 * strict IEEE binary32 on SSE).
 */
#include "flexq_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* binary16 <-> binary32                                                      */
/* ------------------------------------------------------------------------- */

float oracle_f16_to_f32(uint16_t h) {
  uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  uint32_t e = (h >> 10) & 0x1F;
  uint32_t m = h & 0x3FF;
  uint32_t bits;
  if (e == 0x1F) {
    bits = sign | 0x7F800000u | (m << 13);
  } else if (e != 0) {
    bits = sign | ((e - 15 + 127) << 23) | (m << 13);
  } else if (m == 0) {
    bits = sign;
  } else {
    /* subnormal: value = m * 2^-24, renormalise */
    int shift = 0;
    while ((m & 0x400) == 0) {
      m <<= 1;
      ++shift;
    }
    m &= 0x3FF;
    bits = sign | ((uint32_t)(127 - 15 + 1 - shift) << 23) | (m << 13);
  }
  float f;
  memcpy(&f, &bits, 4);
  return f;
}

uint16_t oracle_f32_to_f16(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  uint16_t sign = (uint16_t)((b >> 16) & 0x8000u);
  int e = (int)((b >> 23) & 0xFF);
  uint32_t mant = b & 0x7FFFFF;
  if (e == 0xFF) return sign | (mant ? 0x7E00u : 0x7C00u);
  if (e == 0) return sign; /* binary32 subnormals are far below binary16's range */
  int exp = e - 127;
  uint32_t sig = mant | 0x800000u; /* 24-bit significand */
  int shift;
  int out_exp;
  if (exp >= -14) {
    if (exp > 15) return sign | 0x7C00u;
    shift = 13;
    out_exp = exp + 15;
  } else {
    shift = 13 + (-14 - exp);
    out_exp = 0;
    if (shift > 24) return sign;
  }
  uint32_t kept = sig >> shift;
  uint32_t rem = sig & ((1u << shift) - 1);
  uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (kept & 1))) kept += 1;
  if (out_exp == 0) return sign | (uint16_t)kept; /* carry into 0x400 is the right answer */
  if (kept == 0x800) {
    kept >>= 1;
    out_exp += 1;
    if (out_exp >= 31) return sign | 0x7C00u;
  }
  return sign | (uint16_t)((out_exp << 10) | (kept & 0x3FF));
}

/* ------------------------------------------------------------------------- */
/* Weight quantizer                                                           */
/* FlexQ abstract: uniform 6-bit weights in every layer.  Blog "Fine-Grained  */
/* Quantization ...": a group shares one scale.  Blog "Bridging ... BTC":     */
/* groups run along K.  Symmetric grid [-31, 31], max-abs scale, stored fp16, */
/* round half to even.                                                        */
/* ------------------------------------------------------------------------- */

int oracle_quant_w6(const uint16_t* w, int64_t N, int64_t K, int64_t group,
                    int8_t* qw, uint16_t* sw) {
  if (!w || !qw || !sw || N <= 0 || K <= 0 || group <= 0 || K % group) return -1;
  int64_t G = K / group;
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t g = 0; g < G; ++g) {
      const uint16_t* src = w + n * K + g * group;
      int8_t* dst = qw + n * K + g * group;
      float amax = 0.0f;
      for (int64_t i = 0; i < group; ++i) {
        float a = fabsf(oracle_f16_to_f32(src[i]));
        if (a > amax) amax = a;
      }
      uint16_t s16 = 0;
      float sf = 0.0f;
      if (amax != 0.0f) {
        float s = amax / 31.0f;
        s16 = oracle_f32_to_f16(s);
        sf = oracle_f16_to_f32(s16);
      }
      sw[n * G + g] = s16;
      for (int64_t i = 0; i < group; ++i) {
        int q = 0;
        if (sf != 0.0f) {
          float v = rintf(oracle_f16_to_f32(src[i]) / sf);
          q = (int)v;
          if (q > 31) q = 31;
          if (q < -31) q = -31;
        }
        dst[i] = (int8_t)q;
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------- */
/* Packed 6-bit layout (16 codes -> 3 dwords), the 4+2 split of ZeroQuant(4+2) */
/*   v = q & 63 (two's complement), lo = v & 15, hi = v >> 4.                  */
/*   dword0 byte j: lo[j]    | lo[4+j]  << 4                                   */
/*   dword1 byte j: lo[8+j]  | lo[12+j] << 4                                   */
/*   dword2 byte j: hi[j] | hi[4+j] << 2 | hi[8+j] << 4 | hi[12+j] << 6        */
/* ------------------------------------------------------------------------- */

void oracle_pack_unit(const int8_t q[16], uint32_t d[3]) {
  uint32_t lo[16], hi[16];
  for (int i = 0; i < 16; ++i) {
    uint32_t v = (uint32_t)q[i] & 63u;
    lo[i] = v & 15u;
    hi[i] = v >> 4;
  }
  d[0] = d[1] = d[2] = 0;
  for (int j = 0; j < 4; ++j) {
    uint32_t b0 = lo[j] | (lo[4 + j] << 4);
    uint32_t b1 = lo[8 + j] | (lo[12 + j] << 4);
    uint32_t b2 = hi[j] | (hi[4 + j] << 2) | (hi[8 + j] << 4) | (hi[12 + j] << 6);
    d[0] |= b0 << (8 * j);
    d[1] |= b1 << (8 * j);
    d[2] |= b2 << (8 * j);
  }
}

void oracle_unpack_unit(const uint32_t d[3], int8_t q[16]) {
  for (int j = 0; j < 4; ++j) {
    uint32_t b0 = (d[0] >> (8 * j)) & 0xFF;
    uint32_t b1 = (d[1] >> (8 * j)) & 0xFF;
    uint32_t b2 = (d[2] >> (8 * j)) & 0xFF;
    uint32_t lo[4] = {b0 & 15u, b0 >> 4, b1 & 15u, b1 >> 4};
    uint32_t hi[4] = {b2 & 3u, (b2 >> 2) & 3u, (b2 >> 4) & 3u, b2 >> 6};
    for (int p = 0; p < 4; ++p) {
      int v = (int)((hi[p] << 4) | lo[p]);
      q[4 * p + j] = (int8_t)(v >= 32 ? v - 64 : v);
    }
  }
}

/* Units of 16 consecutive rows n share a tile; inside the tile the unit index
   u = k/16 is major and the row n%16 minor. */
int64_t oracle_unit_offset(int64_t n, int64_t u, int64_t K) {
  int64_t units_per_row = K / 16;
  return 3 * (((n / 16) * units_per_row + u) * 16 + (n % 16));
}

int oracle_pack_codes(const int8_t* qw, int64_t N, int64_t K, uint32_t* wp) {
  if (!qw || !wp || N <= 0 || K <= 0 || N % 16 || K % 16) return -1;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t u = 0; u < K / 16; ++u)
      oracle_pack_unit(qw + n * K + u * 16, wp + oracle_unit_offset(n, u, K));
  return 0;
}

int oracle_unpack_codes(const uint32_t* wp, int64_t N, int64_t K, int8_t* qw) {
  if (!qw || !wp || N <= 0 || K <= 0 || N % 16 || K % 16) return -1;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t u = 0; u < K / 16; ++u)
      oracle_unpack_unit(wp + oracle_unit_offset(n, u, K), qw + n * K + u * 16);
  return 0;
}

int oracle_pack_w6(const uint16_t* w, int64_t N, int64_t K, int64_t group,
                   uint32_t* wp, uint16_t* sw) {
  if (!w || !wp || !sw || N <= 0 || K <= 0 || group <= 0 || K % group || N % 16 || K % 16)
    return -1;
  int8_t* qw = (int8_t*)malloc((size_t)(N * K));
  if (!qw) return -2;
  int rc = oracle_quant_w6(w, N, K, group, qw, sw);
  if (rc == 0) rc = oracle_pack_codes(qw, N, K, wp);
  free(qw);
  return rc;
}

/* ------------------------------------------------------------------------- */
/* Activation quantizer                                                       */
/* Blog "Fine-Grained Quantization ...": activations are group quantized too; */
/* 6-bit in most layers, 8-bit in sensitive ones.  Per token m, groups of     */
/* consecutive k, symmetric, max-abs scale kept in fp32, half to even.        */
/* ------------------------------------------------------------------------- */

int oracle_quant_act(const uint16_t* x, int64_t M, int64_t K, int64_t group, int abits,
                     int8_t* qa, float* sa) {
  if (!x || !qa || !sa || M <= 0 || K <= 0 || group <= 0 || K % group) return -1;
  if (abits != 6 && abits != 8) return -1;
  int qmax = abits == 6 ? 31 : 127;
  int64_t G = K / group;
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t g = 0; g < G; ++g) {
      const uint16_t* src = x + m * K + g * group;
      int8_t* dst = qa + m * K + g * group;
      float amax = 0.0f;
      for (int64_t i = 0; i < group; ++i) {
        float a = fabsf(oracle_f16_to_f32(src[i]));
        if (a > amax) amax = a;
      }
      float s = 0.0f;
      if (amax != 0.0f) s = amax / (float)qmax;
      sa[m * G + g] = s;
      for (int64_t i = 0; i < group; ++i) {
        int q = 0;
        if (s != 0.0f) {
          q = (int)rintf(oracle_f16_to_f32(src[i]) / s);
          if (q > qmax) q = qmax;
          if (q < -qmax) q = -qmax;
        }
        dst[i] = (int8_t)q;
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------- */
/* 6-bit activation storage                                                   */
/* FlexQ abstract: W6A6, so activations can be held at 6 bits.  The same      */
/* 16-code unit as the packed weights, laid out row by row: unit u of token   */
/* row m at dword 3 * (m * K/16 + u).                                         */
/* ------------------------------------------------------------------------- */

int oracle_pack_act_a6(const int8_t* qa, int64_t M, int64_t K, uint32_t* qp) {
  if (!qa || !qp || M <= 0 || K <= 0 || K % 16) return -1;
  for (int64_t i = 0; i < M * K; ++i)
    if (qa[i] < -32 || qa[i] > 31) return -3;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t u = 0; u < K / 16; ++u)
      oracle_pack_unit(qa + m * K + u * 16, qp + 3 * (m * (K / 16) + u));
  return 0;
}

int oracle_unpack_act_a6(const uint32_t* qp, int64_t M, int64_t K, int8_t* qa) {
  if (!qa || !qp || M <= 0 || K <= 0 || K % 16) return -1;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t u = 0; u < K / 16; ++u)
      oracle_unpack_unit(qp + 3 * (m * (K / 16) + u), qa + m * K + u * 16);
  return 0;
}

/* ------------------------------------------------------------------------- */
/* Activation codes in 16-row blocks: a layout only, no arithmetic.           */
/* ------------------------------------------------------------------------- */

static int64_t block_offset(int64_t m, int64_t k, int64_t K) {
  int64_t b = m / 16, r = m % 16, g = k / 128, h = (k % 128) / 64, c = k % 64;
  return b * 16 * K + g * 2048 + h * 1024 + r * 64 + c;
}

int oracle_block_act(const int8_t* qa, int64_t M, int64_t K, int8_t* out) {
  if (!qa || !out || M <= 0 || K <= 0 || K % 128) return -1;
  int64_t Mp = (M + 15) / 16 * 16;
  memset(out, 0, (size_t)(Mp * K));
  for (int64_t m = 0; m < M; ++m)
    for (int64_t k = 0; k < K; ++k) out[block_offset(m, k, K)] = qa[m * K + k];
  return 0;
}

int oracle_unblock_act(const int8_t* blk, int64_t M, int64_t K, int8_t* qa) {
  if (!qa || !blk || M <= 0 || K <= 0 || K % 128) return -1;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t k = 0; k < K; ++k) qa[m * K + k] = blk[block_offset(m, k, K)];
  return 0;
}

/* ------------------------------------------------------------------------- */
/* Integer group dots and the fused-dequantization accumulation               */
/* Blog "Bridging ... BTC": exact integer partial products per K-group, then  */
/* dequantization fused into the accumulation.                                */
/* ------------------------------------------------------------------------- */

typedef struct {
  const int8_t* qa;
  const float* sa;
  const int8_t* qw;
  const uint16_t* sw;
  int64_t M, N, K, group;
  int32_t* dots;
  uint16_t* y;
  float* acc_out;
  double* s_out;
  int64_t n0, n1;
} work_t;

static int32_t group_dot(const int8_t* a, const int8_t* b, int64_t len) {
  int32_t d = 0;
  for (int64_t i = 0; i < len; ++i) d += (int32_t)a[i] * (int32_t)b[i];
  return d;
}

static void* dots_worker(void* p) {
  work_t* w = (work_t*)p;
  int64_t G = w->K / w->group;
  for (int64_t n = w->n0; n < w->n1; ++n)
    for (int64_t m = 0; m < w->M; ++m)
      for (int64_t g = 0; g < G; ++g)
        w->dots[(m * w->N + n) * G + g] =
            group_dot(w->qa + m * w->K + g * w->group, w->qw + n * w->K + g * w->group,
                      w->group);
  return NULL;
}

static void* gemm_worker(void* p) {
  work_t* w = (work_t*)p;
  int64_t G = w->K / w->group;
  for (int64_t n = w->n0; n < w->n1; ++n) {
    for (int64_t m = 0; m < w->M; ++m) {
      float acc = 0.0f;
      double s_abs = 0.0;
      for (int64_t g = 0; g < G; ++g) {
        int32_t d = group_dot(w->qa + m * w->K + g * w->group,
                              w->qw + n * w->K + g * w->group, w->group);
        float t = (float)d * oracle_f16_to_f32(w->sw[n * G + g]);
        float s_a = w->sa[m * G + g];
        acc = fmaf(t, s_a, acc);
        s_abs += fabs((double)t * (double)s_a);
      }
      w->y[m * w->N + n] = oracle_f32_to_f16(acc);
      if (w->acc_out) w->acc_out[m * w->N + n] = acc;
      if (w->s_out) w->s_out[m * w->N + n] = s_abs;
    }
  }
  return NULL;
}

static void run_over_n(work_t base, int nthreads, void* (*fn)(void*)) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads > base.N) nthreads = (int)base.N;
  work_t jobs[256];
  pthread_t th[256];
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = base;
    jobs[t].n0 = base.N * t / nthreads;
    jobs[t].n1 = base.N * (t + 1) / nthreads;
  }
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, fn, &jobs[t]);
  fn(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
}

int oracle_group_dots(const int8_t* qa, const int8_t* qw, int64_t M, int64_t N, int64_t K,
                      int64_t group, int32_t* dots, int nthreads) {
  if (!qa || !qw || !dots || M <= 0 || N <= 0 || K <= 0 || group <= 0 || K % group) return -1;
  work_t base = {qa, NULL, qw, NULL, M, N, K, group, dots, NULL, NULL, NULL, 0, N};
  run_over_n(base, nthreads, dots_worker);
  return 0;
}

int oracle_gemm(const int8_t* qa, const float* sa, const int8_t* qw, const uint16_t* sw,
                int64_t M, int64_t N, int64_t K, int64_t group,
                uint16_t* y, float* acc_out, double* s_out, int nthreads) {
  if (!qa || !sa || !qw || !sw || !y || M <= 0 || N <= 0 || K <= 0 || group <= 0 || K % group)
    return -1;
  work_t base = {qa, sa, qw, sw, M, N, K, group, NULL, y, acc_out, s_out, 0, N};
  run_over_n(base, nthreads, gemm_worker);
  return 0;
}

int oracle_gemm_packed(const int8_t* qa, const float* sa, const uint32_t* wp,
                       const uint16_t* sw, int64_t M, int64_t N, int64_t K, int64_t group,
                       uint16_t* y, float* acc_out, double* s_out, int nthreads) {
  if (!wp || N <= 0 || K <= 0 || N % 16 || K % 16) return -1;
  int8_t* qw = (int8_t*)malloc((size_t)(N * K));
  if (!qw) return -2;
  int rc = oracle_unpack_codes(wp, N, K, qw);
  if (rc == 0) rc = oracle_gemm(qa, sa, qw, sw, M, N, K, group, y, acc_out, s_out, nthreads);
  free(qw);
  return rc;
}
