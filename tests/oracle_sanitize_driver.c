/* Drives every function of the CPU oracle (oracle/flexq_oracle.c) on small seeded
 * inputs so that a build with -fsanitize=address,undefined sees every code path run:
 * the quantizers on ordinary, all-zero, extreme and subnormal groups, pack / unpack
 * of every code, the tiled packing of a matrix, the 6-bit activation storage, group dots and the GEMM on one and
 * several threads (with and without the optional accumulator outputs), and the
 * argument checks.  It also checks a few facts the oracle must keep (round trips,
 * thread-count independence) and exits non-zero on any mismatch; the sanitizers
 * abort the run on any memory or undefined-behaviour error. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../oracle/flexq_oracle.h"

static uint64_t state = 0x1234567887654321ull;
static uint64_t next64(void) { /* xorshift64*, only to fill buffers */
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return state * 0x2545F4914F6CDD1Dull;
}
static float uniform(void) { return (float)((next64() >> 11) * (1.0 / 9007199254740992.0)); }

#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      return 1;                                                    \
    }                                                              \
  } while (0)

static void fill_f16(uint16_t* p, int64_t n, float scale) {
  for (int64_t i = 0; i < n; ++i) p[i] = oracle_f32_to_f16((uniform() * 2.0f - 1.0f) * scale);
}

int main(void) {
  const int64_t M = 5, N = 48, K = 384, G = 128, NG = K / G;
  uint16_t* x = malloc(sizeof(uint16_t) * M * K);
  uint16_t* w = malloc(sizeof(uint16_t) * N * K);
  int8_t* qa = malloc(M * K);
  float* sa = malloc(sizeof(float) * M * NG);
  int8_t* qw = malloc(N * K);
  int8_t* qw2 = malloc(N * K);
  uint16_t* sw = malloc(sizeof(uint16_t) * N * NG);
  uint16_t* sw2 = malloc(sizeof(uint16_t) * N * NG);
  uint32_t* wp = malloc(sizeof(uint32_t) * 3 * N * K / 16);
  uint32_t* wp2 = malloc(sizeof(uint32_t) * 3 * N * K / 16);
  int32_t* dots = malloc(sizeof(int32_t) * M * N * NG);
  uint16_t* y1 = malloc(sizeof(uint16_t) * M * N);
  uint16_t* y7 = malloc(sizeof(uint16_t) * M * N);
  uint16_t* yp = malloc(sizeof(uint16_t) * M * N);
  float* acc = malloc(sizeof(float) * M * N);
  double* s = malloc(sizeof(double) * M * N);
  if (!x || !w || !qa || !sa || !qw || !qw2 || !sw || !sw2 || !wp || !wp2 || !dots || !y1 ||
      !y7 || !yp || !acc || !s)
    return 2;

  fill_f16(x, M * K, 20.0f);
  fill_f16(w, N * K, 0.05f);
  /* special groups: all zero, fp16 extremes, subnormals */
  for (int64_t i = 0; i < G; ++i) {
    x[i] = 0;                              /* row 0, group 0: all zero   */
    w[i] = 0;                              /* row 0, group 0: all zero   */
    w[K + i] = (i & 1) ? 0x7BFF : 0xFBFF;  /* row 1, group 0: +-65504    */
    w[2 * K + i] = (uint16_t)(i % 4);      /* row 2, group 0: subnormals */
    x[K + i] = (i & 1) ? 0x0001 : 0x8001;  /* row 1, group 0: subnormals */
  }

  /* fp16 conversions over every pattern */
  for (uint32_t h = 0; h < 65536; ++h) {
    float f = oracle_f16_to_f32((uint16_t)h);
    if (!isnan(f)) CHECK(oracle_f32_to_f16(f) == (uint16_t)h);
  }

  /* packing of single units: every code at every position */
  for (int pos = 0; pos < 16; ++pos)
    for (int code = -32; code < 32; ++code) {
      int8_t q[16], r[16];
      uint32_t d[3];
      for (int i = 0; i < 16; ++i) q[i] = (int8_t)((int)(next64() % 64) - 32);
      q[pos] = (int8_t)code;
      oracle_pack_unit(q, d);
      oracle_unpack_unit(d, r);
      CHECK(memcmp(q, r, 16) == 0);
    }

  /* weights: quantize, pack, unpack, and the one-call form */
  CHECK(oracle_quant_w6(w, N, K, G, qw, sw) == 0);
  CHECK(oracle_pack_codes(qw, N, K, wp) == 0);
  CHECK(oracle_unpack_codes(wp, N, K, qw2) == 0);
  CHECK(memcmp(qw, qw2, N * K) == 0);
  CHECK(oracle_pack_w6(w, N, K, G, wp2, sw2) == 0);
  CHECK(memcmp(wp, wp2, sizeof(uint32_t) * 3 * N * K / 16) == 0);
  CHECK(memcmp(sw, sw2, sizeof(uint16_t) * N * NG) == 0);
  for (int64_t n = 0; n < N; ++n)
    for (int64_t u = 0; u < K / 16; ++u) {
      const int64_t off = oracle_unit_offset(n, u, K);
      CHECK(off >= 0 && off + 3 <= 3 * N * K / 16);
    }

  /* activations, both precisions, then dots and the GEMM on 1 and 7 threads */
  for (int abits = 6; abits <= 8; abits += 2) {
    CHECK(oracle_quant_act(x, M, K, G, abits, qa, sa) == 0);
    CHECK(oracle_group_dots(qa, qw, M, N, K, G, dots, 3) == 0);
    CHECK(oracle_gemm(qa, sa, qw, sw, M, N, K, G, y1, NULL, NULL, 1) == 0);
    CHECK(oracle_gemm(qa, sa, qw, sw, M, N, K, G, y7, acc, s, 7) == 0);
    CHECK(memcmp(y1, y7, sizeof(uint16_t) * M * N) == 0);
    CHECK(oracle_gemm_packed(qa, sa, wp, sw, M, N, K, G, yp, NULL, NULL, 300) == 0);
    CHECK(memcmp(y1, yp, sizeof(uint16_t) * M * N) == 0);
    for (int64_t i = 0; i < M * N; ++i) CHECK(s[i] >= 0.0);
    { /* codes in 16-row blocks: round trip, pad rows zero */
      const int64_t Mp = (M + 15) / 16 * 16;
      int8_t* blk = malloc(Mp * K);
      int8_t* back = malloc(M * K);
      CHECK(blk && back);
      CHECK(oracle_block_act(qa, M, K, blk) == 0);
      CHECK(oracle_unblock_act(blk, M, K, back) == 0);
      CHECK(memcmp(qa, back, M * K) == 0);
      int64_t nz = 0;
      for (int64_t i = 0; i < Mp * K; ++i) nz += blk[i] != 0;
      int64_t nzq = 0;
      for (int64_t i = 0; i < M * K; ++i) nzq += qa[i] != 0;
      CHECK(nz == nzq);
      free(blk);
      free(back);
    }
    if (abits == 6) { /* 6-bit activation storage: pack, unpack, round trip */
      uint32_t* qp = malloc(sizeof(uint32_t) * 3 * M * K / 16);
      int8_t* qa2 = malloc(M * K);
      CHECK(qp && qa2);
      CHECK(oracle_pack_act_a6(qa, M, K, qp) == 0);
      CHECK(oracle_unpack_act_a6(qp, M, K, qa2) == 0);
      CHECK(memcmp(qa, qa2, M * K) == 0);
      free(qp);
      free(qa2);
    } else { /* A8 codes beyond 6 bits are refused */
      uint32_t qp1[3 * K / 16];
      int8_t row[K];
      memset(row, 0, sizeof row);
      row[5] = 127;
      CHECK(oracle_pack_act_a6(row, 1, K, qp1) < 0);
    }
  }

  /* argument checks return errors instead of touching memory */
  CHECK(oracle_quant_w6(NULL, N, K, G, qw, sw) < 0);
  CHECK(oracle_quant_w6(w, N, K + 1, G, qw, sw) < 0);
  CHECK(oracle_quant_act(x, M, K, G, 7, qa, sa) < 0);
  CHECK(oracle_pack_codes(qw, N + 1, K, wp) < 0);
  CHECK(oracle_pack_act_a6(qa, M, K + 1, wp) < 0);
  CHECK(oracle_unpack_act_a6(NULL, M, K, qa) < 0);
  CHECK(oracle_block_act(qa, M, K + 16, (int8_t*)wp) < 0);
  CHECK(oracle_gemm(qa, sa, qw, sw, 0, N, K, G, y1, NULL, NULL, 1) < 0);
  CHECK(oracle_group_dots(qa, qw, M, N, K, 0, dots, 1) < 0);

  free(x); free(w); free(qa); free(sa); free(qw); free(qw2); free(sw); free(sw2);
  free(wp); free(wp2); free(dots); free(y1); free(y7); free(yp); free(acc); free(s);
  puts("oracle sanitizer run: clean");
  return 0;
}
