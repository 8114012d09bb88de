/*
 * flexq_oracle.h -- plain, slow CPU oracle for the W6A6 / W6A8 group-quantized
 * linear layer (FlexQ, arXiv 2508.04405).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code with the GPU library.
 *
 * Sources (the FlexQ pages):
 *   - FlexQ abstract (arXiv): uniform 6-bit weights in every layer, 6- or 8-bit
 *     activations per layer, a W6A6 / W6A8 matrix multiply.
 *   - "Fine-Grained Quantization and Layer Sensitivity" (drgamma blog on FlexQ):
 *     weights and activations are split into small groups that share one scale;
 *     most layers keep 6-bit activations, a few sensitive ones 8-bit.
 *   - "Bridging Software and Hardware with BTC" (same blog): groups run along K,
 *     128 deep; the kernel computes exact integer partial products per group
 *     and fuses the dequantization into the GEMM.
 *   - ZeroQuant(4+2) abstract: the 4+2 split of a 6-bit code, which the packed
 *     layout below follows (a 4-bit plane plus a 2-bit plane).
 *
 * All floating point is IEEE binary32, round to nearest even, no contraction
 * (the only fused multiply-add is the explicit fmaf in the accumulation).
 * Every function returns 0 on success and a negative value on bad arguments.
 */
#ifndef FLEXQ_ORACLE_H
#define FLEXQ_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* exact binary16 -> binary32 widening */
float oracle_f16_to_f32(uint16_t h);
/* binary32 -> binary16, round to nearest even, overflow to inf */
uint16_t oracle_f32_to_f16(float f);

/* Weight quantizer, one scale per (row n, group of `group` consecutive k).
   w [N][K] fp16 bits -> qw [N][K] int8 in [-31, 31], sw [N][K/group] fp16 bits. */
int oracle_quant_w6(const uint16_t* w, int64_t N, int64_t K, int64_t group,
                    int8_t* qw, uint16_t* sw);

/* One 16-code unit -> 3 dwords (4-bit plane in d0/d1, 2-bit plane in d2). */
void oracle_pack_unit(const int8_t q[16], uint32_t d[3]);
/* 3 dwords -> 16 codes in [-32, 31]. */
void oracle_unpack_unit(const uint32_t d[3], int8_t q[16]);
/* First dword of unit (n, u = k/16) inside the packed buffer, N16-tiled. */
int64_t oracle_unit_offset(int64_t n, int64_t u, int64_t K);

/* Pack quantized codes qw [N][K] into wp (0.75*N*K bytes). N % 16 == 0, K % 16 == 0. */
int oracle_pack_codes(const int8_t* qw, int64_t N, int64_t K, uint32_t* wp);
/* Decode wp back into codes [N][K]. */
int oracle_unpack_codes(const uint32_t* wp, int64_t N, int64_t K, int8_t* qw);
/* quant_w6 followed by pack_codes. */
int oracle_pack_w6(const uint16_t* w, int64_t N, int64_t K, int64_t group,
                   uint32_t* wp, uint16_t* sw);

/* Activation quantizer, one fp32 scale per (token m, group). abits 6 -> [-31,31],
   abits 8 -> [-127,127].  x [M][K] fp16 bits -> qa [M][K], sa [M][K/group]. */
int oracle_quant_act(const uint16_t* x, int64_t M, int64_t K, int64_t group, int abits,
                     int8_t* qa, float* sa);

/* 6-bit activation storage (FlexQ abstract: W6A6, activations held at 6 bits): the
   codes qa [M][K] (each in [-32, 31], else -3) packed 16 per unit as above, the
   units of a token row one after another: unit u = k/16 of row m at dword
   3 * (m * K/16 + u), 0.75 * K bytes per row.  K % 16 == 0. */
int oracle_pack_act_a6(const int8_t* qa, int64_t M, int64_t K, uint32_t* qp);
/* Decode qp back into codes [M][K]. */
int oracle_unpack_act_a6(const uint32_t* qp, int64_t M, int64_t K, int8_t* qa);

/* Activation codes in 16-row blocks (the order the weight-streaming kernel feeds its
   MFMAs): rows padded with zero codes to a multiple of 16; block b = m / 16, group g,
   64-deep half h of the group, row r = m % 16 and byte c of the half at
   b*16*K + g*2048 + h*1024 + r*64 + c.  K % 128 == 0.  out: ceil(M/16)*16*K bytes. */
int oracle_block_act(const int8_t* qa, int64_t M, int64_t K, int8_t* out);
/* The inverse on the first M rows. */
int oracle_unblock_act(const int8_t* blk, int64_t M, int64_t K, int8_t* qa);

/* Integer group dot products d[m][n][g] = sum over k in group g of qa[m][k]*qw[n][k]. */
int oracle_group_dots(const int8_t* qa, const int8_t* qw, int64_t M, int64_t N, int64_t K,
                      int64_t group, int32_t* dots, int nthreads);

/* Y[m][n] = fp16( acc ),  acc = +0; for g ascending:
       t   = RN32( float(d[m][n][g]) * float(sw[n][g]) )
       acc = fmaf( t, sa[m][g], acc ).
   acc_out (optional) receives the fp32 acc, s_out (optional) sum_g |t*sa| in binary64. */
int oracle_gemm(const int8_t* qa, const float* sa, const int8_t* qw, const uint16_t* sw,
                int64_t M, int64_t N, int64_t K, int64_t group,
                uint16_t* y, float* acc_out, double* s_out, int nthreads);

/* Same as oracle_gemm but takes the packed weights and decodes them first. */
int oracle_gemm_packed(const int8_t* qa, const float* sa, const uint32_t* wp,
                       const uint16_t* sw, int64_t M, int64_t N, int64_t K, int64_t group,
                       uint16_t* y, float* acc_out, double* s_out, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
