/*
 * flexq_peaks.h -- on-device measurements of what this GPU reaches, next to which
 * the W6Ax kernels' figures are reported (the FlexQ pages compare their kernel only
 * against other systems, "What the Numbers Tell Us" in the blog "Meet FlexQ: A
 * Six-Bit Quantization Breakthrough"; these put the kernels against the hardware).
 *
 * Each measurement enqueues one kernel on `stream` (a hipStream_t as void*, NULL = the null
 * stream) and return 0, or -1 for a bad argument (nothing enqueued), or -2 when the
 * runtime rejected the launch.  The caller times them (HIP events) and owns every
 * buffer.
 */
#ifndef FLEXQ_PEAKS_H
#define FLEXQ_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes the sink of every measurement must hold on the current device. */
size_t flexq_peak_sink_bytes(void);

/* Plain streaming read: every 16-byte word of buf[0 .. bytes) is loaded once
   (non-temporal, as the decode kernel loads packed weights) by a grid of eight
   256-thread workgroups per compute unit, and folded into sink so nothing is
   skipped.  buf: device memory, 16-byte aligned, bytes a positive multiple of 16.
   sink: device memory of flexq_peak_sink_bytes() bytes (overwritten). */
int flexq_peak_hbm_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Back-to-back v_mfma_i32_32x32x32_i8 (the prefill kernel's instruction): two
   256-thread workgroups per compute unit (two waves per SIMD), each wave running
   `iters` rounds of 4 MFMAs on 4 independent accumulators, with `valu_per_mfma`
   (0, 4, 8 or 12) independent fp32 FMAs issued after every MFMA -- 8 is the
   fused rescale's count per MFMA (two per output and group).  Ops per call =
   2 * 32768 * 4 * iters * (waves in the grid).  clock[0] receives the shader
   cycles and clock[1] the 100 MHz reference ticks that wave 0 of workgroup 0
   spent in its loop (shader clock = clock[0] / clock[1] * 100 MHz).
   iters in [1, 2^24]; sink as above; clock: device memory of 2 uint64. */
int flexq_peak_mfma_i8(int64_t iters, int32_t valu_per_mfma, uint32_t* sink, uint64_t* clock,
                       void* stream);

/* Workgroups in the grid of flexq_peak_mfma_i8 on the current device (4 waves each). */
int64_t flexq_peak_mfma_i8_workgroups(void);

/* The instruction mix the exact group rescale sets a floor on (blog, "Bridging
   Software and Hardware with BTC": the dequantization is fused into the GEMM, two
   fp32 FMAs per output and group here), without global memory: one 512-thread
   workgroup per compute unit (two waves per SIMD); per wave and round (one 128-deep
   group) four 32 x 32 int8 tiles, each a chain of four v_mfma_i32_32x32x32_i8, the
   previous tile's results rescaled under each chain (4 fma + 4 DPP-broadcast fmac
   per MFMA, as in the prefill kernel), one 16-byte LDS read per MFMA, and one
   workgroup barrier per round.  Ops per call = 2 * 32768 * 16 * iters * waves, with
   waves = flexq_peak_mfma_i8_rescale_waves().  clock as for flexq_peak_mfma_i8;
   iters in [1, 2^24]; sink of flexq_peak_sink_bytes() bytes (overwritten). */
int flexq_peak_mfma_i8_rescale(int64_t iters, uint32_t* sink, uint64_t* clock, void* stream);

/* Waves in the grid of flexq_peak_mfma_i8_rescale on the current device. */
int64_t flexq_peak_mfma_i8_rescale_waves(void);

#ifdef __cplusplus
}
#endif
#endif /* FLEXQ_PEAKS_H */
