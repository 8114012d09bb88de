/*
 * flexq.h -- C ABI of the MI355X (gfx950) W6A6 / W6A8 group-quantized linear layer.
 *
 * The method is FlexQ (arXiv 2508.04405, "FlexQ: Efficient Post-training INT6
 * Quantization for LLM Serving via Algorithm-System Co-Design"):
 *   - abstract: uniform 6-bit weights in every layer; activations kept at 6 bits
 *     in most layers and at 8 bits in sensitive ones; a kernel for the W6A6 and
 *     W6A8 matrix multiply;
 *   - blog "Meet FlexQ: A Six-Bit Quantization Breakthrough", section
 *     "Fine-Grained Quantization and Layer Sensitivity": weights and activations
 *     are split into small groups that share one scale factor;
 *   - same blog, section "Bridging Software and Hardware with BTC": the groups run
 *     along K (128 deep), every group yields an exact integer partial product, and
 *     the dequantization is fused into the GEMM.
 *
 * All tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA tensors) and
 * are owned by the caller; the library allocates no memory the caller sees.
 * `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every call
 * validates its arguments on the host first; on error it returns without touching
 * the GPU.  On success the work is enqueued and the call returns; a fault during
 * execution surfaces at the caller's next synchronisation, as in HIP.
 *
 * Layouts (row-major, contiguous):
 *   W   fp16 [N][K]         nn.Linear weight ([out][in]); Y = X * W^T
 *   X   fp16 [M][K]         activations, one row per token
 *   q_a int8 [M][K]         quantized activations (one code per byte)
 *   s_a fp32 [K/128][M]     activation scales, group-major: s_a[g][m] at g*M + m
 *   s_w fp16 [K/128][N]     weight scales, group-major: s_w[g][n] at g*N + n
 *                           (group-major so one group's scales are contiguous)
 *   w_packed                6-bit weight codes, 16 codes per 3 dwords:
 *       v = q & 63, lo = v & 15, hi = v >> 4 (q in [-31, 31]; -32 decodes but is
 *       never produced), for byte j = 0..3 of each dword:
 *         dword0.byte[j] = lo[j]   | lo[4+j]  << 4
 *         dword1.byte[j] = lo[8+j] | lo[12+j] << 4
 *         dword2.byte[j] = hi[j] | hi[4+j] << 2 | hi[8+j] << 4 | hi[12+j] << 6
 *       (a 4-bit plane plus a 2-bit plane, the 4+2 split of ZeroQuant(4+2)).
 *       The unit of rows n, codes k = 16u .. 16u+15 starts at dword
 *         3 * (((n / 16) * (K / 16) + u) * 16 + n % 16),
 *       i.e. 16-row tiles, unit index major, row-in-tile minor.
 *   q_a6p                   A6 codes packed (flexq_quant_act_a6_packed): the w_packed
 *       unit encoding above, 16 codes per 3 dwords; the unit of row m, codes
 *       k = 16u .. 16u+15 starts at dword 3 * (m * (K / 16) + u), i.e. the units of
 *       a token row one after another, 0.75 * K bytes per row.
 *   q_a_blk                 activation codes in 16-row blocks (flexq_quant_act_blocked),
 *       the order the weight-streaming kernel feeds its MFMAs: rows padded with zero
 *       codes to a multiple of 16; the code of row m, column k at byte
 *         (m / 16) * 16 * K + (k / 128) * 2048 + ((k % 128) / 64) * 1024
 *           + (m % 16) * 64 + k % 64,
 *       i.e. per 16-row block and group, each 64-deep half as the 16 rows' 64-byte
 *       segments in turn; ceil(M / 16) * 16 * K bytes.
 *   Y   fp16 [M][N]
 *
 * Quantizers (symmetric, round half to even, IEEE binary32 division):
 *   weights, per (n, group g):    amax = max |w|;  s16 = fp16(amax / 31)  (0 if amax = 0);
 *                                 q = clamp(rint(w / float(s16)), -31, 31)  (0 if s16 = 0)
 *   activations, per (m, g):      amax = max |x|;  s = amax / qmax in fp32 (0 if amax = 0);
 *                                 q = clamp(rint(x / s), -qmax, qmax), qmax = 31 (A6) or 127 (A8)
 * Product:
 *   d[m][n][g] = sum_{k in g} q_a[m][k] * q_w[n][k]           (exact int32)
 *   acc = +0;  for g ascending:  t = RN32(float(d) * float(s_w[n][g]));
 *                                acc = fma(t, s_a[m][g], acc)
 *   Y[m][n] = fp16(acc).
 *
 * Preconditions: finite inputs; outputs must not overlap inputs; group_size == 128;
 * K a positive multiple of 128; N a multiple of 16; pointers aligned as stated.
 * The functions may be called from any thread.  Their only global state is a
 * per-device cache of the compute-unit count, filled on first use (atomically), and
 * the staging array of flexq_linear_w6ax_noalloc (one per GPU, with its address
 * cached per device the same way).
 */
#ifndef FLEXQ_H
#define FLEXQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FLEXQ_SUCCESS = 0,
  FLEXQ_ERROR_INVALID_VALUE = 1, /* null pointer, negative size, abits not 6/8, overlap */
  FLEXQ_ERROR_UNSUPPORTED = 2,   /* group_size != 128, K % 128 != 0, N % 16 != 0, misalignment */
  FLEXQ_ERROR_LAUNCH = 3         /* hipLaunchKernel rejected one of the call's launches (its
                                    own status, never an earlier call's sticky error);
                                    kernels the call enqueued before it may still run */
} flexq_status;

typedef enum {
  FLEXQ_PATH_AUTO = 0,    /* see flexq_gemm_w6ax_auto_path */
  FLEXQ_PATH_DECODE = 1,  /* HBM-streaming kernel for few tokens (any M is accepted) */
  FLEXQ_PATH_PREFILL = 2, /* MFMA-bound tiled kernel for many tokens (any M is accepted),
                             tile chosen as flexq_gemm_w6ax_prefill_tile reports, with
                             the tail split flexq_gemm_w6ax_prefill_main_cols reports */
  /* the prefill kernel with a fixed workgroup tile (rows x columns), for tests and
     tuning; every tile accepts every shape and gives the same bits */
  FLEXQ_PATH_PREFILL_256X128 = 3,
  FLEXQ_PATH_PREFILL_128X128 = 4,
  FLEXQ_PATH_PREFILL_128X64 = 5,
  /* 256 x 128 tiles computed by 4 MFMA waves while 4 loader waves stage the operands */
  FLEXQ_PATH_PREFILL_256X128_WS = 6,
  /* the prefill kernel with 64 x 128 tiles (two waves, two workgroups per compute
     unit), for few tokens on wide layers */
  FLEXQ_PATH_PREFILL_64X128 = 7
} flexq_path;

#define FLEXQ_ABI_VERSION 1
#define FLEXQ_PACK_FORMAT_VERSION 1
#define FLEXQ_GROUP_SIZE 128
#define FLEXQ_DECODE_MAX_M 64

/* FLEXQ_ABI_VERSION of the loaded library. */
int flexq_abi_version(void);

/* Static text for a status code; never NULL. */
const char* flexq_status_string(flexq_status status);

/* Bytes of w_packed for an N x K weight: 0.75 * N * K (12 bytes per 16 codes).
   Returns 0 for N <= 0, K <= 0 or K not a multiple of 16. */
size_t flexq_packed_w6_bytes(int64_t N, int64_t K);

/* Weight group quantization and packing (offline; FlexQ abstract: uniform 6-bit
   weights; blog, "Fine-Grained Quantization ...": one scale per group).
     w_fp16   [N][K] fp16 bits, 16-byte aligned          (input)
     w_packed flexq_packed_w6_bytes(N, K) bytes, 16-byte aligned (output)
     s_w_fp16 [K/128][N] fp16 bits, 2-byte aligned        (output)
   N == 0 is a no-op.  Errors: INVALID_VALUE (null, N < 0, K <= 0, overlap),
   UNSUPPORTED (group_size != 128, K % 128, N % 16, alignment). */
flexq_status flexq_pack_w6(const uint16_t* w_fp16, int64_t N, int64_t K, int32_t group_size,
                           uint32_t* w_packed, uint16_t* s_w_fp16, void* stream);

/* Per-token, per-group symmetric activation quantization to INT6 (abits = 6) or
   INT8 (abits = 8) (blog, "Fine-Grained Quantization ...": 6-bit activations in most
   layers, 8-bit in sensitive ones).
     x_fp16 [M][K] fp16 bits, 16-byte aligned (input)
     q_a    [M][K] int8, 8-byte aligned       (output)
     s_a    [K/128][M] fp32, 4-byte aligned   (output; M is its row stride)
   M == 0 is a no-op.  Errors as for flexq_pack_w6, plus INVALID_VALUE for abits. */
flexq_status flexq_quant_act(const uint16_t* x_fp16, int64_t M, int64_t K, int32_t group_size,
                             int32_t abits, int8_t* q_a, float* s_a, void* stream);

/* Bytes of q_a6p for an M x K activation: 0.75 * M * K (12 bytes per 16 codes).
   Returns 0 for M <= 0, K <= 0 or K not a multiple of 16. */
size_t flexq_packed_a6_bytes(int64_t M, int64_t K);

/* flexq_quant_act with abits = 6, the codes stored at 6 bits (FlexQ abstract: W6A6
   holds activations at 6 bits; layout q_a6p in the preamble): the same codes and
   the same s_a bits as flexq_quant_act(..., abits = 6, ...), at 0.75 bytes per code.
     x_fp16 [M][K] fp16 bits, 16-byte aligned                      (input)
     q_a6p  flexq_packed_a6_bytes(M, K) bytes, 16-byte aligned      (output)
     s_a    [K/128][M] fp32, 4-byte aligned                          (output)
   M == 0 is a no-op.  Errors as for flexq_quant_act (without abits). */
flexq_status flexq_quant_act_a6_packed(const uint16_t* x_fp16, int64_t M, int64_t K,
                                       int32_t group_size, uint32_t* q_a6p, float* s_a,
                                       void* stream);

/* The W6A6 GEMM over packed A6 activations (q_a6p from flexq_quant_act_a6_packed):
   the weight-streaming kernel of FLEXQ_PATH_DECODE, which unpacks each activation
   unit as it unpacks the weights.  Y is bit-identical to flexq_gemm_w6ax on the
   unpacked codes (abits = 6).  Any M is accepted; it is meant for few tokens
   (M <= FLEXQ_DECODE_MAX_M), since above that the weights are streamed once per 64
   rows.
     q_a6p  packed codes, 16-byte aligned     s_a, w_packed, s_w_fp16, y_fp16 as for
                                              flexq_gemm_w6ax
   M == 0 or N == 0 is a no-op.  Errors as for flexq_gemm_w6ax (without abits). */
flexq_status flexq_gemm_w6a6_packed(const uint32_t* q_a6p, const float* s_a,
                                    const uint32_t* w_packed, const uint16_t* s_w_fp16,
                                    int64_t M, int64_t N, int64_t K, int32_t group_size,
                                    uint16_t* y_fp16, void* stream);

/* Bytes of q_a_blk for an M x K activation: ceil(M / 16) * 16 * K.  Returns 0 for
   M <= 0, K <= 0 or K not a multiple of 128. */
size_t flexq_blocked_act_bytes(int64_t M, int64_t K);

/* flexq_quant_act writing the codes in 16-row blocks (layout q_a_blk in the preamble)
   for the weight-streaming GEMM: the same codes, the rows past M as zero codes, and
   the same s_a bits as flexq_quant_act.
     x_fp16  [M][K] fp16 bits, 16-byte aligned                       (input)
     q_a_blk flexq_blocked_act_bytes(M, K) bytes, 16-byte aligned     (output)
     s_a     [K/128][M] fp32, 4-byte aligned                           (output)
   M == 0 is a no-op.  Errors as for flexq_quant_act. */
flexq_status flexq_quant_act_blocked(const uint16_t* x_fp16, int64_t M, int64_t K,
                                     int32_t group_size, int32_t abits, int8_t* q_a_blk,
                                     float* s_a, void* stream);

/* The GEMM over blocked activation codes: the weight-streaming kernel of
   FLEXQ_PATH_DECODE with each MFMA fragment loaded as one contiguous kilobyte (whole
   cache lines) instead of sixteen 64-byte row segments: on LLaMA-2-70B layers as fast
   as the row-major codes at 1 to 4 tokens and 1-24 % faster from 8 to 64.  Y is
   bit-identical to flexq_gemm_w6ax on the row-major codes.  Any M is accepted; it
   is meant for few tokens (M <= FLEXQ_DECODE_MAX_M), since above that the weights
   are streamed once per 64 rows.
     q_a_blk  flexq_blocked_act_bytes(M, K) bytes, 16-byte aligned (its pad rows may
              hold anything: they only meet outputs that are never written)
     s_a, w_packed, s_w_fp16, y_fp16 as for flexq_gemm_w6ax
   M == 0 or N == 0 is a no-op.  Errors as for flexq_gemm_w6ax. */
flexq_status flexq_gemm_w6ax_blocked(const int8_t* q_a_blk, const float* s_a,
                                     const uint32_t* w_packed, const uint16_t* s_w_fp16,
                                     int64_t M, int64_t N, int64_t K, int32_t group_size,
                                     int32_t abits, uint16_t* y_fp16, void* stream);

/* Y = sum over groups of int32 group dot x s_w x s_a, fp32 accumulation, fp16 out
   (blog, "Bridging Software and Hardware with BTC": exact integer group products,
   dequantization fused into the GEMM).  The result is bit-identical to the formula
   in this header's preamble on every path.
     q_a      [M][K] int8, 16-byte aligned     s_a [K/128][M] fp32, 4-byte aligned
     w_packed packed codes, 16-byte aligned   s_w [K/128][N] fp16, 2-byte aligned
     y_fp16   [M][N] fp16, 4-byte aligned (output)
   abits (6 or 8) is validated; both are stored as int8 so the product is the same.
   M == 0 or N == 0 is a no-op. */
flexq_status flexq_gemm_w6ax(const int8_t* q_a, const float* s_a, const uint32_t* w_packed,
                             const uint16_t* s_w_fp16, int64_t M, int64_t N, int64_t K,
                             int32_t group_size, int32_t abits, uint16_t* y_fp16, void* stream);

/* The kernel FLEXQ_PATH_AUTO runs for an M x N x K product: FLEXQ_PATH_DECODE (the
   weight-streaming kernel) for M <= FLEXQ_DECODE_MAX_M, FLEXQ_PATH_PREFILL above,
   and also for 48 <= M <= FLEXQ_DECODE_MAX_M where flexq_gemm_w6ax_prefill_tile
   reports the 64 x 128 tile (a layer at least 1.5 * 128 columns wide per compute
   unit).  K does not enter the choice.  Never fails (M <= 0 or N <= 0 report
   FLEXQ_PATH_DECODE). */
int flexq_gemm_w6ax_auto_path(int64_t M, int64_t N, int64_t K);

/* The tile FLEXQ_PATH_PREFILL uses for an M x N x K product on the current device
   (one of FLEXQ_PATH_PREFILL_256X128 / _128X128 / _128X64 / _64X128): 64 x 128 for
   M <= 64 when the 128-column tiles number at least 1.5 per compute unit; otherwise
   the 256 x 128 tile when the grid of 128 x 128 tiles needs enough more rounds of one
   tile per compute unit (rounds256 * 1.46 < rounds128), else 128 x 64 when 128 x 128
   tiles would number no more than the compute units, else 128 x 128.  K does not
   enter the choice.  Never fails. */
int flexq_gemm_w6ax_prefill_tile(int64_t M, int64_t N, int64_t K);

/* Tail split of FLEXQ_PATH_PREFILL.  When the 256 x 128 grid ends in a partly filled
   round of one tile per compute unit, the 128-column blocks that fill whole rounds
   run as one launch of that tile and the remaining columns as a second launch of
   128 x 64 tiles on the same stream (at most two per compute unit), when the costs
   measured for the tiles predict a saving of at least a twentieth.  Y is the same either way.  Returns how many
   leading columns the first launch covers: N when there is no split, 0 for
   N <= 0.  K does not enter the choice.  Never fails. */
int64_t flexq_gemm_w6ax_prefill_main_cols(int64_t M, int64_t N, int64_t K);

/* flexq_gemm_w6ax with an explicit kernel choice (flexq_path); every kernel and
   tile accepts every M and gives identical results. */
flexq_status flexq_gemm_w6ax_path(const int8_t* q_a, const float* s_a,
                                  const uint32_t* w_packed, const uint16_t* s_w_fp16,
                                  int64_t M, int64_t N, int64_t K, int32_t group_size,
                                  int32_t abits, int32_t path, uint16_t* y_fp16, void* stream);

/* Split-K form of the GEMM, for mid-sized M (tens to a few hundred tokens), where
   the tile grid of the prefill kernel leaves compute units idle and each tile walks
   all of K alone.  K is cut at group boundaries into S slices: slice s covers the
   groups [s*G/S, (s+1)*G/S) (G = K/128) of every tile, in its own workgroup, and
   accumulates them from +0 in ascending order with the preamble's t / fma steps into
   fp32 plane s of the workspace ([S][M][N]).  A second kernel then adds the planes in
   ascending s in fp32 and rounds once to fp16.  The integer group products are the
   same as on every path; only the fp32 summation order differs from the preamble's
   single ascending chain, so Y agrees with it to within one fp16 ulp, or else the
   fp32 sum (acc_f32) agrees with the sequential accumulator to within 1e-5 times
   sum_g |t * s_a| (the blog's "Bridging Software and Hardware with BTC" fixes the
   exact integer group products and the fused dequantization, not an fp32 order).
   With S = 1 the result is bit-identical to flexq_gemm_w6ax.  Deterministic: the
   same inputs give the same bits on every call.
     q_a, s_a, w_packed, s_w_fp16, y_fp16 as for flexq_gemm_w6ax
     path      FLEXQ_PATH_PREFILL (the tile flexq_gemm_w6ax_splitk_plan reports) or
               FLEXQ_PATH_PREFILL_256X128 / _128X128 / _128X64 / _64X128
     splits    S, 1 <= S <= min(K/128, 64); 0 takes flexq_gemm_w6ax_splitk_plan's
     workspace at least flexq_gemm_w6ax_splitk_workspace_bytes(M, N, K, S) bytes,
               16-byte aligned, owned by the caller; overwritten, and not to be used
               by other work until this call's kernels have run
     acc_f32   NULL, or [M][N] fp32, 16-byte aligned: receives the fp32 sums that
               Y rounds (for verification)
   M == 0 or N == 0 is a no-op.  Errors: INVALID_VALUE (null, negative size, abits,
   path, splits out of range, workspace too small, overlap of an output with an
   input or of any two of workspace, y and acc), UNSUPPORTED (as for flexq_gemm_w6ax,
   and M * N * S above 2^40 elements). */
flexq_status flexq_gemm_w6ax_splitk(const int8_t* q_a, const float* s_a,
                                    const uint32_t* w_packed, const uint16_t* s_w_fp16,
                                    int64_t M, int64_t N, int64_t K, int32_t group_size,
                                    int32_t abits, int32_t path, int32_t splits,
                                    void* workspace, size_t workspace_bytes, uint16_t* y_fp16,
                                    float* acc_f32, void* stream);

/* Bytes of workspace flexq_gemm_w6ax_splitk needs with `splits` slices (0 = the
   planned count): splits * M * N * 4.  0 for M <= 0, N <= 0, K not a positive
   multiple of 128 or splits outside 0 .. min(K/128, 64). */
size_t flexq_gemm_w6ax_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t splits);

/* The slice count S and tile (written to *tile_path when it is not NULL) that
   flexq_gemm_w6ax_splitk takes for an M x N x K product on the current device when
   asked to choose.  S = 1 means splitting is not expected to pay: not against the
   tile grid alone and, up to 64 tokens, not against the weight-streaming kernel on
   blocked codes (flexq_gemm_w6ax_blocked), the faster choice there.  Never fails
   (degenerate shapes report 1 and FLEXQ_PATH_PREFILL_128X64). */
int32_t flexq_gemm_w6ax_splitk_plan(int64_t M, int64_t N, int64_t K, int32_t* tile_path);

/* Bytes of workspace flexq_linear_w6ax needs for an M x K activation: the codes
   (ceil(M/16)*16*K bytes, the blocked layout of the weight-streaming kernel, for
   M <= FLEXQ_DECODE_MAX_M; M*K row-major bytes above), rounded up to a multiple of 256,
   followed by s_a (M*(K/128)*4 bytes).  Returns 0 for M <= 0, K <= 0 or K not a
   multiple of 128. */
size_t flexq_linear_w6ax_workspace_bytes(int64_t M, int64_t K);

/* One W6A6 / W6A8 linear layer from fp16 activations in one call: the activation
   quantization into the workspace, then the GEMM with the automatic kernel choice --
   flexq_quant_act_blocked + flexq_gemm_w6ax_blocked where that choice is the
   weight-streaming kernel, flexq_quant_act + flexq_gemm_w6ax otherwise (blog,
   "Bridging Software and Hardware with BTC": quantized operands feed the integer
   GEMM; FlexQ abstract: activations at 6 or 8 bits).  Y is bit-identical to those
   two calls.  Nothing is allocated, so the call can be captured in a HIP graph.
     x_fp16    [M][K] fp16, 16-byte aligned (input)
     w_packed, s_w_fp16 as for flexq_gemm_w6ax (input)
     workspace device memory of at least flexq_linear_w6ax_workspace_bytes(M, K)
               bytes, 16-byte aligned; owned by the caller.  Its contents are
               overwritten (q_a, then s_a) and it must not be used by other work
               until this call's kernels have run.
     y_fp16    [M][N] fp16, 4-byte aligned (output)
   M == 0 or N == 0 is a no-op.  Errors: INVALID_VALUE (null, negative size, abits,
   workspace too small, overlap of any two of x, weights, workspace and y),
   UNSUPPORTED (group_size, K % 128, N % 16, size limits, alignment). */
flexq_status flexq_linear_w6ax(const uint16_t* x_fp16, const uint32_t* w_packed,
                               const uint16_t* s_w_fp16, int64_t M, int64_t N, int64_t K,
                               int32_t group_size, int32_t abits, void* workspace,
                               size_t workspace_bytes, uint16_t* y_fp16, void* stream);

/* Bytes of device memory the library keeps on each GPU for
   flexq_linear_w6ax_noalloc (64 MiB). */
#define FLEXQ_NOALLOC_SCRATCH_BYTES (64u << 20)

/* flexq_linear_w6ax for callers that cannot allocate device memory or bring a
   workspace: code under HIP graph capture, tight serving loops, harnesses that forbid
   hipMalloc.  Same arguments and result (bit for bit) without the workspace: q_a and
   s_a are staged in a file-scope device array of FLEXQ_NOALLOC_SCRATCH_BYTES bytes
   inside the library, one per GPU, held until the process ends; its address is
   looked up on the first call made with that device current.  The call allocates
   nothing.  Shapes with flexq_linear_w6ax_workspace_bytes(M, K) above
   FLEXQ_NOALLOC_SCRATCH_BYTES return FLEXQ_ERROR_UNSUPPORTED (e.g. K = 8192 allows
   M <= 7943, K = 28672 allows M <= 2269).  All calls on one GPU share the array and
   it keeps the last call's contents (nothing in it needs to start at zero): calls
   ordered on one stream are safe, calls that may overlap in time on one GPU (other
   streams, unordered host threads) race on it and must be serialized by the caller.
   FLEXQ_ERROR_LAUNCH also when the runtime cannot resolve the array's address. */
flexq_status flexq_linear_w6ax_noalloc(const uint16_t* x_fp16, const uint32_t* w_packed,
                                       const uint16_t* s_w_fp16, int64_t M, int64_t N, int64_t K,
                                       int32_t group_size, int32_t abits, uint16_t* y_fp16,
                                       void* stream);

/* The int32 group dots d[m][n][g] (the integer products of the BTC section) computed
   with the same weight unpack and int8 MFMA as the GEMM; for verification.
     dots [M][N][K/128] int32, 4-byte aligned (output). */
flexq_status flexq_gemm_w6ax_group_dots(const int8_t* q_a, const uint32_t* w_packed,
                                        int64_t M, int64_t N, int64_t K, int32_t group_size,
                                        int32_t* dots, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* FLEXQ_H */
