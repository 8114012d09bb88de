// gemm_decode.hip -- W6Ax GEMM for few tokens (M <= 64): an HBM-streaming kernel.
//
// FlexQ blog, "Bridging Software and Hardware with BTC": K is cut into 128-deep
// groups, each group gives an exact integer product, partial results are
// reduced and the dequantization is fused; the kernel is meant to use the
// memory hierarchy well at small batch.  On gfx950 the integer product is an
// int8 MFMA (v_mfma_i32_16x16x64_i8) over weights unpacked in registers, and
// the time goes to streaming the 0.75 B/weight packed matrix from HBM.
//
// Work items are (T adjacent 16-column tiles, pass of up to 64 token rows); a wave
// unpacks the weights of all T tiles of its group against one set of activation
// fragments, so activations are fetched once per T tiles.  The grid is
// persistent: every workgroup owns a contiguous run of items (so of packed weight
// memory) and streams through it without a break, its load ring running on from
// one item into the next.  Inside an item, round r hands group g = r*S + w to
// wave w, so a round reads S*1536 contiguous bytes of the tile.  Every wave keeps
// P rounds of loads in flight (weights, activations and both scales, issued
// together so the in-order vmcnt never waits on a younger load); the weight loads
// are non-temporal since each weight byte is read exactly once.  After its two
// MFMAs a wave parks the 16 x rows int32 dots and the group's scales in LDS; after
// one barrier the block folds the S groups into the fp32 accumulators in
// ascending group order, so the result equals the sequential definition bit for
// bit.  The last round of an item stores its fp16 outputs.
#include <atomic>
#include <type_traits>

#include "kernels.h"
#include "w6_device.h"

namespace flexq {

namespace {

constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw 32-bit dword buffer, gfx9 style
constexpr int kNonTemporal = 2;                // cache-policy bit of buffer loads

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           kRsrcWord3);
}

// Activation fragment as loaded: 16 int8 codes, or (PA) one packed 6-bit unit.
template <bool PA>
using AFrag = typename std::conditional<PA, u32x3, i32x4>::type;

template <int MT, int T, bool PA>
struct Bundle {
  u32x3 w[T][2];        // per 16-column tile: two weight units (k-blocks of 64)
  AFrag<PA> a[MT][2];   // activation fragments, rows ms*16 + lane%16
  float sa;             // s_a[row = lane][g]
  uint32_t sw;          // s_w[col = lane % (16*T)][g] (fp16 bits)
};

// Position of a step in a workgroup's stream.  The workgroup's items are cut into
// chunks of up to C consecutive items of one pass; a chunk runs round-major (round
// r of all its items, then round r+1), so the activation fragments of a round are
// fetched once per chunk.  A step is (chunk, round r, item i of the chunk); i runs
// over all C slots, slots past the chunk's end are empty steps.
struct Cursor {
  int chunk_begin, chunk_n, tile0, pass, r, i;
  __device__ __forceinline__ void start_chunk(int C, int item_end, int ntiles) {
    chunk_n = min(C, min(item_end - chunk_begin, ntiles - tile0));
  }
  __device__ __forceinline__ void next(int C, int R, int item_end, int ntiles) {
    if (++i == C) {
      i = 0;
      if (++r == R) {
        r = 0;
        chunk_begin += chunk_n;
        tile0 += chunk_n;
        if (tile0 == ntiles) {
          tile0 = 0;
          ++pass;
        }
        start_chunk(C, item_end, ntiles);
      }
    }
  }
  __device__ __forceinline__ bool live(int item_end) const {
    return chunk_begin < item_end && i < chunk_n;
  }
};

}  // namespace

// Where the activation codes come from (AL):
// kActBytes: q_a row-major, one byte per code.
// kActFused: the activation quantization fused in front (one pass of up to 16 rows):
//   the workgroup quantizes fp16 X (x, qmax) once into LDS -- the same per-group rule
//   and helper as flexq_quant_act, so codes and scales are bit-identical -- and the
//   activation fragments and scales are read from there instead of q_a / s_a.
// kActPacked6: qa holds A6 codes packed 16 per 3 dwords, the units of a row in order
//   (0.75 K bytes per row); each fragment is one 12-byte unit, unpacked like the
//   weights into bytes 4 * q_a, so the MFMA dots are 16 d and the fold scales by
//   s_w / 16 instead of s_w / 4 (both exact).
// kActBlocked: qa holds the codes in 16-row blocks, each group's two 64-deep halves
//   stored as the 16 rows' 64-byte segments in turn (rows padded to a multiple of
//   16): a fragment load reads 1 KB in one piece, 8 whole 128-byte lines, where the
//   row-major codes give 16 half-used lines, and that line traffic is what makes 16
//   and more rows slower than a few.
constexpr int kActBytes = 0, kActFused = 1, kActPacked6 = 2, kActBlocked = 3;

template <int MT, int T, int S, int P, int C, int AL>
__global__ __launch_bounds__(64 * S) void gemm_decode_kernel(
    const int8_t* __restrict__ qa, const float* __restrict__ sa, const uint32_t* __restrict__ wp,
    const uint16_t* __restrict__ sw, int M, int N, int K, uint16_t* __restrict__ y, int ntiles16,
    int ntiles, int items, int per_wg, const uint16_t* __restrict__ x, int qmax) {
  constexpr bool FQ = AL == kActFused, PA = AL == kActPacked6, BL = AL == kActBlocked;
  static_assert(!FQ || MT == 1, "the fused quantizer covers one pass of up to 16 rows");
  static_assert(P % 2 == 0, "slot parity must be static");
  constexpr int U = C > P ? C : P;  // steps per loop iteration: ring slot and item static
  static_assert(U % P == 0 && U % C == 0, "step unroll");
  constexpr int ROWS = MT * 16;
  constexpr int COLS = T * 16;
  constexpr int OUTS = ROWS * COLS;
  constexpr int THREADS = 64 * S;
  // Fold layout.  With 16 waves (up to 32 rows): dots parked row-major, one output
  // per thread and round.  With 8 waves or from 48 rows: parked column-major (padded
  // pitch, conflict-free), each thread folding a 4-row segment of one column with
  // 16-byte LDS reads: a quarter of the LDS instructions; the four accumulators per
  // thread fit the 8-wave register budget.
  constexpr bool QUAD = MT >= 3 || S <= 8;
  constexpr int PITCH = QUAD ? ROWS + 4 : COLS;  // int32s per parked column / row
  constexpr int PARK = QUAD ? COLS * PITCH : OUTS;
  constexpr int QUADS = (ROWS / 4) * COLS;
  constexpr int OPT = QUAD ? 4 * ((QUADS + THREADS - 1) / THREADS) : (OUTS + THREADS - 1) / THREADS;

  const int G = K >> 7;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int R = (G + S - 1) / S;  // rounds per item
  const int item_begin = blockIdx.x * per_wg;
  const int item_end = min(items, item_begin + per_wg);

  __shared__ __attribute__((aligned(16))) int32_t lds_d[2][S][PARK];
  __shared__ __attribute__((aligned(16))) float lds_sa[2][S][ROWS];
  __shared__ float lds_sw[2][S][COLS];
  // FQ: the quantized activations, [rows][K] codes then [G][rows] scales
  extern __shared__ __attribute__((aligned(16))) int8_t lds_x[];
  const int fq_rows = FQ ? min(ROWS, M) : 0;
  const int8_t* lq = lds_x;
  const float* lsc = reinterpret_cast<const float*>(lds_x + (fq_rows * K + 15) / 16 * 16);

  // bytes per activation row (a 16-row block is 16 rows), and the strides of a group
  // and of a 64-deep k-block, and the lane's offset in them
  const uint32_t a_row = PA ? (uint32_t)K / 4u * 3u : (uint32_t)K;
  constexpr uint32_t a_grp = BL ? 2048u : (PA ? 96u : 128u);
  constexpr uint32_t a_blk = BL ? 1024u : (PA ? 48u : 64u);
  const uint32_t a_lane_off =
      BL ? (uint32_t)(lane & 15) * 64u + (uint32_t)(lane >> 4) * 16u
         : (uint32_t)(lane & 15) * a_row + (uint32_t)(lane >> 4) * (a_blk / 4u);

  // Loads of step c.  Out-of-range buffer loads return zero: rows past the pass and
  // groups >= G vanish; empty steps read from empty buffers.  The activation
  // fragments are loaded by the chunk's first item slot only.
  auto load = [&](Bundle<MT, T, PA>& b, const Cursor& c, auto first_slot) {
    const bool live = c.live(item_end);
    const int tile = live ? c.tile0 + c.i : 0;  // in units of COLS columns
    const int row0 = live ? c.pass * 64 : 0;
    // rows of the pass the activation buffer holds (blocked: padded to whole blocks)
    const int rows = live ? min(ROWS, (BL ? (M + 15) / 16 * 16 : M) - row0) : 0;
    const auto ra = make_rsrc(qa + (size_t)row0 * a_row, (uint32_t)rows * a_row);
    // blocked: a lane whose row is a pad row reads past the buffer instead (zero, and no
    // memory traffic), as the row-major codes' lanes past M do
    const int real_rows = live ? min(ROWS, M - row0) : 0;
    // scales are group-major (s_a[g][m] at g*M + m, s_w[g][n] at g*N + n); entries of
    // rows past the pass or columns past N are read but never used
    const auto rsa = make_rsrc(sa + row0, live ? (uint32_t)((size_t)G * M - row0) * 4u : 0u);
    const auto rsw = make_rsrc(sw + (size_t)tile * COLS,
                               live ? (uint32_t)((size_t)G * N - tile * COLS) * 2u : 0u);
    const uint32_t g = (uint32_t)(c.r * S + wave);
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int t16 = tile * T + t;
      const bool in = live && t16 < ntiles16;
      const auto rw = make_rsrc(wp + (size_t)(in ? t16 : 0) * 3 * K, in ? 12u * (uint32_t)K : 0u);
      b.w[t][0] =
          __builtin_amdgcn_raw_buffer_load_b96(rw, (g * 128u + lane) * 12u, 0, kNonTemporal);
      b.w[t][1] =
          __builtin_amdgcn_raw_buffer_load_b96(rw, (g * 128u + 64u + lane) * 12u, 0, kNonTemporal);
    }
    if constexpr (decltype(first_slot)::value && !FQ) {
#pragma unroll
      for (int ms = 0; ms < MT; ++ms) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          uint32_t off = a_lane_off + (uint32_t)(ms * 16) * a_row + g * a_grp + j * a_blk;
          if constexpr (BL)
            if (ms * 16 + (lane & 15) >= real_rows) off = 0x80000000u;
          if constexpr (PA)
            b.a[ms][j] = __builtin_amdgcn_raw_buffer_load_b96(ra, off, 0, 0);
          else
            b.a[ms][j] = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);
        }
      }
    }
    // (every offset goes in the VGPR operand: the range check that zeroes reads
    // past the buffer does not cover the scalar offset)
    if constexpr (!FQ)
      b.sa = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(rsa, ((uint32_t)lane + g * (uint32_t)M) * 4u, 0, 0));
    b.sw = __builtin_amdgcn_raw_buffer_load_b16(
        rsw, ((uint32_t)(lane % COLS) + g * (uint32_t)N) * 2u, 0, 0);
  };

  Cursor start{item_begin, 0, item_begin % ntiles, item_begin / ntiles, 0, 0};
  start.start_chunk(C, item_end, ntiles);
  Cursor cl = start;  // next step to load; step k goes to ring slot k % P
  Bundle<MT, T, PA> ring[P];
  unroll([&](auto pc) {
    constexpr int p = decltype(pc)::value;
    load(ring[p], cl, std::integral_constant<bool, p % C == 0>{});
    cl.next(C, R, item_end, ntiles);
  }, std::make_integer_sequence<int, P>{});

  if constexpr (FQ) {
    // quantize the pass's rows into LDS while the weight loads above are in flight:
    // unit u = 8 consecutive values; the 16 units of a 128-deep group sit in the 16
    // lanes of one DPP row (rows * K / 8 and the loop step are multiples of 16, so a
    // DPP row is wholly inside or outside the range)
    int8_t* wq = lds_x;
    float* ws = reinterpret_cast<float*>(lds_x + (fq_rows * K + 15) / 16 * 16);
    const int upr = K >> 3, units = fq_rows * upr;
    for (int u0 = 0; u0 < units; u0 += THREADS) {
      const int u = u0 + (int)threadIdx.x;
      if (u < units) {
        const int row = u / upr, k0 = (u - row * upr) * 8;
        const u32x4 h = *reinterpret_cast<const u32x4*>(x + (size_t)row * K + k0);
        float s;
        const u32x2 codes = quant8_row16(h, qmax, s);
        *reinterpret_cast<u32x2*>(wq + row * K + k0) = codes;
        if ((threadIdx.x & 15) == 0) ws[(k0 >> 7) * fq_rows + row] = s;
      }
    }
    __syncthreads();
  }

  float acc[C][OPT];
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int i = 0; i < OPT; ++i) acc[c][i] = 0.0f;
  i32x4 a_cur[MT][2];  // activation fragments of the current round

  Cursor cp = start;  // step being processed
  const i32x4 zero = {0, 0, 0, 0};
  while (cp.chunk_begin < item_end) {  // workgroup-uniform
    unroll([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      constexpr int slot = p & 1;
      constexpr int ci = p % C;  // item slot of this step
      Bundle<MT, T, PA>& b = ring[p % P];
      // FQ: this step's group in the LDS copy (clamped: rounds past the last group
      // are never folded), and a row that exists (rows past M are never stored)
      const int fq_g = FQ ? min(cp.r * S + wave, G - 1) : 0;
      if constexpr (ci == 0) {
        if constexpr (FQ) {
          const int row = min(lane & 15, fq_rows - 1);
#pragma unroll
          for (int j = 0; j < 2; ++j)
            a_cur[0][j] = *reinterpret_cast<const i32x4*>(lq + row * K + fq_g * 128 + j * 64 +
                                                          (lane >> 4) * 16);
        } else {
#pragma unroll
          for (int ms = 0; ms < MT; ++ms) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              if constexpr (PA)
                a_cur[ms][j] = unpack_unit_x4(b.a[ms][j][0], b.a[ms][j][1], b.a[ms][j][2]);
              else
                a_cur[ms][j] = b.a[ms][j];
            }
          }
        }
      }
      // exact integer group products (4*d, see w6_device.h; PA: 16*d)
      i32x4 d[T][MT];
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const i32x4 b0 = unpack_unit_x4(b.w[t][0][0], b.w[t][0][1], b.w[t][0][2]);
        const i32x4 b1 = unpack_unit_x4(b.w[t][1][0], b.w[t][1][1], b.w[t][1][2]);
#pragma unroll
        for (int ms = 0; ms < MT; ++ms) {
          d[t][ms] = mfma16(a_cur[ms][0], b0, zero);
          d[t][ms] = mfma16(a_cur[ms][1], b1, d[t][ms]);
        }
      }
      // park dots 4d (row-major [row][col]) and this group's scales, s_w as s_w / 4
      // (exact), so the fold forms t = RN(d * s_w) as float(4d) * (s_w / 4); with PA
      // as float(16d) * (s_w / 16), exact too: |16d| <= 16 * 128 * 32 * 32 = 2^21
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int ms = 0; ms < MT; ++ms) {
          if constexpr (QUAD) {
            *reinterpret_cast<i32x4*>(
                &lds_d[slot][wave][(t * 16 + (lane & 15)) * PITCH + ms * 16 + 4 * (lane >> 4)]) =
                d[t][ms];
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              lds_d[slot][wave][(ms * 16 + 4 * (lane >> 4) + i) * COLS + t * 16 + (lane & 15)] =
                  d[t][ms][i];
          }
        }
      if constexpr (FQ) {
        if (lane < ROWS) lds_sa[slot][wave][lane] = lsc[fq_g * fq_rows + min(lane, fq_rows - 1)];
      } else {
        if (lane < ROWS) lds_sa[slot][wave][lane] = b.sa;
      }
      if (lane < COLS)
        lds_sw[slot][wave][lane] = (PA ? 0.0625f : 0.25f) * half_bits_to_float((uint16_t)b.sw);
      // the step P ahead lands in this ring slot; it is the chunk's first item slot
      // exactly when this one is (P is a multiple of C, or C of P)
      load(b, cl, std::integral_constant<bool, ((p + P) % C) == 0>{});
      cl.next(C, R, item_end, ntiles);
      __syncthreads();
      if (cp.live(item_end)) {  // workgroup-uniform
        // fold the S groups of this round into item ci's accumulators, ascending g
        const int row0 = cp.pass * 64;
        const int rows = min(ROWS, M - row0);
        const int ng = min(S, G - cp.r * S);
        if constexpr (QUAD) {
#pragma unroll
          for (int j = 0; j < OPT / 4; ++j) {
            const int q = threadIdx.x + j * THREADS;
            const int col = q % COLS, r0 = 4 * (q / COLS);
            if (q < QUADS && r0 < rows) {
              i32x4 dv[S];
              f32x4 sav[S];
              float swv[S];
#pragma unroll
              for (int w = 0; w < S; ++w) {
                dv[w] = *reinterpret_cast<const i32x4*>(&lds_d[slot][w][col * PITCH + r0]);
                sav[w] = *reinterpret_cast<const f32x4*>(&lds_sa[slot][w][r0]);
                swv[w] = lds_sw[slot][w][col];
              }
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                float a = acc[ci][4 * j + r];
#pragma unroll
                for (int w = 0; w < S; ++w) {
                  if (w < ng) {
                    const float t = (float)dv[w][r] * swv[w];  // float(4d) exact
                    a = fmaf(t, sav[w][r], a);
                  }
                }
                acc[ci][4 * j + r] = a;
              }
            }
          }
        } else {
#pragma unroll
        for (int i = 0; i < OPT; ++i) {
          const int o = threadIdx.x + i * THREADS;
          if (o < OUTS && o / COLS < rows) {
            const int row = o / COLS, col = o % COLS;
            // all reads first, then the dependent chain
            int dv[S];
            float swv[S], sav[S];
#pragma unroll
            for (int w = 0; w < S; ++w) {
              dv[w] = lds_d[slot][w][o];
              swv[w] = lds_sw[slot][w][col];
              sav[w] = lds_sa[slot][w][row];
            }
            float a = acc[ci][i];
#pragma unroll
            for (int w = 0; w < S; ++w) {
              if (w < ng) {
                const float t = (float)dv[w] * swv[w];  // float(4d) is exact
                a = fmaf(t, sav[w], a);
              }
            }
            acc[ci][i] = a;
          }
        }
        }
        if (cp.r == R - 1) {  // item complete: store and restart its accumulators
          const int tile = cp.tile0 + ci;
#pragma unroll
          for (int i = 0; i < OPT; ++i) {
            // output i of this thread: (row, col) in the item
            int row, col;
            bool in;
            if constexpr (QUAD) {
              const int q = threadIdx.x + (i / 4) * THREADS;
              col = q % COLS;
              row = 4 * (q / COLS) + i % 4;
              in = q < QUADS;
            } else {
              const int o = threadIdx.x + i * THREADS;
              col = o % COLS;
              row = o / COLS;
              in = o < OUTS;
            }
            const int n = tile * COLS + col;
            if (in && row < rows && n < N)
              y[(size_t)(row0 + row) * N + n] = float_to_half_bits(acc[ci][i]);
            acc[ci][i] = 0.0f;
          }
        }
      }
      cp.next(C, R, item_end, ntiles);
    }, std::make_integer_sequence<int, U>{});
  }
}

int device_cu_count() {
  // per device, 0 = not yet queried; threads that race on the first query store the
  // same value
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

bool fused_quant_eligible(int64_t M, int64_t N, int64_t K) {
  // Every workgroup quantizes all of X, so the prologue grows with M * K while the
  // kernel boundary it saves is fixed.  In HIP graphs of 20 calls on the
  // LLaMA-2-70B layers (us, fused / quant_act + GEMM): qkv M = 1, 2, 4: 15.6 / 17.7,
  // 16.9 / 17.7, 19.3 / 18.0; o 12.4 / 13.7, 13.2 / 13.8, 15.8 / 14.2; gate_up M = 1
  // 58.4 / 59.2, M = 2 57.5 / 57.0; down (K = 28672) M = 1 35.0 / 33.6.
  (void)N;
  return M >= 1 && M <= 4 && M * K <= 16384;
}

size_t fused_quant_lds_bytes(int64_t M, int64_t K) {
  const int64_t rows = M < 16 ? M : 16;
  return (size_t)((rows * K + 15) / 16 * 16 + rows * (K / kGroup) * 4);
}

// Time model of the weight-streaming kernel on codes in 16-row blocks at 33 to 64
// rows (its paired-tile, 8-wave forms), in microseconds, fitted to the LLaMA-2 7B,
// 13B and 70B layers and their 8-way tensor-parallel shares on MI355X (20 launches
// back to back, weights rotated through HBM): 4.3 plus, per group each workgroup
// walks, 0.205 up to 48 rows and 0.005 more per row above; workgroups that own two
// or more items share each round's activation fragments over a chunk (x 0.8); a grid
// that leaves CUs idle gives each workgroup more of the HBM bandwidth (x (0.7 + 0.3 *
// workgroups / CUs)).  Over 90 shapes at 33-64 rows the split plan this model informs
// takes in total within 1 % of the best of the streaming kernel, split-K and the
// tile grid per shape (its largest miss: 2 us on the 8-way share of 70B qkv).
double predict_decode_us(int64_t M, int64_t N, int64_t G, int64_t cu) {
  const int64_t items = std::max<int64_t>(1, (N + 31) / 32);  // paired 16-column tiles
  const int64_t grid = std::max<int64_t>(1, std::min(items, cu));
  const int64_t per_wg = (items + grid - 1) / grid;
  double c = 0.205 + (M > 48 ? 0.005 * (double)(M - 48) : 0.0);
  if (per_wg >= 2) c *= 0.8;
  c *= 0.7 + 0.3 * (double)grid / (double)cu;
  return 4.3 + (double)(per_wg * G) * c;
}

int auto_gemm_path(int64_t M, int64_t N) {
  // Up to one 64-row pass the streaming kernel is faster than the 128-row prefill
  // tiles on every LLaMA-2-70B layer (M = 64, weights cold: qkv 37.5 vs 38.8 us, o 27
  // vs 37, gate_up 108 vs 121, down 87 vs 127); beyond it the weights would be
  // streamed once per 64 rows and the tiled kernel wins.  From 48 rows on wide
  // layers, where the 64 x 128 tile's grid fills the GPU (prefill_tile), that tile
  // wins instead: gate_up M = 64 96 -> 78 us, M = 48 79 -> 76 us (it loses at 32 rows
  // and below, and on narrow layers, whose grids it leaves half empty).
  if (M > kDecodeRowsPerPass) return 2;
  return M >= 48 && prefill_tile(M, N) == kTile64x128 ? 2 : 1;
}

template <int MT, int T, int S, int P, int C, int AL = kActBytes>
static hipError_t launch_decode_c(const int8_t* qa, const float* sa, const uint32_t* wp,
                                  const uint16_t* sw, int64_t M, int64_t N, int64_t K,
                                  uint16_t* y, int64_t ntiles16, int64_t ntiles, int64_t items,
                                  int64_t per_wg, int64_t grid, hipStream_t stream,
                                  const uint16_t* x = nullptr, int qmax = 0) {
  const size_t lds_x = AL == kActFused ? fused_quant_lds_bytes(M, K) : 0;
  return launch_kernel_lds(gemm_decode_kernel<MT, T, S, P, C, AL>, dim3((unsigned)grid),
                           dim3(64 * S), lds_x, stream, qa, sa, wp, sw, (int)M, (int)N, (int)K, y,
                           (int)ntiles16, (int)ntiles, (int)items, (int)per_wg, x, qmax);
}

template <int MT, int T, int S, int P, int CMAX, int AL = kActBytes>
static hipError_t launch_decode_t(const int8_t* qa, const float* sa, const uint32_t* wp,
                                  const uint16_t* sw, int64_t M, int64_t N, int64_t K,
                                  uint16_t* y, hipStream_t stream, bool chunk_few_rows = false,
                                  const uint16_t* x = nullptr, int qmax = 0) {
  const int64_t ntiles16 = N / 16;
  const int64_t ntiles = (ntiles16 + T - 1) / T;
  const int64_t items = ntiles * ((M + 63) / 64);
  if (items > INT32_MAX) return hipErrorInvalidValue;  // item indices are 32-bit
  // one resident workgroup per CU; each takes an equal contiguous share of items
  const int64_t grid0 = std::min<int64_t>(items, device_cu_count());
  const int64_t per_wg = (items + grid0 - 1) / grid0;
  const int64_t grid = (items + per_wg - 1) / per_wg;
  // chunk: the workgroup's items share each round's activation fragments (with only a
  // few token rows not worth the empty steps of a partial chunk, except where the
  // caller found it pays)
  if (M <= 4 && !chunk_few_rows)
    return launch_decode_c<MT, T, S, P, 1, AL>(qa, sa, wp, sw, M, N, K, y, ntiles16, ntiles,
                                                   items, per_wg, grid, stream, x, qmax);
  if (CMAX >= 8 && per_wg >= 5)
    return launch_decode_c<MT, T, S, P, (CMAX >= 8 ? 8 : 1), AL>(
        qa, sa, wp, sw, M, N, K, y, ntiles16, ntiles, items, per_wg, grid, stream, x, qmax);
  if (CMAX >= 4 && per_wg >= 3)
    return launch_decode_c<MT, T, S, P, (CMAX >= 4 ? 4 : 1), AL>(
        qa, sa, wp, sw, M, N, K, y, ntiles16, ntiles, items, per_wg, grid, stream, x, qmax);
  if (CMAX >= 2 && per_wg >= 2)
    return launch_decode_c<MT, T, S, P, (CMAX >= 2 ? 2 : 1), AL>(
        qa, sa, wp, sw, M, N, K, y, ntiles16, ntiles, items, per_wg, grid, stream, x, qmax);
  return launch_decode_c<MT, T, S, P, 1, AL>(qa, sa, wp, sw, M, N, K, y, ntiles16, ntiles,
                                                 items, per_wg, grid, stream, x, qmax);
}

// The kernel configuration for an M x N x K product, activations as AL says.
template <int AL>
static hipError_t launch_decode_any(const int8_t* qa, const float* sa, const uint32_t* wp,
                                    const uint16_t* sw, int64_t M, int64_t N, int64_t K,
                                    uint16_t* y, hipStream_t stream) {
  // rows per pass: 16 * MT; more passes over W only when M > 64
  const int64_t rows = M > 64 ? 64 : M;
  const int64_t cu = device_cu_count();
  if (rows <= 16) {
    // Narrow, short layers (up to 3 single-tile items per CU, K <= 16384) run single
    // tiles: the workgroups' shares of the weights come out more even (10 % faster on
    // the 70B qkv and o shapes); elsewhere pairing tiles halves the activation
    // fragment loads per weight byte and wins.  Up to 4 rows, chunks of 2 items share
    // the activation fragments, and layers with more than 2 single tiles per CU pair
    // their tiles (back-to-back launches, 70B at M = 1: qkv 16.3 -> 14.8 us with
    // paired tiles, o 12.3 -> 11.3 us with chunks of single tiles).
    if (N / 16 <= 3 * cu && K <= 16384) {
      if (rows <= 4 && N / 16 > 2 * cu)
        return launch_decode_t<1, 2, 16, 2, 2, AL>(qa, sa, wp, sw, M, N, K, y, stream,
                                                          true);
      if (rows <= 4)
        return launch_decode_t<1, 1, 16, 2, 2, AL>(qa, sa, wp, sw, M, N, K, y, stream,
                                                          true);
      return launch_decode_t<1, 1, 16, 2, 8, AL>(qa, sa, wp, sw, M, N, K, y, stream);
    }
    // Paired tiles: 16 waves for up to 4 rows; from 5 rows 8 waves with the
    // column-segment fold (70B down at M = 16: 39 -> 36 us; 16 waves stay faster
    // at M = 1, where the fold is tiny and more waves keep more loads in flight).
    if (rows <= 4)
      return launch_decode_t<1, 2, 16, 2, 8, AL>(qa, sa, wp, sw, M, N, K, y, stream);
    return launch_decode_t<1, 2, 8, 2, 8, AL>(qa, sa, wp, sw, M, N, K, y, stream);
  }
  if (rows <= 32) {
    // Paired tiles with 8 waves on every layer: the register budget allows chunks of
    // 8 items (activation fragments shared 8 ways; 16 waves fit only 2) and the
    // column-segment fold (70B gate_up at M = 24 / 32: 80 -> 67 / 90 -> 73 us).  From
    // 17 rows the narrow layers gain from it too (single 16-column tiles in chunks of
    // up to 4, 16 waves: qkv M = 24 / 32 22.3 / 24.5 -> 20.9 / 23.2 us, o M = 24
    // 15.6 -> 14.5 us, o M = 32 equal).
    return launch_decode_t<2, 2, 8, 2, 8, AL>(qa, sa, wp, sw, M, N, K, y, stream);
  }
  if (rows <= 48)
    return launch_decode_t<3, 2, 8, 2, 8, AL>(qa, sa, wp, sw, M, N, K, y, stream);
  return launch_decode_t<4, 2, 8, 2, 8, AL>(qa, sa, wp, sw, M, N, K, y, stream);
}

hipError_t launch_gemm_decode(const int8_t* qa, const float* sa, const uint32_t* wp,
                              const uint16_t* sw, int64_t M, int64_t N, int64_t K, uint16_t* y,
                              hipStream_t stream) {
  return launch_decode_any<kActBytes>(qa, sa, wp, sw, M, N, K, y, stream);
}

hipError_t launch_gemm_decode_a6p(const uint32_t* qp, const float* sa, const uint32_t* wp,
                                  const uint16_t* sw, int64_t M, int64_t N, int64_t K,
                                  uint16_t* y, hipStream_t stream) {
  return launch_decode_any<kActPacked6>(reinterpret_cast<const int8_t*>(qp), sa, wp, sw, M, N, K,
                                        y, stream);
}

hipError_t launch_gemm_decode_blocked(const int8_t* qb, const float* sa, const uint32_t* wp,
                                      const uint16_t* sw, int64_t M, int64_t N, int64_t K,
                                      uint16_t* y, hipStream_t stream) {
  return launch_decode_any<kActBlocked>(qb, sa, wp, sw, M, N, K, y, stream);
}

hipError_t launch_linear_decode_fused(const uint16_t* x, int64_t M, int64_t K, int qmax,
                                      const uint32_t* wp, const uint16_t* sw, int64_t N,
                                      uint16_t* y, hipStream_t stream) {
  // the kernel configurations launch_gemm_decode takes for up to 4 rows
  const int64_t cu = device_cu_count();
  if (N / 16 <= 3 * cu && K <= 16384) {
    if (N / 16 > 2 * cu)
      return launch_decode_t<1, 2, 16, 2, 2, kActFused>(nullptr, nullptr, wp, sw, M, N, K, y,
                                                        stream, true, x, qmax);
    return launch_decode_t<1, 1, 16, 2, 2, kActFused>(nullptr, nullptr, wp, sw, M, N, K, y,
                                                      stream, true, x, qmax);
  }
  return launch_decode_t<1, 2, 16, 2, 8, kActFused>(nullptr, nullptr, wp, sw, M, N, K, y, stream,
                                                    false, x, qmax);
}

}  // namespace flexq
