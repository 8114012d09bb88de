// gemm_prefill.hip -- W6Ax GEMM for many tokens: an MFMA-bound tiled kernel.
//
// FlexQ blog, "Bridging Software and Hardware with BTC": 128-deep K groups, an
// exact integer product per group, a bank-conflict-free shared-memory layout and
// the dequantization fused into the GEMM.  On gfx950 the integer product is
// v_mfma_i32_32x32x32_i8, the staging buffer is LDS, and the fused dequant is
// two fp32 FMAs per output and group:
//
//   * the first MFMA of a group takes C = 0x4B400000 (the float 1.5 * 2^23), so
//     the int32 result is 0x4B400000 + 4d; since |4d| < 2^22 those bits are the
//     float F = 12582912 + 4d exactly;
//   * with s4 = s_w / 4 (exact), t = fma(F, s4, -12582912 * s4) is the single
//     rounding of 4d * s4 = d * s_w, i.e. exactly RN32(float(d) * s_w);
//   * acc = fma(t, s_a, acc), groups in ascending order.
//
// So every output is bit-identical to the sequential definition.
//
// Tile: BM x BN per workgroup, 4 waves in a 2 x 2 grid, each wave 2 x 2 MFMA
// tiles of 32 x 32.  Per group, the workgroup stages the int8 activation tile and
// the unpacked weight tile (4*q bytes) in LDS, double-buffered; rows are padded
// by 16 bytes so the 16-byte fragment reads of a wave spread over all banks.
#include "kernels.h"
#include "w6_device.h"

namespace flexq {

namespace {

constexpr uint32_t kRsrcWord3 = 0x00020000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           kRsrcWord3);
}

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int LDA = kGroup + 16;  // padded LDS row (bytes)
constexpr int THREADS = 256;
constexpr uint32_t kMagic = 0x4B400000u;
constexpr float kMagicF = 12582912.0f;

}  // namespace

__global__ __launch_bounds__(THREADS) void gemm_prefill_kernel(
    const int8_t* __restrict__ qa, const float* __restrict__ sa, const uint32_t* __restrict__ wp,
    const uint16_t* __restrict__ sw, int M, int N, int K, uint16_t* __restrict__ y) {
  const int G = K >> 7;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const int mrows = min(BM, M - m0);
  const int ncols = min(BN, N - n0);

  __shared__ __attribute__((aligned(16))) int8_t lds_a[2][BM * LDA];
  __shared__ __attribute__((aligned(16))) int8_t lds_b[2][BN * LDA];
  __shared__ float lds_sa[2][BM];
  __shared__ float lds_sw[2][BN];

  // Out-of-range loads return zero: rows >= M and columns >= N vanish.
  const auto ra = make_rsrc(qa + (size_t)m0 * K, (uint32_t)mrows * (uint32_t)K);
  const auto rw = make_rsrc(wp + (size_t)(n0 / 16) * 3 * K, (uint32_t)(ncols / 16) * 12u * K);
  const auto rsa = make_rsrc(sa + (size_t)m0 * G, (uint32_t)mrows * G * 4u);
  const auto rsw = make_rsrc(sw + (size_t)n0 * G, (uint32_t)ncols * G * 2u);

  // global -> register staging for one group
  i32x4 ga[4];   // A: 16 B chunks c = tid + i*256 -> row c/8, col (c%8)*16
  u32x4 gb[3];   // B: 48 contiguous bytes = 4 units of tile tid/32
  float gsa = 0.0f;
  uint32_t gsw = 0;

  auto gload = [&](int g) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * THREADS;
      ga[i] = __builtin_amdgcn_raw_buffer_load_b128(
          ra, (uint32_t)(c >> 3) * (uint32_t)K + (uint32_t)g * 128u + (uint32_t)(c & 7) * 16u, 0, 0);
    }
    const uint32_t tb = (uint32_t)(tid >> 5) * 12u * (uint32_t)K + (uint32_t)g * 1536u +
                        (uint32_t)(tid & 31) * 48u;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rw, tb + 16u * i, 0, 0);
      gb[i] = __builtin_bit_cast(u32x4, v);
    }
    if (tid < BM)
      gsa = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(rsa, ((uint32_t)tid * G + g) * 4u, 0, 0));
    else
      gsw = __builtin_amdgcn_raw_buffer_load_b16(
          rsw, ((uint32_t)(tid - BM) * G + g) * 2u, 0, 0);
  };

  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * THREADS;
      *reinterpret_cast<i32x4*>(&lds_a[buf][(c >> 3) * LDA + (c & 7) * 16]) = ga[i];
    }
    // 48 bytes = units us0 .. us0+3 of the group in tile tid/32 (us = unit*16 + row%16)
    const uint32_t w[12] = {gb[0][0], gb[0][1], gb[0][2], gb[0][3], gb[1][0], gb[1][1],
                            gb[1][2], gb[1][3], gb[2][0], gb[2][1], gb[2][2], gb[2][3]};
    const int tile = tid >> 5;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int us = (tid & 31) * 4 + q;
      const int n = tile * 16 + (us & 15);
      const int kb = (us >> 4) * 16;
      *reinterpret_cast<i32x4*>(&lds_b[buf][n * LDA + kb]) =
          unpack_unit_x4(w[3 * q], w[3 * q + 1], w[3 * q + 2]);
    }
    if (tid < BM)
      lds_sa[buf][tid] = gsa;
    else
      lds_sw[buf][tid - BM] = half_bits_to_float((uint16_t)gsw);
  };

  float acc[2][2][16];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  i32x16 magic;
#pragma unroll
  for (int r = 0; r < 16; ++r) magic[r] = (int32_t)kMagic;

  gload(0);
  lstore(0);
  __syncthreads();

  const int frag_row = lane & 31;
  const int frag_k = (lane >> 5) * 16;

  for (int g = 0; g < G; ++g) {
    const int buf = g & 1;
    if (g + 1 < G) gload(g + 1);

    i32x16 d[2][2];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      i32x4 af[2], bf[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        af[t] = *reinterpret_cast<const i32x4*>(
            &lds_a[buf][(wm * 64 + t * 32 + frag_row) * LDA + c * 32 + frag_k]);
        bf[t] = *reinterpret_cast<const i32x4*>(
            &lds_b[buf][(wn * 64 + t * 32 + frag_row) * LDA + c * 32 + frag_k]);
      }
#pragma unroll
      for (int tm = 0; tm < 2; ++tm)
#pragma unroll
        for (int tn = 0; tn < 2; ++tn)
          d[tm][tn] = mfma32(af[tm], bf[tn], c == 0 ? magic : d[tm][tn]);
    }

    // fused dequantization
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) {
      const float s4 = 0.25f * lds_sw[buf][wn * 64 + tn * 32 + frag_row];
      const float bias = -kMagicF * s4;
#pragma unroll
      for (int tm = 0; tm < 2; ++tm) {
        const float* sar = &lds_sa[buf][wm * 64 + tm * 32 + 4 * (lane >> 5)];
        // reinterpret the whole vector: with hipcc 7.2 (clang 22) a bit_cast of a
        // single subscripted vector element silently reads element 0 instead
        const f32x16 Fv = __builtin_bit_cast(f32x16, d[tm][tn]);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float F = Fv[r];
          const float t = fmaf(F, s4, bias);
          acc[tm][tn][r] = fmaf(t, sar[8 * (r >> 2) + (r & 3)], acc[tm][tn][r]);
        }
      }
    }

    if (g + 1 < G) lstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: fp16 stores, column = lane % 32
#pragma unroll
  for (int tm = 0; tm < 2; ++tm)
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) {
      const int col = wn * 64 + tn * 32 + frag_row;
      if (col < ncols) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * 64 + tm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (row < mrows)
            y[(size_t)(m0 + row) * N + n0 + col] = float_to_half_bits(acc[tm][tn][r]);
        }
      }
    }
}

hipError_t launch_gemm_prefill(const int8_t* qa, const float* sa, const uint32_t* wp,
                               const uint16_t* sw, int64_t M, int64_t N, int64_t K, uint16_t* y,
                               hipStream_t stream) {
  dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  hipLaunchKernelGGL(gemm_prefill_kernel, grid, dim3(THREADS), 0, stream, qa, sa, wp, sw,
                     (int)M, (int)N, (int)K, y);
  return hipGetLastError();
}

}  // namespace flexq
