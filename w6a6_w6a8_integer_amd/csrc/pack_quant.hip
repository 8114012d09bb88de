// pack_quant.hip -- weight group quantization + 6-bit packing, and activation
// group quantization (FlexQ blog, "Fine-Grained Quantization and Layer
// Sensitivity": one scale per small group of weights or activations; FlexQ
// abstract: 6-bit weights everywhere, 6- or 8-bit activations per layer).
//
// The activation quantizer can also write A6 codes packed 16 per 3 dwords (the
// weight unit, FlexQ abstract: W6A6 holds activations at 6 bits), or the codes in
// 16-row blocks in the order the weight-streaming kernel feeds its MFMAs.
//
// Both kernels are HBM-bound elementwise passes.  Arithmetic follows the
// formulas of the public header exactly (IEEE division, round half to even),
// so their outputs are bit-identical to the plain definition.
#include "kernels.h"
#include "w6_device.h"

namespace flexq {

// One workgroup = one 16-row tile x one 128-deep group.  Thread t handles row
// t/8 of the tile and unit t%8 of the group (16 codes); the 8 threads of a row
// are adjacent lanes, so the group max is a 3-step butterfly.
__global__ __launch_bounds__(128) void pack_w6_kernel(const uint16_t* __restrict__ w, int N,
                                                      int K, uint32_t* __restrict__ wp,
                                                      uint16_t* __restrict__ sw) {
  const int t = threadIdx.x;
  const int r = t >> 3, j = t & 7;
  const int64_t n = (int64_t)blockIdx.x * 16 + r;
  const int g = blockIdx.y;
  const u32x4* src = reinterpret_cast<const u32x4*>(w + n * K + g * kGroup + j * 16);
  u32x4 h0 = src[0], h1 = src[1];
  float v[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = half_bits_to_float((uint16_t)(h0[i] & 0xFFFFu));
    v[2 * i + 1] = half_bits_to_float((uint16_t)(h0[i] >> 16));
    v[8 + 2 * i] = half_bits_to_float((uint16_t)(h1[i] & 0xFFFFu));
    v[8 + 2 * i + 1] = half_bits_to_float((uint16_t)(h1[i] >> 16));
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  amax = fmaxf(amax, __shfl_xor(amax, 4));
  const uint16_t s16 = float_to_half_bits(amax / 31.0f);
  const float sf = half_bits_to_float(s16);
  int q[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    int c = 0;
    if (sf != 0.0f) c = (int)rintf(v[i] / sf);
    q[i] = c > 31 ? 31 : (c < -31 ? -31 : c);
  }
  const u32x3 d = pack_unit(q);
  uint32_t* dst = wp + unit_dword(n, (int64_t)g * kUnitsPerGroup + j, K);
  dst[0] = d[0];
  dst[1] = d[1];
  dst[2] = d[2];
  if (j == 0) sw[(int64_t)g * N + n] = s16;  // group-major scales
}

// Thread = 8 consecutive activations; 16 adjacent lanes (one DPP row) = one
// 128-deep group.  blockIdx.x = token row, blockIdx.y = chunk of 2048 columns.
// kOutPackedA6: the codes of lanes 2i and 2i+1 form one 16-code unit, which the even
// lane writes (12 bytes at unit (m, k0 / 16) of the row-major unit grid).
// kOutBlocked: the grid covers M rounded up to 16 rows; row m's 8 codes go to block
// m / 16, group g, half h, row m % 16, byte c at (m/16)*16*K + g*2048 + h*1024 +
// (m%16)*64 + c, and the rows past M write zero codes (no scale).
constexpr int kOutBytes = 0, kOutPackedA6 = 1, kOutBlocked = 2;

template <int OUT>
__global__ __launch_bounds__(256) void quant_act_kernel(const uint16_t* __restrict__ x, int M,
                                                        int K, int qmax, int8_t* __restrict__ qa,
                                                        float* __restrict__ sa) {
  const int64_t m = blockIdx.x;
  const int k0 = (blockIdx.y * 256 + threadIdx.x) * 8;
  if (k0 >= K) return;  // whole groups drop out together (K % 128 == 0)
  if constexpr (OUT == kOutBlocked) {
    const int64_t off = (m >> 4) * 16 * K + (k0 >> 7) * 2048 + ((k0 >> 6) & 1) * 1024 +
                        (m & 15) * 64 + (k0 & 63);
    if (m >= M) {  // a pad row of the last block (the whole workgroup)
      *reinterpret_cast<u32x2*>(qa + off) = u32x2{0u, 0u};
      return;
    }
    const u32x4 h = *reinterpret_cast<const u32x4*>(x + m * K + k0);
    float s;
    const u32x2 codes = quant8_row16(h, qmax, s);
    *reinterpret_cast<u32x2*>(qa + off) = codes;
    if ((threadIdx.x & 15) == 0) sa[(int64_t)(k0 >> 7) * M + m] = s;
    return;
  }
  const u32x4 h = *reinterpret_cast<const u32x4*>(x + m * K + k0);
  float s;
  const u32x2 codes = quant8_row16(h, qmax, s);
  if constexpr (OUT == kOutPackedA6) {
    // the partner lane is in the same group, so it is active whenever this one is
    const uint32_t p0 = (uint32_t)__shfl_xor((int)codes[0], 1);
    const uint32_t p1 = (uint32_t)__shfl_xor((int)codes[1], 1);
    if ((threadIdx.x & 1) == 0) {
      const u32x3 d = pack_codes16(codes[0], codes[1], p0, p1);
      uint32_t* dst = reinterpret_cast<uint32_t*>(qa) + 3 * ((m * K + k0) >> 4);
      dst[0] = d[0];
      dst[1] = d[1];
      dst[2] = d[2];
    }
  } else {
    *reinterpret_cast<u32x2*>(qa + m * K + k0) = codes;
  }
  if ((threadIdx.x & 15) == 0) sa[(int64_t)(k0 >> 7) * M + m] = s;  // group-major scales
}

hipError_t launch_pack_w6(const uint16_t* w, int64_t N, int64_t K, uint32_t* wp, uint16_t* sw,
                          hipStream_t stream) {
  dim3 grid((unsigned)(N / 16), (unsigned)(K / kGroup));
  return launch_kernel(pack_w6_kernel, grid, dim3(128), stream, w, (int)N, (int)K, wp, sw);
}

hipError_t launch_quant_act(const uint16_t* x, int64_t M, int64_t K, int qmax, int8_t* qa,
                            float* sa, hipStream_t stream) {
  dim3 grid((unsigned)M, (unsigned)((K + 2047) / 2048));
  return launch_kernel(quant_act_kernel<kOutBytes>, grid, dim3(256), stream, x, (int)M, (int)K,
                       qmax, qa, sa);
}

hipError_t launch_quant_act_a6_packed(const uint16_t* x, int64_t M, int64_t K, uint32_t* qp,
                                      float* sa, hipStream_t stream) {
  dim3 grid((unsigned)M, (unsigned)((K + 2047) / 2048));
  return launch_kernel(quant_act_kernel<kOutPackedA6>, grid, dim3(256), stream, x, (int)M,
                       (int)K, 31, reinterpret_cast<int8_t*>(qp), sa);
}

hipError_t launch_quant_act_blocked(const uint16_t* x, int64_t M, int64_t K, int qmax,
                                    int8_t* qb, float* sa, hipStream_t stream) {
  dim3 grid((unsigned)((M + 15) / 16 * 16), (unsigned)((K + 2047) / 2048));
  return launch_kernel(quant_act_kernel<kOutBlocked>, grid, dim3(256), stream, x, (int)M,
                       (int)K, qmax, qb, sa);
}

}  // namespace flexq
