// group_dots.hip -- the int32 group products d[m][n][g] of the FlexQ BTC section
// ("Bridging Software and Hardware with BTC": each 128-deep K group gives an exact
// integer partial product), computed with the same unpack and int8 MFMA as the
// GEMM kernels and written out for verification.
//
// One wave per (16-column tile, 16-row block, group): two v_mfma_i32_16x16x64_i8,
// whose accumulator holds 4*d (weights enter the MFMA as 4*q); d = acc >> 2 exactly.
#include "kernels.h"
#include "w6_device.h"

namespace flexq {

namespace {
constexpr uint32_t kRsrcWord3 = 0x00020000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           kRsrcWord3);
}
}  // namespace

__global__ __launch_bounds__(64) void group_dots_kernel(const int8_t* __restrict__ qa,
                                                        const uint32_t* __restrict__ wp, int M,
                                                        int N, int K, int32_t* __restrict__ dots) {
  const int G = K >> 7;
  const int lane = threadIdx.x;
  const int tile = blockIdx.x;
  const int row0 = blockIdx.y * 16;
  const int g = blockIdx.z;
  const int rows = min(16, M - row0);
  const auto ra = make_rsrc(qa + (size_t)row0 * K, (uint32_t)rows * (uint32_t)K);
  const uint32_t* wt = wp + (size_t)tile * 3 * K;
  i32x4 acc = {0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t* u = wt + (size_t)(g * 128 + j * 64 + lane) * 3;
    const i32x4 b = unpack_unit_x4(u[0], u[1], u[2]);
    const i32x4 a = __builtin_amdgcn_raw_buffer_load_b128(
        ra, (uint32_t)(lane & 15) * (uint32_t)K + (uint32_t)(g * 128 + j * 64 + (lane >> 4) * 16),
        0, 0);
    acc = mfma16(a, b, acc);
  }
  const int n = tile * 16 + (lane & 15);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * (lane >> 4) + i;
    if (r < rows) dots[((size_t)(row0 + r) * N + n) * G + g] = acc[i] >> 2;
  }
}

hipError_t launch_group_dots(const int8_t* qa, const uint32_t* wp, int64_t M, int64_t N,
                             int64_t K, int32_t* dots, hipStream_t stream) {
  dim3 grid((unsigned)(N / 16), (unsigned)((M + 15) / 16), (unsigned)(K / kGroup));
  return launch_kernel(group_dots_kernel, grid, dim3(64), stream, qa, wp, (int)M, (int)N, (int)K,
                       dots);
}

}  // namespace flexq
