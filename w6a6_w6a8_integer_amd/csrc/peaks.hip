// peaks.hip -- measurements of the GPU's reachable HBM read rate and int8 MFMA rate
// (declared in include/flexq_peaks.h), reported beside the W6Ax kernels' figures.
#include "../../include/flexq_peaks.h"
#include "kernels.h"
#include "w6_device.h"

namespace flexq {

namespace {

constexpr int kReadWgsPerCu = 8;   // enough loads in flight to saturate HBM
constexpr int kMfmaWgsPerCu = 2;   // two waves per SIMD
constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void peak_read_kernel(const u32x4* __restrict__ p,
                                                             size_t n16, uint32_t* sink) {
  u32x4 s = {0u, 0u, 0u, 0u};
  const size_t stride = (size_t)gridDim.x * kThreads;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride)
    s ^= __builtin_nontemporal_load(p + i);
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

template <int V>
__global__ __launch_bounds__(kThreads, kMfmaWgsPerCu) void peak_mfma_kernel(
    int iters, uint32_t* sink, uint64_t* clock) {
  const int lane = threadIdx.x & 63;
  const i32x4 a = {lane, lane * 3, lane ^ 5, 7};
  const i32x4 b = {lane * 7, 3, lane, 1};
  i32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = c + r;
  float f[V > 0 ? V : 1];
#pragma unroll
  for (int v = 0; v < (V > 0 ? V : 1); ++v) f[v] = (float)(lane + v) * 1e-3f;
  const float x = 0.999f, y = 1e-3f;
  const uint64_t t0 = clock64(), r0 = wall_clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      acc[c] = mfma32(a, b, acc[c]);
#pragma unroll
      for (int v = 0; v < V; ++v) f[v] = fmaf(f[v], x, y);
      // one MFMA, then its V independent FMAs, in this order
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (V > 0) __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
    }
  }
  const uint64_t t1 = clock64(), r1 = wall_clock64();
  uint32_t s = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += (uint32_t)acc[c][r];
#pragma unroll
  for (int v = 0; v < (V > 0 ? V : 1); ++v) s += __float_as_uint(f[v]);
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    clock[0] = t1 - t0;
    clock[1] = r1 - r0;
  }
}

}  // namespace

}  // namespace flexq

extern "C" {

size_t flexq_peak_sink_bytes(void) {
  const size_t wgs = (size_t)flexq::device_cu_count() *
                     (size_t)(flexq::kReadWgsPerCu > flexq::kMfmaWgsPerCu
                                  ? flexq::kReadWgsPerCu : flexq::kMfmaWgsPerCu);
  return wgs * flexq::kThreads * sizeof(uint32_t);
}

int flexq_peak_hbm_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 || (reinterpret_cast<uintptr_t>(buf) & 15))
    return -1;
  const unsigned grid = (unsigned)(flexq::device_cu_count() * flexq::kReadWgsPerCu);
  const hipError_t e = flexq::launch_kernel(
      flexq::peak_read_kernel, dim3(grid), dim3(flexq::kThreads), (hipStream_t)stream,
      static_cast<const flexq::u32x4*>(buf), bytes / 16, sink);
  return e == hipSuccess ? 0 : -2;
}

int64_t flexq_peak_mfma_i8_workgroups(void) {
  return (int64_t)flexq::device_cu_count() * flexq::kMfmaWgsPerCu;
}

int flexq_peak_mfma_i8(int64_t iters, int32_t valu_per_mfma, uint32_t* sink, uint64_t* clock,
                       void* stream) {
  if (!sink || !clock || iters < 1 || iters > (1 << 24)) return -1;
  const dim3 grid((unsigned)flexq_peak_mfma_i8_workgroups()), block(flexq::kThreads);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  switch (valu_per_mfma) {
    case 0: e = flexq::launch_kernel(flexq::peak_mfma_kernel<0>, grid, block, s, (int)iters, sink, clock); break;
    case 4: e = flexq::launch_kernel(flexq::peak_mfma_kernel<4>, grid, block, s, (int)iters, sink, clock); break;
    case 8: e = flexq::launch_kernel(flexq::peak_mfma_kernel<8>, grid, block, s, (int)iters, sink, clock); break;
    case 12: e = flexq::launch_kernel(flexq::peak_mfma_kernel<12>, grid, block, s, (int)iters, sink, clock); break;
    default: return -1;
  }
  return e == hipSuccess ? 0 : -2;
}

}  // extern "C"
