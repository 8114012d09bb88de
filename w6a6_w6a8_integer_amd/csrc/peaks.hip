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

// acc += S' * t with S' = lane R of the caller's 16-lane DPP row of S (the prefill
// kernel's form of the rescale's second FMA)
template <int R>
__device__ __forceinline__ void fmac_row_bcast(float& acc, float S, float t) {
  asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
      : "+v"(acc)
      : "v"(S), "v"(t), "i"(R));
}

constexpr int kRescaleThreads = 512;  // one workgroup per CU, two waves per SIMD

// The loop the exact group rescale puts a lower bound on: per wave and 128-deep group,
// four 32 x 32 output tiles, each a chain of four int8 MFMAs started from the bits of
// 1.5 * 2^23; while a tile's chain runs, the previous tile's 16 results per lane are
// rescaled (t = fma(F, s/4, bias), then acc += S' * t with the DPP row broadcast: 8
// VALU per MFMA), one 16-byte LDS read per MFMA supplies an operand two MFMAs later,
// and the workgroup meets at one barrier per group.  No global memory, no unpack: the
// prefill kernel's instruction mix minus its loads.
__global__ __launch_bounds__(kRescaleThreads, 1) void peak_rescale_kernel(int iters, uint32_t* sink,
                                                                         uint64_t* clock) {
  __shared__ i32x4 lds[1024];
  const int lane = threadIdx.x & 63, tid = threadIdx.x;
  for (int i = tid; i < 1024; i += kRescaleThreads) lds[i] = i32x4{i, i * 3, i ^ 7, 1};
  __syncthreads();
  i32x4 a[4], b[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    a[k] = i32x4{lane + k, lane * 3, lane ^ 5, 7};
    b[k] = i32x4{lane * 7, 3 + k, lane, 1};
  }
  i32x16 magic;
#pragma unroll
  for (int r = 0; r < 16; ++r) magic[r] = (int32_t)kMagic;
  float acc[4][16];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
  const float S = 1.0f + lane * 1e-6f;
  const float s4 = 0.25f * (1.0f + lane * 1e-5f), bias = -kMagicF * s4;
  i32x16 dd[2] = {magic, magic};
  const uint64_t t0 = clock64(), r0 = wall_clock64();
  int lo = tid;
  for (int it = 0; it < iters; ++it) {
    unroll([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const f32x16 Fp = __builtin_bit_cast(f32x16, dd[(j + 1) & 1]);
      i32x16& d = dd[j & 1];
#pragma unroll
      for (int k = 0; k < 4; ++k) asm volatile("" : "+v"(a[k]));  // no reuse across tiles
      unroll([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        a[(k + 2) & 3] = lds[(lo + 64 * k) & 1023];
        d = mfma32(a[k], b[k], k == 0 ? magic : d);
        unroll([&](auto rc) {
          constexpr int r = 4 * k + decltype(rc)::value;
          fmac_row_bcast<r>(acc[(j + 3) & 3][r], S, fmaf(Fp[r], s4, bias));
        }, std::make_integer_sequence<int, 4>{});
        __builtin_amdgcn_sched_barrier(0);
      }, std::make_integer_sequence<int, 4>{});
    }, std::make_integer_sequence<int, 4>{});
    lo += 17;
    __builtin_amdgcn_s_barrier();
  }
  const uint64_t t1 = clock64(), r1 = wall_clock64();
  uint32_t s = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += __float_as_uint(acc[j][r]) + (uint32_t)dd[j & 1][r];
  sink[(size_t)blockIdx.x * kRescaleThreads + tid] = s;
  if (blockIdx.x == 0 && tid == 0) {
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

int64_t flexq_peak_mfma_i8_rescale_waves(void) {
  return (int64_t)flexq::device_cu_count() * (flexq::kRescaleThreads / 64);
}

int flexq_peak_mfma_i8_rescale(int64_t iters, uint32_t* sink, uint64_t* clock, void* stream) {
  if (!sink || !clock || iters < 1 || iters > (1 << 24)) return -1;
  const hipError_t e = flexq::launch_kernel(
      flexq::peak_rescale_kernel, dim3((unsigned)flexq::device_cu_count()),
      dim3(flexq::kRescaleThreads), (hipStream_t)stream, (int)iters, sink, clock);
  return e == hipSuccess ? 0 : -2;
}

}  // extern "C"
