// kernels.h -- host-side launchers of the gfx950 kernels (internal to libflexq).
// Arguments are already validated by the C ABI layer (api.hip) when these run.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>

namespace flexq {

// Enqueue `kernel` on `stream` and return the status of this launch alone: the
// runtime's answer to hipLaunchKernel, not the thread's sticky last error (which an
// earlier failed HIP call, the caller's included, may have left behind).  The
// arguments are converted to the kernel's parameter types first.
template <typename... Params, typename... Args>
hipError_t launch_kernel(void (*kernel)(Params...), dim3 grid, dim3 block, hipStream_t stream,
                         Args... args) {
  static_assert(sizeof...(Params) == sizeof...(Args), "kernel argument count");
  std::tuple<Params...> values(static_cast<Params>(args)...);
  void* ptrs[sizeof...(Params)];
  std::apply([&ptrs](auto&... v) {
    int i = 0;
    ((ptrs[i++] = static_cast<void*>(&v)), ...);
  }, values);
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, 0, stream);
}

hipError_t launch_pack_w6(const uint16_t* w, int64_t N, int64_t K, uint32_t* wp, uint16_t* sw,
                          hipStream_t stream);

hipError_t launch_quant_act(const uint16_t* x, int64_t M, int64_t K, int qmax, int8_t* qa,
                            float* sa, hipStream_t stream);

hipError_t launch_gemm_decode(const int8_t* qa, const float* sa, const uint32_t* wp,
                              const uint16_t* sw, int64_t M, int64_t N, int64_t K, uint16_t* y,
                              hipStream_t stream);

// Prefill tile shapes (rows x columns per workgroup); kTileAuto = prefill_tile(M, N).
constexpr int kTileAuto = 0, kTile256x128 = 1, kTile128x128 = 2, kTile128x64 = 3;

// The tile the prefill kernel uses for an M x N product on the current device.
int prefill_tile(int64_t M, int64_t N);
// columns the main prefill launch covers (N unless a launch of 128 x 64 tiles takes
// the rest)
int64_t prefill_main_cols(int64_t M, int64_t N);

hipError_t launch_gemm_prefill(const int8_t* qa, const float* sa, const uint32_t* wp,
                               const uint16_t* sw, int64_t M, int64_t N, int64_t K, uint16_t* y,
                               hipStream_t stream, int tile = kTileAuto);

hipError_t launch_group_dots(const int8_t* qa, const uint32_t* wp, int64_t M, int64_t N,
                             int64_t K, int32_t* dots, hipStream_t stream);

// Largest M the decode kernel handles in one pass (rows are processed in
// passes of this many tokens above it).
constexpr int64_t kDecodeRowsPerPass = 64;

// Compute units of the current device (cached per device).
int device_cu_count();

// The kernel the automatic path runs for an M x N product: 1 = decode, 2 = prefill.
int auto_gemm_path(int64_t M, int64_t N);

}  // namespace flexq
