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

// 6-bit activation storage: A6 codes packed 16 per 3 dwords in the weight unit
// encoding, unit (m, u = k/16) at dword 3 * (m * K/16 + u).  The quantizer gives the
// codes and scales of launch_quant_act with qmax = 31; the streaming GEMM over them
// gives the bits of launch_gemm_decode on the unpacked codes.
hipError_t launch_quant_act_a6_packed(const uint16_t* x, int64_t M, int64_t K, uint32_t* qp,
                                      float* sa, hipStream_t stream);
hipError_t launch_gemm_decode_a6p(const uint32_t* qp, const float* sa, const uint32_t* wp,
                                  const uint16_t* sw, int64_t M, int64_t N, int64_t K,
                                  uint16_t* y, hipStream_t stream);

// Activation codes in 16-row blocks, the order the streaming kernel feeds its MFMAs:
// block b = m / 16, group g, 64-deep half h, row m % 16 and byte c at
// b*16*K + g*2048 + h*1024 + (m%16)*64 + c, rows padded with zero codes to a multiple
// of 16.  The quantizer gives the codes and scales of launch_quant_act; the streaming
// GEMM over them gives the bits of launch_gemm_decode on the row-major codes.
hipError_t launch_quant_act_blocked(const uint16_t* x, int64_t M, int64_t K, int qmax,
                                    int8_t* qb, float* sa, hipStream_t stream);
hipError_t launch_gemm_decode_blocked(const int8_t* qb, const float* sa, const uint32_t* wp,
                                      const uint16_t* sw, int64_t M, int64_t N, int64_t K,
                                      uint16_t* y, hipStream_t stream);

// launch_kernel with `lds_bytes` of dynamic LDS.
template <typename... Params, typename... Args>
hipError_t launch_kernel_lds(void (*kernel)(Params...), dim3 grid, dim3 block, size_t lds_bytes,
                             hipStream_t stream, Args... args) {
  static_assert(sizeof...(Params) == sizeof...(Args), "kernel argument count");
  std::tuple<Params...> values(static_cast<Params>(args)...);
  void* ptrs[sizeof...(Params)];
  std::apply([&ptrs](auto&... v) {
    int i = 0;
    ((ptrs[i++] = static_cast<void*>(&v)), ...);
  }, values);
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, lds_bytes,
                         stream);
}

// Activation quantization fused into the decode kernel: for up to 4 token rows with
// rows * K <= 16384 each workgroup quantizes fp16 X into LDS (codes and scales
// bit-identical to launch_quant_act) and streams the weights against it, so one
// kernel does both steps.
bool fused_quant_eligible(int64_t M, int64_t N, int64_t K);
size_t fused_quant_lds_bytes(int64_t M, int64_t K);
hipError_t launch_linear_decode_fused(const uint16_t* x, int64_t M, int64_t K, int qmax,
                                      const uint32_t* wp, const uint16_t* sw, int64_t N,
                                      uint16_t* y, hipStream_t stream);

// Prefill tile shapes (rows x columns per workgroup); kTileAuto = prefill_tile(M, N).
constexpr int kTileAuto = 0, kTile256x128 = 1, kTile128x128 = 2, kTile128x64 = 3,
              kTile64x128 = 4;

// The tile the prefill kernel uses for an M x N product on the current device.
int prefill_tile(int64_t M, int64_t N);
// columns the main prefill launch covers (N unless a launch of 128 x 64 tiles takes
// the rest)
int64_t prefill_main_cols(int64_t M, int64_t N);

hipError_t launch_gemm_prefill(const int8_t* qa, const float* sa, const uint32_t* wp,
                               const uint16_t* sw, int64_t M, int64_t N, int64_t K, uint16_t* y,
                               hipStream_t stream, int tile = kTileAuto);

// Split-K prefill: the tile grid times S workgroups, slice s accumulating groups
// [s*G/S, (s+1)*G/S) (G = K/128) into fp32 plane s of part ([S][M][N]), then
// Y = fp16(sum of the planes in ascending order), the fp32 sums also into acc when
// it is not null.  tile is kTile256x128, kTile128x128, kTile128x64 or kTile64x128;
// 1 <= S <= G.
hipError_t launch_gemm_splitk(const int8_t* qa, const float* sa, const uint32_t* wp,
                              const uint16_t* sw, int64_t M, int64_t N, int64_t K, int tile,
                              int S, float* part, uint16_t* y, float* acc, hipStream_t stream);

// The tile and slice count split-K takes for an M x N x K product on the current
// device (S = 1 when splitting is not expected to pay).
void splitk_plan(int64_t M, int64_t N, int64_t K, int* tile, int* S);

// The prefill kernel with loader and MFMA waves (256 x 128 tiles) over columns
// n0 .. n0 + N - 1 of a product whose Y and s_w rows are ldn columns apart.
hipError_t launch_gemm_prefill_ws(const int8_t* qa, const float* sa, const uint32_t* wp,
                                  const uint16_t* sw, int64_t M, int64_t n0, int64_t N, int64_t K,
                                  int64_t ldn, uint16_t* y, hipStream_t stream);

hipError_t launch_group_dots(const int8_t* qa, const uint32_t* wp, int64_t M, int64_t N,
                             int64_t K, int32_t* dots, hipStream_t stream);

// Largest M the decode kernel handles in one pass (rows are processed in
// passes of this many tokens above it).
constexpr int64_t kDecodeRowsPerPass = 64;

// Compute units of the current device (cached per device).
int device_cu_count();

// The kernel the automatic path runs for an M x N product: 1 = decode, 2 = prefill.
int auto_gemm_path(int64_t M, int64_t N);

// Predicted time (us) of the weight-streaming kernel on blocked codes for an
// M x N product with G groups, 33 <= M <= 64, on `cu` compute units.
double predict_decode_us(int64_t M, int64_t N, int64_t G, int64_t cu);

}  // namespace flexq
