// api.hip -- the C ABI of libflexq (declared in include/flexq.h).
//
// Every entry point validates its arguments on the host before any HIP call and
// returns an error without enqueuing anything; otherwise it enqueues the kernels on
// the caller's stream and returns FLEXQ_SUCCESS (or FLEXQ_ERROR_LAUNCH if the runtime
// rejected a launch).  No memory is allocated; the only global state is the
// per-device compute-unit count that the launch geometry uses (gemm_decode.hip).
#include <algorithm>
#include <atomic>

#include "../../include/flexq.h"
#include "kernels.h"

// Staging memory of flexq_linear_w6ax_noalloc (activation codes, then their scales):
// one copy of this array per GPU, held by the library until the process ends.  In
// host code `scratch` is a host-side stand-in for the symbol, not a device address;
// the address each GPU's copy has is looked up once per device (scratch_address).
static __device__ __align__(256) unsigned char scratch[FLEXQ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int64_t kGroup = FLEXQ_GROUP_SIZE;

// Size limits keep every in-kernel 32-bit buffer offset and grid dimension in range.
constexpr int64_t kMaxM = 65535LL * 16;  // 1,048,560 tokens
constexpr int64_t kMaxN = 1LL << 24;
constexpr int64_t kMaxK = 1LL << 22;

struct Range {
  uintptr_t lo, hi;
};

inline Range range_of(const void* p, uint64_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return {a, a + (uintptr_t)bytes};
}

inline bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

inline bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

inline flexq_status check_k(int64_t K, int32_t group_size) {
  if (K <= 0) return FLEXQ_ERROR_INVALID_VALUE;
  if (group_size != kGroup || K % kGroup != 0 || K > kMaxK) return FLEXQ_ERROR_UNSUPPORTED;
  return FLEXQ_SUCCESS;
}

inline flexq_status check_n(int64_t N) {
  if (N < 0) return FLEXQ_ERROR_INVALID_VALUE;
  if (N % 16 != 0 || N > kMaxN) return FLEXQ_ERROR_UNSUPPORTED;
  return FLEXQ_SUCCESS;
}

// the group-major scale arrays are addressed with 32-bit byte offsets
inline flexq_status check_scales(int64_t rows, int64_t K) {
  return rows * (K / kGroup) < (1LL << 29) ? FLEXQ_SUCCESS : FLEXQ_ERROR_UNSUPPORTED;
}

inline flexq_status check_m(int64_t M) {
  if (M < 0) return FLEXQ_ERROR_INVALID_VALUE;
  if (M > kMaxM) return FLEXQ_ERROR_UNSUPPORTED;
  return FLEXQ_SUCCESS;
}

inline flexq_status launched(hipError_t e) {
  return e == hipSuccess ? FLEXQ_SUCCESS : FLEXQ_ERROR_LAUNCH;
}

// most K slices flexq_gemm_w6ax_splitk accepts
constexpr int64_t kMaxSplits = 64;

int path_of_tile(int tile) {
  return tile == flexq::kTile256x128   ? FLEXQ_PATH_PREFILL_256X128
         : tile == flexq::kTile128x128 ? FLEXQ_PATH_PREFILL_128X128
         : tile == flexq::kTile64x128  ? FLEXQ_PATH_PREFILL_64X128
                                       : FLEXQ_PATH_PREFILL_128X64;
}

// the tile of a fixed-tile prefill path (kTileAuto for FLEXQ_PATH_PREFILL)
int tile_of_path(int path) {
  return path == FLEXQ_PATH_PREFILL_256X128   ? flexq::kTile256x128
         : path == FLEXQ_PATH_PREFILL_128X128 ? flexq::kTile128x128
         : path == FLEXQ_PATH_PREFILL_128X64  ? flexq::kTile128x64
         : path == FLEXQ_PATH_PREFILL_64X128  ? flexq::kTile64x128
                                              : flexq::kTileAuto;
}

#define FLEXQ_TRY(expr)                       \
  do {                                        \
    const flexq_status s_ = (expr);           \
    if (s_ != FLEXQ_SUCCESS) return s_;       \
  } while (0)

flexq_status validate_gemm_operands(const int8_t* q_a, const float* s_a, const uint32_t* w_packed,
                                    const uint16_t* s_w, int64_t M, int64_t N, int64_t K,
                                    const void* out, uint64_t out_bytes) {
  if (!q_a || !s_a || !w_packed || !s_w || !out) return FLEXQ_ERROR_INVALID_VALUE;
  if (!aligned(q_a, 16) || !aligned(w_packed, 16) || !aligned(s_a, 4) || !aligned(s_w, 2) ||
      !aligned(out, 4))
    return FLEXQ_ERROR_UNSUPPORTED;
  const uint64_t G = (uint64_t)(K / kGroup);
  const Range o = range_of(out, out_bytes);
  if (overlap(o, range_of(q_a, (uint64_t)M * K)) || overlap(o, range_of(s_a, (uint64_t)M * G * 4)) ||
      overlap(o, range_of(w_packed, (uint64_t)N * K * 3 / 4)) ||
      overlap(o, range_of(s_w, (uint64_t)N * G * 2)))
    return FLEXQ_ERROR_INVALID_VALUE;
  return FLEXQ_SUCCESS;
}

// Argument checks of the one-call layer apart from its workspace.
flexq_status validate_linear(const uint16_t* x_fp16, const uint32_t* w_packed,
                             const uint16_t* s_w_fp16, int64_t M, int64_t N, int64_t K,
                             int32_t group_size, int32_t abits, const uint16_t* y_fp16) {
  FLEXQ_TRY(check_m(M));
  FLEXQ_TRY(check_n(N));
  FLEXQ_TRY(check_k(K, group_size));
  FLEXQ_TRY(check_scales(M, K));
  FLEXQ_TRY(check_scales(N, K));
  if (abits != 6 && abits != 8) return FLEXQ_ERROR_INVALID_VALUE;
  if (M == 0 || N == 0) return FLEXQ_SUCCESS;
  if (!x_fp16 || !w_packed || !s_w_fp16 || !y_fp16) return FLEXQ_ERROR_INVALID_VALUE;
  if (!aligned(x_fp16, 16) || !aligned(w_packed, 16) || !aligned(s_w_fp16, 2) ||
      !aligned(y_fp16, 4))
    return FLEXQ_ERROR_UNSUPPORTED;
  const uint64_t G = (uint64_t)(K / kGroup);
  const Range ry = range_of(y_fp16, (uint64_t)M * N * 2);
  if (overlap(ry, range_of(x_fp16, (uint64_t)M * K * 2)) ||
      overlap(ry, range_of(w_packed, (uint64_t)N * K * 3 / 4)) ||
      overlap(ry, range_of(s_w_fp16, (uint64_t)N * G * 2)))
    return FLEXQ_ERROR_INVALID_VALUE;
  return FLEXQ_SUCCESS;
}

// Device address of this GPU's copy of `scratch`: looked up with the current device
// on the first call that needs it and kept per device (every GPU holds its own copy
// at its own address).  nullptr if the runtime cannot resolve it.
void* scratch_address() {
  static std::atomic<void*> addr[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return nullptr;
    addr[dev].store(p, std::memory_order_release);
  }
  return p;
}

// Bytes of the one-call layer's code area: the blocked codes of the streaming kernel
// (whole 16-row blocks) up to one 64-row pass, the row-major codes above.
size_t linear_code_bytes(int64_t M, int64_t K) {
  const int64_t rows = M <= flexq::kDecodeRowsPerPass ? (M + 15) / 16 * 16 : M;
  return ((size_t)rows * (size_t)K + 255) / 256 * 256;
}

// The one-call layer on validated arguments: quantize X into the workspace (the codes,
// then s_a at the next 256-byte boundary), then the GEMM with the automatic choice --
// the streaming kernel on codes in 16-row blocks, or the tiled kernel on row-major
// codes.
flexq_status run_linear(const uint16_t* x_fp16, const uint32_t* w_packed,
                        const uint16_t* s_w_fp16, int64_t M, int64_t N, int64_t K, int32_t abits,
                        void* workspace, uint16_t* y_fp16, hipStream_t s) {
  const int qmax = abits == 6 ? 31 : 127;
  if (flexq::fused_quant_eligible(M, N, K))   // one kernel; the workspace is not touched
    return launched(flexq::launch_linear_decode_fused(x_fp16, M, K, qmax, w_packed, s_w_fp16, N,
                                                      y_fp16, s));
  int8_t* q_a = static_cast<int8_t*>(workspace);
  float* s_a =
      reinterpret_cast<float*>(static_cast<char*>(workspace) + linear_code_bytes(M, K));
  if (flexq::auto_gemm_path(M, N) == FLEXQ_PATH_DECODE) {
    FLEXQ_TRY(launched(flexq::launch_quant_act_blocked(x_fp16, M, K, qmax, q_a, s_a, s)));
    return launched(
        flexq::launch_gemm_decode_blocked(q_a, s_a, w_packed, s_w_fp16, M, N, K, y_fp16, s));
  }
  FLEXQ_TRY(launched(flexq::launch_quant_act(x_fp16, M, K, qmax, q_a, s_a, s)));
  return launched(flexq::launch_gemm_prefill(q_a, s_a, w_packed, s_w_fp16, M, N, K, y_fp16, s));
}

}  // namespace

extern "C" {

int flexq_abi_version(void) { return FLEXQ_ABI_VERSION; }

const char* flexq_status_string(flexq_status status) {
  switch (status) {
    case FLEXQ_SUCCESS:
      return "FLEXQ_SUCCESS";
    case FLEXQ_ERROR_INVALID_VALUE:
      return "FLEXQ_ERROR_INVALID_VALUE: null pointer, negative size, bad abits or overlapping buffers";
    case FLEXQ_ERROR_UNSUPPORTED:
      return "FLEXQ_ERROR_UNSUPPORTED: group size, shape multiple, size limit or pointer alignment";
    case FLEXQ_ERROR_LAUNCH:
      return "FLEXQ_ERROR_LAUNCH: the HIP runtime rejected a kernel launch";
  }
  return "unknown flexq_status";
}

size_t flexq_packed_w6_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || K % 16 != 0) return 0;
  return (size_t)N * (size_t)K / 16 * 12;
}

flexq_status flexq_pack_w6(const uint16_t* w_fp16, int64_t N, int64_t K, int32_t group_size,
                           uint32_t* w_packed, uint16_t* s_w_fp16, void* stream) {
  FLEXQ_TRY(check_n(N));
  FLEXQ_TRY(check_k(K, group_size));
  FLEXQ_TRY(check_scales(N, K));
  if (N == 0) return FLEXQ_SUCCESS;
  if (!w_fp16 || !w_packed || !s_w_fp16) return FLEXQ_ERROR_INVALID_VALUE;
  if (!aligned(w_fp16, 16) || !aligned(w_packed, 16) || !aligned(s_w_fp16, 2))
    return FLEXQ_ERROR_UNSUPPORTED;
  const Range in = range_of(w_fp16, (uint64_t)N * K * 2);
  const Range op = range_of(w_packed, flexq_packed_w6_bytes(N, K));
  const Range os = range_of(s_w_fp16, (uint64_t)N * (K / kGroup) * 2);
  if (overlap(in, op) || overlap(in, os) || overlap(op, os)) return FLEXQ_ERROR_INVALID_VALUE;
  return launched(flexq::launch_pack_w6(w_fp16, N, K, w_packed, s_w_fp16, (hipStream_t)stream));
}

flexq_status flexq_quant_act(const uint16_t* x_fp16, int64_t M, int64_t K, int32_t group_size,
                             int32_t abits, int8_t* q_a, float* s_a, void* stream) {
  FLEXQ_TRY(check_m(M));
  FLEXQ_TRY(check_k(K, group_size));
  FLEXQ_TRY(check_scales(M, K));
  if (abits != 6 && abits != 8) return FLEXQ_ERROR_INVALID_VALUE;
  if (M == 0) return FLEXQ_SUCCESS;
  if (!x_fp16 || !q_a || !s_a) return FLEXQ_ERROR_INVALID_VALUE;
  if (!aligned(x_fp16, 16) || !aligned(q_a, 8) || !aligned(s_a, 4)) return FLEXQ_ERROR_UNSUPPORTED;
  const Range in = range_of(x_fp16, (uint64_t)M * K * 2);
  const Range oq = range_of(q_a, (uint64_t)M * K);
  const Range os = range_of(s_a, (uint64_t)M * (K / kGroup) * 4);
  if (overlap(in, oq) || overlap(in, os) || overlap(oq, os)) return FLEXQ_ERROR_INVALID_VALUE;
  return launched(flexq::launch_quant_act(x_fp16, M, K, abits == 6 ? 31 : 127, q_a, s_a,
                                          (hipStream_t)stream));
}

size_t flexq_packed_a6_bytes(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0 || K % 16 != 0) return 0;
  return (size_t)M * (size_t)K / 16 * 12;
}

flexq_status flexq_quant_act_a6_packed(const uint16_t* x_fp16, int64_t M, int64_t K,
                                       int32_t group_size, uint32_t* q_a6p, float* s_a,
                                       void* stream) {
  FLEXQ_TRY(check_m(M));
  FLEXQ_TRY(check_k(K, group_size));
  FLEXQ_TRY(check_scales(M, K));
  if (M == 0) return FLEXQ_SUCCESS;
  if (!x_fp16 || !q_a6p || !s_a) return FLEXQ_ERROR_INVALID_VALUE;
  if (!aligned(x_fp16, 16) || !aligned(q_a6p, 16) || !aligned(s_a, 4))
    return FLEXQ_ERROR_UNSUPPORTED;
  const Range in = range_of(x_fp16, (uint64_t)M * K * 2);
  const Range oq = range_of(q_a6p, flexq_packed_a6_bytes(M, K));
  const Range os = range_of(s_a, (uint64_t)M * (K / kGroup) * 4);
  if (overlap(in, oq) || overlap(in, os) || overlap(oq, os)) return FLEXQ_ERROR_INVALID_VALUE;
  return launched(
      flexq::launch_quant_act_a6_packed(x_fp16, M, K, q_a6p, s_a, (hipStream_t)stream));
}

flexq_status flexq_gemm_w6a6_packed(const uint32_t* q_a6p, const float* s_a,
                                    const uint32_t* w_packed, const uint16_t* s_w_fp16,
                                    int64_t M, int64_t N, int64_t K, int32_t group_size,
                                    uint16_t* y_fp16, void* stream) {
  FLEXQ_TRY(check_m(M));
  FLEXQ_TRY(check_n(N));
  FLEXQ_TRY(check_k(K, group_size));
  FLEXQ_TRY(check_scales(M, K));
  FLEXQ_TRY(check_scales(N, K));
  if (M == 0 || N == 0) return FLEXQ_SUCCESS;
  if (!q_a6p || !s_a || !w_packed || !s_w_fp16 || !y_fp16) return FLEXQ_ERROR_INVALID_VALUE;
  if (!aligned(q_a6p, 16) || !aligned(w_packed, 16) || !aligned(s_a, 4) ||
      !aligned(s_w_fp16, 2) || !aligned(y_fp16, 4))
    return FLEXQ_ERROR_UNSUPPORTED;
  const uint64_t G = (uint64_t)(K / kGroup);
  const Range o = range_of(y_fp16, (uint64_t)M * N * 2);
  if (overlap(o, range_of(q_a6p, flexq_packed_a6_bytes(M, K))) ||
      overlap(o, range_of(s_a, (uint64_t)M * G * 4)) ||
      overlap(o, range_of(w_packed, (uint64_t)N * K * 3 / 4)) ||
      overlap(o, range_of(s_w_fp16, (uint64_t)N * G * 2)))
    return FLEXQ_ERROR_INVALID_VALUE;
  return launched(flexq::launch_gemm_decode_a6p(q_a6p, s_a, w_packed, s_w_fp16, M, N, K, y_fp16,
                                                (hipStream_t)stream));
}

size_t flexq_blocked_act_bytes(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0 || K % kGroup != 0) return 0;
  return (size_t)((M + 15) / 16 * 16) * (size_t)K;
}

flexq_status flexq_quant_act_blocked(const uint16_t* x_fp16, int64_t M, int64_t K,
                                     int32_t group_size, int32_t abits, int8_t* q_a_blk,
                                     float* s_a, void* stream) {
  FLEXQ_TRY(check_m(M));
  FLEXQ_TRY(check_k(K, group_size));
  FLEXQ_TRY(check_scales(M, K));
  if (abits != 6 && abits != 8) return FLEXQ_ERROR_INVALID_VALUE;
  if (M == 0) return FLEXQ_SUCCESS;
  if (!x_fp16 || !q_a_blk || !s_a) return FLEXQ_ERROR_INVALID_VALUE;
  if (!aligned(x_fp16, 16) || !aligned(q_a_blk, 16) || !aligned(s_a, 4))
    return FLEXQ_ERROR_UNSUPPORTED;
  const Range in = range_of(x_fp16, (uint64_t)M * K * 2);
  const Range oq = range_of(q_a_blk, flexq_blocked_act_bytes(M, K));
  const Range os = range_of(s_a, (uint64_t)M * (K / kGroup) * 4);
  if (overlap(in, oq) || overlap(in, os) || overlap(oq, os)) return FLEXQ_ERROR_INVALID_VALUE;
  return launched(flexq::launch_quant_act_blocked(x_fp16, M, K, abits == 6 ? 31 : 127, q_a_blk,
                                                  s_a, (hipStream_t)stream));
}

flexq_status flexq_gemm_w6ax_blocked(const int8_t* q_a_blk, const float* s_a,
                                     const uint32_t* w_packed, const uint16_t* s_w_fp16,
                                     int64_t M, int64_t N, int64_t K, int32_t group_size,
                                     int32_t abits, uint16_t* y_fp16, void* stream) {
  FLEXQ_TRY(check_m(M));
  FLEXQ_TRY(check_n(N));
  FLEXQ_TRY(check_k(K, group_size));
  FLEXQ_TRY(check_scales(M, K));
  FLEXQ_TRY(check_scales(N, K));
  if (abits != 6 && abits != 8) return FLEXQ_ERROR_INVALID_VALUE;
  if (M == 0 || N == 0) return FLEXQ_SUCCESS;
  if (!q_a_blk || !s_a || !w_packed || !s_w_fp16 || !y_fp16) return FLEXQ_ERROR_INVALID_VALUE;
  if (!aligned(q_a_blk, 16) || !aligned(w_packed, 16) || !aligned(s_a, 4) ||
      !aligned(s_w_fp16, 2) || !aligned(y_fp16, 4))
    return FLEXQ_ERROR_UNSUPPORTED;
  const uint64_t G = (uint64_t)(K / kGroup);
  const Range o = range_of(y_fp16, (uint64_t)M * N * 2);
  if (overlap(o, range_of(q_a_blk, flexq_blocked_act_bytes(M, K))) ||
      overlap(o, range_of(s_a, (uint64_t)M * G * 4)) ||
      overlap(o, range_of(w_packed, (uint64_t)N * K * 3 / 4)) ||
      overlap(o, range_of(s_w_fp16, (uint64_t)N * G * 2)))
    return FLEXQ_ERROR_INVALID_VALUE;
  return launched(flexq::launch_gemm_decode_blocked(q_a_blk, s_a, w_packed, s_w_fp16, M, N, K,
                                                    y_fp16, (hipStream_t)stream));
}

flexq_status flexq_gemm_w6ax_path(const int8_t* q_a, const float* s_a, const uint32_t* w_packed,
                                  const uint16_t* s_w_fp16, int64_t M, int64_t N, int64_t K,
                                  int32_t group_size, int32_t abits, int32_t path,
                                  uint16_t* y_fp16, void* stream) {
  FLEXQ_TRY(check_m(M));
  FLEXQ_TRY(check_n(N));
  FLEXQ_TRY(check_k(K, group_size));
  FLEXQ_TRY(check_scales(M, K));
  FLEXQ_TRY(check_scales(N, K));
  if (abits != 6 && abits != 8) return FLEXQ_ERROR_INVALID_VALUE;
  if (path < FLEXQ_PATH_AUTO || path > FLEXQ_PATH_PREFILL_64X128)
    return FLEXQ_ERROR_INVALID_VALUE;
  if (M == 0 || N == 0) return FLEXQ_SUCCESS;
  FLEXQ_TRY(validate_gemm_operands(q_a, s_a, w_packed, s_w_fp16, M, N, K, y_fp16,
                                   (uint64_t)M * N * 2));
  if (path == FLEXQ_PATH_AUTO) path = flexq::auto_gemm_path(M, N);
  hipStream_t s = (hipStream_t)stream;
  if (path == FLEXQ_PATH_DECODE)
    return launched(flexq::launch_gemm_decode(q_a, s_a, w_packed, s_w_fp16, M, N, K, y_fp16, s));
  if (path == FLEXQ_PATH_PREFILL_256X128_WS)
    return launched(
        flexq::launch_gemm_prefill_ws(q_a, s_a, w_packed, s_w_fp16, M, 0, N, K, N, y_fp16, s));
  const int tile = tile_of_path(path);
  return launched(
      flexq::launch_gemm_prefill(q_a, s_a, w_packed, s_w_fp16, M, N, K, y_fp16, s, tile));
}

int flexq_gemm_w6ax_prefill_tile(int64_t M, int64_t N, int64_t K) {
  (void)K;
  if (M <= 0 || N <= 0) return FLEXQ_PATH_PREFILL_128X64;
  return path_of_tile(flexq::prefill_tile(M, N));
}

int64_t flexq_gemm_w6ax_prefill_main_cols(int64_t M, int64_t N, int64_t K) {
  (void)K;
  if (M <= 0 || N <= 0) return N > 0 ? N : 0;
  return flexq::prefill_main_cols(M, N);
}

int flexq_gemm_w6ax_auto_path(int64_t M, int64_t N, int64_t K) {
  (void)K;  // the choice depends on the token count and the layer width only
  if (M <= 0 || N <= 0) return FLEXQ_PATH_DECODE;
  return flexq::auto_gemm_path(M, N);
}

flexq_status flexq_gemm_w6ax(const int8_t* q_a, const float* s_a, const uint32_t* w_packed,
                             const uint16_t* s_w_fp16, int64_t M, int64_t N, int64_t K,
                             int32_t group_size, int32_t abits, uint16_t* y_fp16, void* stream) {
  return flexq_gemm_w6ax_path(q_a, s_a, w_packed, s_w_fp16, M, N, K, group_size, abits,
                              FLEXQ_PATH_AUTO, y_fp16, stream);
}

int32_t flexq_gemm_w6ax_splitk_plan(int64_t M, int64_t N, int64_t K, int32_t* tile_path) {
  int tile = flexq::kTile128x64, S = 1;
  if (M > 0 && N > 0 && K > 0 && K % kGroup == 0) flexq::splitk_plan(M, N, K, &tile, &S);
  if (tile_path) *tile_path = path_of_tile(tile);
  return S;
}

size_t flexq_gemm_w6ax_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t splits) {
  if (M <= 0 || N <= 0 || K <= 0 || K % kGroup != 0) return 0;
  if (splits == 0) splits = flexq_gemm_w6ax_splitk_plan(M, N, K, nullptr);
  if (splits < 1 || splits > std::min<int64_t>(K / kGroup, kMaxSplits)) return 0;
  return (size_t)splits * (size_t)M * (size_t)N * 4;
}

flexq_status flexq_gemm_w6ax_splitk(const int8_t* q_a, const float* s_a, const uint32_t* w_packed,
                                    const uint16_t* s_w_fp16, int64_t M, int64_t N, int64_t K,
                                    int32_t group_size, int32_t abits, int32_t path,
                                    int32_t splits, void* workspace, size_t workspace_bytes,
                                    uint16_t* y_fp16, float* acc_f32, void* stream) {
  FLEXQ_TRY(check_m(M));
  FLEXQ_TRY(check_n(N));
  FLEXQ_TRY(check_k(K, group_size));
  FLEXQ_TRY(check_scales(M, K));
  FLEXQ_TRY(check_scales(N, K));
  if (abits != 6 && abits != 8) return FLEXQ_ERROR_INVALID_VALUE;
  if (path != FLEXQ_PATH_PREFILL && path != FLEXQ_PATH_PREFILL_256X128 &&
      path != FLEXQ_PATH_PREFILL_128X128 && path != FLEXQ_PATH_PREFILL_128X64 &&
      path != FLEXQ_PATH_PREFILL_64X128)
    return FLEXQ_ERROR_INVALID_VALUE;
  const int64_t G = K / kGroup;
  if (splits < 0 || splits > std::min<int64_t>(G, kMaxSplits)) return FLEXQ_ERROR_INVALID_VALUE;
  if (M == 0 || N == 0) return FLEXQ_SUCCESS;
  int plan_tile = flexq::kTile128x64, plan_S = 1;
  flexq::splitk_plan(M, N, K, &plan_tile, &plan_S);
  const int S = splits == 0 ? plan_S : splits;
  const int tile = path == FLEXQ_PATH_PREFILL ? plan_tile : tile_of_path(path);
  if ((double)M * (double)N * (double)S > (double)(1LL << 40)) return FLEXQ_ERROR_UNSUPPORTED;
  const uint64_t ws = (uint64_t)S * (uint64_t)M * (uint64_t)N * 4;
  FLEXQ_TRY(validate_gemm_operands(q_a, s_a, w_packed, s_w_fp16, M, N, K, y_fp16,
                                   (uint64_t)M * N * 2));
  if (!workspace || workspace_bytes < ws) return FLEXQ_ERROR_INVALID_VALUE;
  if (!aligned(workspace, 16) || (acc_f32 && !aligned(acc_f32, 16)))
    return FLEXQ_ERROR_UNSUPPORTED;
  const Range rw = range_of(workspace, ws), ry = range_of(y_fp16, (uint64_t)M * N * 2);
  const Range inputs[4] = {range_of(q_a, (uint64_t)M * K), range_of(s_a, (uint64_t)M * G * 4),
                           range_of(w_packed, (uint64_t)N * K * 3 / 4),
                           range_of(s_w_fp16, (uint64_t)N * G * 2)};
  for (const Range& in : inputs)
    if (overlap(rw, in)) return FLEXQ_ERROR_INVALID_VALUE;
  if (overlap(rw, ry)) return FLEXQ_ERROR_INVALID_VALUE;
  if (acc_f32) {
    const Range ra = range_of(acc_f32, (uint64_t)M * N * 4);
    for (const Range& in : inputs)
      if (overlap(ra, in)) return FLEXQ_ERROR_INVALID_VALUE;
    if (overlap(ra, rw) || overlap(ra, ry)) return FLEXQ_ERROR_INVALID_VALUE;
  }
  return launched(flexq::launch_gemm_splitk(q_a, s_a, w_packed, s_w_fp16, M, N, K, tile, S,
                                            static_cast<float*>(workspace), y_fp16, acc_f32,
                                            (hipStream_t)stream));
}

size_t flexq_linear_w6ax_workspace_bytes(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0 || K % kGroup != 0) return 0;
  return linear_code_bytes(M, K) + (size_t)M * (size_t)(K / kGroup) * 4;
}

flexq_status flexq_linear_w6ax(const uint16_t* x_fp16, const uint32_t* w_packed,
                               const uint16_t* s_w_fp16, int64_t M, int64_t N, int64_t K,
                               int32_t group_size, int32_t abits, void* workspace,
                               size_t workspace_bytes, uint16_t* y_fp16, void* stream) {
  FLEXQ_TRY(validate_linear(x_fp16, w_packed, s_w_fp16, M, N, K, group_size, abits, y_fp16));
  if (M == 0 || N == 0) return FLEXQ_SUCCESS;
  const size_t ws = flexq_linear_w6ax_workspace_bytes(M, K);
  if (!workspace || workspace_bytes < ws) return FLEXQ_ERROR_INVALID_VALUE;
  if (!aligned(workspace, 16)) return FLEXQ_ERROR_UNSUPPORTED;
  const uint64_t G = (uint64_t)(K / kGroup);
  const Range rk = range_of(workspace, ws);
  if (overlap(rk, range_of(x_fp16, (uint64_t)M * K * 2)) ||
      overlap(rk, range_of(w_packed, (uint64_t)N * K * 3 / 4)) ||
      overlap(rk, range_of(s_w_fp16, (uint64_t)N * G * 2)) ||
      overlap(rk, range_of(y_fp16, (uint64_t)M * N * 2)))
    return FLEXQ_ERROR_INVALID_VALUE;
  return run_linear(x_fp16, w_packed, s_w_fp16, M, N, K, abits, workspace, y_fp16,
                    (hipStream_t)stream);
}

flexq_status flexq_linear_w6ax_noalloc(const uint16_t* x_fp16, const uint32_t* w_packed,
                                       const uint16_t* s_w_fp16, int64_t M, int64_t N, int64_t K,
                                       int32_t group_size, int32_t abits, uint16_t* y_fp16,
                                       void* stream) {
  FLEXQ_TRY(validate_linear(x_fp16, w_packed, s_w_fp16, M, N, K, group_size, abits, y_fp16));
  if (M == 0 || N == 0) return FLEXQ_SUCCESS;
  if (flexq_linear_w6ax_workspace_bytes(M, K) > (size_t)FLEXQ_NOALLOC_SCRATCH_BYTES)
    return FLEXQ_ERROR_UNSUPPORTED;
  void* ws = scratch_address();
  if (ws == nullptr) return FLEXQ_ERROR_LAUNCH;
  // the quantizer writes every byte of q_a and s_a that the GEMM reads, so nothing
  // left in the array by an earlier call is ever used
  return run_linear(x_fp16, w_packed, s_w_fp16, M, N, K, abits, ws, y_fp16, (hipStream_t)stream);
}

flexq_status flexq_gemm_w6ax_group_dots(const int8_t* q_a, const uint32_t* w_packed, int64_t M,
                                        int64_t N, int64_t K, int32_t group_size, int32_t* dots,
                                        void* stream) {
  FLEXQ_TRY(check_m(M));
  FLEXQ_TRY(check_n(N));
  FLEXQ_TRY(check_k(K, group_size));
  if (M == 0 || N == 0) return FLEXQ_SUCCESS;
  if (!q_a || !w_packed || !dots) return FLEXQ_ERROR_INVALID_VALUE;
  if (!aligned(q_a, 16) || !aligned(w_packed, 16) || !aligned(dots, 4))
    return FLEXQ_ERROR_UNSUPPORTED;
  const Range o = range_of(dots, (uint64_t)M * N * (K / kGroup) * 4);
  if (overlap(o, range_of(q_a, (uint64_t)M * K)) ||
      overlap(o, range_of(w_packed, (uint64_t)N * K * 3 / 4)))
    return FLEXQ_ERROR_INVALID_VALUE;
  return launched(flexq::launch_group_dots(q_a, w_packed, M, N, K, dots, (hipStream_t)stream));
}

}  // extern "C"
