// gemm_prefill_ws.hip -- W6Ax GEMM for many tokens with loader and MFMA waves.
//
// FlexQ blog "Meet FlexQ: A Six-Bit Quantization Breakthrough", section "Bridging
// Software and Hardware with BTC": 128-deep K groups, an exact integer product per
// group, operand tiles staged in shared memory, the dequantization fused into the
// GEMM.  Arithmetic is the same as gemm_prefill.hip, bit for bit: the first MFMA of
// a group starts from the bits of 1.5 * 2^23 so the int32 result is the float
// F = 12582912 + 4d exactly; t = fma(F, s_w / 4, -12582912 * s_w / 4) = RN32(d * s_w);
// acc = fma(t, s_a, acc) over ascending groups.
//
// A 256 x 128 output tile per workgroup of 8 waves, one of each kind per SIMD:
//
//   * MFMA waves 0-3 each own 128 rows x 64 columns: 4 x 2 tiles of 32 x 32, each
//     tile one chain of 4 v_mfma_i32_32x32x32_i8 per group.  While chain j runs, the
//     VALU rescales chain j - 1 (two FMAs per output: 8 per MFMA); the last chain of
//     a group is rescaled during the first chain of the next.  These waves touch
//     only LDS: A fragments (one row tile at a time), B fragments (both column tiles
//     for the whole group), the packed activation-scale register of the row tile
//     (lane 16j + r holds the scale of output register r, applied with a DPP
//     row_newbcast FMA) and s_w / 4 per column.
//   * Loader waves 4-7 do every global load: the activation tile and its scales go
//     global -> LDS by buffer_load ... lds (no registers), the packed weights and
//     their scales come through registers, two groups ahead, and are unpacked into
//     the fragment-linear B stage one group ahead.
//
// A 3-stage LDS ring per 128-deep group: in iteration g the MFMA waves read stage
// g % 3 while the loaders complete stage (g + 1) % 3 (unpacked weights, landing
// copies) and start the copies of group g + 2 into stage (g + 2) % 3, which the MFMA
// waves left at the previous barrier.  One s_barrier per group.
#include <utility>

#include "kernels.h"
#include "w6_device.h"

namespace flexq {

namespace {

constexpr uint32_t kWsRsrcWord3 = 0x00020000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t ws_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           kWsRsrcWord3);
}

typedef __attribute__((address_space(3))) void* ws_lds_ptr_t;

// s_waitcnt vmcnt(n) lgkmcnt(0) (gfx9 encoding)
template <int N>
__device__ __forceinline__ void ws_wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

__device__ __forceinline__ void ws_barrier() { asm volatile("s_barrier" ::: "memory"); }

// acc += S' * t with S' = lane R of this lane's 16-lane row of S (DPP row_newbcast);
// S is written only by LDS loads, so no VALU-to-DPP wait states are needed.
template <int R>
__device__ __forceinline__ void ws_fmac_bcast(float& acc, float S, float t) {
  asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
      : "+v"(acc)
      : "v"(S), "v"(t), "i"(R));
}

// Outputs R0 .. R0 + 3 of one 32 x 32 tile: t = RN(d * s_w) from F = 12582912 + 4d,
// then acc = RN(t * s_a + acc).
template <int R0>
__device__ __forceinline__ void ws_rescale4(float (&a)[16], const f32x16& F, float s4,
                                            float bias, float S) {
  const float t0 = fmaf(F[R0 + 0], s4, bias);
  const float t1 = fmaf(F[R0 + 1], s4, bias);
  const float t2 = fmaf(F[R0 + 2], s4, bias);
  const float t3 = fmaf(F[R0 + 3], s4, bias);
  ws_fmac_bcast<R0 + 0>(a[R0 + 0], S, t0);
  ws_fmac_bcast<R0 + 1>(a[R0 + 1], S, t1);
  ws_fmac_bcast<R0 + 2>(a[R0 + 2], S, t2);
  ws_fmac_bcast<R0 + 3>(a[R0 + 3], S, t3);
}

constexpr int WS_BM = 256, WS_BN = 128;
constexpr int WS_STAGES = 3;
constexpr int WS_A_BYTES = WS_BM * kGroup;              // 32 KB activation tile
constexpr int WS_B_BYTES = WS_BN * kGroup;              // 16 KB unpacked weight tile
constexpr int WS_SA_OFF = WS_A_BYTES + WS_B_BYTES;      // 256 fp32 activation scales
constexpr int WS_S4_OFF = WS_SA_OFF + WS_BM * 4;        // 128 fp32 s_w / 4
constexpr int WS_STAGE = WS_S4_OFF + WS_BN * 4;         // 50688 bytes
constexpr int WS_RT = 4, WS_CT = 2;                     // 32 x 32 tiles per MFMA wave
constexpr int WS_OUT_PITCH = 144;                       // staged output row: 128 B + pad
// vector-memory instructions a loader issues per group: 8 activation copies, one
// activation-scale copy, 4 weight loads, and for loaders 0 and 1 one weight-scale load
constexpr int WS_LD_OPS_SW = 14, WS_LD_OPS = 13;

}  // namespace

__global__ __launch_bounds__(512, 1) void gemm_prefill_ws_kernel(
    const int8_t* __restrict__ qa, const float* __restrict__ sa, const uint32_t* __restrict__ wp,
    const uint16_t* __restrict__ sw, int M, int N, int K, int ldn, int GM,
    uint16_t* __restrict__ y) {
  static_assert(WS_STAGES * WS_STAGE <= 160 * 1024, "LDS ring");
  static_assert(4 * 128 * WS_OUT_PITCH <= WS_STAGES * WS_STAGE, "output staging fits");
  const int G = K >> 7;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // ---- logical tile from the workgroup id (XCD-contiguous, row-band order)
  const int nbm = (M + WS_BM - 1) / WS_BM, nbn = (N + WS_BN - 1) / WS_BN;
  const int total = nbm * nbn;
  int pid = blockIdx.x;
  if ((total & 7) == 0) pid = (pid & 7) * (total >> 3) + (pid >> 3);
  const int band = GM * nbn;
  const int first_m = (pid / band) * GM;
  const int gm = min(GM, nbm - first_m);
  const int in_band = pid - (pid / band) * band;
  const int bm = first_m + in_band % gm;
  const int bn = in_band / gm;
  const int m0 = bm * WS_BM, n0 = bn * WS_BN;
  const int mrows = min(WS_BM, M - m0);
  const int ncols = min(WS_BN, N - n0);

  __shared__ __attribute__((aligned(1024))) int8_t lds[WS_STAGES * WS_STAGE];
  const int glast = G - 1;

  if (wave >= 4) {
    // =========================== loader waves ===========================
    const int l = wave - 4;
    // Out-of-range loads return zero: rows >= M and columns >= N vanish.
    const auto ra = ws_rsrc(qa + (size_t)m0 * K, (uint32_t)mrows * (uint32_t)K);
    const auto rw = ws_rsrc(wp + (size_t)(n0 / 16) * 3 * K, (uint32_t)(ncols / 16) * 12u * K);
    const auto rsa = ws_rsrc(sa + m0, (uint32_t)((size_t)G * M - m0) * 4u);
    const auto rsw = ws_rsrc(sw + n0, (uint32_t)((size_t)(G - 1) * ldn + N - n0) * 2u);
    // Activation tile: row-major, 128 B per row, the 16-byte chunk j of row r stored
    // at chunk j ^ ((r >> 1) & 7).  Copy i of loader l moves rows R0 = (8l + i) * 8 ..
    // R0 + 7: lane t takes physical chunk t % 8 of row R0 + t / 8, i.e. logical chunk
    // (t % 8) ^ (4 * (i % 2) + t / 16).  The row part of the offset stays in the VGPR
    // operand (the range check zeroes rows >= M); the group's column offset goes in the
    // scalar offset.
    uint32_t a_voff[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      a_voff[i] = (uint32_t)((8 * l + i) * 8 + (lane >> 3)) * (uint32_t)K +
                  (uint32_t)(((lane & 7) ^ (4 * (i & 1) + (lane >> 4))) * 16);
    const uint32_t sa_voff = (uint32_t)(64 * l + lane) * 4u;
    // Weights: loader l takes 16-column tiles 2l and 2l + 1 of the group (1536
    // contiguous bytes each, unit slot j = u * 16 + n % 16); load i reads slot
    // (i % 2) * 64 + lane of tile 2l + i / 2 (768 contiguous bytes per instruction).
    uint32_t b_voff[4];
    int b_lds[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 2 * l + (i >> 1);
      b_voff[i] = (uint32_t)t * 12u * (uint32_t)K + (uint32_t)((i & 1) * 64 + lane) * 12u;
      const int u = (i & 1) * 4 + (lane >> 4);          // unit in the group (16 codes)
      const int n = 16 * t + (lane & 15);               // column in the tile
      // fragment-linear B: block (chunk u / 2, column tile n / 32), lane (n % 32) + 32 (u % 2)
      b_lds[i] = WS_A_BYTES + (((u >> 1) * (WS_BN / 32) + (n >> 5)) * 64 + (n & 31) + 32 * (u & 1)) * 16;
    }
    const bool sw_loader = l < 2;
    const uint32_t sw_voff = (uint32_t)(64 * l + lane) * 2u;

    u32x3 breg[2][4];
    uint32_t sreg[2] = {0u, 0u};
    auto issue = [&](int g, int so, u32x3 (&b)[4], uint32_t& s) {
      int8_t* la = lds + so;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (ws_lds_ptr_t)(la + (8 * l + i) * 1024), 16,
                                                 a_voff[i], (uint32_t)g * 128u, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (ws_lds_ptr_t)(la + WS_SA_OFF + 256 * l), 4,
                                               sa_voff + (uint32_t)g * (uint32_t)M * 4u, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        b[i] = __builtin_amdgcn_raw_buffer_load_b96(rw, b_voff[i] + (uint32_t)g * 1536u, 0, 0);
      if (sw_loader)
        s = __builtin_amdgcn_raw_buffer_load_b16(rsw, sw_voff + (uint32_t)g * (uint32_t)ldn * 2u,
                                                 0, 0);
      asm volatile("" ::: "memory");  // no load of this group moves past what follows
    };
    auto fill = [&](int so, const u32x3 (&b)[4], uint32_t s) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<i32x4*>(lds + so + b_lds[i]) = unpack_unit_x4(b[i][0], b[i][1], b[i][2]);
      if (sw_loader)
        *reinterpret_cast<float*>(lds + so + WS_S4_OFF + (64 * l + lane) * 4) =
            0.25f * half_bits_to_float((uint16_t)s);   // exact
    };
    // everything but the group just issued has landed (loads complete in order)
    auto wait_prev = [&]() {
      __builtin_amdgcn_sched_barrier(0);
      if (sw_loader)
        ws_wait_vm_lgkm0<WS_LD_OPS_SW>();
      else
        ws_wait_vm_lgkm0<WS_LD_OPS>();
      __builtin_amdgcn_sched_barrier(0);
    };
    // prologue: groups 0 and 1 issued, group 0 staged.  Past the last group the last
    // group is read again into stages that are never read (no branch in the loop).
    issue(0, 0, breg[0], sreg[0]);
    issue(min(1, glast), WS_STAGE, breg[1], sreg[1]);
    ws_wait_vm_lgkm0<0>();
    fill(0, breg[0], sreg[0]);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    ws_barrier();
    // iteration g: copies of group g + 2 into stage (g + 2) % 3 (left by the MFMA
    // waves at the last barrier), then group g + 1 completed in stage (g + 1) % 3.
    int so0 = 0, so1 = WS_STAGE, so2 = 2 * WS_STAGE;
    for (int g = 0; g < G; g += 2) {
      issue(min(g + 2, glast), so2, breg[0], sreg[0]);
      wait_prev();
      fill(so1, breg[1], sreg[1]);
      __builtin_amdgcn_s_waitcnt(0xC07F);
      ws_barrier();
      if (g + 1 >= G) break;
      issue(min(g + 3, glast), so0, breg[1], sreg[1]);
      wait_prev();
      fill(so2, breg[0], sreg[0]);
      __builtin_amdgcn_s_waitcnt(0xC07F);
      ws_barrier();
      // two groups move the ring by two stages
      const int t = so0;
      so0 = so2;
      so2 = so1;
      so1 = t;
    }
    ws_wait_vm_lgkm0<0>();  // no copy into LDS may outlive the workgroup
    ws_barrier();           // the MFMA waves' epilogue barrier
    return;
  }

  // ============================== MFMA waves ==============================
  const int wm = wave & 1, wn = wave >> 1;   // rows wm*128.., columns wn*64..
  const int r32 = lane & 31, hl = lane >> 5;
  // A fragment (row tile rt, k-chunk c): row wm*128 + rt*32 + r32, logical chunk
  // 2c + hl; the swizzle (row >> 1) & 7 does not depend on rt, so row tile rt is the
  // row tile 0 offset + rt * 4096
  int a_off[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int row = wm * 128 + r32;
    a_off[c] = row * 128 + (((2 * c + hl) ^ ((row >> 1) & 7)) * 16);
  }
  // B fragment (column tile ct, chunk c): fragment-linear block c * 4 + 2wn + ct
  const int b_off = WS_A_BYTES + (2 * wn) * 1024 + lane * 16;
  // this lane's s_a in the packed scale register of row tile rt (+128 rt)
  const int sa_off =
      WS_SA_OFF + (wm * 128 + 8 * ((lane >> 2) & 3) + 4 * hl + (lane & 3)) * 4;
  const int s4_off = WS_S4_OFF + (wn * 64 + r32) * 4;

  auto ldA = [&](int so, int rt, int c) {
    return *reinterpret_cast<const i32x4*>(lds + so + a_off[c] + rt * 4096);
  };
  auto ldB = [&](int so, int ct, int c) {
    return *reinterpret_cast<const i32x4*>(lds + so + b_off + c * 4096 + ct * 1024);
  };
  auto ldS = [&](int so, int rt) {
    return *reinterpret_cast<const float*>(lds + so + sa_off + rt * 128);
  };
  auto ldS4 = [&](int so, int ct) {
    return *reinterpret_cast<const float*>(lds + so + s4_off + ct * 128);
  };

  float acc[WS_RT][WS_CT][16];
#pragma unroll
  for (int a = 0; a < WS_RT; ++a)
#pragma unroll
    for (int b = 0; b < WS_CT; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;
  i32x16 magic;
#pragma unroll
  for (int r = 0; r < 16; ++r) magic[r] = (int32_t)kMagic;

  // MFMA results of the running and the previous chain.  When a group ends d[1] holds
  // its last chain (row tile 3, column tile 1), rescaled during the next group's
  // first chain with the scales kept below; the starting values make that first
  // deferred rescale add exactly +0 to a zero accumulator.
  i32x16 d[2] = {magic, magic};
  float s4last = 0.0f, blast = -0.0f, Slast = 0.0f;

  ws_barrier();  // group 0 staged
  int so = 0;
  for (int g = 0; g < G; ++g) {
    // this group's B fragments (both column tiles), scales and row tile 0
    // (first what chain 0 needs, so its first MFMA waits only for those reads)
    i32x4 b[WS_CT][4], a[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      a[c] = ldA(so, 0, c);
      b[0][c] = ldB(so, 0, c);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) b[1][c] = ldB(so, 1, c);
    float s4[WS_CT], bias[WS_CT], S[2];
#pragma unroll
    for (int ct = 0; ct < WS_CT; ++ct) s4[ct] = ldS4(so, ct);
    S[0] = ldS(so, 0);
    // chains j = 0 .. 7: (rt, ct) = (j / 2, j % 2); while chain j runs, chain j - 1
    // is rescaled (chain -1 = the previous group's last chain).  During a row tile's
    // second chain each A fragment, once its last MFMA is issued, is reloaded with the
    // next row tile's.
    unroll([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      constexpr int rt = j / 2, ct = j % 2;
      if constexpr (ct == 1 && rt + 1 < WS_RT) S[(rt + 1) & 1] = ldS(so, rt + 1);
      unroll([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        d[j & 1] = mfma32(a[c], b[ct][c], c == 0 ? magic : d[j & 1]);
        if constexpr (ct == 1 && rt + 1 < WS_RT) a[c] = ldA(so, rt + 1, c);
        // four of the sixteen outputs of the previous chain per MFMA
        if constexpr (j == 0) {
          // (d[1] is overwritten only by chain 1, after this rescale)
          ws_rescale4<4 * c>(acc[WS_RT - 1][WS_CT - 1], __builtin_bit_cast(f32x16, d[1]),
                             s4last, blast, Slast);
          if constexpr (c == 3) {  // needed from chain 1 on
#pragma unroll
            for (int t = 0; t < WS_CT; ++t) bias[t] = -kMagicF * s4[t];
          }
        } else {
          constexpr int pj = j - 1, prt = pj / 2, pct = pj % 2;
          ws_rescale4<4 * c>(acc[prt][pct], __builtin_bit_cast(f32x16, d[pj & 1]), s4[pct],
                             bias[pct], S[prt & 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }, std::make_integer_sequence<int, 4>{});
    }, std::make_integer_sequence<int, WS_RT * WS_CT>{});
    s4last = s4[WS_CT - 1];
    blast = bias[WS_CT - 1];
    Slast = S[(WS_RT - 1) & 1];
    __builtin_amdgcn_s_waitcnt(0xC07F);  // this stage's reads done before it is refilled
    ws_barrier();
    so = so == 2 * WS_STAGE ? 0 : so + WS_STAGE;
  }
  {
    const f32x16 F = __builtin_bit_cast(f32x16, d[1]);
    unroll([&](auto qc) {
      constexpr int q = decltype(qc)::value;
      ws_rescale4<4 * q>(acc[WS_RT - 1][WS_CT - 1], F, s4last, blast, Slast);
    }, std::make_integer_sequence<int, 4>{});
  }

  // Epilogue.  With a 16-byte aligned Y each MFMA wave stages its 128 x 64 fp16 outputs
  // in LDS (its own region, row pitch WS_OUT_PITCH) and stores 16-byte row chunks; the
  // barrier keeps the stages' last copies and reads out of the way.
  ws_barrier();
  if ((reinterpret_cast<uintptr_t>(y) & 15u) == 0) {
    uint8_t* tw = reinterpret_cast<uint8_t*>(lds) + wave * 128 * WS_OUT_PITCH;
#pragma unroll
    for (int rt = 0; rt < WS_RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < WS_CT; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = rt * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          *reinterpret_cast<uint16_t*>(tw + lr * WS_OUT_PITCH + (ct * 32 + r32) * 2) =
              float_to_half_bits(acc[rt][ct][r]);
        }
    __builtin_amdgcn_wave_barrier();
    // 128 rows x 8 chunks of 16 bytes: lane takes chunk lane % 8 of rows 8i + lane / 8
    const int col = wn * 64 + (lane & 7) * 8;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int lr = i * 8 + (lane >> 3);
      const i32x4 v = *reinterpret_cast<const i32x4*>(tw + lr * WS_OUT_PITCH + (lane & 7) * 16);
      const int row = wm * 128 + lr;
      if (row < mrows && col < ncols)
        *reinterpret_cast<i32x4*>(y + (size_t)(m0 + row) * ldn + n0 + col) = v;
    }
    return;
  }
#pragma unroll
  for (int rt = 0; rt < WS_RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < WS_CT; ++ct) {
      const int col = wn * 64 + ct * 32 + r32;
      if (col < ncols) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * 128 + rt * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (row < mrows)
            y[(size_t)(m0 + row) * ldn + n0 + col] = float_to_half_bits(acc[rt][ct][r]);
        }
      }
    }
}

hipError_t launch_gemm_prefill_ws(const int8_t* qa, const float* sa, const uint32_t* wp,
                                  const uint16_t* sw, int64_t M, int64_t n0, int64_t N, int64_t K,
                                  int64_t ldn, uint16_t* y, hipStream_t stream) {
  const int64_t nbm = (M + WS_BM - 1) / WS_BM, nbn = (N + WS_BN - 1) / WS_BN;
  return launch_kernel(gemm_prefill_ws_kernel, dim3((unsigned)(nbm * nbn)), dim3(512), stream,
                       qa, sa, wp + (n0 / 16) * 3 * K, sw + n0, (int)M, (int)N, (int)K, (int)ldn, 4,
                       y + n0);
}

}  // namespace flexq
