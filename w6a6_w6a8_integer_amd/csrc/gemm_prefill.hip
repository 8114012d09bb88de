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
// Tile: BM x 128 per workgroup, BM/64 x 2 waves, each wave 64 x 64 = 2 x 2 MFMA
// tiles of 32 x 32, handled as two halves (row tile 0, row tile 1).  The 2 fp32
// FMAs of the rescale equal the MFMA time of a group at the chip's rates, so the
// loop is software-pipelined: the MFMAs of one half run while the VALU rescales the
// other half (the previous group's second half, then this group's first half).
//
// Staging: a 3-deep LDS ring per group holds the int8 activation tile, the
// unpacked weight tile (bytes 4*q) and both scale vectors, all in
// "fragment-linear" order: every 1 KB block is one 32 x 32 MFMA operand with lane
// l's 16 bytes at offset 16*l, so fills and fragment reads are linear 16-byte
// accesses.  Activations and activation scales go global -> LDS directly
// (buffer_load ... lds, no registers); packed weights and weight scales come
// through registers (two sets) and are unpacked into the ring.  Loads run two
// groups ahead; one barrier per group, with the counter waits written out so the
// loads of group g+2 stay in flight across it.
//
// Workgroups are numbered so that the 8 XCDs each take a contiguous run of
// logical tiles (hardware hands workgroup i to XCD i % 8), and logical tiles run
// over a band of GM row blocks before moving to the next column block.
#include "kernels.h"
#include "w6_device.h"

namespace flexq {

namespace {

constexpr uint32_t kRsrcWord3 = 0x00020000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           kRsrcWord3);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int BN = 128;
constexpr int STAGES = 3;
constexpr uint32_t kMagic = 0x4B400000u;
constexpr float kMagicF = 12582912.0f;

// s_waitcnt vmcnt(n) lgkmcnt(0) (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8],
// vmcnt[5:4] in [15:14]).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

}  // namespace

template <int BM>
struct PrefillCfg {
  static constexpr int THREADS = BM * 2;
  static constexpr int WAVES = THREADS / 64;
  static constexpr int RB = BM / 32;                 // 32-row blocks
  static constexpr int A_BYTES = BM * kGroup;        // activation stage
  static constexpr int B_BYTES = BN * kGroup;        // unpacked weight stage
  static constexpr int A_BLOCKS = A_BYTES / 1024;    // 1 KB fragment blocks
  static constexpr int A_BLOCKS_PER_WAVE = A_BLOCKS / WAVES;  // 4
  static constexpr int B_UNITS = BN * 8 / THREADS;   // packed units per thread
  static constexpr int SA_WAVES = BM / 64;           // waves that copy s_a
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES + BM * 4 + BN * 4;
  // global -> LDS copies a wave issues per group (activation blocks + one scale row)
  static constexpr int DMA_OPS = A_BLOCKS_PER_WAVE + 1;
};

template <int BM>
__global__ __launch_bounds__(BM * 2, 512 / (BM * 2)) void gemm_prefill_kernel(
    const int8_t* __restrict__ qa, const float* __restrict__ sa, const uint32_t* __restrict__ wp,
    const uint16_t* __restrict__ sw, int M, int N, int K, int GM, uint16_t* __restrict__ y) {
  using C = PrefillCfg<BM>;
  static_assert(C::A_BLOCKS_PER_WAVE == 4, "tile/thread mismatch");
  static_assert(C::B_UNITS * C::THREADS == BN * 8, "B split");

  const int G = K >> 7;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % (BM / 64), wn = wave / (BM / 64);

  // ---- logical tile from the workgroup id (XCD-contiguous, row-band order)
  const int nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN;
  const int total = nbm * nbn;
  int pid = blockIdx.x;
  if ((total & 7) == 0) pid = (pid & 7) * (total >> 3) + (pid >> 3);
  const int band = GM * nbn;
  const int first_m = (pid / band) * GM;
  const int gm = min(GM, nbm - first_m);
  const int in_band = pid - (pid / band) * band;
  const int bm = first_m + in_band % gm;
  const int bn = in_band / gm;
  const int m0 = bm * BM, n0 = bn * BN;
  const int mrows = min(BM, M - m0);
  const int ncols = min(BN, N - n0);

  __shared__ __attribute__((aligned(1024))) int8_t lds[STAGES * C::STAGE_BYTES];
  auto stage_a = [&](int s) { return lds + s * C::STAGE_BYTES; };
  auto stage_b = [&](int s) { return lds + s * C::STAGE_BYTES + C::A_BYTES; };
  auto stage_sa = [&](int s) {
    return reinterpret_cast<float*>(lds + s * C::STAGE_BYTES + C::A_BYTES + C::B_BYTES);
  };
  auto stage_s4 = [&](int s) {
    return reinterpret_cast<float*>(lds + s * C::STAGE_BYTES + C::A_BYTES + C::B_BYTES + BM * 4);
  };

  // Out-of-range loads return zero: rows >= M and columns >= N vanish.
  const auto ra = make_rsrc(qa + (size_t)m0 * K, (uint32_t)mrows * (uint32_t)K);
  const auto rw = make_rsrc(wp + (size_t)(n0 / 16) * 3 * K, (uint32_t)(ncols / 16) * 12u * K);
  // scales are group-major: s_a[g][m] at g*M + m, s_w[g][n] at g*N + n
  const auto rsa = make_rsrc(sa + m0, (uint32_t)((size_t)G * M - m0) * 4u);
  const auto rsw = make_rsrc(sw + n0, (uint32_t)((size_t)G * N - n0) * 2u);

  // A stage: row-major, 128 bytes per row, the 16-byte chunk j of row r stored at
  // chunk j ^ ((r >> 1) & 7) (so the 32x32 fragment reads below touch every bank
  // once per 16 lanes).  The copy into it is coalesced: DMA instruction i of wave w
  // moves rows R0 = (4w + i) * 8 .. R0 + 7, lane l taking physical chunk l % 8 of row
  // R0 + l / 8, i.e. logical chunk (l % 8) ^ (4 * (i % 2) + l / 16).
  const uint32_t a_vrow = (uint32_t)(wave * 32 + (lane >> 3)) * (uint32_t)K;
  const uint32_t a_voff0 = a_vrow + (uint32_t)(((lane & 7) ^ (lane >> 4)) * 16);
  const uint32_t a_voff1 = a_vrow + (uint32_t)(((lane & 7) ^ (4 + (lane >> 4))) * 16);
  // fragment read offsets (32x32x32 operand: row l % 32, logical chunk 2c + l / 32)
  int a_frag[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int r = lane & 31;
    a_frag[c] = (wm * 64 + r) * 128 + (((2 * c + (lane >> 5)) ^ ((r >> 1) & 7)) * 16);
  }
  // s_a: waves w and w + SA_WAVES copy the same 64 rows (identical data, so the
  // duplicate write is harmless and every wave runs the same instruction stream)
  const int sa_row0 = (wave % C::SA_WAVES) * 64;
  const uint32_t sa_voff = (uint32_t)(sa_row0 + lane) * 4u;
  // B: thread t owns B_UNITS consecutive unit slots (u_local*16 + n%16) of one
  // 16-column tile of the group; they share u_local, so their fragment slots are
  // 16 bytes apart.
  constexpr int THREADS_PER_TILE = C::THREADS / (BN / 16);
  const int b_tile = tid / THREADS_PER_TILE;
  const int b_us0 = (tid % THREADS_PER_TILE) * C::B_UNITS;
  const uint32_t b_voff = (uint32_t)b_tile * 12u * (uint32_t)K + (uint32_t)b_us0 * 12u;
  // s_w: thread t handles column t % 128 (duplicates write identical values)
  const int sw_col = tid % BN;
  const uint32_t sw_voff = (uint32_t)sw_col * 2u;
  int b_lds0;
  {
    const int ul = b_us0 >> 4;
    const int n = b_tile * 16 + (b_us0 & 15);
    b_lds0 = (((ul >> 1) * (BN / 32) + (n >> 5)) * 64 + (n & 31) + 32 * (ul & 1)) * 16;
  }

  struct BRegs {
    u32x3 u[C::B_UNITS];
    uint32_t s;
  };
  BRegs breg[2];  // group h lives in set h % 2 from its issue until its fill

  // Register half of group g's reads: packed weights and weight scales.
  auto issue_regs = [&](int g, BRegs& r) {
    const uint32_t bo = b_voff + (uint32_t)g * 1536u;
#pragma unroll
    for (int i = 0; i < C::B_UNITS; ++i)
      r.u[i] = __builtin_amdgcn_raw_buffer_load_b96(rw, bo + 12u * i, 0, 0);
    r.s = __builtin_amdgcn_raw_buffer_load_b16(rsw, sw_voff + (uint32_t)g * (uint32_t)N * 2u, 0, 0);
  };
  // DMA half of group g's reads: activations and activation scales into stage s.
  auto issue_dma = [&](int g, int s) {
    int8_t* la = stage_a(s);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (lds_ptr_t)(la + (wave * 4 + i) * 1024), 16,
          ((i & 1) ? a_voff1 : a_voff0) + (uint32_t)g * 128u + (uint32_t)(i * 8) * K, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr_t)(stage_sa(s) + sa_row0), 4,
                                             sa_voff + (uint32_t)g * (uint32_t)M * 4u, 0, 0, 0);
  };
  // Unpack a register set into stage s.
  auto fill = [&](int s, const BRegs& r) {
    int8_t* lb = stage_b(s);
#pragma unroll
    for (int i = 0; i < C::B_UNITS; ++i)
      *reinterpret_cast<i32x4*>(lb + b_lds0 + 16 * i) =
          unpack_unit_x4(r.u[i][0], r.u[i][1], r.u[i][2]);
    stage_s4(s)[sw_col] = 0.25f * half_bits_to_float((uint16_t)r.s);  // exact
  };
  // vector-memory instructions issued per group: register loads + DMA
  constexpr int OPS_PER_GROUP = C::B_UNITS + 1 + C::DMA_OPS;

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

  // deferred second half of the previous group: MFMA results + its scales; starting
  // values make the first deferred rescale add exactly 0 (t = fma(F0, 0, 0) = 0)
  i32x16 dprev[2] = {magic, magic};
  float saprev[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) saprev[r] = 0.0f;
  float s4prev[2] = {0.0f, 0.0f};

  auto rescale = [&](float (&a)[2][16], const i32x16 (&d)[2], const float (&sav)[16],
                     const float (&s4v)[2]) {
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) {
      const float bias = -kMagicF * s4v[tn];
      // reinterpret the whole vector: with hipcc 7.2 a bit_cast of one subscripted
      // vector element silently reads element 0
      const f32x16 Fv = __builtin_bit_cast(f32x16, d[tn]);
#pragma unroll
      for (int r = 0; r < 16; ++r) a[tn][r] = fmaf(fmaf(Fv[r], s4v[tn], bias), sav[r], a[tn][r]);
    }
  };

  // Pin values to this point of the instruction stream (keeps each rescale inside
  // the MFMA phase it is meant to overlap instead of being sunk to the loop end).
  auto anchor = [](auto& v) {
    if constexpr (sizeof(v) == 2 * 16 * sizeof(float)) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(v[t][r]));
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t) asm volatile("" : "+v"(v[t]));
    }
  };

  // ---- prologue: group 0 staged, group 1 in flight.  Past the last group (here
  // and in the loop) the last group is simply read again into stages that are
  // never read, so the loop body has no branches and no read leaves the buffers.
  const int glast = G - 1;
  issue_regs(0, breg[0]);
  issue_dma(0, 0);
  issue_regs(min(1, glast), breg[1]);
  issue_dma(min(1, glast), 1);
  wait_vm_lgkm0<OPS_PER_GROUP>();  // group 0 landed
  fill(0, breg[0]);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  barrier();

  const int frag = lane * 16;
  // One group.  `mine` held group g (unpacked during the previous group) and now
  // receives group g+2; `other` holds group g+1, unpacked here.
  auto step = [&](int g, BRegs& mine, const BRegs& other) __attribute__((always_inline)) {
    const int s = g % STAGES;
    // group g+2: registers, and DMA into the stage group g-1 used; both stay in
    // flight across this group's barrier
    issue_regs(min(g + 2, glast), mine);
    issue_dma(min(g + 2, glast), (g + 2) % STAGES);
    __builtin_amdgcn_sched_barrier(0);

    const int8_t* la = stage_a(s);
    const int8_t* lb = stage_b(s);
    const float* lsa = stage_sa(s);
    const float* ls4 = stage_s4(s);
    const int rowoff0 = wm * 64 + 4 * (lane >> 5);

    // phase 1: MFMAs of row tile 0 (both column tiles) while the VALU rescales the
    // previous group's row tile 1; also fetch this group's scales for phase 2
    i32x16 d0[2];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const i32x4 af = *reinterpret_cast<const i32x4*>(la + a_frag[c]);
#pragma unroll
      for (int tn = 0; tn < 2; ++tn) {
        const i32x4 bf =
            *reinterpret_cast<const i32x4*>(lb + (c * (BN / 32) + wn * 2 + tn) * 1024 + frag);
        d0[tn] = mfma32(af, bf, c == 0 ? magic : d0[tn]);
      }
    }
    rescale(acc[1], dprev, saprev, s4prev);
    anchor(acc[1]);
    anchor(d0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);  // eight VALU
    }
    __builtin_amdgcn_sched_barrier(0);

    // phase 2: MFMAs of row tile 1 while the VALU rescales row tile 0 of this group
    float sa0[16], s4c[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) sa0[r] = lsa[rowoff0 + 8 * (r >> 2) + (r & 3)];
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) s4c[tn] = ls4[wn * 64 + tn * 32 + (lane & 31)];
    i32x16 d1[2];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const i32x4 af = *reinterpret_cast<const i32x4*>(la + a_frag[c] + 32 * 128);
#pragma unroll
      for (int tn = 0; tn < 2; ++tn) {
        const i32x4 bf =
            *reinterpret_cast<const i32x4*>(lb + (c * (BN / 32) + wn * 2 + tn) * 1024 + frag);
        d1[tn] = mfma32(af, bf, c == 0 ? magic : d1[tn]);
      }
    }
    rescale(acc[0], d0, sa0, s4c);
    fill((g + 1) % STAGES, other);  // group g+1, loaded during the previous group
#pragma unroll
    for (int r = 0; r < 16; ++r) saprev[r] = lsa[rowoff0 + 32 + 8 * (r >> 2) + (r & 3)];
    anchor(acc[0]);
    anchor(d1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
    }
    __builtin_amdgcn_sched_barrier(0);

    // the second half is rescaled during the next group's first half
    dprev[0] = d1[0];
    dprev[1] = d1[1];
    s4prev[0] = s4c[0];
    s4prev[1] = s4c[1];

    // everything issued before this group's loads has landed (group g+1's DMA), and
    // this group's fills and LDS reads are done before anyone passes the barrier
    wait_vm_lgkm0<OPS_PER_GROUP>();
    barrier();
  };
  // Unrolled by two so each register set is named statically; no branch sits
  // between a load and the unpack that consumes it.
  int g = 0;
  for (; g + 1 < G; g += 2) {
    step(g, breg[0], breg[1]);
    step(g + 1, breg[1], breg[0]);
  }
  if (g < G) step(g, breg[0], breg[1]);
  wait_vm_lgkm0<0>();  // no copy into LDS may outlive the workgroup
  rescale(acc[1], dprev, saprev, s4prev);

  // epilogue: fp16 stores, column = lane % 32
#pragma unroll
  for (int tm = 0; tm < 2; ++tm)
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) {
      const int col = wn * 64 + tn * 32 + (lane & 31);
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

template <int BM>
static void launch_prefill_t(const int8_t* qa, const float* sa, const uint32_t* wp,
                             const uint16_t* sw, int64_t M, int64_t N, int64_t K, uint16_t* y,
                             hipStream_t stream) {
  const int64_t nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN;
  const int GM = 8;
  hipLaunchKernelGGL(gemm_prefill_kernel<BM>, dim3((unsigned)(nbm * nbn)), dim3(BM * 2), 0,
                     stream, qa, sa, wp, sw, (int)M, (int)N, (int)K, GM, y);
}

hipError_t launch_gemm_prefill(const int8_t* qa, const float* sa, const uint32_t* wp,
                               const uint16_t* sw, int64_t M, int64_t N, int64_t K, uint16_t* y,
                               hipStream_t stream) {
  if (M >= 1024)
    launch_prefill_t<256>(qa, sa, wp, sw, M, N, K, y, stream);
  else
    launch_prefill_t<128>(qa, sa, wp, sw, M, N, K, y, stream);
  return hipGetLastError();
}

}  // namespace flexq
