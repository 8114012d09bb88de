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
// Tile: BM x BN per workgroup (256 x 128, 128 x 128 or 128 x 64, see prefill_tile),
// BM/32 waves, each wave 64 x 32*TN outputs = 2 x TN MFMA tiles of 32 x 32 (TN = 2,
// or 1 for the 64-wide tile), handled as two row tiles.  A group is written out as
// 8*TN steps of one MFMA each: the 4*TN steps of row tile 0 overlap the rescale of
// the previous group's row tile 1, the 4*TN steps of row tile 1 the rescale of this
// group's row tile 0 and the unpack of the next group.
// The 16 activation scales a lane needs for one 32 x 32 tile arrive in one register
// (lane 16j + r holds the scale of output register r) and the accumulate is a
// v_fmac_f32 with DPP row_newbcast:r, which hands lane r of each 16-lane row to
// the whole row.
//
// Staging: a 3-deep LDS ring per 128-deep group holds the int8 activation tile,
// the unpacked weight tile (bytes 4*q) and both scale vectors.  The activation
// tile is row-major with a 16-byte-chunk XOR swizzle (conflict-free fragment
// reads); the weight tile is "fragment-linear" (every 1 KB block one 32 x 32 MFMA
// operand, lane l's 16 bytes at 16*l).  Activations and their scales go global ->
// LDS directly (buffer_load ... lds, no registers); packed weights and weight
// scales come through registers (two sets) and are unpacked into the ring; each
// scale vector is loaded by just the waves that cover it.  Loads run two groups
// ahead, at most one vector-memory instruction per MFMA step; one barrier
// per group, with the counter waits written out so the loads of group g+2 stay in
// flight across it.
//
// Workgroups are numbered so that the 8 XCDs each take a contiguous run of
// logical tiles (hardware hands workgroup i to XCD i % 8), and logical tiles run
// over a band of GM row blocks before moving to the next column block.
#include <algorithm>
#include <utility>

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

constexpr int STAGES = 3;
constexpr int kOutPitch = 144;  // bytes per staged output row: 128 + 16 of padding
// which scale vectors a wave loads in the main loop (both: the 64-row tile, whose one
// activation-scale wave also covers half the weight scales)
constexpr int kRoleNone = 0, kRoleSa = 1, kRoleSw = 2, kRoleBoth = 3;

// s_waitcnt vmcnt(n) lgkmcnt(0) (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8],
// vmcnt[5:4] in [15:14]).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// acc += S' * t, where S' is lane R of the caller's 16-lane row of S (DPP
// row_newbcast on the first source; S is only ever written by LDS loads, so no
// VALU-to-DPP wait states are needed).
template <int R>
__device__ __forceinline__ void fmac_row_bcast(float& acc, float S, float t) {
  asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
      : "+v"(acc)
      : "v"(S), "v"(t), "i"(R));
}

// Rescale outputs R0 .. R0+3 of one 32x32 tile: t = RN(d * s_w) from the biased
// MFMA result F = 12582912 + 4d, then acc = RN(t * s_a + acc).  The s_a of output r
// sits in lane r of each 16-lane row of the packed register S.
template <int R0>
__device__ __forceinline__ void rescale4(float (&a)[16], const f32x16& F, float s4, float bias,
                                         float S) {
  const float t0 = fmaf(F[R0 + 0], s4, bias);
  const float t1 = fmaf(F[R0 + 1], s4, bias);
  const float t2 = fmaf(F[R0 + 2], s4, bias);
  const float t3 = fmaf(F[R0 + 3], s4, bias);
  fmac_row_bcast<R0 + 0>(a[R0 + 0], S, t0);
  fmac_row_bcast<R0 + 1>(a[R0 + 1], S, t1);
  fmac_row_bcast<R0 + 2>(a[R0 + 2], S, t2);
  fmac_row_bcast<R0 + 3>(a[R0 + 3], S, t3);
}


}  // namespace

// Order of the instructions inside one MFMA step: the MFMA first, then the step's
// LDS reads and vector-memory loads, then its VALU work (rescale, unpack) and LDS
// writes, so that the step's VALU work issues while its MFMA runs (left to itself the
// compiler puts the MFMAs of neighbouring steps back to back).  Used by the tiles with
// two 32-column MFMA tiles per wave: 2-8 % faster on 128 x 128 tiles, neutral on
// 256 x 128 (where it also frees the registers that spilled), 2 % slower on 128 x 64.
__device__ __forceinline__ void step_order() {
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // LDS reads
  __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);   // vector-memory reads
  __builtin_amdgcn_sched_group_barrier(0x002, 48, 0);  // VALU
  __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);   // LDS writes
}

template <int BM, int BN>
struct PrefillCfg {
  static constexpr int THREADS = BM * 2;
  static constexpr int WAVES = THREADS / 64;
  static constexpr int WM = BM / 64;                 // waves along M (64 rows each)
  static constexpr int WN = WAVES / WM;              // waves along N
  static constexpr int TN = BN / WN / 32;            // 32-column MFMA tiles per wave
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

// PARTIAL: split-K.  The grid is S times the tile grid; slice s of a tile takes the
// groups [s*G/S, (s+1)*G/S) (G = K/128), accumulates them from +0 in ascending order
// exactly as the whole product would, and stores its fp32 accumulators as plane s of
// `part` ([S][M][ldn]) instead of fp16 Y.  The planes are summed afterwards in
// ascending slice order (launch_splitk_reduce).
template <int BM, int BN, bool PARTIAL>
__global__ __launch_bounds__(BM * 2, 1) void gemm_prefill_kernel(
    const int8_t* __restrict__ qa, const float* __restrict__ sa, const uint32_t* __restrict__ wp,
    const uint16_t* __restrict__ sw, int M, int N, int K, int ldn, int GM,
    uint16_t* __restrict__ y, int S, float* __restrict__ part) {
  using C = PrefillCfg<BM, BN>;
  constexpr int TN = C::TN;
  static_assert(TN == 1 || TN == 2, "one or two 32-column tiles per wave");
  static_assert(C::WN * TN * 32 == BN, "waves cover the tile's columns");
  static_assert(C::A_BLOCKS_PER_WAVE == 4, "tile/thread mismatch");
  static_assert(C::WAVES * 64 * kOutPitch <= STAGES * C::STAGE_BYTES, "output staging fits");
  static_assert(C::B_UNITS * C::THREADS == BN * 8, "B split");
  static_assert(C::B_UNITS == 2 || C::B_UNITS == 4 || C::B_UNITS == 8, "unpack schedule");

  const int Gtot = K >> 7;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % C::WM, wn = wave / C::WM;

  // ---- logical tile from the workgroup id (XCD-contiguous, row-band order)
  const int nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN;
  const int tiles = nbm * nbn;
  const int total = tiles * S;
  int pid = blockIdx.x;
  if ((total & 7) == 0) pid = (pid & 7) * (total >> 3) + (pid >> 3);
  // K slice: groups g0 .. g0 + G - 1 (the whole of K when S = 1)
  const int slice = pid / tiles;
  pid -= slice * tiles;
  const int g0 = (int)((int64_t)slice * Gtot / S);
  const int G = (int)((int64_t)(slice + 1) * Gtot / S) - g0;
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

  // Out-of-range loads return zero: rows >= M and columns >= N vanish.
  const auto ra = make_rsrc(qa + (size_t)m0 * K, (uint32_t)mrows * (uint32_t)K);
  const auto rw = make_rsrc(wp + (size_t)(n0 / 16) * 3 * K, (uint32_t)(ncols / 16) * 12u * K);
  // scales are group-major: s_a[g][m] at g*M + m, s_w[g][n] at g*ldn + n (the launch
  // covers columns 0 .. N-1 of a matrix whose Y rows and s_w rows are ldn apart)
  const auto rsa = make_rsrc(sa + m0, (uint32_t)((size_t)Gtot * M - m0) * 4u);
  const auto rsw = make_rsrc(sw + n0, (uint32_t)((size_t)(Gtot - 1) * ldn + N - n0) * 2u);

  // A stage: row-major, 128 bytes per row, the 16-byte chunk j of row r stored at
  // chunk j ^ ((r >> 1) & 7) (so the 32x32 fragment reads below touch every bank
  // once per 16 lanes).  The copy into it is coalesced: DMA instruction i of wave w
  // moves rows R0 = (4w + i) * 8 .. R0 + 7, lane l taking physical chunk l % 8 of row
  // R0 + l / 8, i.e. logical chunk (l % 8) ^ (4 * (i % 2) + l / 16).
  // The row part of every offset stays in the VGPR operand, which the range check
  // that zeroes rows >= M covers; the group's column offset (always inside the row)
  // goes in the scalar offset.
  const uint32_t a_vrow = (uint32_t)(wave * 32 + (lane >> 3)) * (uint32_t)K;
  uint32_t a_voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    a_voff[i] = a_vrow + (uint32_t)(i * 8) * (uint32_t)K +
                (uint32_t)(((lane & 7) ^ (4 * (i & 1) + (lane >> 4))) * 16);
  // Scales: in the main loop only waves 0 .. SA_WAVES-1 copy s_a (64 rows each) and
  // only BN/64 waves load s_w (one column per thread): the next ones, or with two
  // waves (the 64-row tile) both, the first doing both; each global load instruction
  // costs issue time whatever its size, so no wave loads a copy another wave already
  // brings.  The main loop exists once per role (kRoleSa, kRoleSw, kRoleBoth,
  // kRoleNone) so that no branch splits it.  (The prologue loads the scales in every
  // wave; duplicates write identical values.)
  constexpr int SW0 = C::SA_WAVES < C::WAVES - BN / 64 ? C::SA_WAVES : C::WAVES - BN / 64;
  static_assert(SW0 >= 0, "enough waves for the weight scales");
  const bool sa_wave = wave < C::SA_WAVES;
  const bool sw_wave = wave >= SW0 && wave < SW0 + BN / 64;
  const int sa_row0 = (wave % C::SA_WAVES) * 64;
  const uint32_t sa_voff = (uint32_t)(sa_row0 + lane) * 4u;
  // B: wave w loads the 16-column tiles TPW*w .. TPW*w + TPW - 1 of the group
  // (1536 contiguous bytes per tile and group, unit slot j = u_local*16 + n%16).
  // Load i of a lane takes slot (i%2)*64 + lane of tile TPW*w + i/2, so every load
  // instruction reads 768 contiguous bytes; in fragment order that unit lands at
  // b_lds0 + (i%2)*2*KC_BYTES + ((i/2)%2)*256 + (i/4)*1024 (TPW*w is a multiple of
  // TPW; KC_BYTES is one 32-deep k-chunk of the B stage).
  constexpr int TPW = (BN / 16) / C::WAVES;
  constexpr int KC_BYTES = (BN / 32) * 1024;
  static_assert(C::B_UNITS == 2 * TPW && (TPW == 1 || TPW == 2 || TPW == 4), "B load split");
  const int b_tile0 = wave * TPW;
  const uint32_t b_voff = (uint32_t)b_tile0 * 12u * (uint32_t)K + (uint32_t)lane * 12u;
  auto b_unit_off = [&](int i) -> uint32_t {
    return (uint32_t)(i >> 1) * 12u * (uint32_t)K + (uint32_t)(i & 1) * 768u;
  };
  uint32_t b_voff_u[C::B_UNITS];
#pragma unroll
  for (int i = 0; i < C::B_UNITS; ++i) b_voff_u[i] = b_voff + b_unit_off(i);
  // s_w: thread t handles column t % 128
  const int sw_col = tid % BN;
  const uint32_t sw_voff = (uint32_t)sw_col * 2u;
  int b_lds0;
  {
    const int ul = lane >> 4;
    const int n = b_tile0 * 16 + (lane & 15);
    b_lds0 = (((ul >> 1) * (BN / 32) + (n >> 5)) * 64 + (n & 31) + 32 * (ul & 1)) * 16;
  }

  struct BRegs {
    u32x3 u[C::B_UNITS];
    uint32_t s;
  };
  BRegs breg[2];  // group h lives in set h % 2 from its issue until its fill

  // Prologue reads of group g: packed weights and weight scales into registers, then
  // activations and activation scales into the stage at byte offset `so`.
  auto issue_regs = [&](int gl, BRegs& r) {
    const int g = g0 + gl;
#pragma unroll
    for (int i = 0; i < C::B_UNITS; ++i)
      r.u[i] = __builtin_amdgcn_raw_buffer_load_b96(rw, b_voff_u[i], (uint32_t)g * 1536u, 0);
    r.s = __builtin_amdgcn_raw_buffer_load_b16(rsw, sw_voff + (uint32_t)g * (uint32_t)ldn * 2u, 0, 0);
  };
  auto issue_dma = [&](int gl, int so) {
    const int g = g0 + gl;
    int8_t* la = lds + so;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(la + (wave * 4 + i) * 1024), 16,
                                               a_voff[i], (uint32_t)g * 128u, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsa, (lds_ptr_t)(la + C::A_BYTES + C::B_BYTES + sa_row0 * 4), 4,
        sa_voff + (uint32_t)g * (uint32_t)M * 4u, 0, 0, 0);
  };
  // Unpack unit i of a register set, and its weight scale, into the stage at `so`.
  auto fill_unit = [&](int so, const BRegs& r, int i) {
    *reinterpret_cast<i32x4*>(lds + so + C::A_BYTES + b_lds0 + (i & 1) * 2 * KC_BYTES +
                              ((i >> 1) & 1) * 256 + (i >> 2) * 1024) =
        unpack_unit_x4(r.u[i][0], r.u[i][1], r.u[i][2]);
  };
  auto fill_scale = [&](int so, const BRegs& r) {
    *reinterpret_cast<float*>(lds + so + C::A_BYTES + C::B_BYTES + BM * 4 + sw_col * 4) =
        0.25f * half_bits_to_float((uint16_t)r.s);  // exact
  };
  auto fill = [&](int so, const BRegs& r) {
#pragma unroll
    for (int i = 0; i < C::B_UNITS; ++i) fill_unit(so, r, i);
    fill_scale(so, r);
  };
  // vector-memory instructions of one group: DMA + register loads, and the fewest
  // any wave issues in the main loop (activation blocks and weight units only)
  constexpr int OPS_PER_GROUP = C::B_UNITS + 1 + C::DMA_OPS;
  constexpr int MIN_OPS_PER_GROUP = C::B_UNITS + C::A_BLOCKS_PER_WAVE;
  // Vector-memory instruction i of group g (DMA blocks, the s_a row, weight units,
  // the weight scale), so a group's reads can be spread over the MFMA steps: issued
  // in one burst by every wave right after a barrier, they queue at the texture unit
  // and stall the waves behind them.
  auto vmem_op = [&](auto role, auto ic, int gl, int so, BRegs& r) {
    constexpr int i = decltype(ic)::value;
    const int g = g0 + gl;
    constexpr int kRole = decltype(role)::value;
    if constexpr (i < 4) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(lds + so + (wave * 4 + i) * 1024),
                                               16, a_voff[i], (uint32_t)g * 128u, 0, 0);
    } else if constexpr (i == 4) {
      if constexpr (kRole == kRoleSa || kRole == kRoleBoth)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsa, (lds_ptr_t)(lds + so + C::A_BYTES + C::B_BYTES + sa_row0 * 4), 4,
            sa_voff + (uint32_t)g * (uint32_t)M * 4u, 0, 0, 0);
    } else if constexpr (i < 5 + C::B_UNITS) {
      // (the tile part is in the VGPR operand; a group stays inside its tile)
      r.u[i - 5] = __builtin_amdgcn_raw_buffer_load_b96(rw, b_voff_u[i - 5], (uint32_t)g * 1536u,
                                                        0);
    } else {
      if constexpr (kRole == kRoleSw || kRole == kRoleBoth)
        r.s = __builtin_amdgcn_raw_buffer_load_b16(rsw, sw_voff + (uint32_t)g * (uint32_t)ldn * 2u,
                                                   0, 0);
    }
  };
  static_assert(C::DMA_OPS == 5, "vmem_op numbering");
  static_assert(OPS_PER_GROUP <= 8 * C::TN, "one vector-memory instruction per MFMA step");

  float acc[2][TN][16];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  i32x16 magic;
#pragma unroll
  for (int r = 0; r < 16; ++r) magic[r] = (int32_t)kMagic;

  // Deferred row tile 1 of the previous group: MFMA results, its packed s_a
  // register and s_w / 4.  The starting values make the first deferred rescale add
  // exactly +0 (t = fma(F0, 0, -0) = +0, then acc + S * t with S = 0).
  i32x16 dprev[TN];
  float s4prev[TN], bprev[TN];  // bprev = -12582912 * s4prev
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    dprev[tn] = magic;
    s4prev[tn] = 0.0f;
    bprev[tn] = -0.0f;
  }
  float Sprev = 0.0f;

  // per-lane byte offsets inside a stage
  const int r32 = lane & 31, hl = lane >> 5;
  int a_off[4];  // A fragment of k-chunk c, row tile 0 (row tile 1: +4096)
#pragma unroll
  for (int c = 0; c < 4; ++c)
    a_off[c] = (wm * 64 + r32) * 128 + (((2 * c + hl) ^ ((r32 >> 1) & 7)) * 16);
  // B fragment (c, tn): block c * (BN / 32) + wn * TN + tn, lane-linear
  const int b_off = C::A_BYTES + wn * TN * 1024 + lane * 16;
  // s_a row held by this lane in the packed scale register of row tile tm (+128 * tm)
  const int sa_off =
      C::A_BYTES + C::B_BYTES + (wm * 64 + 8 * ((lane >> 2) & 3) + 4 * hl + (lane & 3)) * 4;
  // s_w / 4 of this lane's column in column tile tn (+128 * tn)
  const int s4_off = C::A_BYTES + C::B_BYTES + BM * 4 + (wn * TN * 32 + r32) * 4;

  auto ldA = [&](int so, int c, int tm) {
    return *reinterpret_cast<const i32x4*>(lds + so + a_off[c] + tm * 4096);
  };
  auto ldB = [&](int so, int c, int tn) {
    return *reinterpret_cast<const i32x4*>(lds + so + b_off + c * KC_BYTES + tn * 1024);
  };
  auto ldS = [&](int so, int tm) {
    return *reinterpret_cast<const float*>(lds + so + sa_off + tm * 128);
  };
  auto ldS4 = [&](int so, int tn) {
    return *reinterpret_cast<const float*>(lds + so + s4_off + tn * 128);
  };

  // ---- prologue: group 0 staged, group 1 in flight.  Past the last group (here
  // and in the loop) the last group is simply read again into stages that are
  // never read, so the loop body has no branches and no read leaves the buffers.
  const int glast = G - 1;
  issue_regs(0, breg[0]);
  issue_dma(0, 0);
  issue_regs(min(1, glast), breg[1]);
  issue_dma(min(1, glast), C::STAGE_BYTES);
  // Group 0 must have landed before its fill.  Wait for every load issued so far:
  // the compiler may sink a load of group 1 below this point, so a count of group
  // 1's loads would not cover all of group 0's; group 1 was issued right after
  // group 0, so waiting for it too costs almost nothing.
  wait_vm_lgkm0<0>();
  fill(0, breg[0]);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  barrier();

  // One group g in stage `so`, written as 8*TN steps of one MFMA each.  The first
  // 4*TN (row tile 0) overlap the rescale of the previous group's row tile 1, the
  // last 4*TN (row tile 1) the rescale of this group's row tile 0 and the unpack of
  // group g+1.  LDS reads run two or more steps ahead of their MFMA; the B
  // fragments stay in registers for both row tiles.  `mine` held group g and now
  // receives group g+2; `other` holds group g+1.
  auto step_group = [&](auto role, int g, int so, int so_next, int so_dma, BRegs& mine,
                        const BRegs& other) __attribute__((always_inline)) {
    // group g+2 goes to registers `mine` (unpacked last group) and to the stage
    // group g-1 used, one vector-memory instruction per MFMA step
    const int gn = min(g + 2, glast);

    i32x4 a0[4], a1[4], b[4][TN];
    i32x16 d0[TN], d1[TN];
    float S0, S1, s4c[TN], bc[TN];
    f32x16 Fp[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) Fp[tn] = __builtin_bit_cast(f32x16, dprev[tn]);
    const float Sp = Sprev;

    // LDS reads of this stage, each at least two steps before its MFMA: k-chunks 0
    // and 1 up front, the rest spread over row tile 0 (schedule per tile width).
    a0[0] = ldA(so, 0, 0);
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) b[0][tn] = ldB(so, 0, tn);
    a0[1] = ldA(so, 1, 0);
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) b[1][tn] = ldB(so, 1, tn);
    rescale4<0>(acc[1][0], Fp[0], s4prev[0], bprev[0], Sp);
    __builtin_amdgcn_sched_barrier(0);

    // ---- row tile 0: 4 * TN steps (k-chunk c = k / TN, column tile tn = k % TN)
    constexpr int STEPS = 4 * TN;
    static_assert(STEPS <= OPS_PER_GROUP, "row tile 0 issues only real loads");
    unroll([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      constexpr int c = k / TN, tn = k % TN;
      vmem_op(role, kc, gn, so_dma, mine);
      if constexpr (TN == 2) {
        if constexpr (k == 0) a0[2] = ldA(so, 2, 0);
        if constexpr (k == 1) b[2][0] = ldB(so, 2, 0);
        if constexpr (k == 2) b[2][TN - 1] = ldB(so, 2, TN - 1);
        if constexpr (k == 3) a0[3] = ldA(so, 3, 0);
        if constexpr (k == 4) b[3][0] = ldB(so, 3, 0);
        if constexpr (k == 5) b[3][TN - 1] = ldB(so, 3, TN - 1);
      } else {
        if constexpr (k == 0) {
          a0[2] = ldA(so, 2, 0);
          b[2][0] = ldB(so, 2, 0);
        }
        if constexpr (k == 1) {
          a0[3] = ldA(so, 3, 0);
          b[3][0] = ldB(so, 3, 0);
        }
      }
      if constexpr (k == STEPS - 2) {
        a1[0] = ldA(so, 0, 1);
        S0 = ldS(so, 0);
#pragma unroll
        for (int t = 0; t < TN; ++t) s4c[t] = ldS4(so, t);
      }
      if constexpr (k == STEPS - 1) {
        a1[1] = ldA(so, 1, 1);
        S1 = ldS(so, 1);
      }
      d0[tn] = mfma32(a0[c], b[c][tn], c == 0 ? magic : d0[tn]);
      // outputs 4 .. 16 * TN - 1 of the deferred tile, four per step
      if constexpr (k < STEPS - 1) {
        constexpr int o = 4 * (k + 1);
        rescale4<o % 16>(acc[1][o / 16], Fp[o / 16], s4prev[o / 16], bprev[o / 16], Sp);
      }
      if constexpr (TN == 2) step_order();
      __builtin_amdgcn_sched_barrier(0);
    }, std::make_integer_sequence<int, STEPS>{});

    // ---- row tile 1
    f32x16 F0[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      F0[tn] = __builtin_bit_cast(f32x16, d0[tn]);
      bc[tn] = -kMagicF * s4c[tn];
    }
    unroll([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      constexpr int c = k / TN, tn = k % TN;
      if constexpr (STEPS + k < OPS_PER_GROUP)
        vmem_op(role, std::integral_constant<int, STEPS + k>{}, gn, so_dma, mine);
      if constexpr (k == 0) a1[2] = ldA(so, 2, 1);
      if constexpr (k == 1) a1[3] = ldA(so, 3, 1);
      d1[tn] = mfma32(a1[c], b[c][tn], c == 0 ? magic : d1[tn]);
      rescale4<4 * (k % 4)>(acc[0][k / 4], F0[k / 4], s4c[k / 4], bc[k / 4], S0);
      // the unpack of group g+1: unit u at step 1 + (STEPS - 2)u/B_UNITS, then its scale
      unroll([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        if constexpr (k == 1 + (u * (STEPS - 2)) / C::B_UNITS) fill_unit(so_next, other, u);
      }, std::make_integer_sequence<int, C::B_UNITS>{});
      if constexpr (k == STEPS - 1) {
        if constexpr (decltype(role)::value == kRoleSw || decltype(role)::value == kRoleBoth)
          fill_scale(so_next, other);
      }
      if constexpr (TN == 2) step_order();
      __builtin_amdgcn_sched_barrier(0);
    }, std::make_integer_sequence<int, STEPS>{});

    // row tile 1 is rescaled during the next group's row tile 0
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      dprev[tn] = d1[tn];
      s4prev[tn] = s4c[tn];
      bprev[tn] = bc[tn];
    }
    Sprev = S1;

    // everything issued before this group's loads has landed (group g+1's DMA), and
    // this group's fills and LDS reads are done before anyone passes the barrier.
    // Waves issue MIN_OPS_PER_GROUP .. OPS_PER_GROUP loads per group; waiting for the
    // fewest is exact for some and one or two loads early for the others.
    wait_vm_lgkm0<MIN_OPS_PER_GROUP>();
    barrier();
  };

  // Unrolled by six, the period of both the two register sets and the three
  // stages: each group's stage offsets are then compile-time constants that fold
  // into the LDS instructions' offset fields instead of costing address additions
  // (10-15 % faster on the large LLaMA-2-70B shapes).  No branch sits between a
  // load and the unpack that consumes it.  The last G % 6 groups run in a loop
  // unrolled by two with the stage offsets in registers.
  auto main_loop = [&](auto role) __attribute__((always_inline)) {
    constexpr int SB = C::STAGE_BYTES;
    int g = 0;
    for (; g + 5 < G; g += 6) {
      step_group(role, g, 0, SB, 2 * SB, breg[0], breg[1]);
      step_group(role, g + 1, SB, 2 * SB, 0, breg[1], breg[0]);
      step_group(role, g + 2, 2 * SB, 0, SB, breg[0], breg[1]);
      step_group(role, g + 3, 0, SB, 2 * SB, breg[1], breg[0]);
      step_group(role, g + 4, SB, 2 * SB, 0, breg[0], breg[1]);
      step_group(role, g + 5, 2 * SB, 0, SB, breg[1], breg[0]);
    }
    // six groups leave the ring and the register sets where they started
    int so = 0, so1 = SB, so2 = 2 * SB;
    auto rotate = [&]() {
      const int t = so;
      so = so1;
      so1 = so2;
      so2 = t;
    };
    for (; g + 1 < G; g += 2) {
      step_group(role, g, so, so1, so2, breg[0], breg[1]);
      rotate();
      step_group(role, g + 1, so, so1, so2, breg[1], breg[0]);
      rotate();
    }
    if (g < G) step_group(role, g, so, so1, so2, breg[0], breg[1]);
  };
  if constexpr (SW0 < C::SA_WAVES) {  // the 64-row tile: wave 0 both, wave 1 s_w
    if (sa_wave)
      main_loop(std::integral_constant<int, kRoleBoth>{});
    else
      main_loop(std::integral_constant<int, kRoleSw>{});
  } else {
    if (sa_wave)
      main_loop(std::integral_constant<int, kRoleSa>{});
    else if (sw_wave)
      main_loop(std::integral_constant<int, kRoleSw>{});
    else
      main_loop(std::integral_constant<int, kRoleNone>{});
  }
  wait_vm_lgkm0<0>();  // no copy into LDS may outlive the workgroup
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    const f32x16 Fp = __builtin_bit_cast(f32x16, dprev[tn]);
    unroll([&](auto kc) {
      constexpr int q = decltype(kc)::value;
      rescale4<4 * q>(acc[1][tn], Fp, s4prev[tn], bprev[tn], Sprev);
    }, std::make_integer_sequence<int, 4>{});
  }

  if constexpr (PARTIAL) {
    // fp32 accumulators of this slice; lanes 0-31 and 32-63 of each store write 128
    // contiguous bytes of two rows
    float* pp = part + (size_t)slice * (size_t)M * (size_t)ldn;
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int col = wn * TN * 32 + tn * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * 64 + tm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (row < mrows && col < ncols) pp[(size_t)(m0 + row) * ldn + n0 + col] = acc[tm][tn][r];
        }
      }
    return;
  }
  // Epilogue.  With a 16-byte aligned Y, each wave stages its 64 x 32TN fp16 outputs
  // in LDS (its own region, row pitch kOutPitch) and stores every row as 16-byte
  // chunks: 4TN store instructions per lane instead of 32TN two-byte ones.  The barrier
  // lets no wave overwrite a stage while another wave's copies into it may still
  // land.  (N and ldn are multiples of 16, so an 8-column chunk is wholly inside or
  // outside the matrix and every row starts 16-byte aligned.)
  if ((reinterpret_cast<uintptr_t>(y) & 15u) == 0) {
    barrier();
    uint8_t* tw = reinterpret_cast<uint8_t*>(lds) + wave * 64 * kOutPitch;
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = tm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          *reinterpret_cast<uint16_t*>(tw + lr * kOutPitch + (tn * 32 + (lane & 31)) * 2) =
              float_to_half_bits(acc[tm][tn][r]);
        }
    __builtin_amdgcn_wave_barrier();
    constexpr int CH = 4 * TN;  // 16-byte chunks per staged row
    const int col = wn * TN * 32 + (lane % CH) * 8;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int lr = i * (64 / CH) + lane / CH;
      const i32x4 v = *reinterpret_cast<const i32x4*>(tw + lr * kOutPitch + (lane % CH) * 16);
      const int row = wm * 64 + lr;
      if (row < mrows && col < ncols)
        *reinterpret_cast<i32x4*>(y + (size_t)(m0 + row) * ldn + n0 + col) = v;
    }
    return;
  }
  // otherwise one fp16 store per output, column = lane % 32
#pragma unroll
  for (int tm = 0; tm < 2; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const int col = wn * TN * 32 + tn * 32 + (lane & 31);
      if (col < ncols) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * 64 + tm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (row < mrows)
            y[(size_t)(m0 + row) * ldn + n0 + col] = float_to_half_bits(acc[tm][tn][r]);
        }
      }
    }
}

// Columns n0 .. n0 + N - 1 of a product whose Y and s_w rows are ldn columns apart.
// With part != nullptr: split-K into S slices, fp32 planes of [M][ldn] into part.
template <int BM, int BN>
static hipError_t launch_prefill_t(const int8_t* qa, const float* sa, const uint32_t* wp,
                                   const uint16_t* sw, int64_t M, int64_t n0, int64_t N,
                                   int64_t K, int64_t ldn, uint16_t* y, hipStream_t stream,
                                   int S = 1, float* part = nullptr) {
  const int64_t nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN;
  const int GM = 4;
  const dim3 grid((unsigned)(nbm * nbn * S)), block(BM * 2);
  if (part != nullptr)
    return launch_kernel(gemm_prefill_kernel<BM, BN, true>, grid, block, stream, qa, sa,
                         wp + (n0 / 16) * 3 * K, sw + n0, (int)M, (int)N, (int)K, (int)ldn, GM,
                         y, S, part + n0);
  return launch_kernel(gemm_prefill_kernel<BM, BN, false>, grid, block, stream, qa, sa,
                       wp + (n0 / 16) * 3 * K, sw + n0, (int)M, (int)N, (int)K, (int)ldn, GM,
                       y + n0, 1, part);
}

static hipError_t launch_tile(int tile, const int8_t* qa, const float* sa, const uint32_t* wp,
                        const uint16_t* sw, int64_t M, int64_t n0, int64_t N, int64_t K,
                        int64_t ldn, uint16_t* y, hipStream_t stream) {
  if (tile == kTile256x128)
    return launch_prefill_t<256, 128>(qa, sa, wp, sw, M, n0, N, K, ldn, y, stream);
  if (tile == kTile128x128)
    return launch_prefill_t<128, 128>(qa, sa, wp, sw, M, n0, N, K, ldn, y, stream);
  if (tile == kTile64x128)
    return launch_prefill_t<64, 128>(qa, sa, wp, sw, M, n0, N, K, ldn, y, stream);
  return launch_prefill_t<128, 64>(qa, sa, wp, sw, M, n0, N, K, ldn, y, stream);
}

namespace {

// Y = fp16(part[0] + part[1] + ... + part[S-1]) element by element, the planes added in
// ascending order in fp32; acc (optional) receives the fp32 sums.  Four outputs per
// thread and step (M * N is a multiple of 16).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int S,
                                                            int64_t n4, int64_t plane,
                                                            uint16_t* __restrict__ y,
                                                            float* __restrict__ acc) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    f32x4 a = *reinterpret_cast<const f32x4*>(part + 4 * i);
    for (int s = 1; s < S; ++s) {
      const f32x4 b = *reinterpret_cast<const f32x4*>(part + (int64_t)s * plane + 4 * i);
      a[0] += b[0];
      a[1] += b[1];
      a[2] += b[2];
      a[3] += b[3];
    }
    if (acc != nullptr) *reinterpret_cast<f32x4*>(acc + 4 * i) = a;
    uint32_t* y2 = reinterpret_cast<uint32_t*>(y) + 2 * i;
    y2[0] = (uint32_t)float_to_half_bits(a[0]) | (uint32_t)float_to_half_bits(a[1]) << 16;
    y2[1] = (uint32_t)float_to_half_bits(a[2]) | (uint32_t)float_to_half_bits(a[3]) << 16;
  }
}

}  // namespace

hipError_t launch_gemm_splitk(const int8_t* qa, const float* sa, const uint32_t* wp,
                              const uint16_t* sw, int64_t M, int64_t N, int64_t K, int tile,
                              int S, float* part, uint16_t* y, float* acc, hipStream_t stream) {
  hipError_t e;
  if (tile == kTile256x128)
    e = launch_prefill_t<256, 128>(qa, sa, wp, sw, M, 0, N, K, N, y, stream, S, part);
  else if (tile == kTile128x128)
    e = launch_prefill_t<128, 128>(qa, sa, wp, sw, M, 0, N, K, N, y, stream, S, part);
  else if (tile == kTile128x64)
    e = launch_prefill_t<128, 64>(qa, sa, wp, sw, M, 0, N, K, N, y, stream, S, part);
  else if (tile == kTile64x128)
    e = launch_prefill_t<64, 128>(qa, sa, wp, sw, M, 0, N, K, N, y, stream, S, part);
  else
    return hipErrorInvalidValue;
  if (e != hipSuccess) return e;
  const int64_t n4 = M * N / 4;
  const int64_t blocks = std::min<int64_t>((n4 + 255) / 256, (int64_t)device_cu_count() * 8);
  return launch_kernel(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), stream, part, S,
                       n4, M * N, y, acc);
}

namespace {

// Time model of one launch of the prefill kernel, in microseconds, fitted to
// LLaMA-2-70B-shaped layers (M = 16 .. 512) on MI355X: the grid runs in rounds of
// one workgroup per compute unit; a round costs a per-group time times the groups
// each workgroup walks plus a fixed part; split-K adds the write and read of its fp32
// planes (per MB of S * M * N * 4) and the reduce launch.  Median error 3 %.
struct TileCost {
  int tile, bm, bn;
  double per_group, per_round, per_mb, fixed;
};
constexpr TileCost kCost[2] = {{kTile256x128, 256, 128, 1.108, 3.09, 0.362, 2.65},
                               {kTile128x128, 128, 128, 0.784, 3.32, 0.324, 2.28}};

double predict_us(const TileCost& c, int64_t M, int64_t N, int64_t G, int64_t S, int64_t cu,
                  bool partial) {
  const int64_t tiles = (M + c.bm - 1) / c.bm * ((N + c.bn - 1) / c.bn);
  const int64_t rounds = (tiles * S + cu - 1) / cu;
  const int64_t g = (G + S - 1) / S;
  return (double)rounds * (c.per_group * (double)g + c.per_round) + c.fixed +
         (partial ? c.per_mb * (double)(S * M * N * 4) / 1e6 : 0.0);
}

}  // namespace

void splitk_plan(int64_t M, int64_t N, int64_t K, int* tile, int* S) {
  const int64_t G = K / kGroup, cu = device_cu_count();
  *tile = prefill_tile(M, N);
  *S = 1;
  // Few tokens: the weight-streaming kernel is faster, unless the layer is narrow
  // (fewer than two 128 x 64 tiles per compute unit) and M is above 32.
  if (M <= 32 || (M <= 64 && (M + 127) / 128 * ((N + 63) / 64) >= 2 * cu)) return;
  double direct = 0.0;
  for (const TileCost& c : kCost) {
    const double t = predict_us(c, M, N, G, 1, cu, false);
    if (direct == 0.0 || t < direct) direct = t;
  }
  double best = 0.0;
  for (const TileCost& c : kCost)
    for (int64_t s = 2; s <= std::min<int64_t>(G, 16); ++s) {
      const double t = predict_us(c, M, N, G, s, cu, true);
      if (best == 0.0 || t < best) {
        best = t;
        *tile = c.tile;
        *S = (int)s;
      }
    }
  // split only for a predicted gain of a tenth or more over the tile grid and, up to
  // one 64-row pass, over the weight-streaming kernel
  if (best == 0.0 || best * 1.1 > direct ||
      (M <= kDecodeRowsPerPass && best * 1.1 > predict_decode_us(M, N, G, cu))) {
    *tile = prefill_tile(M, N);
    *S = 1;
  }
}

int prefill_tile(int64_t M, int64_t N) {
  // The grid runs in rounds of one 256- or 128-row tile per CU (their LDS rings
  // allow no second one); a round of 256 x 128 tiles takes about 1.46 times as long
  // as a round of 128 x 128 tiles (83 vs 57 us at K = 8192 on the LLaMA-2-70B
  // shapes), so the taller, more efficient tile is taken when it needs enough fewer
  // rounds.  When even the 128 x 128 grid leaves CUs idle (at most one tile per
  // CU), 128 x 64 tiles double the grid: one of them takes about 0.7 of a 128 x 128
  // round, two share a CU (half-size ring) in about 1.0 (LLaMA-2-70B layers at
  // M = 64 ... 512: 25-30 % faster on o and down).
  const int64_t cu = device_cu_count();
  const int64_t nbn = (N + 127) / 128;
  // One 64-row block on a wide layer: 64 x 128 tiles waste no rows, and two share a
  // compute unit, so from 1.5 column tiles per CU their grid fills the GPU (70B
  // gate_up at M = 64: 78 us against 111-113 us for the 128-row tiles).
  if (M <= 64 && nbn * 2 >= 3 * cu) return kTile64x128;
  const int64_t tiles128 = (M + 127) / 128 * nbn;
  const int64_t rounds256 = ((M + 255) / 256 * nbn + cu - 1) / cu;
  const int64_t rounds128 = (tiles128 + cu - 1) / cu;
  if (rounds256 * 146 < rounds128 * 100) return kTile256x128;
  return tiles128 <= cu ? kTile128x64 : kTile128x128;
}

int64_t prefill_main_cols(int64_t M, int64_t N) {
  // When the 256 x 128 grid ends in a partly filled round, the 128-column blocks that
  // fill whole rounds run as 256 x 128 tiles and the remaining columns as a second
  // launch of 128 x 64 tiles, if that is expected to save a twentieth.  Costs in
  // rounds of 256 x 128 tiles, measured on 70B-sized layers (K = 4096 to 8192): up to
  // one 128 x 64 tile per CU 0.48, and 0.6 more per further CU's worth of them (0.74
  // for 1.5 per CU, 1.1 to 1.5 for 2 per CU); tails of more than 2 per CU are not
  // split off.  (A round of 128 x 128 tiles costs about 0.685 for half the columns of
  // a round of 128 x 64 tiles, so it is never the better tail.)
  if (prefill_tile(M, N) != kTile256x128) return N;
  const int64_t cu = device_cu_count();
  const int64_t nbm = (M + 255) / 256, nbn = (N + 127) / 128, tiles = nbm * nbn;
  const int64_t full = tiles / cu;  // whole rounds
  if (full == 0 || tiles % cu == 0) return N;
  const int64_t c = full * cu / nbm;  // column blocks that fit in whole rounds
  if (c == 0 || c >= nbn) return N;
  const int64_t main_rounds = (nbm * c + cu - 1) / cu;
  const int64_t n64 = (M + 127) / 128 * ((N - 128 * c + 63) / 64);  // tail tiles
  if (n64 > 2 * cu) return N;
  const int64_t tail = n64 <= cu ? 480 : 480 + (n64 - cu) * 600 / cu;
  const int64_t split = main_rounds * 1000 + tail;
  return split * 20 <= (full + 1) * 1000 * 19 ? 128 * c : N;
}

hipError_t launch_gemm_prefill(const int8_t* qa, const float* sa, const uint32_t* wp,
                               const uint16_t* sw, int64_t M, int64_t N, int64_t K, uint16_t* y,
                               hipStream_t stream, int tile) {
  if (tile == kTileAuto) {
    const int64_t n_main = prefill_main_cols(M, N);
    const hipError_t e = launch_tile(prefill_tile(M, N), qa, sa, wp, sw, M, 0, n_main, K, N, y,
                                     stream);
    if (e != hipSuccess || n_main == N) return e;
    return launch_tile(kTile128x64, qa, sa, wp, sw, M, n_main, N - n_main, K, N, y, stream);
  }
  if (tile != kTile256x128 && tile != kTile128x128 && tile != kTile128x64 && tile != kTile64x128)
    return hipErrorInvalidValue;
  return launch_tile(tile, qa, sa, wp, sw, M, 0, N, K, N, y, stream);
}

}  // namespace flexq
