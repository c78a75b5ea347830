// Streaming bf16 MFMA tile mainloop for gfx950, shared by the grouped expert GEMMs and the
// router GEMM.
//
// One workgroup of 2*WN wavefronts accumulates a 128 x (128*WN) fp32 tile
// acc += A[128 x K] * B[K x 128*WN] with v_mfma_f32_32x32x16_bf16. Wavefront w, in wave row
// wm = w / WN, owns the 32-row sub-tiles wm and 2 + wm (rows 32*wm .. +32 and 64 + 32*wm .. +32)
// and columns 128*(w % WN) .. +128: 2 x 4 sub-tiles of 32 x 32. WN = 2 gives a
// 128 x 256 tile of four wavefronts (two workgroups per CU); WN = 4 a 128 x 512 tile of eight (one
// workgroup per CU, two wavefronts per SIMD, more of the CU's LDS in flight per FLOP).
//
// Operands move HBM -> LDS with gfx950's direct global-to-LDS loads (16 bytes per lane; lane
// l's bytes land at the instruction's LDS base + 16*l), so no registers hold tiles in flight and
// S stages (8 KB of A + WN * 8 KB of B each) are in flight per workgroup. Each DMA instruction takes
// a wave-uniform 64-bit base (SGPRs) plus a 32-bit per-lane byte offset, and each lane picks its
// offset so that the LDS tile comes out XOR-swizzled at 16-byte granularity:
//   A tile [128 rows][32 K], 64 B per row: chunk c of row m sits at slot c ^ ((m >> 2) & 3).
//     A instruction q (0..7; wave w issues the A_DMA instructions from w*A_DMA) loads rows
//     16q .. 16q+15: lane l takes row 16q + l/4, chunk (l & 3) ^ ((l >> 4) & 3).
//   B tile: WN blocks [32 K][128 N] (N-contiguous as stored in HBM), 256 B per row: chunk c of
//     row k sits at slot c ^ (4 * (k & 3)). B instruction q (0..8*WN-1; wave w issues the B_DMA
//     instructions from w*B_DMA) loads block q/8, rows 4*(q%8) .. +3: lane l takes row
//     4*(q%8) + l/16, chunk (l & 15) ^ (4 * ((l >> 4) & 3)) -- the same per-lane offset for every
//     B instruction.
// A fragments are ds_read_b128 of 8 consecutive K values. B fragments come straight from the
// N-contiguous tile with ds_read_b64_tr_b16: within each 16-lane group, lane 4j+q points at row
// kb+j, columns nb+4q..nb+4q+3, and lane i receives column nb+i at rows kb..kb+3; two such reads
// give the 8 K values of one column that the MFMA takes per lane. The swizzles keep each 32 lanes
// of a B read (4 rows x 4 chunks, 8 bytes per lane) and each 16 lanes of an A read (16 rows,
// 16 bytes per lane) on distinct banks of the 64 x 4-byte LDS banks.
#pragma once

#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace stream {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int SBK = 32;
constexpr int SBM = 128;                     // tile rows
constexpr int BLOCK_BYTES = SBK * 128 * 2;   // one 128-column block of the B tile, 8 KB

template <int WN>
struct Geo {
  static_assert(WN == 2 || WN == 4, "two or four wave columns");
  static constexpr int NW = 2 * WN;                 // wavefronts
  static constexpr int COLS = 128 * WN;             // tile columns
  static constexpr int A_BYTES = SBM * SBK * 2;     // 8 KB
  static constexpr int B_BYTES = WN * BLOCK_BYTES;  // 16 or 32 KB
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_DMA = A_BYTES / 1024 / NW;  // A DMA instructions per wave per stage
  static constexpr int B_DMA = B_BYTES / 1024 / NW;  // B DMA instructions per wave per stage
  static constexpr int DMA = A_DMA + B_DMA;
};

// First row of sub-tile u (0 or 1) of wave row wm (0 or 1). The two wave rows take the tile's
// 32-row sub-tiles in turn (wave row wm: sub-tiles wm and 2 + wm), so the live rows of a partly
// filled tile spread over both and over the CU's SIMDs.
__device__ __forceinline__ int sub_row(int wm, int u) { return (2 * u + wm) * 32; }

// this wave row's live 32-row sub-tiles (0, 1 or 2; a prefix in u) given the rows left
__device__ __forceinline__ int live_subtiles(int rows_left, int wm) {
  return (sub_row(wm, 0) < rows_left) + (sub_row(wm, 1) < rows_left);
}

// A-tile row loaded by this lane's i-th A DMA instruction, and the lane's byte offset inside
// that row (16-byte chunk, swizzled)
template <int WN>
__device__ __forceinline__ int a_dma_row(int wave, int i, int lane) {
  return (wave * Geo<WN>::A_DMA + i) * 16 + (lane >> 2);
}
__device__ __forceinline__ int a_dma_chunk_bytes(int lane) { return ((lane & 3) ^ ((lane >> 4) & 3)) << 4; }
// B: 128-column block and first row of this wave's i-th instruction (uniform; a wave's
// instructions load consecutive 4-row groups of one block), and the lane's offset (row within the
// 4-row group, swizzled chunk) for a matrix with row pitch `pitch` bytes
template <int WN>
__device__ __forceinline__ int b_dma_block(int wave) { return (wave * Geo<WN>::B_DMA) >> 3; }
template <int WN>
__device__ __forceinline__ int b_dma_row0(int wave, int i) { return 4 * ((wave * Geo<WN>::B_DMA + i) & 7); }
__device__ __forceinline__ uint32_t b_dma_lane_offset(int lane, uint32_t pitch) {
  return (uint32_t)(lane >> 4) * pitch + ((((lane & 15) ^ (4 * ((lane >> 4) & 3)))) << 4);
}

// The DMA, the wait on it and the workgroup barrier are asm statements with a memory clobber.
// Through the builtins the compiler cannot tell which LDS stage a DMA writes and drains every
// DMA in flight (vmcnt(0)) before each LDS read; here ordering comes only from the explicit
// vmcnt waits. The DMA has no destination register, so nothing the compiler allocates is
// written behind its back.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void barrier_lds_only() { asm volatile("s_barrier" ::: "memory"); }
// the wave's LDS reads have returned, then the workgroup barrier
__device__ __forceinline__ void barrier_after_lds_reads() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16 bytes per lane from base + voff (base wave-uniform, voff per lane) to LDS byte address
// dst_base + 16 * lane (dst_base wave-uniform). NT: with the non-temporal hint, for weight panels
// that no other workgroup reads (an expert with a single row tile).
template <bool NT = false>
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t dst_base) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(base), "s"(dst_base)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(dst_base)
                 : "memory", "m0");
}

__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ bf16x8_t read_a(const lds_char* st, int m, int c) {
  const int off = m * 64 + ((c ^ ((m >> 2) & 3)) << 4);
  return *(const __attribute__((address_space(3))) bf16x8_t*)(st + off);
}

// sb: start of the B region of a stage; n is the tile column (block n / 128)
__device__ __forceinline__ s16x4_t read_b_tr(const lds_char* sb, int k, int n) {
  const int h = n >> 7, c = n & 127;
  const int off = h * BLOCK_BYTES + k * 256 + (((c >> 3) ^ (4 * (k & 3))) << 4) + ((c & 7) << 1);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(sb + off));
}

// acc[i][j] += A * B over nk K-steps of 32.
//   WN: wave columns (Geo); S: LDS stages (DMA lookahead S k-steps); NL: 32-row sub-tiles of
//     this wave holding any valid row (0, 1 or 2; only those are multiplied);
//   lds: the workgroup's S * Geo<WN>::STAGE bytes of LDS;
//   a_base(kt): uniform base of the A rows at k-step kt; a_off[i]: this lane's byte offset for
//     its i-th A instruction (row offset + swizzled chunk);
//   b_base(kt, i): uniform base of this wave's i-th B instruction at k-step kt (its half, its
//     first row); b_off: this lane's byte offset, common to all B instructions;
//   bcol[j]: tile column of the wave's j-th 32-wide B sub-tile.
//
// Schedule. S stages hold k-steps kt .. kt+S-1. Fragments (the A and B operands of one 16-wide
// K sub-step) are read from LDS one sub-step ahead of the MFMAs that use them. In each k-step the
// second sub-step's fragments are requested, the first sub-step's MFMAs are issued, and then the
// wave waits for its own DMAs of the next stage and for its fragment reads, and meets the others
// at the barrier. Past the barrier every wave holds all of stage kt in registers, so the DMAs for
// k-step kt+S go into it, and the next stage's first fragments are read while the second
// sub-step's MFMAs run: LDS latency after the barrier hides behind MFMAs.

// wait until at most n (0 .. 7; more counts as 7) DMA groups of DMA instructions are outstanding
template <int DMA>
__device__ __forceinline__ void wait_groups(int n) {
  static_assert(7 * DMA < 64, "vmcnt range");
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<DMA>(); break;
    case 2: wait_vmcnt<2 * DMA>(); break;
    case 3: wait_vmcnt<3 * DMA>(); break;
    case 4: wait_vmcnt<4 * DMA>(); break;
    case 5: wait_vmcnt<5 * DMA>(); break;
    case 6: wait_vmcnt<6 * DMA>(); break;
    default: wait_vmcnt<7 * DMA>(); break;
  }
}

template <int WN, int S, int NL, int NAD, bool NT, class ABase, class BBase>
__device__ __forceinline__ void mainloop_v(int nk, lds_char* lds, ABase a_base,
                                           const uint32_t (&a_off)[Geo<WN>::A_DMA], BBase b_base, uint32_t b_off,
                                           const int (&bcol)[4], f32x16_t (&acc)[2][4]) {
  static_assert(S >= 3 && S <= 5, "stages");
  static_assert(NAD >= 0 && NAD <= Geo<WN>::A_DMA, "A instructions");
  using GEO = Geo<WN>;
  constexpr int STG = GEO::STAGE;
  constexpr int DMA = NAD + GEO::B_DMA;  // DMA instructions this wave issues per stage
  constexpr int NA = NL > 0 ? NL : 1;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN;
  const int g16 = lane >> 4;
  const int i16 = lane & 15;
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  // With eight wavefronts (two per SIMD, one workgroup per CU) a wave with two live sub-tiles
  // issues its DMAs after its second sub-step's MFMAs rather than right after the barrier: DMA
  // issue stalls while the memory pipe is full, and behind the queued MFMAs that stall no longer
  // idles the matrix unit (prefill gate/up 14.9 -> 14.1 ms). Waves with less MFMA work (the
  // near-empty tiles of decode, bound by streaming the weights) issue at once, keeping the most
  // bytes in flight. The stage is free from the barrier on, and the DMAs still go out before the
  // wave's next wait. (Four-wave tiles, two workgroups per CU, measured no better this way.)
  constexpr bool late = GEO::NW == 8 && NL == 2;

  auto issue = [&](int kt, int stage) {
    const uint32_t dst = lds_base + stage * STG;
    const char* ab = a_base(kt);
#pragma unroll
    for (int i = 0; i < NAD; ++i) dma16(ab, a_off[i], dst + (wave * GEO::A_DMA + i) * 1024);
#pragma unroll
    for (int i = 0; i < GEO::B_DMA; ++i)
      dma16<NT>(b_base(kt, i), b_off, dst + GEO::A_BYTES + (wave * GEO::B_DMA + i) * 1024);
  };
  // fragments of sub-step s (0 or 1) of the stage at st
  auto read = [&](const lds_char* st, int s, bf16x8_t (&a)[NA], bf16x8_t (&b)[4]) {
    if constexpr (NL > 0) {
#pragma unroll
      for (int u = 0; u < NL; ++u) a[u] = read_a(st, sub_row(wm, u) + (lane & 31), 2 * s + (lane >> 5));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kb = 16 * s + 8 * (g16 >> 1) + (i16 >> 2);
        const int n = bcol[j] + 16 * (g16 & 1) + 4 * (i16 & 3);
        const s16x4_t lo = read_b_tr(st + GEO::A_BYTES, kb, n);
        const s16x4_t hi = read_b_tr(st + GEO::A_BYTES, kb + 4, n);
        b[j] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  };
  auto mma = [&](const bf16x8_t (&a)[NA], const bf16x8_t (&b)[4]) {
    if constexpr (NL > 0) {
#pragma unroll
      for (int u = 0; u < NL; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[u][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], b[j], acc[u][j], 0, 0, 0);
    }
  };

  // prologue: S stages in flight, stage 0 complete
#pragma unroll
  for (int i = 0; i < S; ++i)
    if (i < nk) issue(i, i);
  wait_groups<DMA>(min(S - 1, nk - 1));
  barrier_lds_only();

  bf16x8_t a0[NA], b0[4], a1[NA], b1[4];
  read(lds, 0, a0, b0);
  // The last k-step is peeled off: inside the loop every path crosses the barrier, so the
  // compiler's LDS wait before the second sub-step's MFMAs covers only their own fragments (read
  // before the barrier). With the barrier under a branch its merged wait also covered the next
  // stage's fresh reads, and their latency stalled the MFMAs it is meant to hide behind.
  int stage = 0;
  for (int kt = 0; kt < nk - 1; ++kt) {
    const lds_char* cur = lds + stage * STG;
    const int next = stage == S - 1 ? 0 : stage + 1;
    read(cur, 1, a1, b1);
    mma(a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    // stage kt+1 complete once at most the DMAs of k-steps kt+2 .. kt+S-1 are outstanding
    wait_groups<DMA>(min(S - 2, nk - kt - 2));
    barrier_after_lds_reads();
    if (!late && kt + S < nk) issue(kt + S, stage);
    read(lds + next * STG, 0, a0, b0);
    mma(a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    if (late && kt + S < nk) issue(kt + S, stage);
    stage = next;
  }
  if (nk >= 1) {  // k-step nk-1: all DMAs issued (nk-2+S >= nk), no barrier
    read(lds + stage * STG, 1, a1, b1);
    mma(a0, b0);
    mma(a1, b1);
  }
}

// Dispatch outside the K loop on this wave's live 32-row sub-tiles (0, 1 or 2) and on the A
// instructions it must issue: only those whose 16 rows hold a valid row of the tile (rows of them).
// A tile rows past `rows` are then never loaded; the LDS holds stale values there, which only
// reach accumulator rows that are not stored. Every wave takes part in the barriers.
template <int WN, int S, int NL, bool NT, class ABase, class BBase>
__device__ __forceinline__ void mainloop_a(int nad, int nk, lds_char* lds, ABase a_base,
                                           const uint32_t (&a_off)[Geo<WN>::A_DMA], BBase b_base, uint32_t b_off,
                                           const int (&bcol)[4], f32x16_t (&acc)[2][4]) {
  if constexpr (Geo<WN>::A_DMA == 2) {
    if (nad >= 2) mainloop_v<WN, S, NL, 2, NT>(nk, lds, a_base, a_off, b_base, b_off, bcol, acc);
    else if (nad == 1) mainloop_v<WN, S, NL, 1, NT>(nk, lds, a_base, a_off, b_base, b_off, bcol, acc);
    else mainloop_v<WN, S, NL, 0, NT>(nk, lds, a_base, a_off, b_base, b_off, bcol, acc);
  } else {
    if (nad >= 1) mainloop_v<WN, S, NL, 1, NT>(nk, lds, a_base, a_off, b_base, b_off, bcol, acc);
    else mainloop_v<WN, S, NL, 0, NT>(nk, lds, a_base, a_off, b_base, b_off, bcol, acc);
  }
}

// A instructions this wave needs for a tile with `rows` valid rows (instruction q holds rows 16q ..)
template <int WN>
__device__ __forceinline__ int needed_a_dma(int rows, int wave) {
  const int n = (rows + 15) / 16 - wave * Geo<WN>::A_DMA;
  return n < 0 ? 0 : (n > Geo<WN>::A_DMA ? Geo<WN>::A_DMA : n);
}

// nt: B (weight) DMAs with the non-temporal hint -- for panels no other workgroup reads
template <int WN, int S, bool NT, class ABase, class BBase>
__device__ __forceinline__ void mainloop_n(int nk, int nl, int nad, lds_char* lds, ABase a_base,
                                           const uint32_t (&a_off)[Geo<WN>::A_DMA], BBase b_base, uint32_t b_off,
                                           const int (&bcol)[4], f32x16_t (&acc)[2][4]) {
  if (nl >= 2) mainloop_a<WN, S, 2, NT>(nad, nk, lds, a_base, a_off, b_base, b_off, bcol, acc);
  else if (nl == 1) mainloop_a<WN, S, 1, NT>(nad, nk, lds, a_base, a_off, b_base, b_off, bcol, acc);
  else mainloop_a<WN, S, 0, NT>(nad, nk, lds, a_base, a_off, b_base, b_off, bcol, acc);
}

template <int WN, int S, class ABase, class BBase>
__device__ __forceinline__ void mainloop(int nk, int nl, int rows, lds_char* lds, ABase a_base,
                                         const uint32_t (&a_off)[Geo<WN>::A_DMA], BBase b_base, uint32_t b_off,
                                         const int (&bcol)[4], f32x16_t (&acc)[2][4], bool nt = false) {
  const int nad = needed_a_dma<WN>(rows, __builtin_amdgcn_readfirstlane(threadIdx.x >> 6));
  if (nt) mainloop_n<WN, S, true>(nk, nl, nad, lds, a_base, a_off, b_base, b_off, bcol, acc);
  else mainloop_n<WN, S, false>(nk, nl, nad, lds, a_base, a_off, b_base, b_off, bcol, acc);
}


__device__ __forceinline__ void zero(f32x16_t (&acc)[2][4]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}

// ------------------------------------------------------------------------------------------------
// Tall tiles for groups of a few hundred rows: 160 x 512, eight wavefronts, each holding every row
// of the tile (five 32-row sub-tiles) and 64 columns (two 32-wide sub-tiles), 160 fp32
// accumulators per lane. An expert's rows are split over ceil(rows / 160) row tiles in whole
// 32-row sub-tiles, as evenly as possible: ~320 rows take two row tiles instead of the three of
// 128 rows, so the weight panels are streamed from L2 into LDS twice instead of three times, and
// the two tiles do equal work, run in step and share each panel through L2. Per K step the CU
// moves 10 KB of A and 32 KB of B for 5.2 MFLOP (128 x 512 tiles: 40 KB for 4.2 MFLOP).
//   LDS per stage: A [160 rows][32 K] (10 instructions of 16 rows; wave w issues instructions w
//   and w + 8) in the layout and swizzle of the 128-row tiles, then the same B tile of four
//   128-column blocks (wave w fills rows 16 (w % 2) .. +16 of block w / 2).
// ------------------------------------------------------------------------------------------------
namespace tall {
constexpr int ROWS = 160;                  // tile rows: five 32-row sub-tiles
constexpr int SUB = ROWS / 32;
constexpr int NW = 8;                      // wavefronts
constexpr int A_BYTES = ROWS * SBK * 2;    // 10 KB
constexpr int A_INSTR = A_BYTES / 1024;    // 10
constexpr int B_BYTES = 4 * BLOCK_BYTES;   // 32 KB
constexpr int B_DMA = B_BYTES / 1024 / NW; // 4 per wave
constexpr int STAGE = A_BYTES + B_BYTES;   // 42 KB
constexpr int A_DMA = (A_INSTR + NW - 1) / NW;  // at most 2 A instructions per wave

// A instructions this wave issues for a tile with `rows` valid rows: instructions w and w + 8,
// those whose 16 rows hold a valid row
__device__ __forceinline__ int needed_a(int rows, int wave) {
  const int n = (rows + 15) / 16;  // instructions 0 .. n-1 hold valid rows
  return (wave < n) + (wave + NW < n);
}

template <int S, int NL, int NAD, bool NT, class ABase, class BBase>
__device__ __forceinline__ void mainloop_v(int nk, lds_char* lds, ABase a_base, const uint32_t (&a_off)[A_DMA],
                                           BBase b_base, uint32_t b_off, const int (&bcol)[2],
                                           f32x16_t (&acc)[SUB][2]) {
  static_assert(S >= 2 && S <= 3, "stages");
  static_assert(NL >= 0 && NL <= SUB, "sub-tiles");
  constexpr int DMA = NAD + B_DMA;
  constexpr int NA = NL > 0 ? NL : 1;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g16 = lane >> 4;
  const int i16 = lane & 15;
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  // a wave with three or more live sub-tiles issues its DMAs behind its second sub-step's
  // MFMAs, so that a stalled DMA issue does not idle the matrix unit (as in the 128 x 512 tiles)
  constexpr bool late = NL >= 3;

  auto issue = [&](int kt, int stage) {
    const uint32_t dst = lds_base + stage * STAGE;
    const char* ab = a_base(kt);
#pragma unroll
    for (int i = 0; i < NAD; ++i) dma16(ab, a_off[i], dst + (wave + NW * i) * 1024);
#pragma unroll
    for (int i = 0; i < B_DMA; ++i) dma16<NT>(b_base(kt, i), b_off, dst + A_BYTES + (wave * B_DMA + i) * 1024);
  };
  auto read = [&](const lds_char* st, int s, bf16x8_t (&a)[NA], bf16x8_t (&b)[2]) {
    if constexpr (NL > 0) {
#pragma unroll
      for (int u = 0; u < NL; ++u) a[u] = read_a(st, u * 32 + (lane & 31), 2 * s + (lane >> 5));
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int kb = 16 * s + 8 * (g16 >> 1) + (i16 >> 2);
        const int n = bcol[j] + 16 * (g16 & 1) + 4 * (i16 & 3);
        const s16x4_t lo = read_b_tr(st + A_BYTES, kb, n);
        const s16x4_t hi = read_b_tr(st + A_BYTES, kb + 4, n);
        b[j] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  };
  // operands swapped (B fragment first): each accumulator holds the transposed 32 x 32 block, so
  // that a lane ends up with four consecutive columns of one row per register group (the
  // epilogue then stages 8 bytes per store instead of 2)
  auto mma = [&](const bf16x8_t (&a)[NA], const bf16x8_t (&b)[2]) {
    if constexpr (NL > 0) {
#pragma unroll
      for (int u = 0; u < NL; ++u)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[u][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[u], acc[u][j], 0, 0, 0);
    }
  };

  // prologue: S stages in flight, stage 0 complete
#pragma unroll
  for (int i = 0; i < S; ++i)
    if (i < nk) issue(i, i);
  wait_groups<DMA>(min(S - 1, nk - 1));
  barrier_lds_only();

  bf16x8_t a0[NA], b0[2], a1[NA], b1[2];
  read(lds, 0, a0, b0);
  // k-steps 0 .. nk-2 cross the barrier; the last one is peeled (see the 128-row mainloop)
  int stage = 0;
  for (int kt = 0; kt < nk - 1; ++kt) {
    const lds_char* cur = lds + stage * STAGE;
    const int next = stage == S - 1 ? 0 : stage + 1;
    read(cur, 1, a1, b1);
    mma(a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    wait_groups<DMA>(min(S - 2, nk - kt - 2));
    barrier_after_lds_reads();
    if (!late && kt + S < nk) issue(kt + S, stage);
    read(lds + next * STAGE, 0, a0, b0);
    mma(a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    if (late && kt + S < nk) issue(kt + S, stage);
    stage = next;
  }
  if (nk >= 1) {
    read(lds + stage * STAGE, 1, a1, b1);
    mma(a0, b0);
    mma(a1, b1);
  }
}

template <int S, int NL, bool NT, class ABase, class BBase>
__device__ __forceinline__ void mainloop_a(int nad, int nk, lds_char* lds, ABase a_base,
                                           const uint32_t (&a_off)[A_DMA], BBase b_base, uint32_t b_off,
                                           const int (&bcol)[2], f32x16_t (&acc)[SUB][2]) {
  if (nad >= 2) mainloop_v<S, NL, 2, NT>(nk, lds, a_base, a_off, b_base, b_off, bcol, acc);
  else if (nad == 1) mainloop_v<S, NL, 1, NT>(nk, lds, a_base, a_off, b_base, b_off, bcol, acc);
  else mainloop_v<S, NL, 0, NT>(nk, lds, a_base, a_off, b_base, b_off, bcol, acc);
}

// acc[u][j] += A * B over nk K-steps for a tile with `rows` valid rows (1 .. 160): dispatch on the
// live sub-tiles (every wave multiplies all of them) and on this wave's A instructions
template <int S, bool NT, class ABase, class BBase>
__device__ __forceinline__ void mainloop_n(int nk, int rows, lds_char* lds, ABase a_base,
                                           const uint32_t (&a_off)[A_DMA], BBase b_base, uint32_t b_off,
                                           const int (&bcol)[2], f32x16_t (&acc)[SUB][2]) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nad = needed_a(rows, wave);
  const int nl = (rows + 31) / 32;
  switch (nl) {
    case 5: mainloop_a<S, 5, NT>(nad, nk, lds, a_base, a_off, b_base, b_off, bcol, acc); break;
    case 4: mainloop_a<S, 4, NT>(nad, nk, lds, a_base, a_off, b_base, b_off, bcol, acc); break;
    case 3: mainloop_a<S, 3, NT>(nad, nk, lds, a_base, a_off, b_base, b_off, bcol, acc); break;
    case 2: mainloop_a<S, 2, NT>(nad, nk, lds, a_base, a_off, b_base, b_off, bcol, acc); break;
    default: mainloop_a<S, 1, NT>(nad, nk, lds, a_base, a_off, b_base, b_off, bcol, acc); break;
  }
}

// nt: B (weight) DMAs with the non-temporal hint, for a group with a single row tile (the only
// reader of its weight panels)
template <int S, class ABase, class BBase>
__device__ __forceinline__ void mainloop(int nk, int rows, lds_char* lds, ABase a_base,
                                         const uint32_t (&a_off)[A_DMA], BBase b_base, uint32_t b_off,
                                         const int (&bcol)[2], f32x16_t (&acc)[SUB][2], bool nt) {
  if (nt) mainloop_n<S, true>(nk, rows, lds, a_base, a_off, b_base, b_off, bcol, acc);
  else mainloop_n<S, false>(nk, rows, lds, a_base, a_off, b_base, b_off, bcol, acc);
}

__device__ __forceinline__ void zero(f32x16_t (&acc)[SUB][2]) {
#pragma unroll
  for (int i = 0; i < SUB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}
}  // namespace tall

// ------------------------------------------------------------------------------------------------
// 192-row tiles, for the groups that need fewer row tiles of 192 than of 160 rows, at most two
// (161 .. 192 and 321 .. 384 rows): 192 x 512 on eight wavefronts in two wave rows of four. Wave
// (wm, wn) holds the 32-row sub-tiles wm, wm + 2, wm + 4 (a partly filled tile keeps its live rows
// spread over both wave rows, so over every SIMD) and columns 128 wn .. +128 (gate/up: gate
// columns 64 wn .. +64 and the up columns with the same indices), 192 accumulators per lane, two
// wavefronts per SIMD. Against 160-row tiles such a group's weight panels cross from L2 into LDS
// once fewer, and per FLOP the CU moves 7.0 instead of 8.0 KB per MFLOP from L2 into LDS -- the
// prefill GEMMs run power-limited, with the clock set mostly by that traffic.
//   LDS per stage: A [192 rows][32 K] (12 instructions of 16 rows; wave w issues w and w + 8 when
//   < 12) in the swizzle of the 128-row tiles, then the B tile of four 128-column blocks (wave w
//   fills rows 16 (w % 2) .. +16 of block w / 2).
// ------------------------------------------------------------------------------------------------
namespace wide {
constexpr int ROWS = 192;
constexpr int NW = 8;
constexpr int A_BYTES = ROWS * SBK * 2;     // 12 KB
constexpr int A_INSTR = A_BYTES / 1024;     // 12
constexpr int A_DMA = 2;                    // at most two A instructions per wave
constexpr int B_BYTES = 4 * BLOCK_BYTES;    // 32 KB
constexpr int B_DMA = B_BYTES / 1024 / NW;  // 4 per wave
constexpr int STAGE = A_BYTES + B_BYTES;    // 44 KB

// this wave row's live sub-tiles (a prefix of u = 0, 1, 2: tile sub-tile wm + 2u) given the rows
__device__ __forceinline__ int live(int rows, int wm) {
  const int n = (rows + 31) / 32;
  return (wm < n) + (wm + 2 < n) + (wm + 4 < n);
}
__device__ __forceinline__ int needed_a(int rows, int wave) {
  const int n = (rows + 15) / 16;
  return (wave < n) + (wave + NW < n);
}

template <int S, int NL, int NAD, bool NT, class ABase, class BBase>
__device__ __forceinline__ void mainloop_v(int nk, lds_char* lds, ABase a_base, const uint32_t (&a_off)[A_DMA],
                                           BBase b_base, uint32_t b_off, const int (&bcol)[4],
                                           f32x16_t (&acc)[3][4]) {
  static_assert(S >= 2 && S <= 3, "stages");
  static_assert(NL >= 0 && NL <= 3, "sub-tiles");
  constexpr int DMA = NAD + B_DMA;
  constexpr int NA = NL > 0 ? NL : 1;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 2;
  const int g16 = lane >> 4;
  const int i16 = lane & 15;
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  constexpr bool late = NL >= 2;

  auto issue = [&](int kt, int stage) {
    const uint32_t dst = lds_base + stage * STAGE;
    const char* ab = a_base(kt);
#pragma unroll
    for (int i = 0; i < NAD; ++i) dma16(ab, a_off[i], dst + (wave + NW * i) * 1024);
#pragma unroll
    for (int i = 0; i < B_DMA; ++i) dma16<NT>(b_base(kt, i), b_off, dst + A_BYTES + (wave * B_DMA + i) * 1024);
  };
  auto read = [&](const lds_char* st, int s, bf16x8_t (&a)[NA], bf16x8_t (&b)[4]) {
    if constexpr (NL > 0) {
#pragma unroll
      for (int u = 0; u < NL; ++u) a[u] = read_a(st, (wm + 2 * u) * 32 + (lane & 31), 2 * s + (lane >> 5));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kb = 16 * s + 8 * (g16 >> 1) + (i16 >> 2);
        const int n = bcol[j] + 16 * (g16 & 1) + 4 * (i16 & 3);
        const s16x4_t lo = read_b_tr(st + A_BYTES, kb, n);
        const s16x4_t hi = read_b_tr(st + A_BYTES, kb + 4, n);
        b[j] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  };
  auto mma = [&](const bf16x8_t (&a)[NA], const bf16x8_t (&b)[4]) {
    if constexpr (NL > 0) {
#pragma unroll
      for (int u = 0; u < NL; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[u][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[u], acc[u][j], 0, 0, 0);
    }
  };

#pragma unroll
  for (int i = 0; i < S; ++i)
    if (i < nk) issue(i, i);
  wait_groups<DMA>(min(S - 1, nk - 1));
  barrier_lds_only();

  bf16x8_t a0[NA], b0[4], a1[NA], b1[4];
  read(lds, 0, a0, b0);
  int stage = 0;
  for (int kt = 0; kt < nk - 1; ++kt) {
    const lds_char* cur = lds + stage * STAGE;
    const int next = stage == S - 1 ? 0 : stage + 1;
    read(cur, 1, a1, b1);
    mma(a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    wait_groups<DMA>(min(S - 2, nk - kt - 2));
    barrier_after_lds_reads();
    if (!late && kt + S < nk) issue(kt + S, stage);
    read(lds + next * STAGE, 0, a0, b0);
    mma(a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    if (late && kt + S < nk) issue(kt + S, stage);
    stage = next;
  }
  if (nk >= 1) {
    read(lds + stage * STAGE, 1, a1, b1);
    mma(a0, b0);
    mma(a1, b1);
  }
}

template <int S, int NL, bool NT, class ABase, class BBase>
__device__ __forceinline__ void mainloop_a(int nad, int nk, lds_char* lds, ABase a_base,
                                           const uint32_t (&a_off)[A_DMA], BBase b_base, uint32_t b_off,
                                           const int (&bcol)[4], f32x16_t (&acc)[3][4]) {
  if (nad >= 2) mainloop_v<S, NL, 2, NT>(nk, lds, a_base, a_off, b_base, b_off, bcol, acc);
  else if (nad == 1) mainloop_v<S, NL, 1, NT>(nk, lds, a_base, a_off, b_base, b_off, bcol, acc);
  else mainloop_v<S, NL, 0, NT>(nk, lds, a_base, a_off, b_base, b_off, bcol, acc);
}

template <int S, class ABase, class BBase>
__device__ __forceinline__ void mainloop(int nk, int rows, lds_char* lds, ABase a_base,
                                         const uint32_t (&a_off)[A_DMA], BBase b_base, uint32_t b_off,
                                         const int (&bcol)[4], f32x16_t (&acc)[3][4], bool nt) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nad = needed_a(rows, wave);
  const int nl = live(rows, wave >> 2);
  auto go = [&](auto ntc) {
    constexpr bool N = decltype(ntc)::value;
    switch (nl) {
      case 3: mainloop_a<S, 3, N>(nad, nk, lds, a_base, a_off, b_base, b_off, bcol, acc); break;
      case 2: mainloop_a<S, 2, N>(nad, nk, lds, a_base, a_off, b_base, b_off, bcol, acc); break;
      case 1: mainloop_a<S, 1, N>(nad, nk, lds, a_base, a_off, b_base, b_off, bcol, acc); break;
      default: mainloop_a<S, 0, N>(nad, nk, lds, a_base, a_off, b_base, b_off, bcol, acc); break;
    }
  };
  if (nt) go(std::true_type());
  else go(std::false_type());
}
}  // namespace wide

// Workgroup-index remap so that consecutive logical tiles run on the same XCD: workgroups are
// dispatched round-robin over the 8 XCDs, so physical block b runs on XCD b % 8. Logical tiles
// [x*q + min(x, r), ...) of n = 8q + r go to XCD x, in order. Returns -1 for b >= n.
__device__ __forceinline__ int xcd_remap(int b, int n) {
  if (b >= n) return -1;
  const int q = n >> 3, r = n & 7;
  const int x = b & 7, i = b >> 3;
  return x * q + min(x, r) + i;
}

}  // namespace stream
}  // namespace moe
