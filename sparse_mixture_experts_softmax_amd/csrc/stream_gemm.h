// Streaming bf16 MFMA tile mainloop for gfx950, shared by the grouped expert GEMMs and the
// router GEMM.
//
// One 256-thread workgroup (4 wavefronts in 2x2) accumulates a 128 x 256 fp32 tile
// acc += A[128 x K] * B[K x 256] with v_mfma_f32_32x32x16_bf16 (each wavefront 64 x 128).
//
// Operands move HBM -> LDS with gfx950's direct global-to-LDS loads (16 bytes per lane; lane
// l's bytes land at the instruction's LDS base + 16*l), so no registers hold tiles in flight and
// three 24 KB stages are in flight per workgroup. Each DMA instruction takes a wave-uniform
// 64-bit base (SGPRs) plus a 32-bit per-lane byte offset, and each lane picks its offset so
// that the LDS tile comes out XOR-swizzled at 16-byte granularity:
//   A tile [128 rows][32 K], 64 B per row: chunk c of row m sits at slot c ^ ((m >> 2) & 3).
//     A instruction q (0..7, wave w issues q = 2w, 2w+1) loads rows 16q .. 16q+15:
//     lane l takes row 16q + l/4, chunk (l & 3) ^ ((l >> 4) & 3).
//   B tile: two halves [32 K][128 N] (N-contiguous as stored in HBM), 256 B per row: chunk c
//     of row k sits at slot c ^ (2 * (k & 3)). B instruction q (0..15, wave w issues 4w..4w+3)
//     loads half q/8, rows 4*(q%8) .. +3: lane l takes row 4*(q%8) + l/16, chunk
//     (l & 15) ^ (2 * ((l >> 4) & 3)) -- the same per-lane offset for every B instruction.
// A fragments are ds_read_b128 of 8 consecutive K values. B fragments come straight from the
// N-contiguous tile with ds_read_b64_tr_b16: within each 16-lane group, lane 4j+q points at row
// kb+j, columns nb+4q..nb+4q+3, and lane i receives column nb+i at rows kb..kb+3; two such reads
// give the 8 K values of one column that the MFMA takes per lane. Both swizzles keep the 16
// lanes of a B read and each 8 lanes of an A read on distinct banks.
#pragma once

#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace stream {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int SBM = 128;
constexpr int SBK = 32;
constexpr int SBN = 256;
constexpr int A_BYTES = SBM * SBK * 2;       // 8 KB
constexpr int B_BYTES = SBK * SBN * 2;       // 16 KB
constexpr int STAGE = A_BYTES + B_BYTES;     // 24 KB
constexpr int A_DMA = A_BYTES / 1024 / 4;    // DMA instructions per wave per stage: 2
constexpr int B_DMA = B_BYTES / 1024 / 4;    // 4
constexpr int DMA_PER_STAGE = A_DMA + B_DMA;

constexpr int HALF_BYTES = B_BYTES / 2;     // one 128-column half of the B tile

// A-tile row loaded by this lane's i-th A DMA instruction, and the lane's byte offset inside
// that row (16-byte chunk, swizzled)
__device__ __forceinline__ int a_dma_row(int wave, int i, int lane) { return (wave * A_DMA + i) * 16 + (lane >> 2); }
__device__ __forceinline__ int a_dma_chunk_bytes(int lane) { return ((lane & 3) ^ ((lane >> 4) & 3)) << 4; }
// B: half and first row of this wave's i-th instruction (uniform), and the lane's offset
// (row within the 4-row block, swizzled chunk) for a matrix with row pitch `pitch` bytes
__device__ __forceinline__ int b_dma_half(int wave) { return wave >> 1; }
__device__ __forceinline__ int b_dma_row0(int wave, int i) { return 4 * ((wave * B_DMA + i) & 7); }
__device__ __forceinline__ uint32_t b_dma_lane_offset(int lane, uint32_t pitch) {
  return (uint32_t)(lane >> 4) * pitch + ((((lane & 15) ^ (2 * ((lane >> 4) & 3)))) << 4);
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

// 16 bytes per lane from base + voff (base wave-uniform, voff per lane) to LDS byte address
// dst_base + 16 * lane (dst_base wave-uniform)
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t dst_base) {
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

// n is the tile column 0..255 (half n / 128)
__device__ __forceinline__ s16x4_t read_b_tr(const lds_char* st, int k, int n) {
  const int h = n >> 7, c = n & 127;
  const int off = A_BYTES + h * HALF_BYTES + k * 256 + (((c >> 3) ^ (2 * (k & 3))) << 4) + ((c & 7) << 1);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(st + off));
}

// acc[i][j] += A * B over nk K-steps of 32, for a wave with NI (1 or 2) live 32-row sub-tiles.
//   lds: the workgroup's 3 * STAGE bytes of LDS;
//   a_base(kt): uniform base of the A rows at k-step kt; a_off[i]: this lane's byte offset for
//     its i-th A instruction (row offset + swizzled chunk);
//   b_base(kt, i): uniform base of this wave's i-th B instruction at k-step kt (its half, its
//     first row); b_off: this lane's byte offset, common to all B instructions;
//   bcol[j]: tile column of the wave's j-th 32-wide B sub-tile.
template <int NI, class ABase, class BBase>
__device__ __forceinline__ void mainloop_n(int nk, lds_char* lds, ABase a_base, const uint32_t (&a_off)[A_DMA],
                                           BBase b_base, uint32_t b_off, const int (&bcol)[4],
                                           f32x16_t (&acc)[2][4]) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1;
  const int g16 = lane >> 4;
  const int i16 = lane & 15;
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);

  auto issue = [&](int kt, int stage) {
    const uint32_t dst = lds_base + stage * STAGE;
    const char* ab = uniform_ptr(a_base(kt));
#pragma unroll
    for (int i = 0; i < A_DMA; ++i) dma16(ab, a_off[i], dst + (wave * A_DMA + i) * 1024);
#pragma unroll
    for (int i = 0; i < B_DMA; ++i)
      dma16(uniform_ptr(b_base(kt, i)), b_off, dst + A_BYTES + (wave * B_DMA + i) * 1024);
  };

  auto compute = [&](const lds_char* st) {
    if constexpr (NI > 0) {
#pragma unroll
    for (int s = 0; s < SBK / 16; ++s) {
      bf16x8_t a[NI], b[4];
#pragma unroll
      for (int i = 0; i < NI; ++i) a[i] = read_a(st, wm * 64 + i * 32 + (lane & 31), 2 * s + (lane >> 5));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kb = 16 * s + 8 * (g16 >> 1) + (i16 >> 2);
        const int n = bcol[j] + 16 * (g16 & 1) + 4 * (i16 & 3);
        const s16x4_t lo = read_b_tr(st, kb, n);
        const s16x4_t hi = read_b_tr(st, kb + 4, n);
        b[j] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    }
  };

  issue(0, 0);
  if (nk > 1) issue(1, 1);
  // k-step kt: stage kt is complete once at most one later stage's DMAs are outstanding. Each
  // wave waits for its own DMAs, then the bare barrier makes stage kt whole for everyone; it
  // also guarantees every wave finished reading stage kt-1, which the next DMAs overwrite.
  int stage = 0;
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) wait_vmcnt<DMA_PER_STAGE>();
    else wait_vmcnt<0>();
    barrier_lds_only();
    if (kt + 2 < nk) issue(kt + 2, stage == 0 ? 2 : stage - 1);
    compute(lds + stage * STAGE);
    stage = stage == 2 ? 0 : stage + 1;
  }
}

// Dispatch on the wave's live 32-row sub-tiles (0, 1 or 2) outside the K loop.
template <class ABase, class BBase>
__device__ __forceinline__ void mainloop(int nk, int nlive, lds_char* lds, ABase a_base,
                                         const uint32_t (&a_off)[A_DMA], BBase b_base, uint32_t b_off,
                                         const int (&bcol)[4], f32x16_t (&acc)[2][4]) {
  // every wave must take part in the barriers even when it has no live rows
  if (nlive >= 2) mainloop_n<2>(nk, lds, a_base, a_off, b_base, b_off, bcol, acc);
  else if (nlive == 1) mainloop_n<1>(nk, lds, a_base, a_off, b_base, b_off, bcol, acc);
  else mainloop_n<0>(nk, lds, a_base, a_off, b_base, b_off, bcol, acc);
}

__device__ __forceinline__ void zero(f32x16_t (&acc)[2][4]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}

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
