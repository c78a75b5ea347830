// Routed and shared SwiGLU experts as grouped GEMMs.
//
// Each expert is a feed-forward network with the silu activation and three
// bias-free matrices, gate and up [d, I] and down [I, d] (Qwen3.8-Max
// architecture page, config.json listing: hidden_act, moe_intermediate_size,
// shared_expert_intermediate_size; the overview page's parameter table counts
// 3*d*I per expert). For the rows of group g (expert g's sorted slots, or all T
// tokens for the shared expert, g = E):
//
//   ffn1:  H = silu(A Wg) * (A Wu),  A = x gathered through sorted_token
//   ffn2:  Y = H Wd
//
// Paths, chosen per call by ffn_plan:
//   - bf16, aligned shapes: the streaming MFMA kernel (ffn_mfma_stream_kernel, mainloop in
//     stream_gemm.h) on 128 x 256 or 128 x 512 tiles, global-to-LDS DMA, K split for few tokens;
//   - bf16, one or two tokens: the skinny kernels (grouped_ffn_skinny.hip), weight streams on the
//     vector ALUs;
//   - bf16, other shapes: the generic MFMA kernel (ffn_mfma_kernel): 256-thread workgroups (4
//     wavefronts in 2x2) on 128-row tiles with v_mfma_f32_32x32x16_bf16, K step 32,
//     double-buffered LDS; the weights are stored N-contiguous ([K, N] row-major) while MFMA wants
//     8 consecutive K values per lane, so each thread loads a 4(K) x 8(N) block of B with 16-byte
//     loads, transposes it in registers and writes it K-contiguous into LDS;
//   - fp32: 64x64 tiles on the vector ALUs, 4x4 outputs per thread (ffn_f32_kernel).
// In every path ffn1 keeps the gate and up sums of the same (row, column) together, so silu(g)*u
// is applied in registers and H is written once.
//
// Row tiles come from a device-built tile list (group, first row), so the host
// launches an upper bound of tiles without knowing the routing; surplus
// workgroups exit at once.
#include "moe_internal.h"
#include "stream_gemm.h"

namespace moe {
namespace {

using stream::bf16x8_t;
using stream::f32x16_t;

// ------------------------------------------------------------------------------------------
// tile list: for each group with n rows, ceil(n / BM) tiles (group, first row)
// ------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(1024)
build_tiles_kernel(const int32_t* __restrict__ offsets, int64_t T, int E, int has_shared, int BM, int BM2,
                   int32_t* __restrict__ tile_group, int32_t* __restrict__ tile_m0, int32_t* __restrict__ tile_count,
                   int32_t* __restrict__ split_cnt, int64_t cnt_each, int per_tile) {
  __shared__ int s_rows[kMaxGroups];
  __shared__ int s_w[17];
  const int G = E + has_shared;
  for (int g = threadIdx.x; g < G; g += 1024) s_rows[g] = g < E ? offsets[g + 1] - offsets[g] : (int)T;
  __syncthreads();
  build_tile_list(s_rows, G, BM, BM2, s_w, tile_group, tile_m0, tile_count, split_cnt, cnt_each, per_tile);
}

// ------------------------------------------------------------------------------------------
// bf16 MFMA grouped GEMM
// ------------------------------------------------------------------------------------------
constexpr int BM = kMfmaBM;  // 128 rows
constexpr int BK = 32;       // K step
constexpr int LDK = BK + 8;  // LDS row stride in bf16 (80 bytes) to spread banks
constexpr int BNL = 256;     // LDS B tile columns: gate 128 + up 128, or 256 down columns

struct MfmaArgs {
  const bf16_t* a_src;  // ffn1: x [T, d]; ffn2: H [rows_total, ldh]
  const int32_t* offsets;
  const int32_t* sorted_token;
  const bf16_t* w0;  // ffn1: Wg [E, d, I]; ffn2: Wd [E, I, d]
  const bf16_t* w1;  // ffn1: Wu; ffn2: unused
  const bf16_t* w0_s;
  const bf16_t* w1_s;
  bf16_t* out;  // ffn1: H; ffn2: Y
  const int32_t* tile_group;
  const int32_t* tile_m0;
  const int32_t* tile_count;
  int64_t T;
  int d, E, k, I, Is, ldh;
  int n_ntiles;
  // split-K (streaming gate/up kernel): splits > 1 -> fp32 partial rows part[split][row][part_ld],
  // added by gate_up_finish_kernel
  int splits;
  int balance;  // streaming kernel: split each group's rows evenly over its row tiles
  float* part;
  int64_t part_ld, part_sstride;
};

// Transpose a 4(K) x 8(N) block of bf16 (rows r[0..3], each 8 N-consecutive
// values in a uint4) into 8 columns of 4 K-consecutive values (uint2 each).
__device__ __forceinline__ void transpose4x8(const uint4 r[4], uint2 c[8]) {
  const uint32_t* r0 = (const uint32_t*)&r[0];
  const uint32_t* r1 = (const uint32_t*)&r[1];
  const uint32_t* r2 = (const uint32_t*)&r[2];
  const uint32_t* r3 = (const uint32_t*)&r[3];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    // columns 2p (low halves) and 2p+1 (high halves)
    c[2 * p].x = (r0[p] & 0xFFFFu) | (r1[p] << 16);
    c[2 * p].y = (r2[p] & 0xFFFFu) | (r3[p] << 16);
    c[2 * p + 1].x = (r0[p] >> 16) | (r1[p] & 0xFFFF0000u);
    c[2 * p + 1].y = (r2[p] >> 16) | (r3[p] & 0xFFFF0000u);
  }
}

template <bool GATED>
__global__ void __launch_bounds__(256, 2)
ffn_mfma_kernel(MfmaArgs p) {
  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM][LDK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BNL][LDK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;  // wave row block: rows wm*64 .. +64
  const int wn = wave & 1;   // wave column block

  const int mt = blockIdx.x / p.n_ntiles;
  const int nt = blockIdx.x % p.n_ntiles;
  if (mt >= *p.tile_count) return;
  const int g = p.tile_group[mt];
  const int m0 = p.tile_m0[mt];
  const Group G = group_info(g, p.offsets, p.T, p.k, p.E, p.I, p.Is);

  // problem sizes of this GEMM
  const int K = GATED ? p.d : G.n_inter;
  const int N = GATED ? G.n_inter : p.d;
  const int n0 = nt * (GATED ? kMfmaBN1 : kMfmaBN2);
  if (n0 >= N) return;

  const bf16_t* W0;
  const bf16_t* W1 = nullptr;
  if (GATED) {
    W0 = G.shared ? p.w0_s : p.w0 + (size_t)g * p.d * p.I;
    W1 = G.shared ? p.w1_s : p.w1 + (size_t)g * p.d * p.I;
  } else {
    W0 = G.shared ? p.w0_s : p.w0 + (size_t)g * p.I * p.d;
  }

  // ---- A loader: rows tid/4 and tid/4 + 64, 8 K values at (tid%4)*8
  const int a_kq = (tid & 3) * 8;
  const bf16_t* a_ptr[2];
  bool a_ok[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = (tid >> 2) + 64 * h;
    a_ok[h] = m0 + r < G.rows;
    int64_t src_row;
    if (GATED)
      src_row = G.shared ? (int64_t)(m0 + r) : (int64_t)p.sorted_token[G.row0 + m0 + (a_ok[h] ? r : 0)];
    else
      src_row = G.row0 + m0 + (a_ok[h] ? r : 0);
    if (GATED && G.shared && !a_ok[h]) src_row = 0;
    a_ptr[h] = p.a_src + src_row * (GATED ? (int64_t)p.d : (int64_t)p.ldh);
  }
  // ---- B loader: block (kb, nb): rows 4*kb .. +4, 8 columns
  const int b_nb = tid & 31;
  const int b_kb = tid >> 5;  // 0..7
  const bf16_t* b_base;
  int b_col;  // global column of this thread's 8-column block
  int b_lds_n;
  if (GATED) {
    b_base = (b_nb < 16) ? W0 : W1;
    b_col = n0 + (b_nb & 15) * 8;
    b_lds_n = (b_nb >> 4) * 128 + (b_nb & 15) * 8;
  } else {
    b_base = W0;
    b_col = n0 + b_nb * 8;
    b_lds_n = b_nb * 8;
  }
  const bool b_col_ok = b_col < N;

  uint4 ra[2];
  uint4 rb[4];
  auto load_tiles = [&](int k0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kk = k0 + a_kq;
      ra[h] = (a_ok[h] && kk < K) ? *(const uint4*)(a_ptr[h] + kk) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kk = k0 + b_kb * 4 + r;
      rb[r] = (b_col_ok && kk < K) ? *(const uint4*)(b_base + (int64_t)kk * N + b_col) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tiles = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) *(uint4*)&As[buf][(tid >> 2) + 64 * h][a_kq] = ra[h];
    uint2 c[8];
    transpose4x8(rb, c);
#pragma unroll
    for (int j = 0; j < 8; ++j) *(uint2*)&Bs[buf][b_lds_n + j][b_kb * 4] = c[j];
  };

  f32x16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // LDS columns of the wave's four 32-wide B sub-tiles
  int bcol[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) bcol[j] = GATED ? (j >> 1) * 128 + wn * 64 + (j & 1) * 32 : wn * 128 + j * 32;

  const int nk = (K + BK - 1) / BK;
  load_tiles(0);
  store_tiles(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tiles((kt + 1) * BK);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int kofs = s * 16 + (lane >> 5) * 8;
      bf16x8_t a[2], b[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = *(const bf16x8_t*)&As[buf][wm * 64 + i * 32 + (lane & 31)][kofs];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = *(const bf16x8_t*)&Bs[buf][bcol[j] + (lane & 31)][kofs];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_tiles(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue. 32x32 accumulator: lane holds column (lane & 31); register r
  // holds row 8*(r/4) + 4*(lane/32) + (r%4).
  const int col_in = lane & 31;
  const int row_hi = (lane >> 5) * 4;
  if (GATED) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int col = n0 + wn * 64 + jj * 32 + col_in;
        if (col >= N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * 64 + i * 32 + (r >> 2) * 8 + row_hi + (r & 3);
          if (m0 + row < G.rows) {
            const float gv = acc[i][jj][r];
            const float uv = acc[i][jj + 2][r];
            p.out[(G.row0 + m0 + row) * (int64_t)p.ldh + col] = f32_to_bf16(silu_f32(gv) * uv);
          }
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 128 + j * 32 + col_in;
        if (col >= N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * 64 + i * 32 + (r >> 2) * 8 + row_hi + (r & 3);
          if (m0 + row < G.rows) p.out[(G.row0 + m0 + row) * (int64_t)p.d + col] = f32_to_bf16(acc[i][j][r]);
        }
      }
  }
}

// ------------------------------------------------------------------------------------------
// bf16 MFMA grouped GEMM, streaming variant for aligned shapes (K % 32 == 0, N % tile == 0):
// the shared DMA/LDS-transpose mainloop of stream_gemm.h on 128 x (128*WN) tiles. WN = 2: four
// wavefronts per workgroup and two workgroups per CU, so that one workgroup's prologue and
// epilogue overlap the other's mainloop. WN = 4: eight wavefronts and one workgroup per CU, with
// more LDS bytes in flight per FLOP for long K loops. For the gate/up product the tile's columns
// are half gate, half up: columns [0, 64*WN) of the tile are gate columns n0 .. and the next
// 64*WN the up columns with the same indices, so each wavefront holds matching gate and up
// accumulators for the fused silu(g)*u epilogue.
//
// Tiles are ordered expert-major -- (group, column tile, row tile) -- and the workgroup index
// is remapped so that consecutive tiles run on the same XCD: an expert's row tiles share its
// weight panels and its column tiles share its gathered rows through that XCD's L2.
// ------------------------------------------------------------------------------------------
template <bool GATED, int WN, int S>
__global__ void __launch_bounds__(128 * WN, WN == 2 ? 2 : 1) ffn_mfma_stream_kernel(MfmaArgs p) {
  using namespace stream;
  using GEO = Geo<WN>;
  constexpr int TN = GATED ? GEO::COLS / 2 : GEO::COLS;  // output columns per tile
  __shared__ __attribute__((aligned(1024))) char smem[S * GEO::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN;
  const int wn = wave % WN;

  // logical work item -> (tile, K split); tile -> (group, column tile, row tile)
  const int nsp = p.splits;
  const int LS = xcd_remap(blockIdx.x, *p.tile_count * p.n_ntiles * nsp);
  if (LS < 0) return;
  const int L = LS / nsp;
  const int split = LS - L * nsp;
  const int probe = L / p.n_ntiles;
  const int g = p.tile_group[probe];
  const int first = probe - p.tile_m0[probe] / SBM;  // the group's first row tile
  const Group G = group_info(g, p.offsets, p.T, p.k, p.E, p.I, p.Is);
  const int cnt = (G.rows + SBM - 1) / SBM;
  const int local = L - p.n_ntiles * first;
  const int nt = local / cnt;
  // the group's cnt row tiles: 128 rows each and a remainder, or (balance) as equal as possible,
  // so that an expert's tiles do equal work and stream its weight panels in step
  const int mt = local % cnt;
  const int m0 = p.balance ? mt * G.rows / cnt : mt * SBM;
  const int mrows = p.balance ? (mt + 1) * G.rows / cnt - m0 : min(G.rows - m0, SBM);  // valid rows

  const int K = GATED ? p.d : G.n_inter;
  const int N = GATED ? G.n_inter : p.d;
  const int n0 = nt * TN;
  if (n0 >= N) return;

  const bf16_t* W0;
  const bf16_t* W1 = nullptr;
  if (GATED) {
    W0 = G.shared ? p.w0_s : p.w0 + (size_t)g * p.d * p.I;
    W1 = G.shared ? p.w1_s : p.w1 + (size_t)g * p.d * p.I;
  } else {
    W0 = G.shared ? p.w0_s : p.w0 + (size_t)g * p.I * p.d;
  }

  // DMA sources: uniform bases per k-step, 32-bit per-lane byte offsets
  const int64_t a_pitch = (GATED ? (int64_t)p.d : (int64_t)p.ldh) * 2;
  uint32_t a_off[GEO::A_DMA];
#pragma unroll
  for (int i = 0; i < GEO::A_DMA; ++i) {
    const int m = a_dma_row<WN>(wave, i, lane);
    const int r = m < mrows ? m : 0;  // rows past the tile re-read its first row
    int64_t src_row;
    if (GATED)
      src_row = G.shared ? (int64_t)(m0 + r) : (int64_t)p.sorted_token[G.row0 + m0 + r];
    else
      src_row = G.row0 + m0 + r;
    a_off[i] = (uint32_t)(src_row * a_pitch) + a_dma_chunk_bytes(lane);
  }
  // this split's K steps
  const int nk_all = K / SBK;
  const int chunk = (nk_all + nsp - 1) / nsp;
  const int kt0 = split * chunk;
  const int nk = min(chunk, nk_all - kt0);  // <= 0: an empty split, partial sums of zero
  const char* a_src = uniform_ptr((const char*)p.a_src + (int64_t)kt0 * (SBK * 2));
  auto a_base = [=](int kt) { return a_src + kt * (SBK * 2); };

  // B: this wave's DMAs fill one 128-column block of the tile; for gate/up, blocks 0 .. WN/2-1
  // come from W_g and the rest from W_u, at the same columns
  const int64_t b_pitch = (int64_t)N * 2;
  const int blk = b_dma_block<WN>(wave);
  const char* b_mat;
  if (GATED)
    b_mat = (const char*)(blk < WN / 2 ? W0 : W1) + (int64_t)(n0 + 128 * (blk % (WN / 2))) * 2;
  else
    b_mat = (const char*)W0 + (int64_t)(n0 + 128 * blk) * 2;
  const int64_t b_kstep = (int64_t)SBK * b_pitch;
  const char* b0 = uniform_ptr(b_mat + (int64_t)b_dma_row0<WN>(wave, 0) * b_pitch + (int64_t)kt0 * b_kstep);
  // the wave's B instructions load consecutive 4-row groups of one block
  auto b_base = [=](int kt, int i) { return b0 + kt * b_kstep + i * 4 * b_pitch; };
  const uint32_t b_off = b_dma_lane_offset(lane, (uint32_t)b_pitch);

  int bcol[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) bcol[j] = GATED ? (j >> 1) * TN + wn * 64 + (j & 1) * 32 : wn * 128 + j * 32;
  const int nl = live_subtiles(mrows, wm);

  f32x16_t acc[2][4];
  zero(acc);
  // An expert with a single row tile is the only reader of its weight panels (few tokens): they
  // stream with the non-temporal hint (decode gate/up 2.68 -> 2.39 ms, down 1.29 -> 1.23 ms). The
  // row tiles of a larger group share each panel through L2, where the hint would evict it
  // (prefill gate/up 13.4 -> 15.6 ms with it on every panel).
  if (nk > 0) mainloop<WN, S>(nk, nl, mrows, (lds_char*)smem, a_base, a_off, b_base, b_off, bcol, acc, cnt == 1);

  // 32x32 accumulator layout -- lane holds column (lane & 31); register r holds row
  // 8*(r/4) + 4*(lane/32) + (r%4)
  const int col_in = lane & 31;
  const int row_hi = (lane >> 5) * 4;

  if constexpr (GATED) {
    if (nsp > 1) {
      // Split K, gate/up: every split stores its fp32 partial rows with plain stores and ends; the
      // next kernel on the stream (gate_up_finish_kernel) adds them in split order and applies
      // silu * up. (The down product is launched with one split.)
      float* mine = p.part + (int64_t)split * p.part_sstride;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t pc = (j >> 1) * p.ldh + n0 + wn * 64 + (j & 1) * 32 + col_in;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = sub_row(wm, i) + (r >> 2) * 8 + row_hi + (r & 3);
            if (row < mrows) mine[(G.row0 + m0 + row) * p.part_ld + pc] = acc[i][j][r];
          }
        }
      return;
    }
  }

  // Epilogue through LDS: the output tile (silu(g)*u for gate/up) is staged in bf16, row-major, in
  // the LDS stages (free once every wave is past its mainloop), and then each lane writes 16
  // contiguous bytes of a row instead of single 2-byte elements (mid down product 181 -> 168 us).
  constexpr int PITCH = TN * 2 + 16;  // bytes per staged row; the pad moves row r + 4 to other banks
  static_assert(SBM * PITCH <= S * GEO::STAGE, "the staged tile fits the LDS stages");
  __syncthreads();
  char* st = smem;
  if (GATED) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int c = wn * 64 + jj * 32 + col_in;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = sub_row(wm, i) + (r >> 2) * 8 + row_hi + (r & 3);
          if (row < mrows)
            *(bf16_t*)(st + row * PITCH + c * 2) = f32_to_bf16(silu_f32(acc[i][jj][r]) * acc[i][jj + 2][r]);
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = wn * 128 + j * 32 + col_in;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = sub_row(wm, i) + (r >> 2) * 8 + row_hi + (r & 3);
          if (row < mrows) *(bf16_t*)(st + row * PITCH + c * 2) = f32_to_bf16(acc[i][j][r]);
        }
      }
  }
  __syncthreads();
  constexpr int CH = TN / 8;  // 16-byte chunks per row
  const int64_t ld = GATED ? p.ldh : p.d;
  bf16_t* out = p.out + (G.row0 + m0) * ld + n0;
  for (int c = tid; c < SBM * CH; c += 128 * WN) {
    const int row = c / CH, ch = c - row * CH;
    if (row < mrows) *(uint4*)(out + row * ld + ch * 8) = *(const uint4*)(st + row * PITCH + ch * 16);
  }
}

// ------------------------------------------------------------------------------------------
// Tall tiles for groups of about a hundred rows and more: 160 x 512 (stream_gemm.h, namespace
// tall: eight wavefronts each holding all rows of the tile and 64 columns; for the gate/up
// product 32 gate and the matching 32 up columns) or 192 x 512 (namespace wide: a 2 x 4 grid of
// wavefronts, each 96 rows x 128 columns), chosen per group by the tile list (kTileRows192 on the
// group's entries): 192 rows where that takes fewer row tiles, at most two, 160 otherwise. A
// group's rows are split over its row tiles in whole 32-row sub-tiles as evenly as possible, so
// its row tiles do equal work and stream each weight panel in step. Tiles are ordered (group,
// column tile, row tile) and remapped per XCD as in the 128-row kernel.
// ------------------------------------------------------------------------------------------
// Logical tile L of a 160-row group.
template <bool GATED, int S>
__device__ __forceinline__ void tile160(const MfmaArgs& p, int L, char* smem) {
  using namespace stream;
  constexpr int TM = tall::ROWS;
  constexpr int TN = GATED ? 256 : 512;  // output columns per tile
  static_assert(S * tall::STAGE <= S * wide::STAGE, "the kernel's LDS holds either tile's stages");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int probe = L / p.n_ntiles;
  const int g = p.tile_group[probe];
  const int first = probe - (p.tile_m0[probe] & ~kTileRows192) / TM;  // the group's first row tile
  const Group G = group_info(g, p.offsets, p.T, p.k, p.E, p.I, p.Is);
  const int cnt = (G.rows + TM - 1) / TM;
  const int local = L - p.n_ntiles * first;
  const int nt = local / cnt;
  const int mt = local % cnt;
  // the group's S32 sub-tiles of 32 rows, split as evenly as possible over its cnt row tiles
  const int S32 = (G.rows + 31) / 32;
  const int m0 = 32 * (mt * S32 / cnt);
  const int mrows = min(32 * ((mt + 1) * S32 / cnt), G.rows) - m0;

  const int K = GATED ? p.d : G.n_inter;
  const int N = GATED ? G.n_inter : p.d;
  const int n0 = nt * TN;
  if (n0 >= N) return;

  const bf16_t* W0;
  const bf16_t* W1 = nullptr;
  if (GATED) {
    W0 = G.shared ? p.w0_s : p.w0 + (size_t)g * p.d * p.I;
    W1 = G.shared ? p.w1_s : p.w1 + (size_t)g * p.d * p.I;
  } else {
    W0 = G.shared ? p.w0_s : p.w0 + (size_t)g * p.I * p.d;
  }

  // A: this wave's instructions q = wave and wave + 8 (16 rows each); rows past the tile re-read
  // its first row
  const int64_t a_pitch = (GATED ? (int64_t)p.d : (int64_t)p.ldh) * 2;
  uint32_t a_off[tall::A_DMA];
#pragma unroll
  for (int i = 0; i < tall::A_DMA; ++i) {
    const int m = (wave + tall::NW * i) * 16 + (lane >> 2);
    const int r = m < mrows ? m : 0;
    int64_t src_row;
    if (GATED)
      src_row = G.shared ? (int64_t)(m0 + r) : (int64_t)p.sorted_token[G.row0 + m0 + r];
    else
      src_row = G.row0 + m0 + r;
    a_off[i] = (uint32_t)(src_row * a_pitch) + a_dma_chunk_bytes(lane);
  }
  const int nk = K / SBK;
  const char* a_src = uniform_ptr((const char*)p.a_src);
  auto a_base = [=](int kt) { return a_src + kt * (SBK * 2); };

  // B: four 128-column blocks; wave w fills rows 16 (w % 2) .. +16 of block w / 2. For gate/up,
  // blocks 0, 1 are W_g columns n0 .. n0 + 255 and blocks 2, 3 the W_u columns with the same indices.
  // B: four 128-column blocks; wave w fills rows 16 (w % 2) .. +16 of block w / 2. For gate/up,
  // blocks 0, 1 are W_g columns n0 .. n0 + 255 and blocks 2, 3 the W_u columns with the same indices.
  const int64_t b_pitch = (int64_t)N * 2;
  const int blk = wave >> 1;
  const char* b_mat;
  if (GATED)
    b_mat = (const char*)(blk < 2 ? W0 : W1) + (int64_t)(n0 + 128 * (blk & 1)) * 2;
  else
    b_mat = (const char*)W0 + (int64_t)(n0 + 128 * blk) * 2;
  const int64_t b_kstep = (int64_t)SBK * b_pitch;
  const char* b0 = uniform_ptr(b_mat + (int64_t)(16 * (wave & 1)) * b_pitch);
  auto b_base = [=](int kt, int i) { return b0 + kt * b_kstep + i * 4 * b_pitch; };
  const uint32_t b_off = b_dma_lane_offset(lane, (uint32_t)b_pitch);

  // the wave's two 32-wide column sub-tiles: gate and up columns wave*32 (gate/up), or
  // wave*64 .. +64 (down)
  int bcol[2];
  if (GATED) {
    bcol[0] = wave * 32;
    bcol[1] = TN + wave * 32;
  } else {
    bcol[0] = wave * 64;
    bcol[1] = wave * 64 + 32;
  }

  f32x16_t acc[tall::SUB][2];
  tall::zero(acc);
  // a group with a single row tile is the only reader of its weight panels: non-temporal hint
  if (nk > 0) tall::mainloop<S>(nk, mrows, (lds_char*)smem, a_base, a_off, b_base, b_off, bcol, acc, cnt == 1);

  // epilogue through LDS (see the 128-row kernel): the output rows staged in bf16, then written
  // with 16-byte row stores; the down tile's 512 columns go in two halves of 256. The mainloop's
  // accumulators hold transposed 32 x 32 blocks: lane l has row 32 u + (l & 31) and, in register
  // 4 g + q, column 8 g + 4 (l >> 5) + q of its 32-wide sub-tile -- four consecutive columns of one
  // row per g, staged with one 8-byte store.
  const int rl = lane & 31;
  const int cq = 4 * (lane >> 5);
  constexpr int HALF = 256;
  constexpr int PITCH = HALF * 2 + 16;
  static_assert(TM * PITCH <= S * tall::STAGE, "a staged half-tile fits the LDS stages");
  const int64_t ld = GATED ? p.ldh : p.d;
  bf16_t* out = p.out + (G.row0 + m0) * ld + n0;
  char* st = smem;
  constexpr int CH = HALF / 8;  // 16-byte chunks per staged row
#pragma unroll
  for (int h = 0; h < TN / HALF; ++h) {
    __syncthreads();  // every wave is past its mainloop (h = 0) or its previous half's copy
    if (GATED) {
#pragma unroll
      for (int u = 0; u < tall::SUB; ++u) {
        const int row = u * 32 + rl;
        if (row < mrows)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int c = wave * 32 + 8 * g + cq;
            float v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = silu_f32(acc[u][0][4 * g + q]) * acc[u][1][4 * g + q];
            *(uint2*)(st + row * PITCH + c * 2) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
          }
      }
    } else if ((wave >> 2) == h) {  // waves 4h .. 4h+3 hold columns 256h .. +256
#pragma unroll
      for (int u = 0; u < tall::SUB; ++u) {
        const int row = u * 32 + rl;
        if (row < mrows)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int c = (wave & 3) * 64 + j * 32 + 8 * g + cq;
              const f32x16_t& a = acc[u][j];
              *(uint2*)(st + row * PITCH + c * 2) =
                  make_uint2(pack_bf16x2(a[4 * g], a[4 * g + 1]), pack_bf16x2(a[4 * g + 2], a[4 * g + 3]));
            }
      }
    }
    __syncthreads();
    for (int c = tid; c < mrows * CH; c += 512) {
      const int row = c / CH, ch = c - row * CH;
      *(uint4*)(out + row * ld + h * HALF + ch * 8) = *(const uint4*)(st + row * PITCH + ch * 16);
    }
  }
}

// Logical tile L of a 192-row group: row split, weight streams and the staged epilogue as in
// tile160.
template <bool GATED, int S>
__device__ __forceinline__ void tile192(const MfmaArgs& p, int L, char* smem) {
  using namespace stream;
  constexpr int TM = wide::ROWS;
  constexpr int TN = GATED ? 256 : 512;  // output columns per tile

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;

  const int probe = L / p.n_ntiles;
  const int g = p.tile_group[probe];
  const int first = probe - (p.tile_m0[probe] & ~kTileRows192) / TM;  // the group's first row tile
  const Group G = group_info(g, p.offsets, p.T, p.k, p.E, p.I, p.Is);
  const int cnt = (G.rows + TM - 1) / TM;
  const int local = L - p.n_ntiles * first;
  const int nt = local / cnt;
  const int mt = local % cnt;
  // the group's S32 sub-tiles of 32 rows, split as evenly as possible over its cnt row tiles
  const int S32 = (G.rows + 31) / 32;
  const int m0 = 32 * (mt * S32 / cnt);
  const int mrows = min(32 * ((mt + 1) * S32 / cnt), G.rows) - m0;

  const int K = GATED ? p.d : G.n_inter;
  const int N = GATED ? G.n_inter : p.d;
  const int n0 = nt * TN;
  if (n0 >= N) return;

  const bf16_t* W0;
  const bf16_t* W1 = nullptr;
  if (GATED) {
    W0 = G.shared ? p.w0_s : p.w0 + (size_t)g * p.d * p.I;
    W1 = G.shared ? p.w1_s : p.w1 + (size_t)g * p.d * p.I;
  } else {
    W0 = G.shared ? p.w0_s : p.w0 + (size_t)g * p.I * p.d;
  }

  // A: this wave's instructions q = wave and wave + 8 (16 rows each; q < 12 only for waves 0 .. 3);
  // rows past the tile re-read its first row
  const int64_t a_pitch = (GATED ? (int64_t)p.d : (int64_t)p.ldh) * 2;
  uint32_t a_off[wide::A_DMA];
#pragma unroll
  for (int i = 0; i < wide::A_DMA; ++i) {
    const int m = min((wave + wide::NW * i) * 16 + (lane >> 2), TM - 1);
    const int r = m < mrows ? m : 0;
    int64_t src_row;
    if (GATED)
      src_row = G.shared ? (int64_t)(m0 + r) : (int64_t)p.sorted_token[G.row0 + m0 + r];
    else
      src_row = G.row0 + m0 + r;
    a_off[i] = (uint32_t)(src_row * a_pitch) + a_dma_chunk_bytes(lane);
  }
  const int nk = K / SBK;
  const char* a_src = uniform_ptr((const char*)p.a_src);
  auto a_base = [=](int kt) { return a_src + kt * (SBK * 2); };

  const int64_t b_pitch = (int64_t)N * 2;
  const int blk = wave >> 1;
  const char* b_mat;
  if (GATED)
    b_mat = (const char*)(blk < 2 ? W0 : W1) + (int64_t)(n0 + 128 * (blk & 1)) * 2;
  else
    b_mat = (const char*)W0 + (int64_t)(n0 + 128 * blk) * 2;
  const int64_t b_kstep = (int64_t)SBK * b_pitch;
  const char* b0 = uniform_ptr(b_mat + (int64_t)(16 * (wave & 1)) * b_pitch);
  auto b_base = [=](int kt, int i) { return b0 + kt * b_kstep + i * 4 * b_pitch; };
  const uint32_t b_off = b_dma_lane_offset(lane, (uint32_t)b_pitch);

  // the wave's four 32-wide column sub-tiles: gate columns 64 wn, 64 wn + 32 and the up columns
  // with the same indices (gate/up), or columns 128 wn .. +128 (down)
  int bcol[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) bcol[j] = GATED ? (j >> 1) * 256 + wn * 64 + (j & 1) * 32 : wn * 128 + j * 32;

  f32x16_t acc[3][4];
#pragma unroll
  for (int u = 0; u < 3; ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[u][j][r] = 0.f;
  // a group with a single row tile is the only reader of its weight panels: non-temporal hint
  if (nk > 0) wide::mainloop<S>(nk, mrows, (lds_char*)smem, a_base, a_off, b_base, b_off, bcol, acc, cnt == 1);

  // epilogue through LDS as in the tall kernel: accumulator u holds transposed 32 x 32 blocks of
  // tile rows 32 (wm + 2u) .. +32, staged 8 bytes per store, copied out with 16-byte row stores;
  // the down tile's 512 columns in two halves of 256
  const int rl = lane & 31;
  const int cq = 4 * (lane >> 5);
  constexpr int HALF = 256;
  constexpr int PITCH = HALF * 2 + 16;
  static_assert(TM * PITCH <= S * wide::STAGE, "a staged half-tile fits the LDS stages");
  const int64_t ld = GATED ? p.ldh : p.d;
  bf16_t* out = p.out + (G.row0 + m0) * ld + n0;
  char* st = smem;
  constexpr int CH = HALF / 8;  // 16-byte chunks per staged row
#pragma unroll
  for (int h = 0; h < TN / HALF; ++h) {
    __syncthreads();  // every wave is past its mainloop (h = 0) or its previous half's copy
    if (GATED) {
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const int row = (wm + 2 * u) * 32 + rl;
        if (row < mrows)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int c = wn * 64 + j * 32 + 8 * g + cq;
              float v[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) v[q] = silu_f32(acc[u][j][4 * g + q]) * acc[u][j + 2][4 * g + q];
              *(uint2*)(st + row * PITCH + c * 2) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            }
      }
    } else if ((wn >> 1) == h) {  // wave columns 2h, 2h + 1 hold columns 256h .. +256
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const int row = (wm + 2 * u) * 32 + rl;
        if (row < mrows)
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int c = (wn & 1) * 128 + j * 32 + 8 * g + cq;
              const f32x16_t& a = acc[u][j];
              *(uint2*)(st + row * PITCH + c * 2) =
                  make_uint2(pack_bf16x2(a[4 * g], a[4 * g + 1]), pack_bf16x2(a[4 * g + 2], a[4 * g + 3]));
            }
      }
    }
    __syncthreads();
    for (int c = tid; c < mrows * CH; c += 512) {
      const int row = c / CH, ch = c - row * CH;
      *(uint4*)(out + row * ld + h * HALF + ch * 8) = *(const uint4*)(st + row * PITCH + ch * 16);
    }
  }
}

template <bool GATED, int S>
__global__ void __launch_bounds__(512, 1) ffn_mfma_tall_kernel(MfmaArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem[S * stream::wide::STAGE];
  const int L = stream::xcd_remap(blockIdx.x, *p.tile_count * p.n_ntiles);
  if (L < 0) return;
  if (p.tile_m0[L / p.n_ntiles] & kTileRows192) tile192<GATED, S>(p, L, smem);
  else tile160<GATED, S>(p, L, smem);
}

// H rows of a gate/up product with K split (streaming MFMA or skinny kernels): each split's fp32
// gate and up sums (row pitch 2 ldh: gate at column c, up at ldh + c) added in split order, then
// silu(gate) * up in bf16.
// Row i < T*k is a routed slot (I columns), the rest shared rows (I_s columns). grid: (ldh / 1024
// rounded up, rows_total); four columns per thread.
__global__ void __launch_bounds__(256)
gate_up_finish_kernel(const float* __restrict__ part, int64_t sstride, int64_t part_ld, int ks, int64_t Tk,
                             int I, int Is, int ldh, bf16_t* __restrict__ H) {
  const int64_t row = blockIdx.y;
  const int c4 = (blockIdx.x * 256 + threadIdx.x) * 4;
  const int N = row < Tk ? I : Is;
  if (c4 >= N) return;
  const float* q = part + row * part_ld + c4;
  float g[4] = {0.f, 0.f, 0.f, 0.f}, u[4] = {0.f, 0.f, 0.f, 0.f};
  constexpr int B = 8;  // splits loaded together
  for (int s0 = 0; s0 < ks; s0 += B) {
    float4 a[B], b[B];
#pragma unroll
    for (int j = 0; j < B; ++j)
      if (s0 + j < ks) {
        a[j] = *(const float4*)(q + (int64_t)(s0 + j) * sstride);
        b[j] = *(const float4*)(q + (int64_t)(s0 + j) * sstride + ldh);
      }
#pragma unroll
    for (int j = 0; j < B; ++j)
      if (s0 + j < ks) {
        g[0] += a[j].x; g[1] += a[j].y; g[2] += a[j].z; g[3] += a[j].w;
        u[0] += b[j].x; u[1] += b[j].y; u[2] += b[j].z; u[3] += b[j].w;
      }
  }
  uint2 o;
  o.x = pack_bf16x2(silu_f32(g[0]) * u[0], silu_f32(g[1]) * u[1]);
  o.y = pack_bf16x2(silu_f32(g[2]) * u[2], silu_f32(g[3]) * u[3]);
  *(uint2*)(H + row * ldh + c4) = o;
}

// K splits for a product whose row x column tiles are expected to number `tiles`: double while
// the grid would not cover two workgroups per CU and every split keeps >= 16 K steps.
int pick_splits(int64_t tiles, int nk_min) {
  int s = 1;
  while (s < 8 && tiles * s < 512 && nk_min / (2 * s) >= 16) s *= 2;
  return s;
}

// wn: wave columns of the streaming tile (2: 128 x 256, 4: 128 x 512)
template <bool GATED>
void launch_stream(int wn, unsigned grid, hipStream_t s, const MfmaArgs& a) {
  if (wn == 4) hipLaunchKernelGGL((ffn_mfma_stream_kernel<GATED, 4, 4>), dim3(grid), dim3(512), 0, s, a);
  else hipLaunchKernelGGL((ffn_mfma_stream_kernel<GATED, 2, 3>), dim3(grid), dim3(256), 0, s, a);
}

// ------------------------------------------------------------------------------------------
// fp32 grouped GEMM (vector ALUs)
// ------------------------------------------------------------------------------------------
struct F32Args {
  const float* a_src;
  const int32_t* offsets;
  const int32_t* sorted_token;
  const float* w0;
  const float* w1;
  const float* w0_s;
  const float* w1_s;
  float* out;
  const int32_t* tile_group;
  const int32_t* tile_m0;
  const int32_t* tile_count;
  int64_t T;
  int d, E, k, I, Is, ldh;
  int n_ntiles;
};

template <bool GATED>
__global__ void __launch_bounds__(256)
ffn_f32_kernel(F32Args p) {
  constexpr int TM = kF32BM, TN = kF32BN, TK = 16;
  constexpr int NB = GATED ? 2 : 1;
  __shared__ __attribute__((aligned(16))) float As[TK][TM + 4];
  __shared__ __attribute__((aligned(16))) float Bs[NB][TK][TN + 4];

  const int tid = threadIdx.x;
  const int mt = blockIdx.x / p.n_ntiles;
  const int nt = blockIdx.x % p.n_ntiles;
  if (mt >= *p.tile_count) return;
  const int g = p.tile_group[mt];
  const int m0 = p.tile_m0[mt];
  const Group G = group_info(g, p.offsets, p.T, p.k, p.E, p.I, p.Is);
  const int K = GATED ? p.d : G.n_inter;
  const int N = GATED ? G.n_inter : p.d;
  const int n0 = nt * TN;
  if (n0 >= N) return;

  const float* Wb[2];
  if (GATED) {
    Wb[0] = G.shared ? p.w0_s : p.w0 + (size_t)g * p.d * p.I;
    Wb[1] = G.shared ? p.w1_s : p.w1 + (size_t)g * p.d * p.I;
  } else {
    Wb[0] = G.shared ? p.w0_s : p.w0 + (size_t)g * p.I * p.d;
    Wb[1] = nullptr;
  }

  const int al_r = tid / 4, al_k = (tid % 4) * 4;
  const bool al_ok = m0 + al_r < G.rows;
  int64_t src_row;
  if (GATED)
    src_row = G.shared ? (al_ok ? (int64_t)(m0 + al_r) : 0)
                       : (int64_t)p.sorted_token[G.row0 + m0 + (al_ok ? al_r : 0)];
  else
    src_row = G.row0 + m0 + (al_ok ? al_r : 0);
  const float* a_row = p.a_src + src_row * (GATED ? (int64_t)p.d : (int64_t)p.ldh);
  const int bl_k = tid / 16, bl_c = (tid % 16) * 4;
  const bool bl_ok = n0 + bl_c < N;

  const int ty = tid / 16, tx = tid % 16;
  float acc[NB][4][4];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[b][i][j] = 0.f;

  for (int k0 = 0; k0 < K; k0 += TK) {
    {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (al_ok && k0 + al_k < K) v = *(const float4*)(a_row + k0 + al_k);
      As[al_k + 0][al_r] = v.x;
      As[al_k + 1][al_r] = v.y;
      As[al_k + 2][al_r] = v.z;
      As[al_k + 3][al_r] = v.w;
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (bl_ok && k0 + bl_k < K) v = *(const float4*)(Wb[b] + (int64_t)(k0 + bl_k) * N + n0 + bl_c);
      *(float4*)&Bs[b][bl_k][bl_c] = v;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      const float4 a = *(const float4*)&As[kk][ty * 4];
      const float av[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float4 w = *(const float4*)&Bs[b][kk][tx * 4];
        const float wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[b][i][j] = fmaf(av[i], wv[j], acc[b][i][j]);
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = ty * 4 + i;
    if (m0 + row >= G.rows) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col >= N) continue;
      if (GATED)
        p.out[(G.row0 + m0 + row) * (int64_t)p.ldh + col] = silu_f32(acc[0][i][j]) * acc[NB - 1][i][j];
      else
        p.out[(G.row0 + m0 + row) * (int64_t)p.d + col] = acc[0][i][j];
    }
  }
}

}  // namespace

hipError_t launch_gate_up_finish(const float* part, int64_t sstride, int64_t part_ld, int ks, int64_t Tk,
                                 int64_t rows_total, int I, int Is, int ldh, bf16_t* H, hipStream_t s) {
  const dim3 grid((unsigned)((ldh + 1023) / 1024), (unsigned)rows_total);
  hipLaunchKernelGGL(gate_up_finish_kernel, grid, dim3(256), 0, s, part, sstride, part_ld, ks, Tk, I, Is, ldh, H);
  return hipGetLastError();
}

const char* ffn_kernel_name(const moe_dims& dm, bool gate_up) {
  if (dm.dtype == MOE_F32) return gate_up ? "ffn_f32_kernel<true>" : "ffn_f32_kernel<false>";
  const FfnPlan P = ffn_plan(dm);
  if (P.skinny) {
    if (P.skinny_rows == 1) return gate_up ? "ffn_skinny_kernel<true, 1>" : "ffn_skinny_kernel<false, 1>";
    return gate_up ? "ffn_skinny_kernel<true, 2>" : "ffn_skinny_kernel<false, 2>";
  }
  if (P.tall) return gate_up ? "ffn_mfma_tall_kernel<true, 3>" : "ffn_mfma_tall_kernel<false, 3>";
  if (P.stream) {
    if ((gate_up ? P.wn1 : P.wn2) == 4)
      return gate_up ? "ffn_mfma_stream_kernel<true, 4, 4>" : "ffn_mfma_stream_kernel<false, 4, 4>";
    return gate_up ? "ffn_mfma_stream_kernel<true, 2, 3>" : "ffn_mfma_stream_kernel<false, 2, 3>";
  }
  return gate_up ? "ffn_mfma_kernel<true>" : "ffn_mfma_kernel<false>";
}

int ffn_tile_rows(const moe_dims& dm) {
  if (dm.dtype == MOE_F32) return kF32BM;
  return ffn_plan(dm).tall ? stream::tall::ROWS : kMfmaBM;
}

int ffn_tile_rows_alt(const moe_dims& dm) {
  if (dm.dtype == MOE_F32) return 0;
  return ffn_plan(dm).tall ? stream::wide::ROWS : 0;
}

hipError_t launch_build_tiles(const moe_dims& dm, const Layout& L, const int32_t* offsets, char* ws, hipStream_t s,
                              int bm) {
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(1024), 0, s, offsets, dm.T, dm.E, dm.I_shared > 0 ? 1 : 0,
                     bm > 0 ? bm : ffn_tile_rows(dm), bm > 0 ? 0 : ffn_tile_rows_alt(dm),
                     (int32_t*)(ws + L.tile_group), (int32_t*)(ws + L.tile_m0),
                     (int32_t*)(ws + L.tile_count), (int32_t*)(ws + L.ffn_cnt), L.ffn_cnt_each,
                     L.ffn_cnt_per_tile);
  return hipGetLastError();
}

FfnPlan ffn_plan(const moe_dims& dm) {
  FfnPlan P;
  const int has_shared = dm.I_shared > 0 ? 1 : 0;
  const int64_t Tk = dm.T * dm.k;
  const int64_t rows_total = Tk + (has_shared ? dm.T : 0);
  const int ldh = dm.I > dm.I_shared ? dm.I : dm.I_shared;
  // the streaming kernel needs whole tiles along N and whole 32-wide K steps
  // (and 32-bit byte offsets for the gathered rows of x and of H)
  P.stream = dm.dtype == MOE_BF16 && dm.d % 256 == 0 && dm.I % 128 == 0 && dm.I_shared % 128 == 0 &&
             (uint64_t)dm.T * dm.d * 2 < (1ull << 32) && (uint64_t)rows_total * ldh * 2 < (1ull << 32);
  // 128 x 512 streaming tiles (one workgroup per CU) for long K loops, where the shape divides
  // them: the gate/up product at d >= 4096, the down product at I >= 2048 with at least 64 rows per
  // expert on average. Short K loops (and the near-empty row tiles of decode) run faster on
  // 128 x 256 tiles, two workgroups per CU, whose prologues and epilogues overlap.
  const double rows_per_expert = (double)Tk / dm.E;
  // Tall 160-row tiles for both products when experts hold ~100 rows or more on average: an
  // expert's rows up to 160 stay in one row tile (its weight panels stream once), ~320 rows are two
  // row tiles rather than three, and under skewed routing the many experts with a few dozen rows
  // stream their weights once, non-temporally. Measured against the 128-row tiles: mid (128 rows
  // per expert) 0.547 -> 0.504 ms, the large shape at T = 6144 (120 rows) 10.7 -> 9.9 ms, skew
  // 14.5 -> 13.7 ms; equal at 64-80 rows; at 48 rows the 128-row tiles are ~2 % faster.
  P.tall = P.stream && rows_per_expert >= 96.0 && dm.I % 256 == 0 && dm.I_shared % 256 == 0 && dm.d % 512 == 0;
  // With the tall tiles each group takes 160- or 192-row tiles, chosen per group when the tile
  // list is built (build_tile_list): 192 rows where they need fewer row tiles and at most two
  // (161-192 and 321-384 rows), 160 otherwise. Against one height per launch chosen from the
  // average rows per expert (192 from 256): prefill 19.9-20.0 -> 19.4 ms, 160 rows per expert
  // under uniform routing 12.3 -> 11.1 ms, mid 0.52 -> 0.51 ms, skew unchanged (192-row tiles on
  // its two 8192-row experts, 43 instead of 52 row tiles, measured 2 % slower).
  P.wn1 = P.stream && dm.I % 256 == 0 && dm.I_shared % 256 == 0 && dm.d >= 4096 ? 4 : 2;
  P.wn2 = P.stream && dm.d % 512 == 0 && dm.I >= 2048 && rows_per_expert >= 64.0 ? 4 : 2;
  const int tn1 = P.tall ? 256 : P.stream ? 64 * P.wn1 : kMfmaBN1;
  const int tn2 = P.tall ? 512 : P.stream ? 128 * P.wn2 : kMfmaBN2;
  P.nt1 = (ldh + tn1 - 1) / tn1;
  P.nt2 = (dm.d + tn2 - 1) / tn2;
  // Split the gate/up product's K when its tiles alone would leave CUs idle (few tokens: each
  // touched expert is one row tile). Expected row tiles: one per group that can be touched, plus
  // the full ones. The down product has 4x the column tiles and measured no faster split.
  P.s1 = 1;
  if (P.stream) {
    const int64_t groups = (Tk < dm.E ? Tk : dm.E) + has_shared;
    const int64_t mt = groups + rows_total / kMfmaBM;
    P.s1 = P.tall ? 1 : pick_splits(mt * P.nt1, dm.d / 32);
  }
  // Equal row tiles where experts hold one to two tiles' worth of rows (HBM-bound shapes): an
  // expert's two tiles then run at the same pace and share each weight panel through L2, instead
  // of a short second tile racing ahead and fetching the panel a second time. At larger row counts
  // the extra partly filled 32-row sub-tiles would cost MFMA time.
  P.balance = P.stream && rows_per_expert <= 192.0;
  P.part_cols1 = 2 * (int64_t)ldh;
  P.part_cols2 = dm.d;
  // One or two tokens: every group holds at most T rows, and both products are weight streams
  // with next to no arithmetic per byte. The skinny kernels split each (group, 256 columns) over K
  // so that up to ~1024 workgroups -- what the CUs hold at once -- stream equal shares in one
  // round. Measured at the large shape against the MFMA path (both with non-temporal weight
  // loads): T = 1 199 vs 206 us for the two products, T = 2 344 vs 351 us; at T = 4 the MFMA path
  // wins (623 vs 681 us: four rows per group need registers for only two workgroups per CU).
  P.skinny = P.stream && dm.T >= 1 && dm.T <= kSkinnyMaxT && dm.I % 256 == 0 && dm.I_shared % 256 == 0;
  P.skinny_rows = dm.T <= 1 ? 1 : 2;
  P.cb1 = ldh / 256;
  P.cb2 = dm.d / 256;
  P.ks1 = P.ks2 = P.kc1 = P.kc2 = 0;
  if (P.skinny) {
    const int64_t groups = (Tk < dm.E ? Tk : dm.E) + has_shared;
    auto split = [&](int K, int cb, int64_t target, int kr, int& ks, int& kc) {
      int64_t want = target / (groups * cb);
      const int64_t most = (K + 255) / 256;  // at least 256 K rows per split
      if (want > most) want = most;
      if (want < (K + kSkinnyMaxKC - 1) / kSkinnyMaxKC) want = (K + kSkinnyMaxKC - 1) / kSkinnyMaxKC;
      if (want < 1) want = 1;
      kc = (int)(((K + want - 1) / want + kr - 1) / kr * kr);  // whole LDS stages
      ks = (K + kc - 1) / kc;
    };
    split(dm.d, P.cb1, kSkinnyWG1, kSkinnyMat1 / 512, P.ks1, P.kc1);
    split(ldh, P.cb2, kSkinnyWG2, kSkinnyMat2 / 512, P.ks2, P.kc2);
  }
  return P;
}

hipError_t launch_grouped_ffn(const moe_dims& dm, const Layout& L, const void* x, const int32_t* offsets,
                              const int32_t* sorted_token, const void* wg, const void* wu, const void* wd,
                              const void* wg_s, const void* wu_s, const void* wd_s, void* y, char* ws,
                              hipStream_t s, const Prof* prof, bool tiles_ready, CombineFuse* combine) {
  const Prof none;
  if (!prof) prof = &none;
  int32_t* tg = (int32_t*)(ws + L.tile_group);
  int32_t* tm = (int32_t*)(ws + L.tile_m0);
  int32_t* tc = (int32_t*)(ws + L.tile_count);
  const int has_shared = dm.I_shared > 0 ? 1 : 0;
  const FfnPlan P = ffn_plan(dm);
  const bool stream_ok = P.stream;
  const int bm = ffn_tile_rows(dm);
  hipError_t e;
  if (!tiles_ready && (e = launch_build_tiles(dm, L, offsets, ws, s)) != hipSuccess) return e;

  // upper bound on row tiles: sum over non-empty groups of ceil(n_g / bm) <= (T*k)/bm + (routed
  // groups with rows, at most min(E, T*k)) + T/bm + 1 for the shared expert
  const int64_t Tk = dm.T * dm.k;
  const int64_t max_mt = Tk / bm + (Tk < dm.E ? Tk : dm.E) + (has_shared ? dm.T / bm + 1 : 0);
  const int nmax = dm.I > dm.I_shared ? dm.I : dm.I_shared;
  char* H = ws + L.H;

  if (P.skinny)
    return launch_ffn_skinny(dm, L, P, x, offsets, sorted_token, wg, wu, wd, wg_s, wu_s, wd_s, y, ws, s, prof,
                             combine);
  if (dm.dtype == MOE_BF16) {
    MfmaArgs a;
    a.offsets = offsets;
    a.sorted_token = sorted_token;
    a.tile_group = tg;
    a.tile_m0 = tm;
    a.tile_count = tc;
    a.T = dm.T;
    a.d = dm.d;
    a.E = dm.E;
    a.k = dm.k;
    a.I = dm.I;
    a.Is = dm.I_shared;
    a.ldh = L.ldh;
    a.part = (float*)(ws + L.ffn_part);
    a.part_sstride = 0;
    a.balance = P.balance ? 1 : 0;
    // ffn1: gate/up
    a.a_src = (const bf16_t*)x;
    a.w0 = (const bf16_t*)wg;
    a.w1 = (const bf16_t*)wu;
    a.w0_s = (const bf16_t*)wg_s;
    a.w1_s = (const bf16_t*)wu_s;
    a.out = (bf16_t*)H;
    a.n_ntiles = P.nt1;
    a.splits = P.s1;
    a.part_ld = P.part_cols1;
    a.part_sstride = L.rows_total * P.part_cols1;
    if ((e = prof->begin(MOE_KERNEL_FFN_GATE_UP, s)) != hipSuccess) return e;
    if (P.tall)
      hipLaunchKernelGGL((ffn_mfma_tall_kernel<true, 3>), dim3((unsigned)(max_mt * a.n_ntiles)), dim3(512), 0, s, a);
    else if (stream_ok)
      launch_stream<true>(P.wn1, (unsigned)(max_mt * a.n_ntiles * a.splits), s, a);
    else
      hipLaunchKernelGGL(ffn_mfma_kernel<true>, dim3((unsigned)(max_mt * a.n_ntiles)), dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (stream_ok && a.splits > 1 &&
        (e = launch_gate_up_finish(a.part, a.part_sstride, a.part_ld, a.splits, dm.T * dm.k, L.rows_total, dm.I,
                                   dm.I_shared, L.ldh, (bf16_t*)H, s)) != hipSuccess)
      return e;
    if ((e = prof->end(MOE_KERNEL_FFN_GATE_UP, s)) != hipSuccess) return e;
    // ffn2: down
    a.a_src = (const bf16_t*)H;
    a.w0 = (const bf16_t*)wd;
    a.w1 = nullptr;
    a.w0_s = (const bf16_t*)wd_s;
    a.w1_s = nullptr;
    a.out = (bf16_t*)y;
    a.n_ntiles = P.nt2;
    a.splits = 1;
    a.part = nullptr;
    a.part_ld = 0;
    a.part_sstride = 0;
    if ((e = prof->begin(MOE_KERNEL_FFN_DOWN, s)) != hipSuccess) return e;
    if (P.tall)
      hipLaunchKernelGGL((ffn_mfma_tall_kernel<false, 3>), dim3((unsigned)(max_mt * a.n_ntiles)), dim3(512), 0, s, a);
    else if (stream_ok)
      launch_stream<false>(P.wn2, (unsigned)(max_mt * a.n_ntiles * a.splits), s, a);
    else
      hipLaunchKernelGGL(ffn_mfma_kernel<false>, dim3((unsigned)(max_mt * a.n_ntiles)), dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return prof->end(MOE_KERNEL_FFN_DOWN, s);
  }

  F32Args a;
  a.offsets = offsets;
  a.sorted_token = sorted_token;
  a.tile_group = tg;
  a.tile_m0 = tm;
  a.tile_count = tc;
  a.T = dm.T;
  a.d = dm.d;
  a.E = dm.E;
  a.k = dm.k;
  a.I = dm.I;
  a.Is = dm.I_shared;
  a.ldh = L.ldh;
  a.a_src = (const float*)x;
  a.w0 = (const float*)wg;
  a.w1 = (const float*)wu;
  a.w0_s = (const float*)wg_s;
  a.w1_s = (const float*)wu_s;
  a.out = (float*)H;
  a.n_ntiles = (nmax + kF32BN - 1) / kF32BN;
  if ((e = prof->begin(MOE_KERNEL_FFN_GATE_UP, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(ffn_f32_kernel<true>, dim3((unsigned)(max_mt * a.n_ntiles)), dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = prof->end(MOE_KERNEL_FFN_GATE_UP, s)) != hipSuccess) return e;
  a.a_src = (const float*)H;
  a.w0 = (const float*)wd;
  a.w1 = nullptr;
  a.w0_s = (const float*)wd_s;
  a.w1_s = nullptr;
  a.out = (float*)y;
  a.n_ntiles = (dm.d + kF32BN - 1) / kF32BN;
  if ((e = prof->begin(MOE_KERNEL_FFN_DOWN, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(ffn_f32_kernel<false>, dim3((unsigned)(max_mt * a.n_ntiles)), dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return prof->end(MOE_KERNEL_FFN_DOWN, s);
}

}  // namespace moe
