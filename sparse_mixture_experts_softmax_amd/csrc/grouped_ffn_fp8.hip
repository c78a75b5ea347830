// Routed and shared SwiGLU experts with FP8 weights: the same grouped GEMMs as grouped_ffn.hip with
// the weight operand in e4m3. The Fondations page of the Qwen3.8-Max report names FP8 among the
// formats without a scheme; the one used here is weight-only OCP e4m3 (bias 7, 3 mantissa bits,
// largest finite 448) with one power-of-two scale per output column, round to nearest even:
//
//   W[k, n] = e4m3(Q[n, k]) * s[n]      so   (A W)[m, n] = s[n] * sum_k A[m, k] e4m3(Q[n, k])
//
// Code layout (per matrix of N columns and K rows; N % 128 == 0, K % 32 == 0): tiles of 128
// columns x 32 K values, 4 KB each, ordered (column tile, K tile), so the codes of one 128-column
// panel are one contiguous stream of K / 32 tiles. Inside a tile, column r holds its 32 K values
// at bytes 32 r .. 32 r + 31, K-contiguous, as two 16-byte halves; half h (K 16h .. 16h+15) sits
// at slot h ^ ((r >> 3) & 1). A tile is thus byte for byte the LDS image the kernel reads, and
// the DMA copies 1 KB runs of it. The MFMA B operand (8 consecutive K values of one column per
// lane) is a plain 8-byte LDS read; each e4m3 value is exact in bf16, so the codes are widened to
// bf16 in registers and the product runs on the bf16 MFMA. The column scale is applied to the
// fp32 accumulator in the epilogue. Half the weight bytes of bf16: the decode shapes, bound by
// streaming the touched experts' weights, move half as much. (Stored plainly K-contiguous, one
// 32-byte run per column and K step, the same kernel ran 12 % slower at decode.)
//
// Tile: 128 x 256 (four wavefronts, wavefront w owning the 32-row sub-tiles w/2 and 2 + w/2 and
// columns 128*(w%2) .. +128), K step 32, S stages of 8 KB of A (bf16) + 8 KB of B (e4m3), two
// workgroups per CU. Schedule, DMA and the A operand as in stream_gemm.h. The B stage holds two
// code tiles (gate and up at the same columns, or two adjacent column tiles of W_d); B instruction
// q (0..7; wave w issues 2w, 2w+1) copies bytes 1024 (q % 4) .. +1023 of tile q / 4, 16 per lane.
// With 32 tokens or fewer every group holds at most 32 rows, only the first 32-row sub-tile is ever
// live, and the stages keep A room for 32 rows (2 KB): four stages of 10 KB per workgroup, four
// workgroups per CU, 128 instead of 80 KB of codes in flight per CU (decode layer 2.00 -> 1.96 ms;
// two workgroups of eight such stages, the same bytes in flight, measured 2.10 ms).
#include "fp8_codec.h"
#include "moe_internal.h"
#include "stream_gemm.h"

namespace moe {
namespace {

using namespace stream;

constexpr int F8_COLS = 256;
constexpr int F8_B_BYTES = F8_COLS * SBK;    // 8 KB
constexpr int F8_A_DMA = 2;                  // per wave per stage (at most)
constexpr int F8_B_DMA = 2;
// A room per stage for AR rows (128: the full tile; 32: few-token launches), and the stage
template <int AR>
struct F8Geo {
  static_assert(AR == 128 || AR == 32, "A rows");
  static constexpr int A_BYTES = AR * SBK * 2;  // 8 KB or 2 KB
  static constexpr int STAGE = A_BYTES + F8_B_BYTES;
};

// 8 e4m3 codes (K-consecutive) -> 8 bf16: exact through fp32 (the top half of each fp32 value)
__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(w0, false);
  const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(w0, true);
  const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(w1, false);
  const auto d = __builtin_amdgcn_cvt_pk_f32_fp8(w1, true);
  auto pk = [](float lo, float hi) { return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u); };
  uint4 u;
  u.x = pk(a[0], a[1]);
  u.y = pk(b[0], b[1]);
  u.z = pk(c[0], c[1]);
  u.w = pk(d[0], d[1]);
  return __builtin_bit_cast(bf16x8_t, u);
}

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// the B fragment of K sub-step s (0 or 1) for tile column n: 8 bytes of the column's 32
__device__ __forceinline__ bf16x8_t read_b_f8(const lds_char* sb, int n, int s, int half) {
  const int off = n * 32 + 16 * (s ^ ((n >> 3) & 1)) + 8 * half;
  const u32x2_t w = *(const __attribute__((address_space(3))) u32x2_t*)(sb + off);
  return e4m3x8_to_bf16(w[0], w[1]);
}

// acc[i][j] += A * dequant(B) over nk K steps; NL live 32-row sub-tiles of this wave.
// a_base(kt) / b_base(kt, i): uniform bases of k-step kt (B: this wave's i-th instruction);
// a_off / b_off[i]: per-lane byte offsets. Same schedule as stream::mainloop_v.
// NAD: A instructions this wave issues (those whose 16 rows hold a valid row of the tile).
// NT: code DMAs with the non-temporal hint (the group's only row tile reads them).
// AR: A rows per stage (F8Geo); with 32, only the first sub-tile of wave row 0 may be live.
template <int S, int NL, int NAD, bool NT, int AR, class ABase, class BBase>
__device__ __forceinline__ void mainloop_f8(int nk, lds_char* lds, ABase a_base, const uint32_t (&a_off)[F8_A_DMA],
                                            BBase b_base, const uint32_t (&b_off)[F8_B_DMA], const int (&bcol)[4],
                                            f32x16_t (&acc)[2][4]) {
  static_assert(S >= 3 && S <= 8, "stages");
  static_assert(AR == SBM || NL <= 1, "32 A rows hold one sub-tile");
  constexpr int F8_A_BYTES = F8Geo<AR>::A_BYTES;
  constexpr int F8_STAGE = F8Geo<AR>::STAGE;
  constexpr int F8_DMA = NAD + F8_B_DMA;
  constexpr int NA = NL > 0 ? NL : 1;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1;
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);

  auto issue = [&](int kt, int stage) {
    const uint32_t dst = lds_base + stage * F8_STAGE;
    const char* ab = a_base(kt);
#pragma unroll
    for (int i = 0; i < NAD; ++i) dma16(ab, a_off[i], dst + (wave * F8_A_DMA + i) * 1024);
#pragma unroll
    for (int i = 0; i < F8_B_DMA; ++i)
      dma16<NT>(b_base(kt, i), b_off[i], dst + F8_A_BYTES + (wave * F8_B_DMA + i) * 1024);
  };
  auto read = [&](const lds_char* st, int s, bf16x8_t (&a)[NA], bf16x8_t (&b)[4]) {
    if constexpr (NL > 0) {
#pragma unroll
      for (int u = 0; u < NL; ++u) a[u] = read_a(st, sub_row(wm, u) + (lane & 31), 2 * s + (lane >> 5));
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = read_b_f8(st + F8_A_BYTES, bcol[j] + (lane & 31), s, lane >> 5);
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

#pragma unroll
  for (int i = 0; i < S; ++i)
    if (i < nk) issue(i, i);
  wait_groups<F8_DMA>(min(S - 1, nk - 1));
  barrier_lds_only();

  bf16x8_t a0[NA], b0[4], a1[NA], b1[4];
  read(lds, 0, a0, b0);
  // last k-step peeled off, as in stream::mainloop_v: the loop body always crosses the barrier
  int stage = 0;
  for (int kt = 0; kt < nk - 1; ++kt) {
    const lds_char* cur = lds + stage * F8_STAGE;
    const int next = stage == S - 1 ? 0 : stage + 1;
    read(cur, 1, a1, b1);
    mma(a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    wait_groups<F8_DMA>(min(S - 2, nk - kt - 2));
    barrier_after_lds_reads();
    if (kt + S < nk) issue(kt + S, stage);
    read(lds + next * F8_STAGE, 0, a0, b0);
    mma(a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    stage = next;
  }
  if (nk >= 1) {
    read(lds + stage * F8_STAGE, 1, a1, b1);
    mma(a0, b0);
    mma(a1, b1);
  }
}

struct Fp8Args {
  const bf16_t* a_src;  // gate/up: x [T, d]; down: H [rows_total, ldh]
  const int32_t* offsets;
  const int32_t* sorted_token;
  const uint8_t* w0;    // gate/up: Wg codes [E, I, d]; down: Wd codes [E, d, I]
  const uint8_t* w1;    // gate/up: Wu codes
  const float* s0;      // column scales of w0 [E, N]
  const float* s1;
  const uint8_t* w0_s;  // shared expert
  const uint8_t* w1_s;
  const float* s0_s;
  const float* s1_s;
  bf16_t* out;          // gate/up: H; down: Y
  const int32_t* tile_group;
  const int32_t* tile_m0;
  const int32_t* tile_count;
  int64_t T;
  int d, E, k, I, Is, ldh;
  int n_ntiles;
};

// AR = 32: launched only when every group holds at most 32 rows (T <= 32)
template <bool GATED, int S, int AR>
__global__ void __launch_bounds__(256, 2) ffn_fp8_stream_kernel(Fp8Args p) {
  constexpr int TN = GATED ? F8_COLS / 2 : F8_COLS;  // output columns per tile
  __shared__ __attribute__((aligned(1024))) char smem[S * F8Geo<AR>::STAGE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1;
  const int wn = wave & 1;

  const int L = xcd_remap(blockIdx.x, *p.tile_count * p.n_ntiles);
  if (L < 0) return;
  const int probe = L / p.n_ntiles;
  const int g = p.tile_group[probe];
  const int first = probe - p.tile_m0[probe] / SBM;
  const Group G = group_info(g, p.offsets, p.T, p.k, p.E, p.I, p.Is);
  const int cnt = (G.rows + SBM - 1) / SBM;
  const int local = L - p.n_ntiles * first;
  const int nt = local / cnt;
  const int m0 = (local % cnt) * SBM;

  const int K = GATED ? p.d : G.n_inter;
  const int N = GATED ? G.n_inter : p.d;
  const int n0 = nt * TN;
  if (n0 >= N) return;

  const uint8_t *W0, *W1 = nullptr;
  const float *S0, *S1 = nullptr;
  if (GATED) {
    W0 = G.shared ? p.w0_s : p.w0 + (size_t)g * p.I * p.d;
    W1 = G.shared ? p.w1_s : p.w1 + (size_t)g * p.I * p.d;
    S0 = G.shared ? p.s0_s : p.s0 + (size_t)g * p.I;
    S1 = G.shared ? p.s1_s : p.s1 + (size_t)g * p.I;
  } else {
    W0 = G.shared ? p.w0_s : p.w0 + (size_t)g * p.d * p.I;
    S0 = G.shared ? p.s0_s : p.s0 + (size_t)g * p.d;
  }

  // A: gathered bf16 rows, as in the bf16 kernel
  const int64_t a_pitch = (GATED ? (int64_t)p.d : (int64_t)p.ldh) * 2;
  uint32_t a_off[F8_A_DMA];
#pragma unroll
  for (int i = 0; i < F8_A_DMA; ++i) {
    const int m = (wave * F8_A_DMA + i) * 16 + (lane >> 2);
    const int r = (m0 + m < G.rows) ? m : 0;  // rows past the group re-read its first row
    int64_t src_row;
    if (GATED)
      src_row = G.shared ? (int64_t)(m0 + r) : (int64_t)p.sorted_token[G.row0 + m0 + r];
    else
      src_row = G.row0 + m0 + r;
    a_off[i] = (uint32_t)(src_row * a_pitch) + a_dma_chunk_bytes(lane);
  }
  const char* a_src = uniform_ptr((const char*)p.a_src);
  auto a_base = [=](int kt) { return a_src + kt * (SBK * 2); };

  // B: waves 0-1 stream the 128-column code panel of tile columns [0, 128), waves 2-3 that of
  // [128, 256): for gate/up the W_g and the W_u panel at columns n0 .., for the down product the
  // panels at n0 and n0 + 128. A panel is K / 32 tiles of 4 KB, one per K step.
  const uint8_t* bmat = (GATED && wave >= 2) ? W1 : W0;
  const int panel = n0 / 128 + (!GATED && wave >= 2 ? 1 : 0);
  const char* b0 = uniform_ptr((const char*)bmat + (int64_t)panel * K * 128 + ((2 * wave) & 3) * 1024);
  uint32_t b_off[F8_B_DMA];
#pragma unroll
  for (int i = 0; i < F8_B_DMA; ++i) b_off[i] = (uint32_t)(i * 1024 + 16 * lane);
  auto b_base = [=](int kt, int) { return b0 + (int64_t)kt * 4096; };

  int bcol[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) bcol[j] = GATED ? (j >> 1) * TN + wn * 64 + (j & 1) * 32 : wn * 128 + j * 32;
  const int nl = live_subtiles(G.rows - m0, wm);
  const int nk = K / SBK;

  f32x16_t acc[2][4];
  zero(acc);
  const int nad = needed_a_dma<2>(G.rows - m0 < SBM ? G.rows - m0 : SBM, wave);
  // the group's only row tile streams its code panels with the non-temporal hint (as in the bf16
  // kernel); row tiles of a larger group share them through L2
  auto run = [&](auto nlc, auto ntc) {
    constexpr int NL = decltype(nlc)::value;
    constexpr bool NT = decltype(ntc)::value;
    if (nad >= 2) mainloop_f8<S, NL, 2, NT, AR>(nk, (lds_char*)smem, a_base, a_off, b_base, b_off, bcol, acc);
    else if (nad == 1) mainloop_f8<S, NL, 1, NT, AR>(nk, (lds_char*)smem, a_base, a_off, b_base, b_off, bcol, acc);
    else mainloop_f8<S, NL, 0, NT, AR>(nk, (lds_char*)smem, a_base, a_off, b_base, b_off, bcol, acc);
  };
  auto run_nt = [&](auto ntc) {
    if constexpr (AR == SBM) {
      if (nl >= 2) run(std::integral_constant<int, 2>(), ntc);
      else if (nl == 1) run(std::integral_constant<int, 1>(), ntc);
      else run(std::integral_constant<int, 0>(), ntc);
    } else {
      if (nl >= 1) run(std::integral_constant<int, 1>(), ntc);
      else run(std::integral_constant<int, 0>(), ntc);
    }
  };
  if (cnt == 1) run_nt(std::true_type());
  else run_nt(std::false_type());

  // epilogue: column scales, then as in the bf16 kernel
  const int col_in = lane & 31;
  const int row_hi = (lane >> 5) * 4;
  if (GATED) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int col = n0 + wn * 64 + jj * 32 + col_in;
        const float sg = S0[col], su = S1[col];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = sub_row(wm, i) + (r >> 2) * 8 + row_hi + (r & 3);
          if (m0 + row < G.rows)
            p.out[(G.row0 + m0 + row) * (int64_t)p.ldh + col] =
                f32_to_bf16(silu_f32(acc[i][jj][r] * sg) * (acc[i][jj + 2][r] * su));
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 128 + j * 32 + col_in;
        const float sd = S0[col];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = sub_row(wm, i) + (r >> 2) * 8 + row_hi + (r & 3);
          if (m0 + row < G.rows) p.out[(G.row0 + m0 + row) * (int64_t)p.d + col] = f32_to_bf16(acc[i][j][r] * sd);
        }
      }
  }
}

// ------------------------------------------------------------------------------------------
// One or two tokens: weight streams over the code tiles on the vector ALUs, as the bf16 skinny
// kernels do (grouped_ffn_skinny.hip). One workgroup (256 threads) per (group, 128-column code
// panel, K split); thread t reads the 16-byte chunk t of every 4 KB code tile of its split --
// column t / 2, one half of the column's 32 K values -- so a wavefront reads 1 KB of contiguous
// codes, and the two threads of a column add their halves at the end. The x (or H) values of the
// split sit in LDS as fp32. Column scales are powers of two, so scaling each split's sums is
// exact: the gate/up product's splits go out scaled, as fp32 partial rows that
// gate_up_finish_kernel adds in split order and finishes with silu * up (H directly with a single
// split); the down product runs unsplit (K = I <= 2048) and writes Y -- in a forward, with
// device-scope stores, and the last group to finish each panel then performs the combine for its
// columns. (A variant that streamed the code tiles into an LDS ring by DMA, as the bf16 skinny
// kernels do, measured slower here: one-token layer 0.132 -> 0.137 ms.)
// ------------------------------------------------------------------------------------------
struct Fp8SkinnyArgs {
  const bf16_t* a_src;  // gate/up: x [T, d]; down: H [rows_total, ldh]
  const int32_t* offsets;
  const int32_t* sorted_token;
  const uint8_t* w0;
  const uint8_t* w1;
  const float* s0;
  const float* s1;
  const uint8_t* w0_s;
  const uint8_t* w1_s;
  const float* s0_s;
  const float* s1_s;
  bf16_t* out;
  const int32_t* tile_group;
  const int32_t* tile_count;
  int64_t T;
  int d, E, k, I, Is, ldh;
  int n_cblk;  // 128-column panels of the widest group
  int ks, kc;  // K splits, K rows per split (multiple of 32, <= kSkinnyMaxKC)
  float* part;  // gate/up with ks > 1: scaled fp32 partial rows part[split][row][part_ld]
  int64_t part_ld, part_sstride;
  // down product with the combine (fout non-null): the block's output rows [T, d], the routing,
  // the residual rows (or null), and one arrival counter per panel, zero on entry
  bf16_t* fout;
  const int32_t* slot_of;
  const float* topk_w;
  const bf16_t* resid;
  int32_t* ccnt;
};

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_codes16(const uint8_t* q) {
  const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)q);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// four e4m3 codes (bytes 0 .. 3 of w, in K order) -> fp32, exactly
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float* f) {
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  f[0] = a[0];
  f[1] = a[1];
  f[2] = b[0];
  f[3] = b[1];
}

template <bool GATED, int R>
__global__ void __launch_bounds__(256, 2) ffn_fp8_skinny_kernel(Fp8SkinnyArgs p) {
  constexpr int NM = GATED ? 2 : 1;  // code matrices
  constexpr int KU = 8;              // code tiles in flight per thread and matrix
  __shared__ __attribute__((aligned(16))) float s_a[R][kSkinnyMaxKC];
  __shared__ int s_last;
  const int tid = threadIdx.x;

  const int per_tile = p.n_cblk * p.ks;
  const int mt = blockIdx.x / per_tile;
  if (mt >= *p.tile_count) return;
  const int rem = blockIdx.x - mt * per_tile;
  const int cb = rem / p.ks;
  const int split = rem - cb * p.ks;
  const int g = p.tile_group[mt];
  const Group G = group_info(g, p.offsets, p.T, p.k, p.E, p.I, p.Is);
  const int K = GATED ? p.d : G.n_inter;
  const int N = GATED ? G.n_inter : p.d;
  const int n0 = cb * 128;
  if (n0 >= N) return;
  const int rows = G.rows;  // <= R
  const int k0 = split * p.kc;
  const int k1 = min(K, k0 + p.kc);  // k1 <= k0: an empty split (partials of zero)

  const uint8_t *W0, *W1 = nullptr;
  const float *S0, *S1 = nullptr;
  if (GATED) {
    W0 = G.shared ? p.w0_s : p.w0 + (size_t)g * p.I * p.d;
    W1 = G.shared ? p.w1_s : p.w1 + (size_t)g * p.I * p.d;
    S0 = G.shared ? p.s0_s : p.s0 + (size_t)g * p.I;
    S1 = G.shared ? p.s1_s : p.s1 + (size_t)g * p.I;
  } else {
    W0 = G.shared ? p.w0_s : p.w0 + (size_t)g * p.d * p.I;
    S0 = G.shared ? p.s0_s : p.s0 + (size_t)g * p.d;
  }
  // chunk tid of each code tile of panel cb: column col, K values 16 half .. +16 of the tile
  const uint8_t* q0 = W0 + (int64_t)cb * K * 128 + 16 * tid;
  const uint8_t* q1 = GATED ? W1 + (int64_t)cb * K * 128 + 16 * tid : nullptr;
  const int col = tid >> 1;
  const int half = (tid & 1) ^ ((col >> 3) & 1);
  const int kt0 = k0 / 32;
  const int ntl = k1 > k0 ? (k1 - k0) / 32 : 0;  // code tiles of this split (K, kc multiples of 32)

  // A rows of this split as fp32 (rows past the group's are zero), as in the bf16 skinny kernel
  const int64_t a_ld = GATED ? p.d : p.ldh;
  int64_t srow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int rr = r < rows ? r : 0;
    srow[r] = GATED ? (G.shared ? (int64_t)rr : (int64_t)p.sorted_token[G.row0 + rr]) : G.row0 + rr;
  }
  const int cpr = p.kc / 8;  // A chunks (8 values) per row; R * cpr <= R * 256
  uint4 av[R];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int i = tid + 256 * j;
    const int r = i / cpr;
    const int c = i - r * cpr;
    int64_t sr = srow[0];
#pragma unroll
    for (int q = 1; q < R; ++q)
      if (r == q) sr = srow[q];
    const bool valid = r < rows && k0 + 8 * c < k1;
    av[j] = *(const uint4*)(p.a_src + (valid ? sr * a_ld + k0 + 8 * c : 0));
    if (!valid) av[j] = make_uint4(0u, 0u, 0u, 0u);
  }

  uint4 buf[NM][KU];
  auto load = [&](int b) {
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int64_t at = (int64_t)(kt0 + KU * b + u) * 4096;
      buf[0][u] = load_codes16(q0 + at);
      if (GATED) buf[NM - 1][u] = load_codes16(q1 + at);
    }
    __builtin_amdgcn_sched_barrier(0);  // the batch's loads go out before the work that follows
  };
  float acc[NM][R];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[m][r] = 0.f;
  // this thread's 16 K values of code tile t (from k0) against the staged rows
  auto tile = [&](const uint4 (&c)[NM], int t) {
    const int kk = t * 32 + 16 * half;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      float w[16];
      e4m3x4_to_f32(c[m].x, w);
      e4m3x4_to_f32(c[m].y, w + 4);
      e4m3x4_to_f32(c[m].z, w + 8);
      e4m3x4_to_f32(c[m].w, w + 12);
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const float4 a = *(const float4*)&s_a[r][kk + 4 * i4];
          acc[m][r] = fmaf(a.x, w[4 * i4], acc[m][r]);
          acc[m][r] = fmaf(a.y, w[4 * i4 + 1], acc[m][r]);
          acc[m][r] = fmaf(a.z, w[4 * i4 + 2], acc[m][r]);
          acc[m][r] = fmaf(a.w, w[4 * i4 + 3], acc[m][r]);
        }
    }
  };
  const int nbw = ntl / KU;  // whole batches
  if (nbw > 0) load(0);  // the first batch goes out before the A rows are staged
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int i = tid + 256 * j;
    const int r = i / cpr;
    const int c = i - r * cpr;
    if (r < R) {
      float* dst = &s_a[r][8 * c];
      *(float4*)dst = make_float4(bf16lo_to_f32(av[j].x), bf16hi_to_f32(av[j].x), bf16lo_to_f32(av[j].y),
                                  bf16hi_to_f32(av[j].y));
      *(float4*)(dst + 4) = make_float4(bf16lo_to_f32(av[j].z), bf16hi_to_f32(av[j].z), bf16lo_to_f32(av[j].w),
                                        bf16hi_to_f32(av[j].w));
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // the code loads stay in flight
  for (int b = 0; b < nbw; ++b) {
    if (b > 0) load(b);
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      uint4 c[NM];
#pragma unroll
      for (int m = 0; m < NM; ++m) c[m] = buf[m][u];
      tile(c, KU * b + u);
    }
  }
  for (int t = nbw * KU; t < ntl; ++t) {  // tiles past the whole batches, one at a time
    uint4 c[NM];
    const int64_t at = (int64_t)(kt0 + t) * 4096;
    c[0] = load_codes16(q0 + at);
    if (GATED) c[NM - 1] = load_codes16(q1 + at);
    tile(c, t);
  }

  // the column's two halves, then one thread per column writes
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[m][r] += __shfl_xor(acc[m][r], 1, 64);
  const int n = n0 + col;
  if (!GATED && p.fout) {
    // Y with device-scope stores, two columns per store (thread 4j holds columns 2j and 2j + 1);
    // the last group to finish this panel (by the counter, after every thread's stores
    // completed) then performs the combine for its 128 columns
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float y0 = acc[0][r] * S0[n];
      const float y1 = __shfl_down(y0, 2, 64);
      if ((tid & 3) == 0 && r < rows)
        __hip_atomic_store((uint32_t*)(p.out + (G.row0 + r) * (int64_t)p.d + n), pack_bf16x2(y0, y1),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0)
      s_last = __hip_atomic_fetch_add(&p.ccnt[cb], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               *p.tile_count - 1;
    __syncthreads();
    const int t = tid >> 6;  // 64 column pairs per token
    if (s_last && t < p.T)
      combine_pair(p.out, p.fout, p.slot_of, p.topk_w, p.resid, p.T, p.d, p.k, p.Is > 0, t, n0 + 2 * (tid & 63));
    return;
  }
  if (tid & 1) return;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r >= rows) break;
    const int64_t row = G.row0 + r;
    if (GATED) {
      const float gs = acc[0][r] * S0[n], us = acc[NM - 1][r] * S1[n];
      if (p.ks > 1) {
        float* q = p.part + (int64_t)split * p.part_sstride + row * p.part_ld + n;
        q[0] = gs;
        q[p.ldh] = us;
      } else {
        p.out[row * p.ldh + n] = f32_to_bf16(silu_f32(gs) * us);
      }
    } else {
      p.out[row * (int64_t)p.d + n] = f32_to_bf16(acc[0][r] * S0[n]);
    }
  }
}

// ------------------------------------------------------------------------------------------
// quantiser: w [batch, K, N] -> codes [batch] x (N / 128 x K / 32 tiles of 4 KB), scales [batch, N]
// ------------------------------------------------------------------------------------------
template <typename WT>
__device__ __forceinline__ float wval(const WT* p, int64_t i);
template <>
__device__ __forceinline__ float wval<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float wval<bf16_t>(const bf16_t* p, int64_t i) { return bf16lo_to_f32(p[i]); }

// grid (N / 64, batch); 256 threads; N % 128 == 0, K % 32 == 0. Pass 1: column maxima (thread:
// column tid % 64, rows tid / 64 + 4i). Pass 2: 64 x 64 blocks through LDS; each thread rounds 16
// K-consecutive values of one column and stores them as one 16-byte half of the column's run in
// its code tile.
template <typename WT>
__global__ void __launch_bounds__(256)
quantize_fp8_kernel(const WT* __restrict__ w, int K, int N, uint8_t* __restrict__ q, float* __restrict__ scale) {
  __shared__ float red[4][64];
  __shared__ int sexp[64];
  __shared__ float tile[64][65];
  const int tid = threadIdx.x;
  const int c = tid & 63;
  const int r0 = tid >> 6;
  const int n = blockIdx.x * 64 + c;
  const int64_t b = blockIdx.y;
  const WT* wb = w + b * (int64_t)K * N;
  float amax = 0.f;
  // maximum of magnitudes that keeps a NaN (fmaxf would drop it): a column holding a non-finite
  // weight gets a NaN scale
  for (int k = r0; k < K; k += 4) {
    const float v = fabsf(wval(wb, (int64_t)k * N + n));
    amax = (v > amax || isnan(v)) ? v : amax;
  }
  red[r0][c] = amax;
  __syncthreads();
  if (r0 == 0) {
    float m = red[0][c];
    for (int i = 1; i < 4; ++i) m = (red[i][c] > m || isnan(red[i][c])) ? red[i][c] : m;
    int e;
    const bool finite = fp8::scale_exp(m, &e);
    sexp[c] = e;
    scale[b * N + n] = finite ? ldexpf(1.0f, e) : __builtin_nanf("");
  }
  __syncthreads();
  uint8_t* qb = q + b * (int64_t)N * K;
  for (int k0 = 0; k0 < K; k0 += 64) {
    for (int i = tid; i < 64 * 64; i += 256) {
      const int kk = i / 64, cc = i % 64;
      const int nn = blockIdx.x * 64 + cc;
      tile[kk][cc] = k0 + kk < K ? wval(wb, (int64_t)(k0 + kk) * N + nn) : 0.f;
    }
    __syncthreads();
    // thread: column tid / 4, K values 16 * (tid % 4) .. +16 of the block
    const int cc = tid >> 2;
    const int kk = k0 + (tid & 3) * 16;
    if (kk < K) {
      const int nn = blockIdx.x * 64 + cc;
      const int e = sexp[cc];
      uint32_t wd[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 16; ++i)
        wd[i >> 2] |= (uint32_t)fp8::e4m3_rne(ldexpf(tile[kk - k0 + i][cc], -e)) << (8 * (i & 3));
      const int r = nn & 127;
      const int h = (kk >> 4) & 1;
      const int64_t at = ((int64_t)(nn >> 7) * (K >> 5) + (kk >> 5)) * 4096 + r * 32 + 16 * (h ^ ((r >> 3) & 1));
      *(uint4*)(qb + at) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    }
    __syncthreads();
  }
}

}  // namespace

bool fp8_shape_ok(const moe_dims& dm) {
  return dm.dtype == MOE_BF16 && dm.d % 256 == 0 && dm.I % 128 == 0 && dm.I_shared % 128 == 0 &&
         (uint64_t)dm.T * dm.d * 2 < (1ull << 32) &&
         (uint64_t)(dm.T * dm.k + dm.T) * (dm.I > dm.I_shared ? dm.I : dm.I_shared) * 2 < (1ull << 32);
}

namespace {

// K split of the skinny gate/up product over the code streams (one or two tokens, ldh <=
// kSkinnyMaxKC): ~1024 workgroups (what the CUs hold at once) with 256 to kSkinnyMaxKC K values
// per split and no more splits than the workspace's partial rows hold. 0: the skinny path does
// not apply (the MFMA tiles run instead).
int fp8_skinny_splits(const moe_dims& dm, const Layout& L) {
  if (dm.T < 1 || dm.T > kSkinnyMaxT || L.ldh > kSkinnyMaxKC) return 0;
  const int64_t Tk = dm.T * dm.k;
  const int64_t groups = (Tk < dm.E ? Tk : dm.E) + (dm.I_shared > 0 ? 1 : 0);
  const int64_t sstride = L.rows_total * 2 * (int64_t)L.ldh;
  const int64_t room = (int64_t)(L.ffn_cnt - L.ffn_part) / (sstride * 4);
  int64_t ks = 1024 / (groups * (L.ldh / 128));
  if (ks > dm.d / 256) ks = dm.d / 256;
  if (ks > room) ks = room;
  const int64_t least = (dm.d + kSkinnyMaxKC - 1) / kSkinnyMaxKC;
  if (ks < least) ks = least;
  if (ks < 1) ks = 1;
  if (ks > 1 && ks > room) return 0;
  const int64_t kc = ((dm.d + ks - 1) / ks + 31) / 32 * 32;
  return (int)((dm.d + kc - 1) / kc);
}

// one or two tokens: the skinny code streams; the down product runs unsplit (and, with `combine`,
// also writes the block's output)
hipError_t launch_fp8_skinny(const moe_dims& dm, const Layout& L, int ks, const void* x, const int32_t* offsets,
                             const int32_t* sorted_token, const Fp8Weights& W, void* y, char* ws, hipStream_t s,
                             const Prof* prof, CombineFuse* combine) {
  const int has_shared = dm.I_shared > 0 ? 1 : 0;
  const int64_t Tk = dm.T * dm.k;
  const int64_t groups = (Tk < dm.E ? Tk : dm.E) + has_shared;  // tiles: one per group with rows
  Fp8SkinnyArgs a{};
  a.offsets = offsets;
  a.sorted_token = sorted_token;
  a.tile_group = (const int32_t*)(ws + L.tile_group);
  a.tile_count = (const int32_t*)(ws + L.tile_count);
  a.T = dm.T;
  a.d = dm.d;
  a.E = dm.E;
  a.k = dm.k;
  a.I = dm.I;
  a.Is = dm.I_shared;
  a.ldh = L.ldh;
  bf16_t* H = (bf16_t*)(ws + L.H);
  // gate/up
  const int cb1 = L.ldh / 128;
  const int64_t part_ld = 2 * (int64_t)L.ldh;
  const int64_t sstride = L.rows_total * part_ld;
  const int kc = (int)(((dm.d + ks - 1) / ks + 31) / 32 * 32);
  a.a_src = (const bf16_t*)x;
  a.w0 = W.wg;
  a.w1 = W.wu;
  a.s0 = W.sg;
  a.s1 = W.su;
  a.w0_s = W.wg_s;
  a.w1_s = W.wu_s;
  a.s0_s = W.sg_s;
  a.s1_s = W.su_s;
  a.out = H;
  a.n_cblk = cb1;
  a.ks = (int)ks;
  a.kc = kc;
  a.part = (float*)(ws + L.ffn_part);
  a.part_ld = part_ld;
  a.part_sstride = sstride;
  hipError_t e;
  if ((e = prof->begin(MOE_KERNEL_FFN_GATE_UP, s)) != hipSuccess) return e;
  const dim3 grid1((unsigned)(groups * cb1 * ks));
  if (dm.T <= 1) hipLaunchKernelGGL((ffn_fp8_skinny_kernel<true, 1>), grid1, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((ffn_fp8_skinny_kernel<true, 2>), grid1, dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ks > 1 && (e = launch_gate_up_finish(a.part, sstride, part_ld, (int)ks, Tk, L.rows_total, dm.I, dm.I_shared,
                                           L.ldh, H, s)) != hipSuccess)
    return e;
  if ((e = prof->end(MOE_KERNEL_FFN_GATE_UP, s)) != hipSuccess) return e;
  // down: K = the group's intermediate width <= ldh <= kSkinnyMaxKC, one split
  a.a_src = H;
  a.w0 = W.wd;
  a.w1 = nullptr;
  a.s0 = W.sd;
  a.s1 = nullptr;
  a.w0_s = W.wd_s;
  a.w1_s = nullptr;
  a.s0_s = W.sd_s;
  a.s1_s = nullptr;
  a.out = (bf16_t*)y;
  a.n_cblk = dm.d / 128;
  a.ks = 1;
  a.kc = L.ldh;
  a.part = nullptr;
  if (combine) {
    // one arrival counter per 128-column panel: the first bank of the split-K counters, which the
    // gate/up product does not use (the layout sizes and the tile list zeroes at least d / 128)
    a.fout = (bf16_t*)combine->out;
    a.slot_of = combine->slot_of;
    a.topk_w = combine->topk_w;
    a.resid = (const bf16_t*)combine->residual;
    a.ccnt = (int32_t*)(ws + L.ffn_cnt);
    combine->done = true;
  }
  if ((e = prof->begin(MOE_KERNEL_FFN_DOWN, s)) != hipSuccess) return e;
  const dim3 grid2((unsigned)(groups * a.n_cblk));
  if (dm.T <= 1) hipLaunchKernelGGL((ffn_fp8_skinny_kernel<false, 1>), grid2, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((ffn_fp8_skinny_kernel<false, 2>), grid2, dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return prof->end(MOE_KERNEL_FFN_DOWN, s);
}

}  // namespace

const char* ffn_fp8_kernel_name(const moe_dims& dm, bool gate_up) {
  if (fp8_skinny_splits(dm, make_layout(dm)) > 0) {
    if (dm.T <= 1) return gate_up ? "ffn_fp8_skinny_kernel<true, 1>" : "ffn_fp8_skinny_kernel<false, 1>";
    return gate_up ? "ffn_fp8_skinny_kernel<true, 2>" : "ffn_fp8_skinny_kernel<false, 2>";
  }
  if (dm.T <= 32) return gate_up ? "ffn_fp8_stream_kernel<true, 4, 32>" : "ffn_fp8_stream_kernel<false, 4, 32>";
  return gate_up ? "ffn_fp8_stream_kernel<true, 5, 128>" : "ffn_fp8_stream_kernel<false, 5, 128>";
}

hipError_t launch_grouped_ffn_fp8(const moe_dims& dm, const Layout& L, const void* x, const int32_t* offsets,
                                  const int32_t* sorted_token, const Fp8Weights& W, void* y, char* ws, hipStream_t s,
                                  const Prof* prof, CombineFuse* combine) {
  const Prof none;
  if (!prof) prof = &none;
  // five stages of 16 KB (80 KB of LDS, still two workgroups per CU): with the non-temporal code
  // stream, the deeper lookahead took decode gate/up from 1.34 to 1.29 ms. At most 32 tokens:
  // four stages of 10 KB (32 A rows), four workgroups per CU.
  constexpr int S = 5, S_THIN = 4;
  const bool thin = dm.T <= 32;
  // 128-row tiles, whatever the bf16 GEMMs would use for these dims
  hipError_t e = launch_build_tiles(dm, L, offsets, ws, s, SBM);
  if (e != hipSuccess) return e;
  const int ks_skinny = fp8_skinny_splits(dm, L);
  if (ks_skinny > 0)
    return launch_fp8_skinny(dm, L, ks_skinny, x, offsets, sorted_token, W, y, ws, s, prof, combine);
  const int has_shared = dm.I_shared > 0 ? 1 : 0;
  const int64_t Tk = dm.T * dm.k;
  const int64_t max_mt = Tk / SBM + (Tk < dm.E ? Tk : dm.E) + (has_shared ? dm.T / SBM + 1 : 0);
  Fp8Args a;
  a.offsets = offsets;
  a.sorted_token = sorted_token;
  a.tile_group = (const int32_t*)(ws + L.tile_group);
  a.tile_m0 = (const int32_t*)(ws + L.tile_m0);
  a.tile_count = (const int32_t*)(ws + L.tile_count);
  a.T = dm.T;
  a.d = dm.d;
  a.E = dm.E;
  a.k = dm.k;
  a.I = dm.I;
  a.Is = dm.I_shared;
  a.ldh = L.ldh;
  bf16_t* H = (bf16_t*)(ws + L.H);
  // gate/up
  a.a_src = (const bf16_t*)x;
  a.w0 = W.wg;
  a.w1 = W.wu;
  a.s0 = W.sg;
  a.s1 = W.su;
  a.w0_s = W.wg_s;
  a.w1_s = W.wu_s;
  a.s0_s = W.sg_s;
  a.s1_s = W.su_s;
  a.out = H;
  a.n_ntiles = (L.ldh + F8_COLS / 2 - 1) / (F8_COLS / 2);
  if ((e = prof->begin(MOE_KERNEL_FFN_GATE_UP, s)) != hipSuccess) return e;
  if (thin)
    hipLaunchKernelGGL((ffn_fp8_stream_kernel<true, S_THIN, 32>), dim3((unsigned)(max_mt * a.n_ntiles)), dim3(256), 0,
                       s, a);
  else
    hipLaunchKernelGGL((ffn_fp8_stream_kernel<true, S, SBM>), dim3((unsigned)(max_mt * a.n_ntiles)), dim3(256), 0, s,
                       a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = prof->end(MOE_KERNEL_FFN_GATE_UP, s)) != hipSuccess) return e;
  // down
  a.a_src = H;
  a.w0 = W.wd;
  a.w1 = nullptr;
  a.s0 = W.sd;
  a.s1 = nullptr;
  a.w0_s = W.wd_s;
  a.w1_s = nullptr;
  a.s0_s = W.sd_s;
  a.s1_s = nullptr;
  a.out = (bf16_t*)y;
  a.n_ntiles = dm.d / F8_COLS;
  if ((e = prof->begin(MOE_KERNEL_FFN_DOWN, s)) != hipSuccess) return e;
  if (thin)
    hipLaunchKernelGGL((ffn_fp8_stream_kernel<false, S_THIN, 32>), dim3((unsigned)(max_mt * a.n_ntiles)), dim3(256), 0,
                       s, a);
  else
    hipLaunchKernelGGL((ffn_fp8_stream_kernel<false, S, SBM>), dim3((unsigned)(max_mt * a.n_ntiles)), dim3(256), 0, s,
                       a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return prof->end(MOE_KERNEL_FFN_DOWN, s);
}

hipError_t launch_quantize_fp8(const void* w, int dtype, int64_t batch, int K, int N, uint8_t* q, float* scale,
                               hipStream_t s) {
  const dim3 grid((unsigned)(N / 64), (unsigned)batch);
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(quantize_fp8_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)w, K, N, q, scale);
  else
    hipLaunchKernelGGL(quantize_fp8_kernel<float>, grid, dim3(256), 0, s, (const float*)w, K, N, q, scale);
  return hipGetLastError();
}

}  // namespace moe
