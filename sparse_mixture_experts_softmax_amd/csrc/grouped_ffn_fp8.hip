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
#include "moe_internal.h"
#include "stream_gemm.h"

namespace moe {
namespace {

using namespace stream;

constexpr int F8_COLS = 256;
constexpr int F8_A_BYTES = SBM * SBK * 2;    // 8 KB
constexpr int F8_B_BYTES = F8_COLS * SBK;    // 8 KB
constexpr int F8_STAGE = F8_A_BYTES + F8_B_BYTES;
constexpr int F8_A_DMA = 2;                  // per wave per stage
constexpr int F8_B_DMA = 2;

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
template <int S, int NL, int NAD, bool NT, class ABase, class BBase>
__device__ __forceinline__ void mainloop_f8(int nk, lds_char* lds, ABase a_base, const uint32_t (&a_off)[F8_A_DMA],
                                            BBase b_base, const uint32_t (&b_off)[F8_B_DMA], const int (&bcol)[4],
                                            f32x16_t (&acc)[2][4]) {
  static_assert(S >= 3 && S <= 6, "stages");
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

template <bool GATED, int S>
__global__ void __launch_bounds__(256, 2) ffn_fp8_stream_kernel(Fp8Args p) {
  constexpr int TN = GATED ? F8_COLS / 2 : F8_COLS;  // output columns per tile
  __shared__ __attribute__((aligned(1024))) char smem[S * F8_STAGE];
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
    if (nad >= 2) mainloop_f8<S, NL, 2, NT>(nk, (lds_char*)smem, a_base, a_off, b_base, b_off, bcol, acc);
    else if (nad == 1) mainloop_f8<S, NL, 1, NT>(nk, (lds_char*)smem, a_base, a_off, b_base, b_off, bcol, acc);
    else mainloop_f8<S, NL, 0, NT>(nk, (lds_char*)smem, a_base, a_off, b_base, b_off, bcol, acc);
  };
  auto run_nt = [&](auto ntc) {
    if (nl >= 2) run(std::integral_constant<int, 2>(), ntc);
    else if (nl == 1) run(std::integral_constant<int, 1>(), ntc);
    else run(std::integral_constant<int, 0>(), ntc);
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
// quantiser: w [batch, K, N] -> codes [batch] x (N / 128 x K / 32 tiles of 4 KB), scales [batch, N]
// ------------------------------------------------------------------------------------------
// nearest e4m3 code of v (|v| <= 448), ties to even, by rounding exactly scaled values to integers
__device__ __forceinline__ uint8_t e4m3_rne(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  int code;
  if (a < 0x1p-6f) {
    code = (int)rintf(a * 512.0f);  // multiples of 2^-9; 8 is the smallest normal's code
  } else {
    int e;
    frexpf(a, &e);  // a in [2^(e-1), 2^e)
    const int E = e - 1;
    int m = (int)rintf(ldexpf(a, 3 - E)) - 8;  // 0 .. 8
    int EE = E;
    if (m == 8) {
      m = 0;
      EE += 1;
    }
    code = ((EE + 7) << 3) | m;
  }
  return code == 0 ? (uint8_t)0 : (uint8_t)(code | sign);
}

// smallest e with |amax| 2^-e <= 448 (0 for amax = 0): the column's scale is 2^e
__device__ __forceinline__ int scale_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  int e = ilogbf(amax) - 10;
  while (ldexpf(amax, -e) > 448.0f) ++e;
  return e;
}

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
  for (int k = r0; k < K; k += 4) amax = fmaxf(amax, fabsf(wval(wb, (int64_t)k * N + n)));
  red[r0][c] = amax;
  __syncthreads();
  if (r0 == 0) {
    const float m = fmaxf(fmaxf(red[0][c], red[1][c]), fmaxf(red[2][c], red[3][c]));
    const int e = scale_exp(m);
    sexp[c] = e;
    scale[b * N + n] = ldexpf(1.0f, e);
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
        wd[i >> 2] |= (uint32_t)e4m3_rne(ldexpf(tile[kk - k0 + i][cc], -e)) << (8 * (i & 3));
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

hipError_t launch_grouped_ffn_fp8(const moe_dims& dm, const Layout& L, const void* x, const int32_t* offsets,
                                  const int32_t* sorted_token, const Fp8Weights& W, void* y, char* ws, hipStream_t s,
                                  const Prof* prof) {
  const Prof none;
  if (!prof) prof = &none;
  // five stages of 16 KB (80 KB of LDS, still two workgroups per CU): with the non-temporal code
  // stream, the deeper lookahead took decode gate/up from 1.34 to 1.29 ms
  constexpr int S = 5;
  hipError_t e = launch_build_tiles(dm, L, offsets, ws, s);
  if (e != hipSuccess) return e;
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
  hipLaunchKernelGGL((ffn_fp8_stream_kernel<true, S>), dim3((unsigned)(max_mt * a.n_ntiles)), dim3(256), 0, s, a);
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
  hipLaunchKernelGGL((ffn_fp8_stream_kernel<false, S>), dim3((unsigned)(max_mt * a.n_ntiles)), dim3(256), 0, s, a);
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
