// Router and softmax top-k.
//
// The router is a linear map from the token's hidden vector to one score per
// expert; a softmax over all experts gives each a probability and the k most
// probable are kept (Qwen3.6 neural-network explorer page, section on the MoE
// router). Selection is made on the fp32 logits (same order as the
// probabilities), ties go to the lower expert index, and the kept
// probabilities are optionally renormalised to sum to one.
//
// Logits, two ways (both fp32-accurate, both optionally split over K with the
// partial sums added by the top-k kernel in a fixed order):
//   router_mfma:   bf16 x and enough tokens. W_r (fp32) is split into three
//                  bf16 parts hi + mid + lo = W_r exactly (each part is the
//                  round-to-nearest bf16 of the remainder; 24 significand bits
//                  fit in three 8-bit ones), stacked along K, so
//                  x W_r = x hi + x mid + x lo with every product exact in fp32;
//                  the streaming bf16 MFMA mainloop runs over K' = 3d.
//   router_logits: fp32 GEMM on the vector ALUs, 64x64 (token x expert) tiles,
//                  4x4 outputs per thread, LDS-staged.
// router_topk: one 64-lane wavefront per token: sums the splits (+ bias) in a
// fixed order, then k (+1 for the gap) rounds of a wave-wide argmax built from
// cross-lane shuffles, then the softmax normaliser as a wave-wide sum.
#include <math.h>

#include "moe_internal.h"
#include "stream_gemm.h"

namespace moe {
namespace {

// W_r [d, E] fp32 -> three bf16 planes [3][d][E]: hi = bf16(w), mid = bf16(w - hi),
// lo = bf16(w - hi - mid); both differences are exact in fp32 and lo is exact in bf16.
__global__ void __launch_bounds__(256)
router_split_kernel(const float* __restrict__ w, bf16_t* __restrict__ planes, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;  // n = d * E is a multiple of 4 (d % 8 == 0)
  const float x[4] = {w[i], w[i + 1], w[i + 2], w[i + 3]};  // w_router is only 4-byte aligned
  uint32_t p0[2], p1[2], p2[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    bf16_t a[2], b[2], c[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float wv = x[2 * h + j];
      a[j] = f32_to_bf16(wv);
      const float r1 = wv - bf16_to_f32(a[j]);
      b[j] = f32_to_bf16(r1);
      const float r2 = r1 - bf16_to_f32(b[j]);
      c[j] = f32_to_bf16(r2);
    }
    p0[h] = (uint32_t)a[0] | ((uint32_t)a[1] << 16);
    p1[h] = (uint32_t)b[0] | ((uint32_t)b[1] << 16);
    p2[h] = (uint32_t)c[0] | ((uint32_t)c[1] << 16);
  }
  *(uint2*)(planes + i) = make_uint2(p0[0], p0[1]);
  *(uint2*)(planes + n + i) = make_uint2(p1[0], p1[1]);
  *(uint2*)(planes + 2 * n + i) = make_uint2(p2[0], p2[1]);
}

// Logits on MFMA: 128 tokens x 128 WN experts per workgroup (the streaming tile of stream_gemm.h:
// WN = 2, four wavefronts, three stages, two workgroups per CU; WN = 4, eight wavefronts, four
// stages, one per CU, fewer L2 -> LDS bytes per FLOP on the long K' = 3d loop), K' split into
// `splits` chunks of `ksteps` 32-wide steps. grid = splits * token tiles * expert tiles.
template <int WN>
__global__ void __launch_bounds__(128 * WN, WN == 2 ? 2 : 1)
router_mfma_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ planes, float* __restrict__ part,
                   int64_t T, int d, int E, int ksteps) {
  using namespace stream;
  using GEO = Geo<WN>;
  constexpr int S = WN == 2 ? 3 : 4;
  constexpr int COLS = 128 * WN;
  constexpr int NT = 128 * WN;  // threads
  __shared__ __attribute__((aligned(1024))) char smem[S * GEO::STAGE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int n_et = E / COLS;
  const int n_mt = (int)((T + 127) / 128);
  const int et = blockIdx.x % n_et;
  const int mt = (blockIdx.x / n_et) % n_mt;
  const int split = blockIdx.x / (n_et * n_mt);
  const int64_t t0 = (int64_t)mt * 128;
  const int e0 = et * COLS;
  const int dk = d / 32;  // K steps per plane
  const int kt0 = split * ksteps;
  const int nk = min(ksteps, 3 * dk - kt0);

  uint32_t a_off[GEO::A_DMA];
#pragma unroll
  for (int i = 0; i < GEO::A_DMA; ++i) {
    const int64_t row = min(t0 + a_dma_row<WN>(wave, i, lane), T - 1);
    a_off[i] = (uint32_t)(row * d * 2) + a_dma_chunk_bytes(lane);
  }
  const char* xb = uniform_ptr((const char*)x);
  auto a_base = [=](int kt) { return xb + ((kt0 + kt) % dk) * (SBK * 2); };
  const int64_t pitch = (int64_t)E * 2;
  const char* pb = uniform_ptr((const char*)planes + (int64_t)(e0 + 128 * b_dma_block<WN>(wave)) * 2 +
                               ((int64_t)kt0 * SBK + b_dma_row0<WN>(wave, 0)) * pitch);
  auto b_base = [=](int kt, int i) { return pb + (int64_t)kt * SBK * pitch + i * 4 * pitch; };
  const uint32_t b_off = b_dma_lane_offset(lane, (uint32_t)pitch);
  int bcol[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) bcol[j] = wn * 128 + j * 32;
  const int nl = live_subtiles((int)min<int64_t>(T - t0, 128), wm);

  f32x16_t acc[2][4];
  zero(acc);
  mainloop<WN, S>(nk, nl, (int)min<int64_t>(T - t0, 128), (lds_char*)smem, a_base, a_off, b_base, b_off, bcol, acc);

  // Partial logits through LDS, 64 tile rows at a time (sub-tile u of both wave rows: tile rows
  // 64u .. 64u+63), so that each lane stores whole 16-byte runs of a row instead of single floats.
  // Row pitch 4 COLS + 32 bytes: the rows r and r + 4 that the two lane halves write fall on
  // disjoint banks.
  constexpr int PITCH = COLS * 4 + 32;
  constexpr int RUNS = COLS / 4;  // 16-byte runs per staged row
  static_assert(64 * PITCH <= S * GEO::STAGE, "64 staged rows fit the LDS stages");
  float* out = part + (int64_t)split * T * E + e0;
  char* st = smem;
  const int col_in = lane & 31;
  const int row_hi = (lane >> 5) * 4;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    __syncthreads();  // every wave is past its mainloop (u = 0) or its stores of the last pass
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = wn * 128 + j * 32 + col_in;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 32 + (r >> 2) * 8 + row_hi + (r & 3);
        *(float*)(st + row * PITCH + c * 4) = acc[u][j][r];
      }
    }
    __syncthreads();
    for (int q = tid; q < 64 * RUNS; q += NT) {  // 64 rows x RUNS runs of 16 bytes
      const int row = q / RUNS, ch = q % RUNS;
      const int64_t t = t0 + 64 * u + row;
      if (t < T) *(float4*)(out + t * E + ch * 4) = *(const float4*)(st + row * PITCH + ch * 16);
    }
  }
}

template <typename XT>
__device__ __forceinline__ void load_x4(const XT* p, float* v);

template <>
__device__ __forceinline__ void load_x4<float>(const float* p, float* v) {
  float4 f = *(const float4*)p;
  v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
}

template <>
__device__ __forceinline__ void load_x4<bf16_t>(const bf16_t* p, float* v) {
  uint2 w = *(const uint2*)p;
  v[0] = bf16lo_to_f32(w.x); v[1] = bf16hi_to_f32(w.x);
  v[2] = bf16lo_to_f32(w.y); v[3] = bf16hi_to_f32(w.y);
}

// grid: (expert tiles, token tiles, splits); 256 threads
template <typename XT>
__global__ void __launch_bounds__(256)
router_logits_kernel(const XT* __restrict__ x, const float* __restrict__ wr, float* __restrict__ part,
                     int64_t T, int d, int E, int kchunk) {
  constexpr int TT = kRouterTileT, TE = kRouterTileE, KS = kRouterKStep;
  __shared__ float xs[KS][TT + 4];
  __shared__ float wsm[KS][TE + 4];

  const int tid = threadIdx.x;
  const int e0 = blockIdx.x * TE;
  const int64_t t0 = (int64_t)blockIdx.y * TT;
  const int split = blockIdx.z;
  const int kbeg = split * kchunk;
  const int kend = min(d, kbeg + kchunk);

  const int tx = tid % 16;  // experts tx*4 .. +4
  const int ty = tid / 16;  // tokens  ty*4 .. +4
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

  // x tile loader: token tid/4, hidden kq = (tid%4)*4 .. +4
  const int xl_t = tid / 4;
  const int xl_k = (tid % 4) * 4;
  const bool xl_ok = t0 + xl_t < T;
  const XT* xrow = x + (xl_ok ? (t0 + xl_t) : 0) * (int64_t)d;
  // W tile loader: hidden row tid/16, experts (tid%16)*4 .. +4
  const int wl_k = tid / 16;
  const int wl_e = (tid % 16) * 4;

  for (int k0 = kbeg; k0 < kend; k0 += KS) {
    {
      float v[4] = {0.f, 0.f, 0.f, 0.f};
      if (xl_ok && k0 + xl_k < kend) load_x4<XT>(xrow + k0 + xl_k, v);  // d % 8 == 0: 4 in or all out
#pragma unroll
      for (int i = 0; i < 4; ++i) xs[xl_k + i][xl_t] = v[i];
    }
    {
      const int kk = k0 + wl_k;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = e0 + wl_e + i;
        wsm[wl_k][wl_e + i] = (kk < kend && e < E) ? wr[(int64_t)kk * E + e] : 0.f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const float4 a = *(const float4*)&xs[kk][ty * 4];
      const float4 b = *(const float4*)&wsm[kk][tx * 4];
      const float av[4] = {a.x, a.y, a.z, a.w};
      const float bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }

  float* out = part + (int64_t)split * T * E;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t t = t0 + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e < E) out[t * E + e] = acc[i][j];
    }
  }
}

// Few tokens (T <= 64): one workgroup per (64 experts, K split) streams its weight rows with all
// of a pass's loads (64 per thread) in flight before the first multiply, the pass's x rows staged
// in LDS. Wavefront q takes rows 16i + 4q .. +4 of each 256-row pass; the four wavefronts' sums
// are added in order q = 0..3 at the end. Writes the same per-split partial logits as
// router_logits_kernel.
constexpr int kSmallRows = 256;

template <typename XT, int TT>
__global__ void __launch_bounds__(256)
router_small_kernel(const XT* __restrict__ x, const float* __restrict__ wr, float* __restrict__ part, int64_t T,
                    int d, int E, int kchunk) {
  __shared__ __attribute__((aligned(16))) float xs[TT * kSmallRows];  // [token][row of the pass]
  const int tid = threadIdx.x;
  const int el = tid & 63;
  const int q = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int e = blockIdx.x * 64 + el;
  const int split = blockIdx.y;
  const int kbeg = split * kchunk;
  const int kend = min(d, kbeg + kchunk);
  float acc[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = 0.f;

  constexpr int NXC = TT * kSmallRows / 4;  // 4-value x chunks per pass
  constexpr int NX = (NXC + 255) / 256;      // per thread
  for (int k0 = kbeg; k0 < kend; k0 += kSmallRows) {
    const int kn = min(kSmallRows, kend - k0);  // a multiple of 8
    // the pass's x values and weights are all requested before any is used: one memory round trip
    float xv[NX][4];
#pragma unroll
    for (int u = 0; u < NX; ++u) {
      const int i = tid + 256 * u;
      const int t = i / (kSmallRows / 4);
      const int r4 = (i % (kSmallRows / 4)) * 4;
      xv[u][0] = xv[u][1] = xv[u][2] = xv[u][3] = 0.f;
      if (i < NXC && t < T && r4 < kn) load_x4<XT>(x + (int64_t)t * d + k0 + r4, xv[u]);
    }
    float w[64];
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int r = 16 * i + 4 * q + c;
        w[4 * i + c] = (r < kn && e < E) ? wr[(int64_t)(k0 + r) * E + e] : 0.f;
      }
    __syncthreads();  // the previous pass is done with xs
#pragma unroll
    for (int u = 0; u < NX; ++u) {
      const int i = tid + 256 * u;
      const int t = i / (kSmallRows / 4);
      const int r4 = (i % (kSmallRows / 4)) * 4;
      if (i < NXC) *(float4*)&xs[t * kSmallRows + r4] = make_float4(xv[u][0], xv[u][1], xv[u][2], xv[u][3]);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 16 * i + 4 * q;
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const float4 xv = *(const float4*)&xs[t * kSmallRows + r];
        acc[t] = fmaf(xv.x, w[4 * i], acc[t]);
        acc[t] = fmaf(xv.y, w[4 * i + 1], acc[t]);
        acc[t] = fmaf(xv.z, w[4 * i + 2], acc[t]);
        acc[t] = fmaf(xv.w, w[4 * i + 3], acc[t]);
      }
    }
  }

  __syncthreads();
  float* red = xs;  // [3][TT][64]
  if (q > 0)
#pragma unroll
    for (int t = 0; t < TT; ++t) red[((q - 1) * TT + t) * 64 + el] = acc[t];
  __syncthreads();
  if (q == 0 && e < E)
#pragma unroll
    for (int t = 0; t < TT; ++t)
      if (t < T)
        part[((int64_t)split * T + t) * E + e] =
            ((acc[t] + red[t * 64 + el]) + red[(TT + t) * 64 + el]) + red[(2 * TT + t) * 64 + el];
}

template <typename XT>
void launch_router_small(const XT* x, const float* wr, float* part, int64_t T, int d, int E, int splits, int kchunk,
                         hipStream_t s) {
  const dim3 grid((unsigned)((E + 63) / 64), (unsigned)splits);
  if (T <= 1) hipLaunchKernelGGL((router_small_kernel<XT, 1>), grid, dim3(256), 0, s, x, wr, part, T, d, E, kchunk);
  else if (T <= 2) hipLaunchKernelGGL((router_small_kernel<XT, 2>), grid, dim3(256), 0, s, x, wr, part, T, d, E, kchunk);
  else if (T <= 8) hipLaunchKernelGGL((router_small_kernel<XT, 8>), grid, dim3(256), 0, s, x, wr, part, T, d, E, kchunk);
  else if (T <= 16) hipLaunchKernelGGL((router_small_kernel<XT, 16>), grid, dim3(256), 0, s, x, wr, part, T, d, E, kchunk);
  else if (T <= 32) hipLaunchKernelGGL((router_small_kernel<XT, 32>), grid, dim3(256), 0, s, x, wr, part, T, d, E, kchunk);
  else hipLaunchKernelGGL((router_small_kernel<XT, 64>), grid, dim3(256), 0, s, x, wr, part, T, d, E, kchunk);
}

// Row-local DPP lane moves (every lane's source lane exists): 0xB1 quad [1,0,3,2], 0x4E quad
// [2,3,0,1], 0x124 row_ror:4, 0x128 row_ror:8. After the four, with a commutative combine, each
// lane of a row of 16 holds the combination of the whole row.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_lane(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// Maximum over the 64 lanes of a wavefront, uniform result: the maximum spreads within each row
// of 16 lanes by the four moves, then the four row maxima are read as scalars.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_move<0xB1>(x));
  x = fmaxf(x, dpp_move<0x4E>(x));
  x = fmaxf(x, dpp_move<0x124>(x));
  x = fmaxf(x, dpp_move<0x128>(x));
  return fmaxf(fmaxf(row_lane(x, 0), row_lane(x, 16)), fmaxf(row_lane(x, 32), row_lane(x, 48)));
}

// Sum over the 64 lanes of a wavefront, uniform result: row sums by the same moves (each lane
// of lanes 0, 16, 32, 48 ends with one fixed association of its row), then the four row sums
// added in row order. Lane moves instead of LDS swizzles: no LDS round trip per step.
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_move<0xB1>(x);
  x += dpp_move<0x4E>(x);
  x += dpp_move<0x124>(x);
  x += dpp_move<0x128>(x);
  return ((row_lane(x, 0) + row_lane(x, 16)) + row_lane(x, 32)) + row_lane(x, 48);
}

// One wavefront per token, 4 tokens per 256-thread workgroup.
// NJ = ceil(E / 64) logits per lane (lane l holds experts l, l+64, ...).
template <int NJ>
__global__ void __launch_bounds__(256)
router_topk_kernel(const float* __restrict__ part, int splits, const float* __restrict__ bias, int64_t T, int E,
                   int k, int renorm, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                   float* __restrict__ topk_gap, float* __restrict__ probs) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave leaves together; no block-wide barrier below

  // partial sums added in split order. The loads of 8 splits for every logit of the lane are all
  // issued before the first add, so a token costs ceil(splits / 8) memory round trips.
  float v[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) v[j] = 0.f;
  for (int sp0 = 0; sp0 < splits; sp0 += 8) {
    float q[NJ][8];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        q[j][u] = (e < E && sp0 + u < splits) ? part[((int64_t)(sp0 + u) * T + t) * E + e] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (sp0 + u < splits) v[j] += q[j][u];
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? (bias ? v[j] + bias[e] : v[j]) : -INFINITY;
  }

  // Round r takes the largest logit not yet taken, ties to the lower expert index: the wave
  // maximum of the lanes' untaken logits, then the lowest index holding it (ballots in index
  // order). Lane r keeps round r's pick. The round loop stays rolled: for a handful of tokens
  // one wavefront walks this code alone, and its length, not its arithmetic, sets the time.
  const int rounds = k < E ? k + 1 : k;
  uint32_t taken = 0;
  float my_v = -INFINITY;
  int my_i = 0x7fffffff;
#pragma unroll 1
  for (int r = 0; r < rounds; ++r) {
    float lv = -INFINITY;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if (lane + 64 * j < E && !((taken >> j) & 1u)) lv = fmaxf(lv, v[j]);
    const float mv = wave_max(lv);
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const unsigned long long b = __ballot(lane + 64 * j < E && !((taken >> j) & 1u) && v[j] == mv);
      if (bi == 0x7fffffff && b != 0ull) bi = 64 * j + (__ffsll(b) - 1);
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == r) {
      my_v = mv;
      my_i = bi;
    }
  }

  // softmax over all E logits; lanes r < k hold the kept ones
  const float m = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(my_v)));
  float z = 0.f;
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    if (lane + 64 * j < E) z += expf(v[j] - m);
  z = wave_sum(z);
  const float p_mine = lane < k ? expf(my_v - m) : 0.f;
  const float denom = renorm ? wave_sum(p_mine) : z;
  if (lane < k) {
    topk_idx[t * k + lane] = my_i;
    topk_w[t * k + lane] = p_mine / denom;
  }
  if (probs) {  // every expert's softmax probability, for the router statistics
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if (lane + 64 * j < E) probs[t * E + lane + 64 * j] = expf(v[j] - m) / z;
  }
  if (topk_gap) {
    const float g = k < E ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_v), k - 1)) -
                                __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_v), k))
                          : INFINITY;
    if (lane == 0) topk_gap[t] = g;
  }
}

// Top-k for few tokens, four wavefronts per token. With one wavefront per token (above) a lone
// token's time is set by its serial rounds over E/64 values per lane and by its split loads. Here
// wavefront w of the token's 256 threads holds experts 256 j + 64 w + lane (j < NJ2, the split
// loads of all its logits in flight, up to 64 per lane at a time) and picks its own best k+1 by the same
// rule (largest logit, lowest index among equals). The four lists go to LDS, where each
// candidate's rank among all of them is counted in one pass (how many candidates beat it by that
// rule); the candidates ranked below k+1 are the token's picks, in order. The softmax normaliser
// is summed per wavefront, then over the four in order.
struct TopkGroupLds {
  uint2 cand[4 * (kMaxK + 1)];  // the four wavefronts' candidate lists: (logit bits, expert)
  float f_v[kMaxK + 1];  // the token's picks by rank (k + 1 when k < E)
  int f_i[kMaxK + 1];
  float s_z[4];
};

// Token t on the 256 threads r = 0 .. 255 of a group, B split loads per logit in flight. Every
// thread of the workgroup must call it (it holds three workgroup barriers); a group with `active`
// false only meets the barriers (its wavefronts would otherwise take issue slots from the active
// groups' on the same SIMDs) and leaves its outputs untouched. Leaves the picks in sm.f_i / sm.f_v.
template <int NJ2, int B>
__device__ __forceinline__ void topk_wide_token(const float* __restrict__ part, int splits,
                                                const float* __restrict__ bias, int64_t T, int E, int k, int renorm,
                                                int64_t t, bool active, int r, TopkGroupLds& sm,
                                                int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                                                float* __restrict__ topk_gap, float* __restrict__ probs) {
  constexpr int NONE = 0x7fffffff;
  const int wave = r >> 6;
  const int lane = r & 63;

  float v[NJ2];
#pragma unroll
  for (int j = 0; j < NJ2; ++j) v[j] = 0.f;
  if (active)
    for (int sp0 = 0; sp0 < splits; sp0 += B) {
      float q[NJ2][B];
#pragma unroll
      for (int j = 0; j < NJ2; ++j) {
        const int e = 256 * j + 64 * wave + lane;
#pragma unroll
        for (int u = 0; u < B; ++u)
          q[j][u] = (e < E && sp0 + u < splits) ? part[((int64_t)(sp0 + u) * T + t) * E + e] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < NJ2; ++j)
#pragma unroll
        for (int u = 0; u < B; ++u)
          if (sp0 + u < splits) v[j] += q[j][u];
    }
#pragma unroll
  for (int j = 0; j < NJ2; ++j) {
    const int e = 256 * j + 64 * wave + lane;
    v[j] = e < E ? (bias ? v[j] + bias[e] : v[j]) : -INFINITY;
  }

  // this wavefront's best `rounds` (index NONE once it has no valid expert left)
  const int rounds = k < E ? k + 1 : k;
  uint32_t taken = 0;
  float my_v = -INFINITY;
  int my_i = NONE;
#pragma unroll 1
  for (int rd = 0; rd < (active ? rounds : 0); ++rd) {
    float lv = -INFINITY;
#pragma unroll
    for (int j = 0; j < NJ2; ++j)
      if (256 * j + 64 * wave + lane < E && !((taken >> j) & 1u)) lv = fmaxf(lv, v[j]);
    const float mv = wave_max(lv);
    int bi = NONE;
#pragma unroll
    for (int j = 0; j < NJ2; ++j) {
      const unsigned long long b =
          __ballot(256 * j + 64 * wave + lane < E && !((taken >> j) & 1u) && v[j] == mv);
      if (bi == NONE && b != 0ull) bi = 256 * j + 64 * wave + (__ffsll(b) - 1);
    }
    if (bi != NONE && (bi & 63) == lane) taken |= 1u << (bi >> 8);
    if (lane == rd) {
      my_v = mv;
      my_i = bi;
    }
  }
  if (active && lane < rounds) sm.cand[wave * rounds + lane] = make_uint2(__float_as_uint(my_v), (uint32_t)my_i);
  __syncthreads();

  // rank of candidate c among the nc = 4 * rounds: the candidates with a larger logit, or an equal
  // logit and a lower expert index (NONE entries, equal among themselves, by position). The ranks
  // are a permutation of 0 .. nc-1, and the ones below `rounds` are the token's picks in order:
  // every valid expert outside the lists is beaten by `rounds` candidates of its own wavefront.
  // Four threads per candidate (a quad of lanes): thread (c, w2) counts the candidates of
  // wavefront w2's list that beat c, all of that list's reads in flight together, and the quad
  // adds its four counts with DPP lane moves. (One thread per candidate reading all 4 (k + 1)
  // entries in turn took ~4 us at k = 10.)
  const int nc = 4 * rounds;  // <= 68 candidates, <= 272 threads: two passes at most
  if (active)
    for (int q = r; q < 4 * nc; q += 256) {
      const int c = q >> 2, w2 = q & 3;
      const uint2 me = sm.cand[c];
      const float cv = __uint_as_float(me.x);
      const int ci = (int)me.y;
      int cnt = 0;
#pragma unroll
      for (int u = 0; u < kMaxK + 1; ++u)
        if (u < rounds) {
          const int c2 = w2 * rounds + u;
          const uint2 o = sm.cand[c2];
          const float v2 = __uint_as_float(o.x);
          const int i2 = (int)o.y;
          cnt += (v2 > cv || (v2 == cv && (i2 < ci || (i2 == ci && c2 < c)))) ? 1 : 0;
        }
      cnt += __builtin_amdgcn_update_dpp(0, cnt, 0xB1, 0xF, 0xF, false);  // quad [1,0,3,2]
      cnt += __builtin_amdgcn_update_dpp(0, cnt, 0x4E, 0xF, 0xF, false);  // quad [2,3,0,1]
      if (w2 == 0 && cnt < rounds) {
        sm.f_v[cnt] = cv;
        sm.f_i[cnt] = ci;
      }
    }
  __syncthreads();

  // softmax over all E logits: per-wavefront sums, then the four in order
  float m = 0.f, z = 0.f;
  if (active) {
    m = sm.f_v[0];
#pragma unroll
    for (int j = 0; j < NJ2; ++j)
      if (256 * j + 64 * wave + lane < E) z += expf(v[j] - m);
    z = wave_sum(z);
    if (lane == 0) sm.s_z[wave] = z;
  }
  __syncthreads();
  if (!active) return;
  z = ((sm.s_z[0] + sm.s_z[1]) + sm.s_z[2]) + sm.s_z[3];
  if (wave == 0) {
    const float fv = lane < rounds ? sm.f_v[lane] : -INFINITY;
    const float p_mine = lane < k ? expf(fv - m) : 0.f;
    const float denom = renorm ? wave_sum(p_mine) : z;
    if (lane < k) {
      topk_idx[t * k + lane] = sm.f_i[lane];
      topk_w[t * k + lane] = p_mine / denom;
    }
    if (topk_gap && lane == 0) topk_gap[t] = k < E ? sm.f_v[k - 1] - sm.f_v[k] : INFINITY;
  }
  if (probs) {
#pragma unroll
    for (int j = 0; j < NJ2; ++j) {
      const int e = 256 * j + 64 * wave + lane;
      if (e < E) probs[t * E + e] = expf(v[j] - m) / z;
    }
  }
}

template <int NJ2>
__global__ void __launch_bounds__(256)
router_topk_wide_kernel(const float* __restrict__ part, int splits, const float* __restrict__ bias, int64_t T, int E,
                        int k, int renorm, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                        float* __restrict__ topk_gap, float* __restrict__ probs) {
  __shared__ TopkGroupLds sm;
  topk_wide_token<NJ2, NJ2 >= 4 ? 16 : 32>(part, splits, bias, T, E, k, renorm, blockIdx.x, true, threadIdx.x, sm, topk_idx, topk_w,
                       topk_gap, probs);
}

// Top-k and the whole dispatch of a few tokens (T <= 4, E > 64) in one workgroup of 1024 threads:
// threads 256 g .. 256 g + 255 pick token g's experts (the device code above), then the T*k picks
// are counted, scanned and scattered from LDS: the same offsets, slots and tile list as the
// dispatch kernels (stable: token-ascending within an expert; a token's experts are distinct).
template <int NJ2>
__global__ void __launch_bounds__(1024)
route_dispatch_kernel(const float* __restrict__ part, int splits, const float* __restrict__ bias, int64_t T, int E,
                      int k, int renorm, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                      float* __restrict__ topk_gap, int32_t* __restrict__ offsets, int32_t* __restrict__ slot_of,
                      int32_t* __restrict__ sorted_token, TileListArgs tl) {
  __shared__ TopkGroupLds sm[4];
  __shared__ int s_rows[kMaxGroups];
  __shared__ int s_off[kMaxGroups];
  __shared__ int s_w[17];
  const int tid = threadIdx.x;
  const int g = tid >> 8;
  // (E <= 256: all 32 split partials in flight at once, one memory round trip; more registers
  // per logit would spill at 1024 threads)
  topk_wide_token<NJ2, NJ2 >= 4 ? 8 : NJ2 == 2 ? 16 : 32>(part, splits, bias, T, E, k, renorm, g, g < T, tid & 255, sm[g], topk_idx, topk_w, topk_gap,
                       nullptr);
  __syncthreads();  // every group's picks in LDS

  const int nt = (int)T;
  int c = 0;
  if (tid < E)
    for (int t = 0; t < nt; ++t)
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) c += (j < k && sm[t].f_i[j] == tid) ? 1 : 0;
  const int excl = block_exclusive_scan_1024t(c, s_w, &s_w[16]);
  if (tid < E) {
    offsets[tid] = excl;
    s_off[tid] = excl;
    s_rows[tid] = c;
  }
  if (tid == 0) offsets[E] = s_w[16];
  if (tid == 0 && tl.tile_group && tl.has_shared) s_rows[E] = (int)T;
  __syncthreads();
  if (tid < nt * k) {
    const int t = tid / k;
    const int e = sm[t].f_i[tid - t * k];
    int rank = 0;  // earlier tokens holding e
    for (int t2 = 0; t2 < t; ++t2)
      for (int j = 0; j < k; ++j) rank += sm[t2].f_i[j] == e ? 1 : 0;
    const int slot = s_off[e] + rank;
    slot_of[tid] = slot;
    sorted_token[slot] = t;
  }
  if (tl.tile_group)
    build_tile_list(s_rows, E + tl.has_shared, tl.BM, tl.BM2, s_w, tl.tile_group, tl.tile_m0, tl.tile_count,
                    tl.split_cnt, tl.cnt_each, tl.per_tile);
}

template <int NJ2>
hipError_t launch_topk_wide(const float* part, int splits, const float* bias, int64_t T, int E, int k, int renorm,
                            int32_t* idx, float* w, float* gap, float* probs, hipStream_t s) {
  hipLaunchKernelGGL(router_topk_wide_kernel<NJ2>, dim3((unsigned)T), dim3(256), 0, s, part, splits, bias, T, E, k,
                     renorm, idx, w, gap, probs);
  return hipGetLastError();
}

template <int NJ>
hipError_t launch_topk(const float* part, int splits, const float* bias, int64_t T, int E, int k, int renorm,
                       int32_t* idx, float* w, float* gap, float* probs, hipStream_t s) {
  const unsigned grid = (unsigned)((T + 3) / 4);
  hipLaunchKernelGGL(router_topk_kernel<NJ>, dim3(grid), dim3(256), 0, s, part, splits, bias, T, E, k, renorm, idx,
                     w, gap, probs);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// router statistics: per expert, the tokens that select it and the mean of its probability.
// Pass 1: one workgroup per (64 experts, 64 tokens); the chunk's selections are staged in LDS,
// wavefront q sums tokens 16q .. +16 of the chunk (lane = expert, all 16 probability loads in
// flight) in fp64, and the four are added in order q = 0..3. Pass 2: one thread per expert adds
// the chunks in order. Fixed orders: the results do not depend on scheduling.
// ------------------------------------------------------------------------------------------
constexpr int kStatChunk = 64;

__global__ void __launch_bounds__(256)
router_stats_partial_kernel(const float* __restrict__ probs, const int32_t* __restrict__ idx, int64_t T, int E,
                            int k, double* __restrict__ part_p, int32_t* __restrict__ part_c) {
  __shared__ int sel[kStatChunk * kMaxK];
  __shared__ double sp[4][64];
  __shared__ int sc[4][64];
  const int lane = threadIdx.x & 63;
  const int q = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  const int64_t c = blockIdx.y;
  const int64_t base = c * kStatChunk;
  const int nt = (int)min<int64_t>(kStatChunk, T - base);
  for (int i = threadIdx.x; i < nt * k; i += 256) sel[i] = idx[base * k + i];
  float p[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int tt = q * 16 + i;
    p[i] = (tt < nt && e < E) ? probs[(base + tt) * E + e] : 0.f;
  }
  __syncthreads();
  double acc = 0.0;
  int n = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int tt = q * 16 + i;
    if (tt < nt) {
      acc += (double)p[i];
      for (int j = 0; j < k; ++j) n += sel[tt * k + j] == e;
    }
  }
  sp[q][lane] = acc;
  sc[q][lane] = n;
  __syncthreads();
  if (q == 0 && e < E) {
    part_p[c * E + e] = ((sp[0][lane] + sp[1][lane]) + sp[2][lane]) + sp[3][lane];
    part_c[c * E + e] = sc[0][lane] + sc[1][lane] + sc[2][lane] + sc[3][lane];
  }
}

__global__ void __launch_bounds__(256)
router_stats_final_kernel(const double* __restrict__ part_p, const int32_t* __restrict__ part_c, int64_t chunks,
                          int64_t T, int E, int32_t* __restrict__ counts, float* __restrict__ prob_mean) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  double acc = 0.0;
  int64_t n = 0;
  for (int64_t c = 0; c < chunks; ++c) {
    acc += part_p[c * E + e];
    n += part_c[c * E + e];
  }
  counts[e] = (int32_t)n;
  prob_mean[e] = T > 0 ? (float)(acc / (double)T) : 0.f;
}

}  // namespace

hipError_t launch_router_logits(const moe_dims& dm, const Layout& L, const void* x, const float* w_router, char* ws,
                                hipStream_t s) {
  float* part = (float*)(ws + L.logits);
  if (L.router_mfma) {
    bf16_t* planes = (bf16_t*)(ws + L.router_planes);
    const int64_t n = (int64_t)dm.d * dm.E;
    hipLaunchKernelGGL(router_split_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, s, w_router, planes,
                       n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t tiles = ((dm.T + 127) / 128) * (dm.E / (128 * L.router_wn));
    const dim3 grid((unsigned)(tiles * L.router_splits));
    if (L.router_wn == 4)
      hipLaunchKernelGGL(router_mfma_kernel<4>, grid, dim3(512), 0, s, (const bf16_t*)x, planes, part, dm.T, dm.d,
                         dm.E, L.router_kchunk);
    else
      hipLaunchKernelGGL(router_mfma_kernel<2>, grid, dim3(256), 0, s, (const bf16_t*)x, planes, part, dm.T, dm.d,
                         dm.E, L.router_kchunk);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  } else if (dm.T <= 64) {
    if (dm.dtype == MOE_F32)
      launch_router_small<float>((const float*)x, w_router, part, dm.T, dm.d, dm.E, L.router_splits,
                                 L.router_kchunk, s);
    else
      launch_router_small<bf16_t>((const bf16_t*)x, w_router, part, dm.T, dm.d, dm.E, L.router_splits,
                                  L.router_kchunk, s);
  } else {
    const dim3 grid((unsigned)((dm.E + kRouterTileE - 1) / kRouterTileE),
                    (unsigned)((dm.T + kRouterTileT - 1) / kRouterTileT), (unsigned)L.router_splits);
    if (dm.dtype == MOE_F32)
      hipLaunchKernelGGL(router_logits_kernel<float>, grid, dim3(256), 0, s, (const float*)x, w_router, part, dm.T,
                         dm.d, dm.E, L.router_kchunk);
    else
      hipLaunchKernelGGL(router_logits_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)x, w_router, part,
                         dm.T, dm.d, dm.E, L.router_kchunk);
  }
  return hipGetLastError();
}

hipError_t launch_topk_dispatch(const moe_dims& dm, const Layout& L, const float* bias, int32_t* topk_idx,
                                float* topk_w, float* topk_gap, int32_t* offsets, int32_t* sorted_token,
                                int32_t* slot_of, char* ws, hipStream_t s, bool with_tiles) {
  if (!L.route_fused) return hipErrorInvalidValue;
  const float* part = (const float*)(ws + L.logits);
  const TileListArgs tl = tile_list_args(dm, L, ws, with_tiles);
  const int nj2 = (dm.E + 255) / 256;
  if (nj2 <= 1)
    hipLaunchKernelGGL(route_dispatch_kernel<1>, dim3(1), dim3(1024), 0, s, part, L.router_splits, bias, dm.T, dm.E,
                       dm.k, dm.renormalize, topk_idx, topk_w, topk_gap, offsets, slot_of, sorted_token, tl);
  else if (nj2 <= 2)
    hipLaunchKernelGGL(route_dispatch_kernel<2>, dim3(1), dim3(1024), 0, s, part, L.router_splits, bias, dm.T, dm.E,
                       dm.k, dm.renormalize, topk_idx, topk_w, topk_gap, offsets, slot_of, sorted_token, tl);
  else
    hipLaunchKernelGGL(route_dispatch_kernel<4>, dim3(1), dim3(1024), 0, s, part, L.router_splits, bias, dm.T, dm.E,
                       dm.k, dm.renormalize, topk_idx, topk_w, topk_gap, offsets, slot_of, sorted_token, tl);
  return hipGetLastError();
}

hipError_t launch_router(const moe_dims& dm, const Layout& L, const void* x, const float* w_router,
                         const float* bias, int32_t* topk_idx, float* topk_w, float* topk_gap, char* ws,
                         hipStream_t s, float* probs) {
  hipError_t e = launch_router_logits(dm, L, x, w_router, ws, s);
  if (e != hipSuccess) return e;
  const float* part = (const float*)(ws + L.logits);
  const int nj = (dm.E + 63) / 64;
  const int sp = L.router_splits;
  if (dm.T <= kTopkWideMaxT && dm.E > 64) {
    const int nj2 = (dm.E + 255) / 256;
    if (nj2 <= 1) return launch_topk_wide<1>(part, sp, bias, dm.T, dm.E, dm.k, dm.renormalize, topk_idx, topk_w, topk_gap, probs, s);
    if (nj2 <= 2) return launch_topk_wide<2>(part, sp, bias, dm.T, dm.E, dm.k, dm.renormalize, topk_idx, topk_w, topk_gap, probs, s);
    return launch_topk_wide<4>(part, sp, bias, dm.T, dm.E, dm.k, dm.renormalize, topk_idx, topk_w, topk_gap, probs, s);
  }
  if (nj <= 1) return launch_topk<1>(part, sp, bias, dm.T, dm.E, dm.k, dm.renormalize, topk_idx, topk_w, topk_gap, probs, s);
  if (nj <= 2) return launch_topk<2>(part, sp, bias, dm.T, dm.E, dm.k, dm.renormalize, topk_idx, topk_w, topk_gap, probs, s);
  if (nj <= 4) return launch_topk<4>(part, sp, bias, dm.T, dm.E, dm.k, dm.renormalize, topk_idx, topk_w, topk_gap, probs, s);
  if (nj <= 8) return launch_topk<8>(part, sp, bias, dm.T, dm.E, dm.k, dm.renormalize, topk_idx, topk_w, topk_gap, probs, s);
  return launch_topk<16>(part, sp, bias, dm.T, dm.E, dm.k, dm.renormalize, topk_idx, topk_w, topk_gap, probs,
                          s);
}

hipError_t launch_router_stats(const moe_dims& dm, const Layout& L, const int32_t* topk_idx, char* ws,
                               int32_t* counts, float* prob_mean, hipStream_t s) {
  const int64_t chunks = (dm.T + kStatChunk - 1) / kStatChunk;
  double* part_p = (double*)(ws + L.stat_p);
  int32_t* part_c = (int32_t*)(ws + L.stat_c);
  hipError_t e;
  if (chunks > 0) {
    hipLaunchKernelGGL(router_stats_partial_kernel, dim3((unsigned)((dm.E + 63) / 64), (unsigned)chunks), dim3(256),
                       0, s, (const float*)(ws + L.probs), topk_idx, dm.T, dm.E, dm.k, part_p, part_c);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(router_stats_final_kernel, dim3((unsigned)((dm.E + 255) / 256)), dim3(256), 0, s, part_p, part_c,
                     chunks, dm.T, dm.E, counts, prob_mean);
  return hipGetLastError();
}

}  // namespace moe
