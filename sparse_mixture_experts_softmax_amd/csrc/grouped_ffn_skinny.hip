// Skinny grouped expert GEMMs for one or two tokens (bf16).
//
// With T <= 2 every group (a routed expert, or the shared expert) holds at most T rows, so the
// products are weight streams: ~1 GB of weights for a handful of rows at the large shape, and
// under one FMA per weight byte per row. A 32 x 32 MFMA tile would be almost all padding; here the
// weights come in with plain 16-byte vector loads and the dot products run on the vector ALUs in
// fp32, which leaves the memory pipe to the weight stream alone.
//
// One workgroup (256 threads) per (group, 256-column block, K split):
//   - the group's rows of A (x rows gathered through sorted_token for the gate/up product, H rows
//     for the down product) over the split's K range are staged in LDS as fp32;
//   - thread (wave w, lane l) owns columns n0 + 8 (l % 32) .. +7 and the K rows
//     k0 + 2w + l / 32 + 8 i, so each wave load covers two weight rows of 512 contiguous bytes; each
//     thread issues eight rows (sixteen for gate and up) of loads at a time;
//   - sums in fixed order: each thread over its K rows in ascending order, then the two lane
//     halves, then the four waves in order, then the K splits in split order (gate/up: a small
//     follow-up kernel adds the splits' fp32 partials; down: the last split to arrive, by an
//     arrival counter per (group, column block), adds them, as the MFMA kernels' split K does);
//   - the gate/up product ends in silu(g) * u rounded to bf16 (H), the down product in bf16 Y rows.
#include "moe_internal.h"

namespace moe {
namespace {

struct SkinnyArgs {
  const bf16_t* a_src;  // gate/up: x [T, d]; down: H [rows_total, ldh]
  const int32_t* offsets;
  const int32_t* sorted_token;
  const bf16_t* w0;  // gate/up: Wg [E, d, I]; down: Wd [E, I, d]
  const bf16_t* w1;  // gate/up: Wu; down: unused
  const bf16_t* w0_s;
  const bf16_t* w1_s;
  bf16_t* out;  // gate/up: H; down: Y
  const int32_t* tile_group;
  const int32_t* tile_count;
  int64_t T;
  int d, E, k, I, Is, ldh;
  int n_cblk;  // 256-column blocks of the widest group
  int ks, kc;  // K splits, K rows per split (multiple of 8, <= kSkinnyMaxKC)
  float* part;  // ks > 1: fp32 partial rows part[split][row][part_ld]
  int64_t part_ld, part_sstride;
  int32_t* cnt;  // ks > 1: arrival counter per (tile, column block), zero on entry
};

constexpr int kU = 8;  // K rows of loads in flight per thread (per weight matrix)

// 16 bytes of weights with the non-temporal hint: each weight byte is read once, and marking the
// stream so (rather than letting it displace cached lines) took the T = 1 gate/up product at the
// large shape from 150 to 134 us and the down product from 68 to 65 us
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_weights16(const bf16_t* q) {
  const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)q);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void fma8(float (&acc)[8], float a, const uint4& w) {
  acc[0] += a * bf16lo_to_f32(w.x);
  acc[1] += a * bf16hi_to_f32(w.x);
  acc[2] += a * bf16lo_to_f32(w.y);
  acc[3] += a * bf16hi_to_f32(w.y);
  acc[4] += a * bf16lo_to_f32(w.z);
  acc[5] += a * bf16hi_to_f32(w.z);
  acc[6] += a * bf16lo_to_f32(w.w);
  acc[7] += a * bf16hi_to_f32(w.w);
}

template <bool GATED, int R>
__global__ void __launch_bounds__(256, 2) ffn_skinny_kernel(SkinnyArgs p) {
  constexpr int NM = GATED ? 2 : 1;  // weight matrices
  __shared__ float s_a[R][kSkinnyMaxKC];
  __shared__ float s_red[4][R][NM][256];
  __shared__ int s_last;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

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
  const int n0 = cb * 256;
  if (n0 >= N) return;  // the whole (tile, column block) leaves: its counter is not used
  const int rows = G.rows;  // <= R
  const int k0 = split * p.kc;
  const int k1 = min(K, k0 + p.kc);  // k1 <= k0: an empty split (partials of zero)

  const bf16_t* W0;
  const bf16_t* W1 = nullptr;
  if (GATED) {
    W0 = G.shared ? p.w0_s : p.w0 + (size_t)g * p.d * p.I;
    W1 = G.shared ? p.w1_s : p.w1 + (size_t)g * p.d * p.I;
  } else {
    W0 = G.shared ? p.w0_s : p.w0 + (size_t)g * p.I * p.d;
  }
  const int cth = lane & 31;
  const int kl = 2 * wave + (lane >> 5);
  const int64_t col = n0 + 8 * cth;
  const bf16_t* w0p = W0 + col;
  const bf16_t* w1p = GATED ? W1 + col : nullptr;
  // this thread's K rows k0 + kl + 8 i, i < steps, in batches of kU rows. k1 - k0 is a multiple of
  // 8 (K and kc are), so every thread of the workgroup has the same count.
  const int steps = k1 > k0 ? (k1 - k0) / 8 : 0;
  auto load = [&](uint4 (&buf)[NM][kU], int b) {
    const int kb = k0 + kl + 8 * kU * b;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      buf[0][u] = load_weights16(w0p + (int64_t)(kb + 8 * u) * N);
      if (GATED) buf[NM - 1][u] = load_weights16(w1p + (int64_t)(kb + 8 * u) * N);
    }
    __builtin_amdgcn_sched_barrier(0);  // the batch's loads go out before the work that follows
  };

  // A rows of this split as fp32 (rows past the group's are zero). The source rows are resolved
  // once; the A chunks (8 values, 16 bytes) then load without branches, all in flight together.
  const int64_t a_ld = GATED ? p.d : p.ldh;
  int64_t srow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int rr = r < rows ? r : 0;  // a group holds >= 1 row
    srow[r] = GATED ? (G.shared ? (int64_t)rr : (int64_t)p.sorted_token[G.row0 + rr]) : G.row0 + rr;
  }
  const int cpr = p.kc / 8;  // A chunks per row
  uint4 av[R];               // R * cpr <= R * 256 chunks over 256 threads
  auto load_a = [&]() {
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
  };
  auto stage_a = [&]() {  // then the LDS barrier alone: weight loads stay in flight
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int i = tid + 256 * j;
      const int r = i / cpr;
      const int c = i - r * cpr;
      if (r < R) {
        float* d = &s_a[r][8 * c];
        *(float4*)d = make_float4(bf16lo_to_f32(av[j].x), bf16hi_to_f32(av[j].x), bf16lo_to_f32(av[j].y),
                                  bf16hi_to_f32(av[j].y));
        *(float4*)(d + 4) = make_float4(bf16lo_to_f32(av[j].z), bf16hi_to_f32(av[j].z), bf16lo_to_f32(av[j].w),
                                        bf16hi_to_f32(av[j].w));
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  float acc[NM][R][8];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[m][r][c] = 0.f;
  auto compute = [&](const uint4 (&buf)[NM][kU], int b) {
    const int ko = kl + 8 * kU * b;  // offset of the batch's first row from k0
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float a = s_a[r][ko + 8 * u];
#pragma unroll
        for (int m = 0; m < NM; ++m) fma8(acc[m][r], a, buf[m][u]);
      }
  };
  auto tail = [&](int from) {  // rows past the whole batches, one at a time
    for (int i = from; i < steps; ++i) {
      const int kk = k0 + kl + 8 * i;
      uint4 wv[NM];
      wv[0] = load_weights16(w0p + (int64_t)kk * N);
      if (GATED) wv[NM - 1] = load_weights16(w1p + (int64_t)kk * N);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float a = s_a[r][kk - k0];
#pragma unroll
        for (int m = 0; m < NM; ++m) fma8(acc[m][r], a, wv[m]);
      }
    }
  };

  if (steps >= kU) {
    // Straight-line streaming: every batch load is unconditional, so the compiler's waits before
    // a batch's FMAs count exactly that batch. The A loads go out before the first batch: waiting
    // for them (loads complete in order) leaves the batch in flight behind the staging. One batch
    // per thread at a time keeps the registers low enough for five workgroups per CU, whose loads
    // together keep the memory pipe full.
    const int nbw = steps / kU;  // whole batches
    uint4 buf[NM][kU];
    load_a();
    load(buf, 0);
    stage_a();
    compute(buf, 0);
    for (int b = 1; b < nbw; ++b) {
      load(buf, b);
      compute(buf, b);
    }
    tail(nbw * kU);
  } else {
    load_a();
    stage_a();
    tail(0);
  }

  // the lane halves hold the even and odd K lanes of the same columns; then the waves via LDS
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[m][r][c] += __shfl_xor(acc[m][r][c], 32, 64);
  if (lane < 32)
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        *(float4*)&s_red[wave][r][m][8 * cth] = make_float4(acc[m][r][0], acc[m][r][1], acc[m][r][2], acc[m][r][3]);
        *(float4*)&s_red[wave][r][m][8 * cth + 4] =
            make_float4(acc[m][r][4], acc[m][r][5], acc[m][r][6], acc[m][r][7]);
      }
  __syncthreads();

  // thread -> row r = tid / 64, columns c4 .. c4 + 3 of the block
  const int r = tid >> 6;
  const int c4 = (tid & 63) * 4;
  float v[NM][4];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int c = 0; c < 4; ++c) v[m][c] = 0.f;
  if (r < R)
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int c = 0; c < 4; ++c) v[m][c] += s_red[w][r][m][c4 + c];
  const bool mine = r < rows;

  if (GATED && p.ks > 1) {
    // gate/up with K split: the fp32 partials go out with plain stores and the follow-up kernel
    // (gate_up_finish_kernel, next on the stream) adds them and applies silu * up. Ending
    // here spares every workgroup the store-acknowledge, counter and reload round trips of the
    // last-arriver sum (T = 1 at the large shape: ~17 us of the product's ~135 us).
    if (mine) {
      float* q = p.part + (int64_t)split * p.part_sstride + (G.row0 + r) * p.part_ld + n0 + c4;
      *(float4*)q = make_float4(v[0][0], v[0][1], v[0][2], v[0][3]);
      *(float4*)(q + p.ldh) = make_float4(v[NM - 1][0], v[NM - 1][1], v[NM - 1][2], v[NM - 1][3]);
    }
    return;
  }
  if (p.ks > 1) {
    // fp32 partials with device-scope relaxed stores (coherent across the XCDs' L2s); the last
    // split to arrive adds them in split order
    auto pcol = [&](int m, int c) { return (GATED ? (int64_t)m * p.ldh : 0) + n0 + c4 + c; };
    float* mine_part = p.part + (int64_t)split * p.part_sstride;
    if (mine)
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          __hip_atomic_store(&mine_part[(G.row0 + r) * p.part_ld + pcol(m, c)], v[m][c], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's partial stores are complete
    __syncthreads();                                  // ... and every thread's
    if (tid == 0)
      s_last = __hip_atomic_fetch_add(&p.cnt[mt * p.n_cblk + cb], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               p.ks - 1;
    __syncthreads();
    if (!s_last) return;
    if (mine)
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int64_t at = (G.row0 + r) * p.part_ld + pcol(m, c);
          float sum = 0.f;
          for (int sp = 0; sp < p.ks; ++sp)
            sum += sp == split ? v[m][c]
                               : __hip_atomic_load(&p.part[sp * p.part_sstride + at], __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
          v[m][c] = sum;
        }
  }
  if (!mine) return;
  uint2 o;
  if (GATED) {
    o.x = pack_bf16x2(silu_f32(v[0][0]) * v[NM - 1][0], silu_f32(v[0][1]) * v[NM - 1][1]);
    o.y = pack_bf16x2(silu_f32(v[0][2]) * v[NM - 1][2], silu_f32(v[0][3]) * v[NM - 1][3]);
    *(uint2*)(p.out + (G.row0 + r) * p.ldh + n0 + c4) = o;
  } else {
    o.x = pack_bf16x2(v[0][0], v[0][1]);
    o.y = pack_bf16x2(v[0][2], v[0][3]);
    *(uint2*)(p.out + (G.row0 + r) * p.d + n0 + c4) = o;
  }
}

template <int R>
void launch_pair(const SkinnyArgs& a1, const SkinnyArgs& a2, unsigned grid1, unsigned grid2, int64_t rows_total,
                 hipStream_t s, const Prof* prof, hipError_t& e) {
  if ((e = prof->begin(MOE_KERNEL_FFN_GATE_UP, s)) != hipSuccess) return;
  hipLaunchKernelGGL((ffn_skinny_kernel<true, R>), dim3(grid1), dim3(256), 0, s, a1);
  if ((e = hipGetLastError()) != hipSuccess) return;
  if (a1.ks > 1 && (e = launch_gate_up_finish(a1.part, a1.part_sstride, a1.part_ld, a1.ks, a1.T * a1.k, rows_total,
                                                 a1.I, a1.Is, a1.ldh, a1.out, s)) != hipSuccess)
    return;
  if ((e = prof->end(MOE_KERNEL_FFN_GATE_UP, s)) != hipSuccess) return;
  if ((e = prof->begin(MOE_KERNEL_FFN_DOWN, s)) != hipSuccess) return;
  hipLaunchKernelGGL((ffn_skinny_kernel<false, R>), dim3(grid2), dim3(256), 0, s, a2);
  if ((e = hipGetLastError()) != hipSuccess) return;
  e = prof->end(MOE_KERNEL_FFN_DOWN, s);
}

}  // namespace

hipError_t launch_ffn_skinny(const moe_dims& dm, const Layout& L, const FfnPlan& P, const void* x,
                             const int32_t* offsets, const int32_t* sorted_token, const void* wg, const void* wu,
                             const void* wd, const void* wg_s, const void* wu_s, const void* wd_s, void* y, char* ws,
                             hipStream_t s, const Prof* prof) {
  SkinnyArgs a;
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
  a.part = (float*)(ws + L.ffn_part);
  int32_t* cnt = (int32_t*)(ws + L.ffn_cnt);
  bf16_t* H = (bf16_t*)(ws + L.H);
  // at most min(E, T*k) routed groups and the shared one hold rows; each is one tile
  const int64_t Tk = dm.T * dm.k;
  const int64_t max_mt = (Tk < dm.E ? Tk : dm.E) + (dm.I_shared > 0 ? 1 : 0);

  SkinnyArgs a1 = a;  // gate/up
  a1.a_src = (const bf16_t*)x;
  a1.w0 = (const bf16_t*)wg;
  a1.w1 = (const bf16_t*)wu;
  a1.w0_s = (const bf16_t*)wg_s;
  a1.w1_s = (const bf16_t*)wu_s;
  a1.out = H;
  a1.n_cblk = P.cb1;
  a1.ks = P.ks1;
  a1.kc = P.kc1;
  a1.part_ld = P.part_cols1;
  a1.part_sstride = L.rows_total * P.part_cols1;
  a1.cnt = cnt;
  SkinnyArgs a2 = a;  // down
  a2.a_src = H;
  a2.w0 = (const bf16_t*)wd;
  a2.w1 = nullptr;
  a2.w0_s = (const bf16_t*)wd_s;
  a2.w1_s = nullptr;
  a2.out = (bf16_t*)y;
  a2.n_cblk = P.cb2;
  a2.ks = P.ks2;
  a2.kc = P.kc2;
  a2.part_ld = P.part_cols2;
  a2.part_sstride = L.rows_total * P.part_cols2;
  a2.cnt = cnt + L.ffn_cnt_each;
  const unsigned grid1 = (unsigned)(max_mt * P.cb1 * P.ks1);
  const unsigned grid2 = (unsigned)(max_mt * P.cb2 * P.ks2);
  hipError_t e = hipSuccess;
  if (P.skinny_rows == 1) launch_pair<1>(a1, a2, grid1, grid2, L.rows_total, s, prof, e);
  else launch_pair<2>(a1, a2, grid1, grid2, L.rows_total, s, prof, e);
  return e;
}

}  // namespace moe
