// Skinny grouped expert GEMMs for one or two tokens (bf16).
//
// With T <= 2 every group (a routed expert, or the shared expert) holds at most T rows, so the
// products are weight streams: ~1 GB of weights for a handful of rows at the large shape, and
// under one FMA per weight byte per row. A 32 x 32 MFMA tile would be almost all padding; here the
// weights stream into LDS by DMA and the dot products run on the vector ALUs in fp32.
//
// One workgroup (256 threads) per (group, 256-column block, K split):
//   - the group's rows of A (x rows gathered through sorted_token for the gate/up product, H rows
//     for the down product) over the split's K range are DMA'd into LDS as bf16;
//   - the weight rows of the split pass through a ring of LDS stages (direct global-to-LDS loads,
//     S - 1 stages in flight while one is multiplied); thread (wave w, lane l) owns columns
//     n0 + 8 (l % 32) .. +7 and the K rows 2w + l / 32 + 8 i of each stage;
//   - sums in fixed order: each thread over its K rows in ascending order, then the two lane
//     halves, then the four waves in order, then the K splits in split order (gate/up: a small
//     follow-up kernel adds the splits' fp32 partials; down: the last split to arrive, by an
//     arrival counter per (group, column block), adds them, as the MFMA kernels' split K does);
//   - the gate/up product ends in silu(g) * u rounded to bf16 (H), the down product in bf16 Y rows;
//     in a forward, the down product's last group per column block also performs the combine
//     (weighted sum of the token's expert rows, shared row, optional residual) for those columns.
#include "moe_internal.h"
#include "stream_gemm.h"

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
  // down product with the combine (fout non-null): the block's output rows [T, d], the routing,
  // the residual rows (or null), and one arrival counter per column block, zero on entry
  bf16_t* fout;
  const int32_t* slot_of;
  const float* topk_w;
  const bf16_t* resid;
  int32_t* ccnt;
};

// Columns n0 .. n0 + 255 of the block's output for every token (T <= 2): thread (t, c), token
// t = tid / 128, columns n0 + 2c and n0 + 2c + 1.
__device__ __forceinline__ void combine_columns(const SkinnyArgs& p, int n0) {
  const int t = threadIdx.x >> 7;
  if (t >= p.T) return;
  combine_pair(p.out, p.fout, p.slot_of, p.topk_w, p.resid, p.T, p.d, p.k, p.Is > 0, t,
               n0 + 2 * (threadIdx.x & 127));
}

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void fma8(float (&acc)[8], float a, const u32x4_t& w) {
  acc[0] += a * bf16lo_to_f32(w.x);
  acc[1] += a * bf16hi_to_f32(w.x);
  acc[2] += a * bf16lo_to_f32(w.y);
  acc[3] += a * bf16hi_to_f32(w.y);
  acc[4] += a * bf16lo_to_f32(w.z);
  acc[5] += a * bf16hi_to_f32(w.z);
  acc[6] += a * bf16lo_to_f32(w.w);
  acc[7] += a * bf16hi_to_f32(w.w);
}

// The weights stream into an LDS ring with gfx950's direct global-to-LDS loads (16 bytes per
// lane, no registers held in flight), with the non-temporal hint, since no other workgroup reads
// these bytes. Each stage holds KR rows of every weight matrix of the 256-column block (512 bytes
// per row, rows one after another): one DMA instruction of a wavefront moves two rows (lane l:
// row l / 32, chunk l % 32). At the large shape this took the one-token layer from 0.214 to
// 0.202 ms against plain 16-byte vector loads of the same stream; 512-column blocks (1 KB runs
// per row) measured slower for both products (gate/up 114 -> 123 us, down 69 -> 73 us).
// Thread mapping: chunk c = tid % 32 (columns 8c .. 8c + 7 of the block), K lane kl = tid / 32
// (rows kl, kl + 8, ... of each stage).
template <bool GATED, int R>
__global__ void __launch_bounds__(256, 2) ffn_skinny_kernel(SkinnyArgs p) {
  constexpr int NC = 256;            // columns of the block
  constexpr int NM = GATED ? 2 : 1;  // weight matrices
  constexpr int ROWB = NC * 2;       // bytes of one weight row of the column block
  constexpr int KR = (GATED ? kSkinnyMat1 : kSkinnyMat2) / ROWB;
  constexpr int S = GATED ? kSkinnyS1 : kSkinnyS2;
  constexpr int CPRL = NC / 8;       // 16-byte chunks per row
  constexpr int NKL = 256 / CPRL;    // K lanes of the workgroup
  constexpr int MAT = KR * ROWB;     // one matrix's rows of a stage
  constexpr int STAGE = NM * MAT;
  constexpr int IPM = MAT / 1024 / 4;  // DMA instructions per wavefront, matrix and stage
  constexpr int D = NM * IPM;          // per wavefront and stage
  constexpr int CPT = NC / 64;         // output columns per thread in the epilogue (4)
  static_assert(KR % NKL == 0 && IPM >= 1 && MAT % 4096 == 0, "stage rows");
  static_assert(S >= 2 && S <= 7 && 7 * D < 64, "ring depth");
  static_assert(4 * R * NM * NC * 4 <= S * STAGE, "the wave sums fit the ring");
  __shared__ __attribute__((aligned(1024))) char s_ring[S * STAGE];
  __shared__ __attribute__((aligned(16))) bf16_t s_a[R][kSkinnyMaxKC];
  __shared__ int s_last;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

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
  const int n0 = cb * NC;
  if (n0 >= N) return;  // the whole (tile, column block) leaves: its counter is not used
  const int rows = G.rows;  // <= R
  const int k0 = split * p.kc;
  const int k1 = min(K, k0 + p.kc);  // k1 <= k0: an empty split (partials of zero)
  // K and kc are multiples of KR, so the split is whole stages
  const int nst = k1 > k0 ? (k1 - k0) / KR : 0;

  const bf16_t* W0;
  const bf16_t* W1 = nullptr;
  if (GATED) {
    W0 = G.shared ? p.w0_s : p.w0 + (size_t)g * p.d * p.I;
    W1 = G.shared ? p.w1_s : p.w1 + (size_t)g * p.d * p.I;
  } else {
    W0 = G.shared ? p.w0_s : p.w0 + (size_t)g * p.I * p.d;
  }
  const int cth = tid % CPRL;
  const int kl = tid / CPRL;

  // DMA: wave-uniform bases at (k0, n0) of each matrix, per-lane offsets below 2^32 (kc rows of at
  // most 16 KB)
  const char* wb0 = stream::uniform_ptr((const char*)(W0 + (int64_t)k0 * N + n0));
  const char* wb1 = GATED ? stream::uniform_ptr((const char*)(W1 + (int64_t)k0 * N + n0)) : nullptr;
  const uint32_t pitch = (uint32_t)N * 2u;
  constexpr int RPI = 1024 / ROWB;  // rows per DMA instruction
  const uint32_t loff = (uint32_t)(lane / CPRL) * pitch + (uint32_t)(lane % CPRL) * 16u;
  stream::lds_char* ring = (stream::lds_char*)s_ring;
  const uint32_t ring_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)ring);
  auto issue = [&](int st) {  // stage st into slot st % S
    const uint32_t dst = ring_base + (uint32_t)(st % S) * STAGE;
#pragma unroll
    for (int q = 0; q < IPM; ++q) {
      const int i = wave * IPM + q;  // rows RPI i .. RPI i + RPI - 1 of the stage
      const uint32_t voff = (uint32_t)(st * KR + RPI * i) * pitch + loff;
      stream::dma16<true>(wb0, voff, dst + i * 1024);
      if (GATED) stream::dma16<true>(wb1, voff, dst + MAT + i * 1024);
    }
  };

  // A rows of this split, bf16, DMA'd into s_a ahead of the ring's first stages (rows past the
  // group's repeat its first row; their sums are never stored). Instruction ia of the workgroup
  // loads 64 chunks of 8 values of row ia / na; lanes past the split's K read the row's first
  // chunk into the unused tail of s_a. No register loads are in flight, so every wait below is an
  // explicit DMA count.
  const int64_t a_ld = GATED ? p.d : p.ldh;
  const int cpr = (k1 - k0) / 8;   // A chunks per row
  const int na = (cpr + 63) / 64;  // A instructions per row
  const uint32_t sa_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(stream::lds_char*)&s_a[0][0]);
  int64_t srow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int rr = r < rows ? r : 0;  // a group holds >= 1 row
    srow[r] = GATED ? (G.shared ? (int64_t)rr : (int64_t)p.sorted_token[G.row0 + rr]) : G.row0 + rr;
  }
  if (nst > 0)
    for (int ia = wave; ia < R * na; ia += 4) {
      const int r = ia / na;
      const int q = ia - r * na;
      int64_t sr = srow[0];
#pragma unroll
      for (int u = 1; u < R; ++u)
        if (r == u) sr = srow[u];
      const int c = 64 * q + lane;
      const uint32_t voff = (uint32_t)((sr * a_ld + k0 + (c < cpr ? 8 * c : 0)) * 2);
      stream::dma16(p.a_src, voff, __builtin_amdgcn_readfirstlane(sa_base + r * (kSkinnyMaxKC * 2) + q * 1024));
    }
  const int pro = nst < S ? nst : S;
#pragma unroll
  for (int st = 0; st < S; ++st)
    if (st < pro) issue(st);

  float acc[NM][R][8];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[m][r][c] = 0.f;
  for (int st = 0; st < nst; ++st) {
    // this wave's DMAs of stage st have landed once at most the later stages' are pending; after
    // the barrier every wave's have, and every wave is done with stage st - 1 (its LDS reads
    // returned), whose slot then takes stage st - 1 + S
    stream::wait_groups<D>(min(st == 0 ? S - 1 : S - 2, nst - 1 - st));
    stream::barrier_after_lds_reads();
    if (st >= 1 && st - 1 + S < nst) issue(st - 1 + S);
    const stream::lds_char* sl = ring + (st % S) * STAGE + cth * 16;
    u32x4_t wv[NM][KR / NKL];
#pragma unroll
    for (int u = 0; u < KR / NKL; ++u)
#pragma unroll
      for (int m = 0; m < NM; ++m)
        wv[m][u] = *(const __attribute__((address_space(3))) u32x4_t*)(sl + m * MAT + (kl + NKL * u) * ROWB);
#pragma unroll
    for (int u = 0; u < KR / NKL; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float a = __uint_as_float((uint32_t)__builtin_bit_cast(uint16_t, s_a[r][st * KR + kl + NKL * u]) << 16);
#pragma unroll
        for (int m = 0; m < NM; ++m) fma8(acc[m][r], a, wv[m][u]);
      }
  }
  __syncthreads();  // every wave is done with the ring: it now holds the K lanes' sums
  float (*s_red)[R][NM][NC] = (float (*)[R][NM][NC])s_ring;

  // the lane halves hold K lanes 2w and 2w + 1 of the same columns; then the waves via LDS
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

  // thread -> row r = tid / 64, columns cc .. cc + CPT - 1 of the block
  const int r = tid >> 6;
  const int cc = (tid & 63) * CPT;
  float v[NM][CPT];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int c = 0; c < CPT; ++c) v[m][c] = 0.f;
  if (r < R)
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int c = 0; c < CPT; ++c) v[m][c] += s_red[w][r][m][cc + c];
  const bool mine = r < rows;

  if (GATED && p.ks > 1) {
    // gate/up with K split: the fp32 partials go out with plain stores and the follow-up kernel
    // (gate_up_finish_kernel, next on the stream) adds them and applies silu * up. Ending
    // here spares every workgroup the store-acknowledge, counter and reload round trips of the
    // last-arriver sum (T = 1 at the large shape: ~17 us of the product's ~135 us).
    if (mine) {
      float* q = p.part + (int64_t)split * p.part_sstride + (G.row0 + r) * p.part_ld + n0 + cc;
#pragma unroll
      for (int c = 0; c < CPT; c += 4) {
        *(float4*)(q + c) = make_float4(v[0][c], v[0][c + 1], v[0][c + 2], v[0][c + 3]);
        *(float4*)(q + p.ldh + c) = make_float4(v[NM - 1][c], v[NM - 1][c + 1], v[NM - 1][c + 2], v[NM - 1][c + 3]);
      }
    }
    return;
  }
  if (p.ks > 1) {
    // fp32 partials with device-scope relaxed stores (coherent across the XCDs' L2s); the last
    // split to arrive adds them in split order
    auto pcol = [&](int m, int c) { return (GATED ? (int64_t)m * p.ldh : 0) + n0 + cc + c; };
    float* mine_part = p.part + (int64_t)split * p.part_sstride;
    if (mine)
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int c = 0; c < CPT; ++c)
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
        for (int c = 0; c < CPT; ++c) {
          const int64_t at = (G.row0 + r) * p.part_ld + pcol(m, c);
          float sum = 0.f;
          for (int sp = 0; sp < p.ks; ++sp)
            sum += sp == split ? v[m][c]
                               : __hip_atomic_load(&p.part[sp * p.part_sstride + at], __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
          v[m][c] = sum;
        }
  }
  if (!GATED && p.fout) {
    // Y rows with device-scope stores; the last group to finish this column block (by the
    // counter, after every thread's stores completed) then writes the block's output columns
    if (mine) {
      uint32_t* q = (uint32_t*)(p.out + (G.row0 + r) * p.d + n0 + cc);
#pragma unroll
      for (int c = 0; c < CPT; c += 2)
        __hip_atomic_store(q + c / 2, pack_bf16x2(v[0][c], v[0][c + 1]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0)
      s_last = __hip_atomic_fetch_add(&p.ccnt[cb], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               *p.tile_count - 1;
    __syncthreads();
    if (s_last) combine_columns(p, n0);
    return;
  }
  if (!mine) return;
  uint32_t o[CPT / 2];
#pragma unroll
  for (int c = 0; c < CPT; c += 2)
    o[c / 2] = GATED ? pack_bf16x2(silu_f32(v[0][c]) * v[NM - 1][c], silu_f32(v[0][c + 1]) * v[NM - 1][c + 1])
                     : pack_bf16x2(v[0][c], v[0][c + 1]);
  bf16_t* dst = p.out + (G.row0 + r) * (GATED ? (int64_t)p.ldh : (int64_t)p.d) + n0 + cc;
  *(uint2*)dst = make_uint2(o[0], o[1]);
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
                             hipStream_t s, const Prof* prof, CombineFuse* combine) {
  SkinnyArgs a{};
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
  if (combine && dm.T <= 2) {
    // the gate/up product uses no arrival counters: the first bank (zeroed for every listed
    // tile, at least one column block's worth) holds one per column block of the output
    a2.fout = (bf16_t*)combine->out;
    a2.slot_of = combine->slot_of;
    a2.topk_w = combine->topk_w;
    a2.resid = (const bf16_t*)combine->residual;
    a2.ccnt = cnt;
    combine->done = true;
  }
  const unsigned grid1 = (unsigned)(max_mt * P.cb1 * P.ks1);
  const unsigned grid2 = (unsigned)(max_mt * P.cb2 * P.ks2);
  hipError_t e = hipSuccess;
  if (P.skinny_rows == 1) launch_pair<1>(a1, a2, grid1, grid2, L.rows_total, s, prof, e);
  else launch_pair<2>(a1, a2, grid1, grid2, L.rows_total, s, prof, e);
  return e;
}

}  // namespace moe
