// Internal declarations shared by the MoE library's translation units:
// workspace layout, element helpers and kernel launchers. Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// ------------------------------------------------------------------------------------------
// element helpers
// ------------------------------------------------------------------------------------------
typedef uint16_t bf16_t;  // bfloat16 bit pattern

__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// round to nearest even; the values here are finite
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }

// ------------------------------------------------------------------------------------------
// tiling constants shared by host and device
// ------------------------------------------------------------------------------------------
constexpr int kPermuteChunk = 256;     // tokens per permute workgroup
constexpr int kRouterTileT = 64;       // router logits tile: tokens
constexpr int kRouterTileE = 64;       // router logits tile: experts
constexpr int kRouterKStep = 16;       // router K step
constexpr int kMaxK = 16;              // largest k (experts per token) accepted
constexpr int kTopkWideMaxT = 64;      // top-k with four wavefronts per token up to this many tokens
constexpr int kMaxGroups = 1025;       // grouped GEMM groups: up to 1024 experts + the shared one
constexpr int kMfmaBM = 128;           // bf16 grouped GEMM tile rows
constexpr int kMfmaBN1 = 128;          // gate/up tile: intermediate columns (x2 for gate and up)
constexpr int kMfmaBN2 = 256;          // down tile: hidden columns
constexpr int kF32BM = 64;             // fp32 grouped GEMM tile rows
constexpr int kF32BN = 64;             // fp32 grouped GEMM tile columns
constexpr int kSkinnyMaxT = 2;         // skinny grouped GEMMs up to this many tokens
constexpr int kSkinnyMaxKC = 2048;     // skinny grouped GEMMs: most K rows per split
// skinny grouped GEMMs (256-column blocks, 512-byte weight rows), gate/up (1) and down (2): bytes
// of one weight matrix per LDS stage (16 and 32 rows), stages in the ring, and the workgroups the
// K split aims at (two per CU: all resident at once)
constexpr int kSkinnyMat1 = 8192;
constexpr int kSkinnyS1 = 4;
constexpr int kSkinnyMat2 = 16384;
constexpr int kSkinnyS2 = 4;
constexpr int kSkinnyWG1 = 512;
constexpr int kSkinnyWG2 = 512;

// The combine for one token t and the two output columns col, col + 1, as combine_kernel sums
// them: out = sum_j w[t, j] * y[slot_of[t k + j]] in the order j = 0 .. k-1 (fp32, fused
// multiply-add from zero), then the shared expert's row T k + t, then the residual row, rounded
// once. Used by the few-token down products that perform the combine themselves: the expert rows
// y were stored by other workgroups with device-scope stores, and are read the same way.
__device__ inline void combine_pair(const bf16_t* y, bf16_t* out, const int32_t* slot_of, const float* topk_w,
                                    const bf16_t* resid, int64_t T, int d, int k, bool has_shared, int64_t t,
                                    int64_t col) {
  uint32_t yv[kMaxK];
  float w[kMaxK];
  bool on[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    on[j] = false;
    if (j < k) {
      const int slot = slot_of[t * k + j];
      w[j] = topk_w[t * k + j];
      on[j] = slot >= 0;
      if (on[j])
        yv[j] = __hip_atomic_load((const uint32_t*)(y + (int64_t)slot * d + col), __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  uint32_t ys = 0, rv = 0;
  if (has_shared)
    ys = __hip_atomic_load((const uint32_t*)(y + (T * k + t) * d + col), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (resid) rv = *(const uint32_t*)(resid + t * d + col);
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (on[j]) {
      a0 = fmaf(w[j], bf16lo_to_f32(yv[j]), a0);
      a1 = fmaf(w[j], bf16hi_to_f32(yv[j]), a1);
    }
  if (has_shared) {
    a0 += bf16lo_to_f32(ys);
    a1 += bf16hi_to_f32(ys);
  }
  if (resid) {
    a0 += bf16lo_to_f32(rv);
    a1 += bf16hi_to_f32(rv);
  }
  *(uint32_t*)(out + t * d + col) = pack_bf16x2(a0, a1);
}

// ------------------------------------------------------------------------------------------
// workspace layout: a pure function of the dims
// ------------------------------------------------------------------------------------------
struct Layout {
  int router_mfma;      // 1: bf16 x with the 3-way bf16 split of W_r on MFMA; 0: fp32 vector ALUs
  int router_wn;        // MFMA router: wave columns of its tile (2: 128 x 256, 4: 128 x 512)
  int router_splits;    // K splits of the router logits GEMM (partial sums summed by top-k)
  int router_kchunk;    // vector path: hidden rows per split; MFMA path: 32-wide K steps per split
  int64_t nchunks;      // permute chunks
  int route_fused;      // few tokens (T <= 4, E > 64, vector router): top-k and dispatch in one kernel
  int64_t max_tiles;    // upper bound on grouped-GEMM row tiles (any BM >= 64)
  int ldh;              // row stride of H = max(I, I_shared)
  int64_t rows_total;   // T*k + (I_shared ? T : 0)
  size_t router_planes, logits, topk_idx, topk_w, topk_gap, chunk_counts, offsets, sorted_token, slot_of;
  size_t tile_group, tile_m0, tile_count, H, Y;
  size_t probs, stat_p, stat_c;  // router statistics: probabilities [T, E], per-chunk sums and counts
  size_t ffn_part;      // split-K partial sums of the grouped GEMMs (small T only)
  size_t ffn_cnt;       // arrival counters of the skinny down product's K split
  size_t hnorm;         // moe_forward_block: the normalised rows [T, d] the router and experts read
  int64_t ffn_cnt_each; // counters per product
  int ffn_cnt_per_tile; // counters per row tile (the widest group's column blocks)
  size_t total;
};

Layout make_layout(const moe_dims& dm);

// How the bf16 grouped GEMMs run for these dims: streaming kernel or not, tile widths (wave
// columns), column tiles, and K splits of the gate/up product.
struct FfnPlan {
  bool stream;
  bool balance;  // equal row tiles per group
  bool tall;     // 160- or 192-row tiles for both products, per group (groups of ~100 rows and more)
  int wn1, wn2;
  int nt1, nt2;
  int s1;  // K splits of the MFMA gate/up product (the MFMA down product is never split)
  int64_t part_cols1, part_cols2;  // columns of the fp32 partial rows (gate | up, or d)
  // few tokens (every group <= kSkinnyMaxT rows): the skinny kernels, 256-column blocks, K in
  // splits of kc1 / kc2 rows (multiples of 8, <= kSkinnyMaxKC)
  bool skinny;
  int skinny_rows;        // rows per group the kernel is built for (1 or 2)
  int cb1, cb2;           // 256-column blocks of the widest group
  int ks1, ks2, kc1, kc2;
};
FfnPlan ffn_plan(const moe_dims& dm);

// ------------------------------------------------------------------------------------------
// optional event pair around one kernel (moe_profile_next_forward)
// ------------------------------------------------------------------------------------------
struct Prof {
  int kernel = MOE_KERNEL_NONE;
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
  hipError_t begin(int which, hipStream_t s) const {
    return kernel == which ? hipEventRecord(start, s) : hipSuccess;
  }
  hipError_t end(int which, hipStream_t s) const {
    return kernel == which ? hipEventRecord(stop, s) : hipSuccess;
  }
};

// ------------------------------------------------------------------------------------------
// grouped GEMM groups: routed expert g < E owns sorted slots [offsets[g], offsets[g+1]); group E
// is the shared expert over all T tokens, whose rows follow the T*k routed ones
// ------------------------------------------------------------------------------------------
struct Group {
  int64_t row0;  // first sorted slot of the group
  int rows;      // rows in the group
  int n_inter;   // intermediate size of the group (I or I_shared)
  bool shared;
};

__device__ __forceinline__ Group group_info(int g, const int32_t* offsets, int64_t T, int k, int E, int I, int Is) {
  Group G;
  if (g < E) {
    G.row0 = offsets[g];
    G.rows = offsets[g + 1] - offsets[g];
    G.n_inter = I;
    G.shared = false;
  } else {
    G.row0 = T * (int64_t)k;
    G.rows = (int)T;
    G.n_inter = Is;
    G.shared = true;
  }
  return G;
}

// Exclusive prefix sum over the 1024 threads of a workgroup: each wavefront scans its 64 values
// with lane shuffles, the 16 wavefront totals go through LDS (s_w, 17 ints), and each thread adds
// the totals of the wavefronts before it. Two barriers instead of one per doubling step.
// Returns the thread's exclusive prefix; *total (LDS) receives the sum of all values.
__device__ inline int block_exclusive_scan_1024t(int x, int* s_w, int* total) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) s_w[wv] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wv; ++w) before += s_w[w];
  if (threadIdx.x == 1023) *total = before + incl;
  __syncthreads();  // s_w may be reused once every thread has read it
  return before + incl - x;
}

// Flag on a tile list entry's first row: the group runs 192-row tiles (its first row is then the
// tile index times 192); without it, tiles of the list's BM rows
constexpr int32_t kTileRows192 = 1 << 30;

// Row-tile list of the grouped GEMMs: group g with s_rows[g] rows gets ceil(rows / BM) tiles,
// listed group after group as (group, first row). BM2 > 0 (192, the tall tiles): a group whose
// rows fit fewer tiles of BM2 rows than of BM, and at most two, takes those, its entries flagged
// kTileRows192 (larger groups measured faster on the 160-row tiles, more of them or not). One
// workgroup of 1024 threads; s_rows and s_w (17 ints) are LDS arrays (G <= 2048 groups). Also
// zeroes the split-K arrival counters of the listed tiles: per_tile for each tile, in two banks
// cnt_each apart.
__device__ inline void build_tile_list(const int* s_rows, int G, int BM, int BM2, int* s_w, int32_t* tile_group,
                                       int32_t* tile_m0, int32_t* tile_count, int32_t* split_cnt, int64_t cnt_each,
                                       int per_tile) {
  const int tid = threadIdx.x;
  // tile heights and counts of groups 2 tid and 2 tid + 1, and their exclusive prefix
  int bm[2], cnts[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int g = 2 * tid + h;
    const int rows = g < G ? s_rows[g] : 0;
    const int c1 = (rows + BM - 1) / BM;
    const int c2 = BM2 > 0 ? (rows + BM2 - 1) / BM2 : c1;
    const bool alt = c2 < c1 && c2 <= 2;
    bm[h] = alt ? BM2 : BM;
    cnts[h] = alt ? c2 : c1;
  }
  const int excl = block_exclusive_scan_1024t(cnts[0] + cnts[1], s_w, &s_w[16]);
  const int starts[2] = {excl, excl + cnts[0]};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int g = 2 * tid + h;
    const int32_t flag = bm[h] == BM2 && BM2 != BM ? kTileRows192 : 0;
    if (g < G)
      for (int i = 0; i < cnts[h]; ++i) {
        tile_group[starts[h] + i] = g;
        tile_m0[starts[h] + i] = (i * bm[h]) | flag;
      }
  }
  if (tid == 1023) *tile_count = excl + cnts[0] + cnts[1];
  const int64_t n = (int64_t)s_w[16] * per_tile;  // the scan's total: tiles listed
  for (int64_t i = tid; i < n; i += 1024) {
    split_cnt[i] = 0;
    split_cnt[cnt_each + i] = 0;
  }
}

// ------------------------------------------------------------------------------------------
// launchers (enqueue only; return hipSuccess or the launch error)
// ------------------------------------------------------------------------------------------
// where the dispatch also writes the grouped GEMM's tile list (tile_group null: it does not)
struct TileListArgs {
  int32_t* tile_group;
  int32_t* tile_m0;
  int32_t* tile_count;
  int32_t* split_cnt;
  int64_t cnt_each;
  int per_tile;
  int64_t T;
  int has_shared;
  int BM;
  int BM2;  // second tile height a group may take (0: none)
};
TileListArgs tile_list_args(const moe_dims& dm, const Layout& L, char* ws, bool with_tiles);

// router logits only: the per-split partial sums in the workspace (top-k adds them)
hipError_t launch_router_logits(const moe_dims& dm, const Layout& L, const void* x, const float* w_router, char* ws,
                                hipStream_t s);

// L.route_fused: top-k and dispatch (and with_tiles, the tile list) in one launch, on the partial
// logits launch_router_logits left in the workspace
hipError_t launch_topk_dispatch(const moe_dims& dm, const Layout& L, const float* bias, int32_t* topk_idx,
                                float* topk_w, float* topk_gap, int32_t* offsets, int32_t* sorted_token,
                                int32_t* slot_of, char* ws, hipStream_t s, bool with_tiles);

// probs: when non-null, every expert's softmax probability [T, E] (for the router statistics)
hipError_t launch_router(const moe_dims& dm, const Layout& L, const void* x, const float* w_router,
                         const float* bias, int32_t* topk_idx, float* topk_w, float* topk_gap, char* ws,
                         hipStream_t s, float* probs = nullptr);

// per-expert selection counts and mean probability from the router's probs (ws) and topk_idx
hipError_t launch_router_stats(const moe_dims& dm, const Layout& L, const int32_t* topk_idx, char* ws,
                               int32_t* counts, float* prob_mean, hipStream_t s);

// with_tiles: the scan also writes the grouped GEMM's tile list (launch_grouped_ffn with
// tiles_ready then skips building it)
hipError_t launch_permute(const moe_dims& dm, const Layout& L, const int32_t* topk_idx, int32_t* offsets,
                          int32_t* sorted_token, int32_t* slot_of, char* ws, hipStream_t s, bool with_tiles = false);

// The combine a forward may hand to the grouped GEMMs: with one or two tokens the skinny down
// product's last workgroup per column block sums the expert rows into `out` (combine_kernel's
// arithmetic, same order) and sets `done`, so that no combine launch follows.
struct CombineFuse {
  void* out;
  const int32_t* slot_of;
  const float* topk_w;
  const void* residual;  // the block's input row added last, or null
  bool done;
};

hipError_t launch_grouped_ffn(const moe_dims& dm, const Layout& L, const void* x, const int32_t* offsets,
                              const int32_t* sorted_token, const void* wg, const void* wu, const void* wd,
                              const void* wg_s, const void* wu_s, const void* wd_s, void* y, char* ws,
                              hipStream_t s, const Prof* prof = nullptr, bool tiles_ready = false,
                              CombineFuse* combine = nullptr);

// gate/up product with K split: H rows from the splits' fp32 partials (gate at column c, up at
// ldh + c of part[split][row], row pitch part_ld), added in split order, then silu(gate) * up
hipError_t launch_gate_up_finish(const float* part, int64_t sstride, int64_t part_ld, int ks, int64_t Tk,
                                 int64_t rows_total, int I, int Is, int ldh, bf16_t* H, hipStream_t s);

// few tokens (plan.skinny): both products on the vector ALUs with the weights streamed into an
// LDS ring by DMA; tile list and counters as for launch_grouped_ffn; with `combine`, the down
// product also writes the block's output
hipError_t launch_ffn_skinny(const moe_dims& dm, const Layout& L, const FfnPlan& P, const void* x,
                             const int32_t* offsets, const int32_t* sorted_token, const void* wg, const void* wu,
                             const void* wd, const void* wg_s, const void* wu_s, const void* wd_s, void* y, char* ws,
                             hipStream_t s, const Prof* prof, CombineFuse* combine);

// names of the grouped GEMM kernels these dims launch (static strings)
const char* ffn_kernel_name(const moe_dims& dm, bool gate_up);
const char* ffn_fp8_kernel_name(const moe_dims& dm, bool gate_up);

// row-tile list of the grouped GEMMs (rows per tile ffn_tile_rows) and zeroed split-K counters
int ffn_tile_rows(const moe_dims& dm);
// the second tile height a group may take instead (192 with the tall tiles), else 0
int ffn_tile_rows_alt(const moe_dims& dm);
// bm: rows per tile of the list (0: ffn_tile_rows(dm), the bf16 grouped GEMMs' choice)
hipError_t launch_build_tiles(const moe_dims& dm, const Layout& L, const int32_t* offsets, char* ws, hipStream_t s,
                              int bm = 0);

// FP8 (e4m3) expert weights: codes in 4 KB tiles of 128 columns x 32 K values (moe_quantize_fp8
// layout) with one fp32 scale per output column
struct Fp8Weights {
  const uint8_t *wg, *wu, *wd;      // per expert d*I bytes each: W_g, W_u (N = I, K = d), W_d (N = d, K = I)
  const float *sg, *su, *sd;        // [E, I], [E, I], [E, d]
  const uint8_t *wg_s, *wu_s, *wd_s;  // [I_s, d], [I_s, d], [d, I_s]
  const float *sg_s, *su_s, *sd_s;    // [I_s], [I_s], [d]
};
bool fp8_shape_ok(const moe_dims& dm);
hipError_t launch_grouped_ffn_fp8(const moe_dims& dm, const Layout& L, const void* x, const int32_t* offsets,
                                  const int32_t* sorted_token, const Fp8Weights& W, void* y, char* ws, hipStream_t s,
                                  const Prof* prof = nullptr, CombineFuse* combine = nullptr);
// w [batch, K, N] (dtype) -> q [batch, N, K] e4m3, scale [batch, N]
hipError_t launch_quantize_fp8(const void* w, int dtype, int64_t batch, int K, int N, uint8_t* q, float* scale,
                               hipStream_t s);

hipError_t launch_combine(const moe_dims& dm, const void* y, const int32_t* slot_of, const float* topk_w,
                          const void* residual, void* out, hipStream_t s);

hipError_t launch_rmsnorm(const moe_dims& dm, const void* x, const void* gamma, double eps, void* h, hipStream_t s);

}  // namespace moe
