// Dispatch: the token is sent to each of its k selected experts (Qwen3.6
// neural-network explorer page, router section). Here that becomes a stable
// grouping of the T*k (token, expert) pairs by expert, so every expert's rows
// are contiguous for the grouped GEMM:
//
//   permute_count   one workgroup per chunk of 256 tokens (one wavefront per 64).
//                   Each wavefront builds, in LDS, a 64-bit mask per expert of
//                   which of its lanes chose it (LDS atomic OR). A pair's rank in
//                   the chunk is the popcount of the masks of earlier wavefronts
//                   plus that of its own mask below its lane -- token order is
//                   kept without any sort. Per-chunk expert counts go to HBM.
//   permute_scan    one workgroup: per expert, an exclusive scan over chunks;
//                   then an exclusive scan over experts gives expert_offsets.
//   permute_scatter slot = chunk base of the expert + rank; writes slot_of and
//                   sorted_token.
// When the tokens fit one chunk (T <= 256, decode) one workgroup does all three
// with the counts in LDS (permute_one_chunk_kernel): two launches fewer.
// A token's expert indices must be distinct (top-k output is). Pairs whose index
// lies outside [0, E) are skipped: slot_of = -1.
// All integer work; results are deterministic.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kWaves = kPermuteChunk / 64;

__global__ void __launch_bounds__(kPermuteChunk)
permute_count_kernel(const int32_t* __restrict__ topk_idx, int64_t T, int E, int k, int32_t* __restrict__ rank,
                     int32_t* __restrict__ chunk_counts) {
  extern __shared__ unsigned long long mask[];  // [kWaves][E]
  const int tid = threadIdx.x;
  for (int i = tid; i < kWaves * E; i += kPermuteChunk) mask[i] = 0ull;
  __syncthreads();

  const int64_t t = (int64_t)blockIdx.x * kPermuteChunk + tid;
  const int w = tid >> 6;
  const int lane = tid & 63;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = topk_idx[t * k + j];
      if ((unsigned)e < (unsigned)E) atomicOr(&mask[w * E + e], 1ull << lane);
    }
  }
  __syncthreads();
  if (t < T) {
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int j = 0; j < k; ++j) {
      const int e = topk_idx[t * k + j];
      int r = 0;
      if ((unsigned)e < (unsigned)E) {
        for (int w2 = 0; w2 < w; ++w2) r += __popcll(mask[w2 * E + e]);
        r += __popcll(mask[w * E + e] & below);
      }
      rank[t * k + j] = (unsigned)e < (unsigned)E ? r : -1;
    }
  }
  for (int e = tid; e < E; e += kPermuteChunk) {
    int c = 0;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) c += __popcll(mask[w2 * E + e]);
    chunk_counts[(int64_t)blockIdx.x * E + e] = c;
  }
}

// Exclusive scan of n (<= 2048) values in s_val, two per thread across 1024 threads, in place;
// *total receives their sum. s_w: 17 ints of LDS.
__device__ void block_exclusive_scan_1024(int* s_val, int n, int* s_w, int* total) {
  const int tid = threadIdx.x;
  const int a = 2 * tid < n ? s_val[2 * tid] : 0;
  const int b = 2 * tid + 1 < n ? s_val[2 * tid + 1] : 0;
  const int excl = block_exclusive_scan_1024t(a + b, s_w, total);
  if (2 * tid < n) s_val[2 * tid] = excl;
  if (2 * tid + 1 < n) s_val[2 * tid + 1] = excl + a;
  __syncthreads();
}

// Chunk counts are loaded 16 at a time before any is rewritten, so each thread has 16 loads in
// flight instead of one dependent load per chunk.
__global__ void __launch_bounds__(1024)
permute_scan_kernel(int32_t* __restrict__ chunk_counts, int64_t nchunks, int E, int32_t* __restrict__ offsets,
                    TileListArgs tl) {
  __shared__ int s_val[2048];
  __shared__ int s_w[17];
  __shared__ int s_rows[kMaxGroups];
  __shared__ int s_total;
  const int tid = threadIdx.x;
  constexpr int B = 16;
  for (int e = tid; e < E; e += 1024) {
    int run = 0;
    for (int64_t c0 = 0; c0 < nchunks; c0 += B) {
      int v[B];
#pragma unroll
      for (int i = 0; i < B; ++i) v[i] = c0 + i < nchunks ? chunk_counts[(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < B; ++i)
        if (c0 + i < nchunks) {
          chunk_counts[(c0 + i) * E + e] = run;
          run += v[i];
        }
    }
    s_val[e] = run;
    s_rows[e] = run;
  }
  __syncthreads();
  block_exclusive_scan_1024(s_val, E, s_w, &s_total);
  for (int e = tid; e < E; e += 1024) {
    const int base = s_val[e];
    offsets[e] = base;
    for (int64_t c0 = 0; c0 < nchunks; c0 += B) {
      int v[B];
#pragma unroll
      for (int i = 0; i < B; ++i) v[i] = c0 + i < nchunks ? chunk_counts[(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < B; ++i)
        if (c0 + i < nchunks) chunk_counts[(c0 + i) * E + e] = v[i] + base;
    }
  }
  if (tid == 0) offsets[E] = s_total;
  if (tl.tile_group) {
    // the grouped GEMM's tile list from the same group sizes (the shared expert last)
    if (tid == 0 && tl.has_shared) s_rows[E] = (int)tl.T;
    __syncthreads();
    build_tile_list(s_rows, E + tl.has_shared, tl.BM, tl.BM2, s_w, tl.tile_group, tl.tile_m0, tl.tile_count, tl.split_cnt,
                    tl.cnt_each, tl.per_tile);
  }
}

__global__ void __launch_bounds__(kPermuteChunk)
permute_scatter_kernel(const int32_t* __restrict__ topk_idx, int64_t T, int E, int k,
                       const int32_t* __restrict__ chunk_counts, int32_t* __restrict__ slot_of,
                       int32_t* __restrict__ sorted_token) {
  const int64_t t = (int64_t)blockIdx.x * kPermuteChunk + threadIdx.x;
  if (t >= T) return;
  for (int j = 0; j < k; ++j) {
    const int e = topk_idx[t * k + j];
    if ((unsigned)e >= (unsigned)E) continue;  // slot_of stays -1
    const int slot = chunk_counts[(int64_t)blockIdx.x * E + e] + slot_of[t * k + j];  // slot_of holds the rank
    slot_of[t * k + j] = slot;
    sorted_token[slot] = (int32_t)t;
  }
}

// All of dispatch in one workgroup when the tokens fit one chunk (T <= 256, decode): the masks and
// ranks of permute_count, the scans of permute_scan (and the tile list) and the scatter, with
// the counts kept in LDS. Same ranks, offsets and slots as the three kernels. 1024 threads;
// threads 0 .. 255 hold one token each.
__global__ void __launch_bounds__(1024)
permute_one_chunk_kernel(const int32_t* __restrict__ topk_idx, int64_t T, int E, int k, int32_t* __restrict__ offsets,
                         int32_t* __restrict__ slot_of, int32_t* __restrict__ sorted_token, TileListArgs tl) {
  extern __shared__ unsigned long long mask[];  // [kWaves][E]
  __shared__ int s_val[2048];
  __shared__ int s_w[17];
  __shared__ int s_rows[kMaxGroups];
  __shared__ int s_total;
  const int tid = threadIdx.x;
  for (int i = tid; i < kWaves * E; i += 1024) mask[i] = 0ull;
  __syncthreads();
  const int t = tid;  // token (chunk 0)
  const int w = tid >> 6;
  const int lane = tid & 63;
  const bool mine = tid < kPermuteChunk && t < T;
  int e_of[kMaxK];
  if (mine)
    for (int j = 0; j < k; ++j) {
      e_of[j] = topk_idx[(int64_t)t * k + j];
      if ((unsigned)e_of[j] < (unsigned)E) atomicOr(&mask[w * E + e_of[j]], 1ull << lane);
    }
  __syncthreads();
  for (int e = tid; e < E; e += 1024) {
    int c = 0;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) c += __popcll(mask[w2 * E + e]);
    s_val[e] = c;
    s_rows[e] = c;
  }
  __syncthreads();
  block_exclusive_scan_1024(s_val, E, s_w, &s_total);
  for (int e = tid; e < E; e += 1024) offsets[e] = s_val[e];
  if (tid == 0) offsets[E] = s_total;
  if (mine) {
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int j = 0; j < k; ++j) {
      const int e = e_of[j];
      if ((unsigned)e >= (unsigned)E) {
        slot_of[(int64_t)t * k + j] = -1;
        continue;
      }
      int r = __popcll(mask[w * E + e] & below);
      for (int w2 = 0; w2 < w; ++w2) r += __popcll(mask[w2 * E + e]);
      const int slot = s_val[e] + r;
      slot_of[(int64_t)t * k + j] = slot;
      sorted_token[slot] = t;
    }
  }
  if (tl.tile_group) {
    if (tid == 0 && tl.has_shared) s_rows[E] = (int)tl.T;
    __syncthreads();
    build_tile_list(s_rows, E + tl.has_shared, tl.BM, tl.BM2, s_w, tl.tile_group, tl.tile_m0, tl.tile_count, tl.split_cnt,
                    tl.cnt_each, tl.per_tile);
  }
}

}  // namespace

TileListArgs tile_list_args(const moe_dims& dm, const Layout& L, char* ws, bool with_tiles) {
  TileListArgs tl{};
  if (with_tiles) {
    tl.tile_group = (int32_t*)(ws + L.tile_group);
    tl.tile_m0 = (int32_t*)(ws + L.tile_m0);
    tl.tile_count = (int32_t*)(ws + L.tile_count);
    tl.split_cnt = (int32_t*)(ws + L.ffn_cnt);
    tl.cnt_each = L.ffn_cnt_each;
    tl.per_tile = L.ffn_cnt_per_tile;
    tl.T = dm.T;
    tl.has_shared = dm.I_shared > 0 ? 1 : 0;
    tl.BM = ffn_tile_rows(dm);
    tl.BM2 = ffn_tile_rows_alt(dm);
  }
  return tl;
}

hipError_t launch_permute(const moe_dims& dm, const Layout& L, const int32_t* topk_idx, int32_t* offsets,
                          int32_t* sorted_token, int32_t* slot_of, char* ws, hipStream_t s, bool with_tiles) {
  const TileListArgs tl = tile_list_args(dm, L, ws, with_tiles);
  int32_t* cc = (int32_t*)(ws + L.chunk_counts);
  const size_t lds = sizeof(unsigned long long) * kWaves * (size_t)dm.E;
  if (L.nchunks == 1) {
    hipLaunchKernelGGL(permute_one_chunk_kernel, dim3(1), dim3(1024), lds, s, topk_idx, dm.T, dm.E, dm.k, offsets,
                       slot_of, sorted_token, tl);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(permute_count_kernel, dim3((unsigned)L.nchunks), dim3(kPermuteChunk), lds, s, topk_idx, dm.T,
                     dm.E, dm.k, slot_of, cc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, s, cc, L.nchunks, dm.E, offsets, tl);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(permute_scatter_kernel, dim3((unsigned)L.nchunks), dim3(kPermuteChunk), 0, s, topk_idx, dm.T,
                     dm.E, dm.k, cc, slot_of, sorted_token);
  return hipGetLastError();
}

}  // namespace moe
