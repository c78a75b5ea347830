// Combine: the kept experts' outputs are summed with their routing weights
// (Qwen3.6 neural-network explorer page, router section: the experts with the
// highest weights process the token) and the always-active shared expert is
// added with no weight (same section; Qwen3-Next article on hyper.ai).
//
//   out[t] = sum_{j<k} w[t,j] * y[slot_of[t*k+j]]  +  y[T*k + t]  (+ residual[t])
//
// One workgroup per token (256 threads; up to 1024 for few tokens); each thread owns
// 8 consecutive hidden elements at a time (16-byte bf16 or 2x16-byte fp32 loads; bf16 expert rows
// with the non-temporal hint when they far exceed the last-level cache),
// issues the loads of all k+1 rows before the first add, accumulates in fp32 in the fixed order j = 0..k-1,
// the shared row, then the residual row (the block's input, when the caller
// asks for the residual add), and rounds once on store. Pairs with slot_of = -1 (an
// expert index outside [0, E) at dispatch) contribute nothing.
#include "moe_internal.h"

namespace moe {
namespace {

// 8 consecutive elements, raw (loaded) and widened to fp32
struct Raw8bf { uint4 w; };
struct Raw8f { float4 a, b; };
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
template <bool NT = false>
__device__ __forceinline__ void load_raw(const bf16_t* p, Raw8bf& r) {
  if constexpr (NT) {
    const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
    r.w = make_uint4(v[0], v[1], v[2], v[3]);
  } else {
    r.w = *(const uint4*)p;
  }
}
template <bool NT = false>
__device__ __forceinline__ void load_raw(const float* p, Raw8f& r) {
  r.a = *(const float4*)p;
  r.b = *(const float4*)(p + 4);
}
__device__ __forceinline__ void widen(const Raw8bf& r, float* v) {
  v[0] = bf16lo_to_f32(r.w.x); v[1] = bf16hi_to_f32(r.w.x);
  v[2] = bf16lo_to_f32(r.w.y); v[3] = bf16hi_to_f32(r.w.y);
  v[4] = bf16lo_to_f32(r.w.z); v[5] = bf16hi_to_f32(r.w.z);
  v[6] = bf16lo_to_f32(r.w.w); v[7] = bf16hi_to_f32(r.w.w);
}
__device__ __forceinline__ void widen(const Raw8f& r, float* v) {
  v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
  v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
}
template <typename ET> struct RawOf;
template <> struct RawOf<bf16_t> { typedef Raw8bf type; };
template <> struct RawOf<float> { typedef Raw8f type; };

__device__ __forceinline__ void store8(bf16_t* p, const float* v) {
  uint4 w;
  w.x = pack_bf16x2(v[0], v[1]);
  w.y = pack_bf16x2(v[2], v[3]);
  w.z = pack_bf16x2(v[4], v[5]);
  w.w = pack_bf16x2(v[6], v[7]);
  *(uint4*)p = w;
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
  *(float4*)(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// NT: the expert output rows y with the non-temporal hint (each is read once here, and at the
// prefill shape they span ~3 GB, past any cache)
template <typename ET, int MAXT, bool NT = false>
__global__ void __launch_bounds__(MAXT)
combine_kernel(const ET* __restrict__ y, const int32_t* __restrict__ slot_of, const float* __restrict__ topk_w,
               const ET* __restrict__ residual, ET* __restrict__ out, int64_t T, int d, int k, int has_shared) {
  __shared__ int s_slot[kMaxK];
  __shared__ float s_w[kMaxK];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < k) {
    s_slot[threadIdx.x] = slot_of[t * k + threadIdx.x];
    s_w[threadIdx.x] = topk_w[t * k + threadIdx.x];
  }
  __syncthreads();
  const int64_t shared_row = T * k + t;
  typedef typename RawOf<ET>::type Raw;
  for (int c = threadIdx.x * 8; c < d; c += blockDim.x * 8) {
    // every row's load is issued before the first add
    Raw raw[kMaxK + 2];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < k && s_slot[j] >= 0) load_raw<NT>(y + (int64_t)s_slot[j] * d + c, raw[j]);
    if (has_shared) load_raw<NT>(y + shared_row * d + c, raw[kMaxK]);
    if (residual) load_raw(residual + t * d + c, raw[kMaxK + 1]);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < k && s_slot[j] >= 0) {
        float v[8];
        widen(raw[j], v);
        const float w = s_w[j];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(w, v[i], acc[i]);
      }
    }
    if (has_shared) {
      float v[8];
      widen(raw[kMaxK], v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    if (residual) {
      float v[8];
      widen(raw[kMaxK + 1], v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    store8(out + t * d + c, acc);
  }
}

}  // namespace

hipError_t launch_combine(const moe_dims& dm, const void* y, const int32_t* slot_of, const float* topk_w,
                          const void* residual, void* out, hipStream_t s) {
  const int hs = dm.I_shared > 0 ? 1 : 0;
  // few tokens: up to d / 8 threads per token (1024 at most), so that all of a token's row loads
  // are in flight at once; otherwise 256 threads, looping over the row
  // (bf16: the eight-element loads fit 128 registers; fp32 stays at 256 threads)
  int threads = 256;
  if (dm.T <= 256 && dm.dtype == MOE_BF16)
    while (threads < 1024 && threads * 8 < dm.d) threads *= 2;
  if (dm.dtype == MOE_BF16 && threads > 256)
    hipLaunchKernelGGL((combine_kernel<bf16_t, 1024>), dim3((unsigned)dm.T), dim3(threads), 0, s, (const bf16_t*)y,
                       slot_of, topk_w, (const bf16_t*)residual, (bf16_t*)out, dm.T, dm.d, dm.k, hs);
  else if (dm.dtype == MOE_BF16 && (uint64_t)(dm.T * dm.k + (hs ? dm.T : 0)) * dm.d * 2 > (512ull << 20))
    // expert outputs at least twice the 256 MB last-level cache: non-temporal reads (prefill
    // combine 636 -> 577 us, skew 322 -> 281 us; at the mid shape, ~150 MB, the rows come from the
    // cache and stay on plain loads)
    hipLaunchKernelGGL((combine_kernel<bf16_t, 256, true>), dim3((unsigned)dm.T), dim3(256), 0, s, (const bf16_t*)y,
                       slot_of, topk_w, (const bf16_t*)residual, (bf16_t*)out, dm.T, dm.d, dm.k, hs);
  else if (dm.dtype == MOE_BF16)
    hipLaunchKernelGGL((combine_kernel<bf16_t, 256>), dim3((unsigned)dm.T), dim3(256), 0, s, (const bf16_t*)y,
                       slot_of, topk_w, (const bf16_t*)residual, (bf16_t*)out, dm.T, dm.d, dm.k, hs);
  else
    hipLaunchKernelGGL((combine_kernel<float, 256>), dim3((unsigned)dm.T), dim3(256), 0, s, (const float*)y, slot_of,
                       topk_w, (const float*)residual, (float*)out, dm.T, dm.d, dm.k, hs);
  return hipGetLastError();
}

}  // namespace moe
