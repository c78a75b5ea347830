// Zero-centred RMSNorm in front of the MoE block. The Qwen3-Next article names Zero-Centered
// RMSNorm, whose parameters start at zero, so the scale is 1 + gamma; the configuration listing on
// the Qwen3.8-Max architecture page gives rms_norm_eps = 1e-6:
//
//   h = x / sqrt(mean_i x_i^2 + eps) * (1 + gamma)
//
// One 256-thread workgroup per row, 8 consecutive elements per thread and step. The row's sum of
// squares and h are computed in fp64 and h is rounded once to the element type of x. The router
// ranks experts on these rows, and an element rounded the other way (as an fp32 computation would
// do now and then) can move a logit by more than the margin that decides the top-k; in fp64 the
// rounding is the correctly rounded one.
#include "moe_internal.h"

namespace moe {
namespace {

// fp64 -> bf16, to nearest with ties to even: the double's significand is rounded at the bf16
// position (45 bits below the top) by an integer add, after which narrowing to fp32 is exact.
// Normal range.
__device__ __forceinline__ bf16_t f64_to_bf16(double v) {
  uint64_t u = (uint64_t)__double_as_longlong(v);
  u += 0x00000FFFFFFFFFFFull + ((u >> 45) & 1ull);  // half of the dropped range, minus one, plus the kept lsb
  u &= ~0x00001FFFFFFFFFFFull;
  const float f = (float)__longlong_as_double((long long)u);
  return (bf16_t)(__float_as_uint(f) >> 16);
}

__device__ __forceinline__ void load8(const bf16_t* p, double* v) {
  const uint4 w = *(const uint4*)p;
  const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = (double)bf16lo_to_f32(a[i]);
    v[2 * i + 1] = (double)bf16hi_to_f32(a[i]);
  }
}
__device__ __forceinline__ void load8(const float* p, double* v) {
  const float4 a = *(const float4*)p;
  const float4 b = *(const float4*)(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void store8(bf16_t* p, const double* v) {
  uint4 w;
  w.x = (uint32_t)f64_to_bf16(v[0]) | ((uint32_t)f64_to_bf16(v[1]) << 16);
  w.y = (uint32_t)f64_to_bf16(v[2]) | ((uint32_t)f64_to_bf16(v[3]) << 16);
  w.z = (uint32_t)f64_to_bf16(v[4]) | ((uint32_t)f64_to_bf16(v[5]) << 16);
  w.w = (uint32_t)f64_to_bf16(v[6]) | ((uint32_t)f64_to_bf16(v[7]) << 16);
  *(uint4*)p = w;
}
__device__ __forceinline__ void store8(float* p, const double* v) {
  *(float4*)p = make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
  *(float4*)(p + 4) = make_float4((float)v[4], (float)v[5], (float)v[6], (float)v[7]);
}

template <typename ET>
__global__ void __launch_bounds__(256)
rmsnorm_kernel(const ET* __restrict__ x, const ET* __restrict__ gamma, double eps, ET* __restrict__ h, int d) {
  __shared__ double part[4];
  const int64_t row = blockIdx.x;
  const ET* xr = x + row * d;
  double ss = 0.0;
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    double v[8];
    load8(xr + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fma(v[i], v[i], ss);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const double inv = 1.0 / sqrt(((part[0] + part[1]) + (part[2] + part[3])) / d + eps);
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    double v[8], g[8];
    load8(xr + c, v);
    load8(gamma + c, g);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = v[i] * inv * (1.0 + g[i]);
    store8(h + row * d + c, v);
  }
}

}  // namespace

hipError_t launch_rmsnorm(const moe_dims& dm, const void* x, const void* gamma, double eps, void* h, hipStream_t s) {
  if (dm.dtype == MOE_BF16)
    hipLaunchKernelGGL(rmsnorm_kernel<bf16_t>, dim3((unsigned)dm.T), dim3(256), 0, s, (const bf16_t*)x,
                       (const bf16_t*)gamma, eps, (bf16_t*)h, dm.d);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<float>, dim3((unsigned)dm.T), dim3(256), 0, s, (const float*)x,
                       (const float*)gamma, eps, (float*)h, dm.d);
  return hipGetLastError();
}

}  // namespace moe
