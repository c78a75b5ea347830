// Device side of the seeded synthetic-input generator (definition in
// synth_core.h). Built with hipcc --offload-arch=gfx950 -ffp-contract=off into
// libsynth_dev.so. The quantile table is the host-built one, copied to the
// device by the caller, so both sides read identical table entries.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "synth_core.h"

namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 8;  // one 16-byte bf16 store or two fp32 16-byte stores

__global__ void __launch_bounds__(kThreads)
fill_kernel(void* __restrict__ out, int dtype, uint64_t n, uint64_t offset, uint64_t key,
            double sigma, const double* __restrict__ q) {
  const uint64_t nchunks = (n + kPerThread - 1) / kPerThread;
  for (uint64_t c = (uint64_t)blockIdx.x * kThreads + threadIdx.x; c < nchunks;
       c += (uint64_t)gridDim.x * kThreads) {
    const uint64_t i0 = c * kPerThread;
    if (dtype == 0) {
      float v[kPerThread];
#pragma unroll
      for (int j = 0; j < kPerThread; ++j)
        v[j] = synth_scale_f32(synth_normal(q, synth_bits(key, offset + i0 + j)), sigma);
      float* o = (float*)out + i0;
      if (i0 + kPerThread <= n) {
        *(float4*)(o) = make_float4(v[0], v[1], v[2], v[3]);
        *(float4*)(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
      } else {
        for (int j = 0; j < kPerThread && i0 + j < n; ++j) o[j] = v[j];
      }
    } else {
      uint16_t b[kPerThread];
#pragma unroll
      for (int j = 0; j < kPerThread; ++j)
        b[j] = synth_f32_to_bf16(synth_scale_f32(synth_normal(q, synth_bits(key, offset + i0 + j)), sigma));
      uint16_t* o = (uint16_t*)out + i0;
      if (i0 + kPerThread <= n) {
        uint4 w;
        w.x = (uint32_t)b[0] | ((uint32_t)b[1] << 16);
        w.y = (uint32_t)b[2] | ((uint32_t)b[3] << 16);
        w.z = (uint32_t)b[4] | ((uint32_t)b[5] << 16);
        w.w = (uint32_t)b[6] | ((uint32_t)b[7] << 16);
        *(uint4*)o = w;
      } else {
        for (int j = 0; j < kPerThread && i0 + j < n; ++j) o[j] = b[j];
      }
    }
  }
}

}  // namespace

// out: device buffer of n elements (fp32 if dtype == 0, bf16 bits if 1),
// 16-byte aligned; q: device copy of the 65537-entry quantile table.
// Returns a hipError_t code (0 on success).
extern "C" int synth_fill_device(void* out, int dtype, uint64_t n, uint64_t offset, uint64_t seed,
                                 uint32_t tensor_id, double sigma, const double* q,
                                 hipStream_t stream) {
  if (n == 0) return 0;
  if (dtype != 0 && dtype != 1) return (int)hipErrorInvalidValue;
  const uint64_t key = synth_stream_key(seed, tensor_id);
  const uint64_t nchunks = (n + kPerThread - 1) / kPerThread;
  uint64_t blocks = (nchunks + kThreads - 1) / kThreads;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, out, dtype, n,
                     offset, key, sigma, q);
  return (int)hipGetLastError();
}
