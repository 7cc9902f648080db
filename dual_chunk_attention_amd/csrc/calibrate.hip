// Reference rates measured on the device for the roofline fractions the benchmark reports next to
// the vendor peaks: a matrix-core loop with no memory traffic (bf16 MFMA 32x32x16, the instruction
// of the prefill passes) and a streaming read of a device buffer (the access of the decode pass).
// Neither is part of the attention path.
#include "common.h"

namespace dca {
namespace {

__global__ __launch_bounds__(256) void probe_mfma_kernel(int32_t iters, float* __restrict__ sink) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (bf16)(1e-3f * (float)((threadIdx.x + e) & 7));
    b[e] = (bf16)(1e-3f * (float)e);
  }
  f32x16 c0 = f32x16{}, c1 = f32x16{}, c2 = f32x16{}, c3 = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {   // 32 MFMAs on four independent accumulators
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
  }
  float t = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) t += c0[e] + c1[e] + c2[e] + c3[e];
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = t;
}

// 16-byte nontemporal loads, eight in flight per thread per step, grid-stride over n16 = bytes / 16
// (of the forms tried on MI355X: four or eight in flight, with or without the nontemporal hint,
// 2048 to 32768 workgroups, this one read fastest)
__global__ __launch_bounds__(256) void probe_read_kernel(const uint4* __restrict__ src, int64_t n16,
                                                         float* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const u32x4* s4 = (const u32x4*)src;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = __builtin_nontemporal_load(s4 + i + k * stride);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = __uint_as_float(acc);
}

}  // namespace

hipError_t launch_probe_mfma(int32_t n_workgroups, int32_t iters, float* sink, hipStream_t stream) {
  hipLaunchKernelGGL(probe_mfma_kernel, dim3((unsigned)n_workgroups), dim3(256), 0, stream, iters, sink);
  return hipGetLastError();
}

hipError_t launch_probe_read(const void* src, int64_t bytes, int32_t n_workgroups, float* sink,
                             hipStream_t stream) {
  hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)n_workgroups), dim3(256), 0, stream,
                     (const uint4*)src, bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace dca
