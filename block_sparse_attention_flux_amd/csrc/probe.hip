// Attainable-peak probes for the roofline figures: a dense bf16 MFMA loop and
// a streaming HBM read.  Measurement helpers only; no attention work here.
#include "flux_probe.h"

#include <hip/hip_runtime.h>

#include "flux_device.h"

namespace flux {
namespace {

// Each wave keeps four independent 32x32x16 accumulators busy; the result is
// written so the loop cannot be removed.
__global__ __launch_bounds__(256) void mfma_probe_kernel(float* sink, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(static_cast<float>(threadIdx.x & 7) * 0.125f);
    b[i] = static_cast<__bf16>(0.5f);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  const float s = c0[0] + c1[1] + c2[2] + c3[3];
  if (threadIdx.x == 0) sink[blockIdx.x] = s;
}

// Grid-stride 16-byte reads folded into one word per workgroup.
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ src, size_t n16,
                                                         uint32_t* sink) {
  const size_t stride = static_cast<size_t>(gridDim.x) * 256 * 4;
  uint32_t acc = 0;
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 * 4 + threadIdx.x; i < n16; i += stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = (i + u * 256 < n16) ? ld16_stream(src + i + u * 256) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
    for (int t = 0; t < 256; ++t) a ^= red[t];
    sink[blockIdx.x] = a;
  }
}

}  // namespace
}  // namespace flux

extern "C" {

int32_t flux_probe_mfma(float* sink, int32_t n_workgroups, int32_t iters, void* stream) {
  if (sink == nullptr || n_workgroups < 1 || iters < 1) return -1;
  flux::mfma_probe_kernel<<<n_workgroups, 256, 0, static_cast<hipStream_t>(stream)>>>(sink, iters);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

double flux_probe_mfma_flops(int32_t n_workgroups, int32_t iters) {
  return 4.0 * n_workgroups * static_cast<double>(iters) * 4.0 * 32.0 * 32.0 * 16.0 * 2.0;
}

int32_t flux_probe_read(const void* src, size_t bytes, uint32_t* sink, int32_t n_workgroups,
                        void* stream) {
  if (src == nullptr || sink == nullptr || n_workgroups < 1 || bytes < 16 || bytes % 16 != 0)
    return -1;
  flux::read_probe_kernel<<<n_workgroups, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const flux::u32x4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
