// Layer Router: pool the first and last 100 prompt rows, two-layer MLP, hard
// threshold (technical summary on gist.science, section 2 "Methodology":
// router pooling, MLP context encoder, hard 0/1 routing at inference).
//
// One workgroup of 1024 threads per request.  The pooled vector and the
// hidden layer stay in LDS; every reduction runs in a fixed order, so the
// logits (and hence the route bits) are bitwise reproducible run to run.
#include "flux_device.h"
#include "flux_internal.h"

namespace flux {
namespace {

constexpr int kPool = 100;        // rows pooled from each end of a prompt
constexpr int kRouterThreads = 1024;
constexpr int kRouterWaves = kRouterThreads / 64;

__device__ __forceinline__ float wave_sum(float v) {
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

template <bool kBf16>
__device__ __forceinline__ float hidden_at(const void* h, int64_t row, int32_t d_in, int32_t j) {
  if constexpr (kBf16) {
    return bf16_bits_to_f32(static_cast<const uint16_t*>(h)[row * d_in + j]);
  } else {
    return static_cast<const float*>(h)[row * d_in + j];
  }
}

template <bool kBf16>
__global__ __launch_bounds__(kRouterThreads) void route_kernel(
    const void* __restrict__ hidden, const int32_t* __restrict__ cu, int32_t d_in,
    const float* __restrict__ w1, const float* __restrict__ b1, int32_t h1,
    const float* __restrict__ w2, const float* __restrict__ b2, int32_t n_layers,
    uint8_t* __restrict__ route, float* __restrict__ logits) {
  extern __shared__ float smem[];  // pooled[d_in] then hid[h1]
  float* pooled = smem;
  float* hid = smem + d_in;
  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  const int64_t start = cu[r];
  const int64_t S = static_cast<int64_t>(cu[r + 1]) - start;
  // pooled set: [0, n_first) U [last_begin, S), disjoint by construction
  const int64_t n_first = S > 0 ? (S < kPool ? S : kPool) : 0;
  const int64_t last_begin = S - kPool > n_first ? S - kPool : n_first;
  const int64_t count = n_first + (S > last_begin ? S - last_begin : 0);

  for (int32_t j = tid; j < d_in; j += kRouterThreads) {
    float acc = 0.0f;
    for (int64_t pos = 0; pos < n_first; ++pos) acc += hidden_at<kBf16>(hidden, start + pos, d_in, j);
    for (int64_t pos = last_begin; pos < S; ++pos) acc += hidden_at<kBf16>(hidden, start + pos, d_in, j);
    pooled[j] = count > 0 ? acc / static_cast<float>(count) : 0.0f;
  }
  __syncthreads();

  for (int32_t j = wave; j < h1; j += kRouterWaves) {
    const float* wr = w1 + static_cast<int64_t>(j) * d_in;
    float acc = 0.0f;
    for (int32_t c = lane; c < d_in; c += 64) acc += wr[c] * pooled[c];
    acc = wave_sum(acc);
    if (lane == 0) hid[j] = fmaxf(acc + b1[j], 0.0f);
  }
  __syncthreads();

  for (int32_t l = wave; l < n_layers; l += kRouterWaves) {
    const float* wr = w2 + static_cast<int64_t>(l) * h1;
    float acc = 0.0f;
    for (int32_t c = lane; c < h1; c += 64) acc += wr[c] * hid[c];
    acc = wave_sum(acc);
    if (lane == 0) {
      const float z = acc + b2[l];
      route[static_cast<int64_t>(r) * n_layers + l] = z >= 0.0f ? 1 : 0;
      if (logits != nullptr) logits[static_cast<int64_t>(r) * n_layers + l] = z;
    }
  }
}

}  // namespace

hipError_t launch_route(const void* hidden, int32_t bf16, const int32_t* cu, int32_t n_req,
                        int32_t d_in, const float* w1, const float* b1, int32_t h1,
                        const float* w2, const float* b2, int32_t n_layers, uint8_t* route,
                        float* logits, hipStream_t s) {
  const size_t lds = static_cast<size_t>(d_in + h1) * sizeof(float);
  if (bf16) {
    route_kernel<true><<<dim3(n_req), dim3(kRouterThreads), lds, s>>>(
        hidden, cu, d_in, w1, b1, h1, w2, b2, n_layers, route, logits);
  } else {
    route_kernel<false><<<dim3(n_req), dim3(kRouterThreads), lds, s>>>(
        hidden, cu, d_in, w1, b1, h1, w2, b2, n_layers, route, logits);
  }
  return hipGetLastError();
}

}  // namespace flux
