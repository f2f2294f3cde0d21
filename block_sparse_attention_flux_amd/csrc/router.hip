// Layer Router: pool the first and last 100 prompt rows, two-layer MLP, hard
// threshold (technical summary on gist.science, section 2 "Methodology":
// router pooling, MLP context encoder, hard 0/1 routing at inference).
//
// Three short kernels, each spread over many workgroups:
//   pool   grid (request, column chunk): 16 row groups x 64 column-chunk
//          threads, 16-byte loads, fp32 sums combined in a fixed order;
//   mlp1   grid (request, 16 rows of W1): one wave per hidden unit, float4
//          loads of the W1 row, h = relu(W1 pooled + b1);
//   mlp2   grid (request): one wave per layer, z = W2 h + b2, route = z >= 0.
// Every reduction runs in a fixed order, so logits and route bits are
// bitwise reproducible.  The pooled vector and the hidden layer live in the
// caller's workspace between the kernels.
#include "flux_device.h"
#include "flux_internal.h"

namespace flux {
namespace {

constexpr int kPool = 100;        // rows pooled from each end of a prompt
constexpr int kPoolGroups = 16;   // row groups per pooling workgroup
constexpr int kPoolChunks = 64;   // column chunks per pooling workgroup

__device__ __forceinline__ float wave_sum(float v) {
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Pooled positions of a request with S rows: [0, n_first) U [last_begin, S).
struct PoolSet {
  int64_t n_first, last_begin, S, count;
  __device__ __forceinline__ PoolSet(int64_t s) : S(s) {
    n_first = S > 0 ? (S < kPool ? S : kPool) : 0;
    last_begin = S - kPool > n_first ? S - kPool : n_first;
    count = n_first + (S > last_begin ? S - last_begin : 0);
  }
  __device__ __forceinline__ int64_t pos(int64_t u) const {
    return u < n_first ? u : last_begin + (u - n_first);
  }
};

// kVec elements per 16-byte load: 8 for bf16, 4 for fp32.
template <bool kBf16>
__global__ __launch_bounds__(kPoolGroups * kPoolChunks) void pool_kernel(
    const void* __restrict__ hidden, const int32_t* __restrict__ cu, int32_t d_in,
    float* __restrict__ pooled) {
  constexpr int kVec = kBf16 ? 8 : 4;
  __shared__ float part[kPoolGroups][kPoolChunks * kVec];
  const int r = blockIdx.y;
  const int grp = threadIdx.x / kPoolChunks, ch = threadIdx.x % kPoolChunks;
  const int col0 = (blockIdx.x * kPoolChunks + ch) * kVec;
  const int64_t start = cu[r];
  const PoolSet ps(static_cast<int64_t>(cu[r + 1]) - start);

  float acc[kVec];
#pragma unroll
  for (int e = 0; e < kVec; ++e) acc[e] = 0.0f;
  const bool full = col0 + kVec <= d_in && (d_in % kVec) == 0 &&
                    (reinterpret_cast<uintptr_t>(hidden) % 16) == 0;
#pragma unroll 4
  for (int64_t u = grp; u < ps.count; u += kPoolGroups) {
    const int64_t row = start + ps.pos(u);
    if constexpr (kBf16) {
      const uint16_t* src = static_cast<const uint16_t*>(hidden) + row * d_in + col0;
      if (full) {
        const u32x4 v = ld16(src);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += u32_as_f32(v[e] << 16);
          acc[2 * e + 1] += u32_as_f32(v[e] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < kVec; ++e)
          if (col0 + e < d_in) acc[e] += bf16_bits_to_f32(src[e]);
      }
    } else {
      const float* src = static_cast<const float*>(hidden) + row * d_in + col0;
      if (full) {
        const u32x4 v = ld16(src);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += u32_as_f32(v[e]);
      } else {
#pragma unroll
        for (int e = 0; e < kVec; ++e)
          if (col0 + e < d_in) acc[e] += src[e];
      }
    }
  }
#pragma unroll
  for (int e = 0; e < kVec; ++e) part[grp][ch * kVec + e] = acc[e];
  __syncthreads();
  for (int i = threadIdx.x; i < kPoolChunks * kVec; i += blockDim.x) {
    const int col = blockIdx.x * kPoolChunks * kVec + i;
    if (col < d_in) {
      float s = part[0][i];
#pragma unroll
      for (int g2 = 1; g2 < kPoolGroups; ++g2) s += part[g2][i];
      pooled[static_cast<int64_t>(r) * d_in + col] =
          ps.count > 0 ? s / static_cast<float>(ps.count) : 0.0f;
    }
  }
}

// Dot product of a row of length n with x, one wave, fixed order.
__device__ __forceinline__ float wave_dot(const float* __restrict__ wrow, const float* __restrict__ x,
                                          int n, int lane) {
  float acc = 0.0f;
  const bool vec = (n % 4) == 0 && (reinterpret_cast<uintptr_t>(wrow) % 16) == 0 &&
                   (reinterpret_cast<uintptr_t>(x) % 16) == 0;
  if (vec) {
    for (int c = lane * 4; c < n; c += 256) {
      const u32x4 a = ld16(wrow + c), b = ld16(x + c);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = __builtin_fmaf(u32_as_f32(a[e]), u32_as_f32(b[e]), acc);
    }
  } else {
    for (int c = lane; c < n; c += 64) acc = __builtin_fmaf(wrow[c], x[c], acc);
  }
  return wave_sum(acc);
}

constexpr int kMlpWaves = 16;

__global__ __launch_bounds__(kMlpWaves * 64) void mlp1_kernel(const float* __restrict__ pooled,
                                                              int32_t d_in, const float* __restrict__ w1,
                                                              const float* __restrict__ b1, int32_t h1,
                                                              float* __restrict__ hid) {
  const int r = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = blockIdx.x * kMlpWaves + wave;
  if (j >= h1) return;
  const float acc = wave_dot(w1 + static_cast<int64_t>(j) * d_in, pooled + static_cast<int64_t>(r) * d_in,
                             d_in, lane);
  if (lane == 0) hid[static_cast<int64_t>(r) * h1 + j] = fmaxf(acc + b1[j], 0.0f);
}

__global__ __launch_bounds__(kMlpWaves * 64) void mlp2_kernel(const float* __restrict__ hid, int32_t h1,
                                                              const float* __restrict__ w2,
                                                              const float* __restrict__ b2, int32_t n_layers,
                                                              uint8_t* __restrict__ route,
                                                              float* __restrict__ logits) {
  const int r = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int l = wave; l < n_layers; l += kMlpWaves) {
    const float acc = wave_dot(w2 + static_cast<int64_t>(l) * h1, hid + static_cast<int64_t>(r) * h1, h1, lane);
    if (lane == 0) {
      const float z = acc + b2[l];
      route[static_cast<int64_t>(r) * n_layers + l] = z >= 0.0f ? 1 : 0;
      if (logits != nullptr) logits[static_cast<int64_t>(r) * n_layers + l] = z;
    }
  }
}

}  // namespace

size_t route_workspace_bytes(int32_t n_req, int32_t d_in, int32_t h1) {
  return static_cast<size_t>(n_req) * (static_cast<size_t>(d_in) + h1) * sizeof(float);
}

hipError_t launch_route(const void* hidden, int32_t bf16, const int32_t* cu, int32_t n_req,
                        int32_t d_in, const float* w1, const float* b1, int32_t h1,
                        const float* w2, const float* b2, int32_t n_layers, uint8_t* route,
                        float* logits, void* workspace, hipStream_t s) {
  float* pooled = static_cast<float*>(workspace);
  float* hid = pooled + static_cast<size_t>(n_req) * d_in;
  const int vec = bf16 ? 8 : 4;
  const dim3 gpool((d_in + kPoolChunks * vec - 1) / (kPoolChunks * vec), n_req);
  if (bf16) {
    pool_kernel<true><<<gpool, dim3(kPoolGroups * kPoolChunks), 0, s>>>(hidden, cu, d_in, pooled);
  } else {
    pool_kernel<false><<<gpool, dim3(kPoolGroups * kPoolChunks), 0, s>>>(hidden, cu, d_in, pooled);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  mlp1_kernel<<<dim3((h1 + kMlpWaves - 1) / kMlpWaves, n_req), dim3(kMlpWaves * 64), 0, s>>>(
      pooled, d_in, w1, b1, h1, hid);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  mlp2_kernel<<<dim3(n_req), dim3(kMlpWaves * 64), 0, s>>>(hid, h1, w2, b2, n_layers, route, logits);
  return hipGetLastError();
}

}  // namespace flux
