// Content-aware SA block mask for gfx950: block importance from mean-pooled
// coarse attention, averaged over the query heads, then Top-tau selection.
//
// The pages only hint at a content-based pattern (the model card's slug,
// page 1 address); the "Daily Papers" page (hugingapi.com, search
// "Head-Centric Sparse Attention") describes block importance from
// coarse-grained attention between mean-pooled blocks (Prism abstract) and an
// adaptive Top-tau selection (RRAttention abstract).  The definition built
// here, step by step:
//   qbar[i][h] / kbar[j][g]  mean of the rows of block i / j (fp32);
//   z[h][i][j] = scale * qbar[i][h] . kbar[j][h / group]  for j <= i;
//   P[i][j]    = mean over h of softmax_j(z[h][i][:]);
//   row i keeps its sink blocks (j < s) and its diagonal block, then the
//   other causal blocks in order of decreasing P (ties: smaller j first)
//   while the mass taken is below tau and the row holds fewer than
//   max_blocks blocks (0: no cap).
// Output: the same CSR form as the static builder (columns ascending), which
// the prefill and decode kernels take as their SA mask.
//
// Four kernels: block means of Q and K (HBM-bound, one read of each); one
// workgroup per (mask row, KV head) for the logits and softmax of that head
// group, summed over its query heads (written per group, then added in a
// fixed order, so the result does not depend on scheduling); one workgroup
// per mask row for the selection (the candidate at sorted rank r is kept iff
// the mass of the r candidates ranked before it, plus the mandatory blocks'
// mass, is below tau: ranks come from pairwise comparisons, so no sort is
// needed); one workgroup per row for the CSR offsets (a sum over the earlier
// rows' counts) and the copy.
#include "flux_device.h"
#include "flux_internal.h"

namespace flux {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// (1) Mean of the rows of block i for one head of Q (y < hq) or K.  Thread t
// sums 16-byte chunk t % CH of rows t / CH, t / CH + RL, ...; the partial sums
// are added in LDS in a fixed order.  qbar is [nb][hq][D]; kbar is stored
// transposed, [hkv][D][nb], so that consecutive key blocks are consecutive
// words for the probability kernel.
template <int D>
__global__ __launch_bounds__(kThreads) void pool_kernel(const uint16_t* __restrict__ q,
                                                        const uint16_t* __restrict__ k, int32_t S,
                                                        int32_t hq, int32_t hkv, int32_t B, int32_t nb,
                                                        float* __restrict__ qbar, float* __restrict__ kbar_t) {
  constexpr int CH = D / 8;
  constexpr int RL = kThreads / CH;
  __shared__ float part[RL][D];
  const int i = blockIdx.x;
  const bool is_q = static_cast<int>(blockIdx.y) < hq;
  const int H = is_q ? hq : hkv;
  const int h = is_q ? blockIdx.y : blockIdx.y - hq;
  const uint16_t* src = is_q ? q : k;
  const int r0 = i * B, r1 = min(S, r0 + B);
  const int c = threadIdx.x % CH, rl = threadIdx.x / CH;
  float acc[8] = {};
#pragma unroll 4
  for (int r = r0 + rl; r < r1; r += RL) {
    const u32x4 v = ld16_stream(src + (static_cast<size_t>(r) * H + h) * D + c * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += bf16_bits_to_f32(static_cast<uint16_t>(v[e] & 0xffffu));
      acc[2 * e + 1] += bf16_bits_to_f32(static_cast<uint16_t>(v[e] >> 16));
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rl][c * 8 + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float s = 0.0f;
    for (int t = 0; t < RL; ++t) s += part[t][threadIdx.x];
    const float mean = s / static_cast<float>(r1 - r0);
    if (is_q)
      qbar[(static_cast<size_t>(i) * hq + h) * D + threadIdx.x] = mean;
    else
      kbar_t[(static_cast<size_t>(h) * D + threadIdx.x) * nb + i] = mean;
  }
}

// Workgroup reduction of N values per thread (slots 0 .. n-1): lanes first
// (a fixed butterfly), then the waves in order; every thread gets the result.
template <int N>
__device__ __forceinline__ void block_reduce(float (&v)[N], int n, bool is_max, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int s = 0; s < N; ++s) {
    if (s < n) {
      float x = v[s];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float y = __shfl_xor(x, o);
        x = is_max ? fmaxf(x, y) : x + y;
      }
      v[s] = x;
    }
  }
  __syncthreads();
  if (lane == 0) {
#pragma unroll
    for (int s = 0; s < N; ++s)
      if (s < n) red[wave * N + s] = v[s];
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < N; ++s) {
    if (s < n) {
      float x = red[s];
      for (int w = 1; w < kWaves; ++w) x = is_max ? fmaxf(x, red[w * N + s]) : x + red[w * N + s];
      v[s] = x;
    }
  }
}

// (2a) One workgroup per (query block i, KV head g): the logits of the query
// heads of g against key blocks j <= i, their softmax over j, and the sum over
// those heads of the probabilities, part[i][g][j].  Thread t owns key blocks
// t, t + 256, ... (at most kOwn).  kGroup is the GQA group size rounded up to
// a power of two (heads past the group are skipped).
template <int D, int kGroup>
__global__ __launch_bounds__(kThreads) void probs_kernel(const float* __restrict__ qbar,
                                                         const float* __restrict__ kbar_t, int32_t nb,
                                                         int32_t hq, int32_t hkv, float scale,
                                                         float* __restrict__ part) {
  constexpr int kOwn = kMaxDynBlocks / kThreads;  // key blocks per thread
  __shared__ __attribute__((aligned(16))) float qs[kGroup * D];  // scale * qbar[i][h] of group g
  __shared__ float red[kWaves * kGroup];

  const int i = blockIdx.x, g = blockIdx.y, n = i + 1, tid = threadIdx.x;
  const int group = hq / hkv;
  for (int e = tid; e < group * D; e += kThreads)
    qs[e] = scale * qbar[(static_cast<size_t>(i) * hq + g * group) * D + e];
  __syncthreads();

  float z[kOwn][kGroup];
#pragma unroll
  for (int o = 0; o < kOwn; ++o) {
    const int j = tid + o * kThreads;
#pragma unroll
    for (int hh = 0; hh < kGroup; ++hh) z[o][hh] = kNegInf;
    if (j < n) {
#pragma unroll
      for (int hh = 0; hh < kGroup; ++hh) z[o][hh] = 0.0f;
      const float* kb = kbar_t + static_cast<size_t>(g) * D * nb + j;
#pragma unroll 2
      for (int c = 0; c < D; c += 4) {
        float kv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) kv[e] = kb[static_cast<size_t>(c + e) * nb];
#pragma unroll
        for (int hh = 0; hh < kGroup; ++hh)
          if (hh < group) {
            const f32x4 qv = *reinterpret_cast<const f32x4*>(qs + hh * D + c);
            z[o][hh] += qv[0] * kv[0] + qv[1] * kv[1] + qv[2] * kv[2] + qv[3] * kv[3];
          }
      }
    }
  }
  float mx[kGroup], sm[kGroup];
#pragma unroll
  for (int hh = 0; hh < kGroup; ++hh) {
    mx[hh] = kNegInf;
#pragma unroll
    for (int o = 0; o < kOwn; ++o) mx[hh] = fmaxf(mx[hh], z[o][hh]);
  }
  block_reduce<kGroup>(mx, group, true, red);
#pragma unroll
  for (int hh = 0; hh < kGroup; ++hh) {
    sm[hh] = 0.0f;
    if (hh < group) {
#pragma unroll
      for (int o = 0; o < kOwn; ++o) {
        z[o][hh] = fast_exp2((z[o][hh] - mx[hh]) * kLog2e);  // 0 for blocks past the row
        sm[hh] += z[o][hh];
      }
    }
  }
  block_reduce<kGroup>(sm, group, false, red);
#pragma unroll
  for (int hh = 0; hh < kGroup; ++hh) sm[hh] = 1.0f / sm[hh];
#pragma unroll
  for (int o = 0; o < kOwn; ++o) {
    const int j = tid + o * kThreads;
    if (j < n) {
      float p = 0.0f;
#pragma unroll
      for (int hh = 0; hh < kGroup; ++hh)
        if (hh < group) p += z[o][hh] * sm[hh];
      part[(static_cast<size_t>(i) * hkv + g) * nb + j] = p;
    }
  }
}

// (2b) One workgroup per query block i: P[i][j] = (sum over g of part[i][g][j])
// / hq, then the selection.
__global__ __launch_bounds__(kThreads) void select_kernel(const float* __restrict__ part, int32_t nb,
                                                          int32_t hq, int32_t hkv, int32_t sink,
                                                          float tau, int32_t max_blocks,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ cols_tmp) {
  __shared__ float P[kMaxDynBlocks];
  __shared__ float red[kWaves];
  __shared__ int32_t scan[kWaves];

  const int i = blockIdx.x, n = i + 1, tid = threadIdx.x;
  const float inv_h = 1.0f / static_cast<float>(hq);
  for (int j = tid; j < n; j += kThreads) {
    float p = 0.0f;
    for (int g = 0; g < hkv; ++g) p += part[(static_cast<size_t>(i) * hkv + g) * nb + j];
    P[j] = p * inv_h;
  }
  __syncthreads();

  // mandatory blocks and their mass
  auto mandatory = [&](int j) { return j < sink || j == i; };
  float mm[1] = {0.0f};
  for (int j = tid; j < n; j += kThreads)
    if (mandatory(j)) mm[0] += P[j];
  block_reduce<1>(mm, 1, false, red);
  const float base = mm[0];
  const int n_mand = min(sink, i) + 1;  // sink blocks left of the diagonal, plus the diagonal

  // selection, then the row's columns in ascending order
  int written = 0;
  for (int j0 = 0; j0 < n; j0 += kThreads) {
    const int j = j0 + tid;
    bool on = false;
    if (j < n) {
      if (mandatory(j)) {
        on = true;
      } else {
        const float pj = P[j];
        int rank = 0;
        float before = 0.0f;
#pragma unroll 8
        for (int kk = 0; kk < n; ++kk) {
          const float pk = P[kk];
          const bool ahead = !mandatory(kk) && (pk > pj || (pk == pj && kk < j));
          rank += ahead ? 1 : 0;
          before += ahead ? pk : 0.0f;
        }
        on = base + before < tau && (max_blocks == 0 || n_mand + rank < max_blocks);
      }
    }
    // exclusive prefix of `on` over this chunk (ballot per wave, waves in order)
    const uint64_t bal = __ballot(on);
    const int lane = tid & 63, wave = tid >> 6;
    const int in_wave = __popcll(bal & ((1ull << lane) - 1ull));
    __syncthreads();
    if (lane == 0) scan[wave] = __popcll(bal);
    __syncthreads();
    int off = 0;
    for (int w = 0; w < wave; ++w) off += scan[w];
    int total = 0;
    for (int w = 0; w < kWaves; ++w) total += scan[w];
    if (on) cols_tmp[static_cast<size_t>(i) * nb + written + off + in_wave] = j;
    written += total;
  }
  if (tid == 0) counts[i] = written;
}

// (3) CSR offsets (sum of the earlier rows' counts) and the copy of row i.
__global__ __launch_bounds__(kThreads) void csr_kernel(const int32_t* __restrict__ counts,
                                                       const int32_t* __restrict__ cols_tmp, int32_t nb,
                                                       int32_t* __restrict__ row_ptr,
                                                       int32_t* __restrict__ col_idx) {
  __shared__ float red[kWaves];
  const int i = blockIdx.x, tid = threadIdx.x;
  float s[1] = {0.0f};
  for (int r = tid; r < i; r += kThreads) s[0] += static_cast<float>(counts[r]);
  block_reduce<1>(s, 1, false, red);  // exact: integers below 2^24
  const int base = static_cast<int>(s[0]);
  const int cnt = counts[i];
  for (int e = tid; e < cnt; e += kThreads) col_idx[base + e] = cols_tmp[static_cast<size_t>(i) * nb + e];
  if (tid == 0) {
    row_ptr[i] = base;
    if (i == nb - 1) row_ptr[nb] = base + cnt;
  }
}

template <int D>
void launch_probs(int group, dim3 grid, hipStream_t s, const float* qbar, const float* kbar_t, int nb, int hq,
                  int hkv, float scale, float* part) {
  if (group <= 1)
    probs_kernel<D, 1><<<grid, kThreads, 0, s>>>(qbar, kbar_t, nb, hq, hkv, scale, part);
  else if (group <= 2)
    probs_kernel<D, 2><<<grid, kThreads, 0, s>>>(qbar, kbar_t, nb, hq, hkv, scale, part);
  else if (group <= 4)
    probs_kernel<D, 4><<<grid, kThreads, 0, s>>>(qbar, kbar_t, nb, hq, hkv, scale, part);
  else if (group <= 8)
    probs_kernel<D, 8><<<grid, kThreads, 0, s>>>(qbar, kbar_t, nb, hq, hkv, scale, part);
  else
    probs_kernel<D, 16><<<grid, kThreads, 0, s>>>(qbar, kbar_t, nb, hq, hkv, scale, part);
}

}  // namespace

size_t dynamic_mask_workspace_bytes(int32_t seqlen, int32_t hq, int32_t hkv, int32_t head_dim,
                                    int32_t block_size) {
  const size_t nb = (static_cast<size_t>(seqlen) + block_size - 1) / block_size;
  return (nb * hq * head_dim + nb * hkv * head_dim + nb * hkv * nb) * sizeof(float) +
         nb * sizeof(int32_t) + nb * nb * sizeof(int32_t);
}

hipError_t launch_dynamic_mask(const DynMaskParams& p, hipStream_t s) {
  const int nb = (p.seqlen + p.block_size - 1) / p.block_size;
  float* qbar = static_cast<float*>(p.workspace);
  float* kbar_t = qbar + static_cast<size_t>(nb) * p.hq * p.head_dim;
  float* part = kbar_t + static_cast<size_t>(nb) * p.hkv * p.head_dim;
  int32_t* counts = reinterpret_cast<int32_t*>(part + static_cast<size_t>(nb) * p.hkv * nb);
  int32_t* cols_tmp = counts + nb;
  const dim3 pool_grid(nb, p.hq + p.hkv), probs_grid(nb, p.hkv);
  const int group = p.hq / p.hkv;
  if (p.head_dim == 128) {
    pool_kernel<128><<<pool_grid, kThreads, 0, s>>>(p.q, p.k, p.seqlen, p.hq, p.hkv, p.block_size, nb, qbar,
                                                    kbar_t);
    launch_probs<128>(group, probs_grid, s, qbar, kbar_t, nb, p.hq, p.hkv, p.scale, part);
  } else {
    pool_kernel<64><<<pool_grid, kThreads, 0, s>>>(p.q, p.k, p.seqlen, p.hq, p.hkv, p.block_size, nb, qbar,
                                                   kbar_t);
    launch_probs<64>(group, probs_grid, s, qbar, kbar_t, nb, p.hq, p.hkv, p.scale, part);
  }
  select_kernel<<<nb, kThreads, 0, s>>>(part, nb, p.hq, p.hkv, p.sink_blocks, p.tau, p.max_blocks, counts,
                                        cols_tmp);
  csr_kernel<<<nb, kThreads, 0, s>>>(counts, cols_tmp, nb, p.row_ptr, p.col_idx);
  return hipGetLastError();
}

}  // namespace flux
