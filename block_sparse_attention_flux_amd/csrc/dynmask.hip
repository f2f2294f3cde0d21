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
// Three kernels: block means of Q and K (HBM-bound, one read of each);
// one workgroup per mask row for the probabilities and the selection (the
// candidate at sorted rank r is kept iff the mass of the r candidates ranked
// before it, plus the mandatory blocks' mass, is below tau: ranks come from
// pairwise comparisons, so no sort is needed); one workgroup per row for the
// CSR offsets (a sum over the earlier rows' counts) and the copy.
#include "flux_device.h"
#include "flux_internal.h"

namespace flux {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// (1) Mean of the rows of block i for one head of Q (y < hq) or K.  Thread t
// sums 16-byte chunk t % CH of rows t / CH, t / CH + RL, ...; the partial sums
// are added in LDS in a fixed order.
template <int D>
__global__ __launch_bounds__(kThreads) void pool_kernel(const uint16_t* __restrict__ q,
                                                        const uint16_t* __restrict__ k, int32_t S,
                                                        int32_t hq, int32_t hkv, int32_t B,
                                                        float* __restrict__ qbar, float* __restrict__ kbar) {
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
  for (int r = r0 + rl; r < r1; r += RL) {
    const u32x4 v = ld16(src + (static_cast<size_t>(r) * H + h) * D + c * 8);
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
    float* dst = is_q ? qbar : kbar;
    dst[(static_cast<size_t>(i) * H + h) * D + threadIdx.x] = s / static_cast<float>(r1 - r0);
  }
}

// Workgroup reductions over kThreads values per slot (n slots at once):
// lanes first (a fixed butterfly), then the waves in order.
template <int N>
__device__ __forceinline__ void block_reduce(float (&v)[N], int n, bool is_max, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int s = 0; s < n; ++s) {
    float x = v[s];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float y = __shfl_xor(x, o);
      x = is_max ? fmaxf(x, y) : x + y;
    }
    v[s] = x;
  }
  __syncthreads();
  if (lane == 0)
    for (int s = 0; s < n; ++s) red[wave * N + s] = v[s];
  __syncthreads();
  for (int s = 0; s < n; ++s) {
    float x = red[s];
    for (int w = 1; w < kWaves; ++w) x = is_max ? fmaxf(x, red[w * N + s]) : x + red[w * N + s];
    v[s] = x;
  }
}

// (2) One workgroup per query block i: P[i][0..i] and the selection.
template <int D>
__global__ __launch_bounds__(kThreads) void select_kernel(const float* __restrict__ qbar,
                                                          const float* __restrict__ kbar, int32_t nb,
                                                          int32_t hq, int32_t hkv, float scale,
                                                          int32_t sink, float tau, int32_t max_blocks,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ cols_tmp) {
  constexpr int kMaxH = kMaxDynHeads;
  __shared__ __attribute__((aligned(16))) float qs[kMaxH * D];  // scale * qbar[i][h]
  __shared__ float P[kMaxDynBlocks];
  __shared__ float red[kWaves * kMaxH];
  __shared__ float stat_m[kMaxH], stat_l[kMaxH];
  __shared__ int32_t scan[kWaves];

  const int i = blockIdx.x, n = i + 1, tid = threadIdx.x;
  const int group = hq / hkv;
  for (int e = tid; e < hq * D; e += kThreads) qs[e] = scale * qbar[static_cast<size_t>(i) * hq * D + e];
  __syncthreads();

  // logits of key block j for the query heads of KV head g, into z[0..group)
  auto logits = [&](int j, int g, float (&z)[16]) {
    const f32x4* kb = reinterpret_cast<const f32x4*>(kbar + (static_cast<size_t>(j) * hkv + g) * D);
    for (int hh = 0; hh < group; ++hh) z[hh] = 0.0f;
    for (int c4 = 0; c4 < D / 4; ++c4) {
      const f32x4 kv = kb[c4];
      for (int hh = 0; hh < group; ++hh) {
        const f32x4 qv = *reinterpret_cast<const f32x4*>(qs + (g * group + hh) * D + c4 * 4);
        z[hh] += qv[0] * kv[0] + qv[1] * kv[1] + qv[2] * kv[2] + qv[3] * kv[3];
      }
    }
  };

  // pass 1: per-head max over the causal key blocks; pass 2: per-head sum
  for (int pass = 0; pass < 2; ++pass) {
    float acc[kMaxH];
    for (int h = 0; h < hq; ++h) acc[h] = pass == 0 ? kNegInf : 0.0f;
    for (int j = tid; j < n; j += kThreads)
      for (int g = 0; g < hkv; ++g) {
        float z[16];
        logits(j, g, z);
        for (int hh = 0; hh < group; ++hh) {
          const int h = g * group + hh;
          acc[h] = pass == 0 ? fmaxf(acc[h], z[hh]) : acc[h] + fast_exp2((z[hh] - stat_m[h]) * kLog2e);
        }
      }
    block_reduce<kMaxH>(acc, hq, pass == 0, red);
    __syncthreads();
    if (tid == 0)
      for (int h = 0; h < hq; ++h) (pass == 0 ? stat_m : stat_l)[h] = acc[h];
    __syncthreads();
  }
  // pass 3: P[j] = mean over heads of the softmax
  const float inv_h = 1.0f / static_cast<float>(hq);
  for (int j = tid; j < n; j += kThreads) {
    float p = 0.0f;
    for (int g = 0; g < hkv; ++g) {
      float z[16];
      logits(j, g, z);
      for (int hh = 0; hh < group; ++hh) {
        const int h = g * group + hh;
        p += fast_exp2((z[hh] - stat_m[h]) * kLog2e) / stat_l[h];
      }
    }
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
        for (int kk = 0; kk < n; ++kk) {
          if (mandatory(kk)) continue;
          const float pk = P[kk];
          if (pk > pj || (pk == pj && kk < j)) {
            ++rank;
            before += pk;
          }
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

}  // namespace

size_t dynamic_mask_workspace_bytes(int32_t seqlen, int32_t hq, int32_t hkv, int32_t head_dim,
                                    int32_t block_size) {
  const size_t nb = (static_cast<size_t>(seqlen) + block_size - 1) / block_size;
  return (nb * hq * head_dim + nb * hkv * head_dim) * sizeof(float) + nb * sizeof(int32_t) +
         nb * nb * sizeof(int32_t);
}

hipError_t launch_dynamic_mask(const DynMaskParams& p, hipStream_t s) {
  const int nb = (p.seqlen + p.block_size - 1) / p.block_size;
  float* qbar = static_cast<float*>(p.workspace);
  float* kbar = qbar + static_cast<size_t>(nb) * p.hq * p.head_dim;
  int32_t* counts = reinterpret_cast<int32_t*>(kbar + static_cast<size_t>(nb) * p.hkv * p.head_dim);
  int32_t* cols_tmp = counts + nb;
  const dim3 pool_grid(nb, p.hq + p.hkv);
  if (p.head_dim == 128) {
    pool_kernel<128><<<pool_grid, kThreads, 0, s>>>(p.q, p.k, p.seqlen, p.hq, p.hkv, p.block_size, qbar, kbar);
    select_kernel<128><<<nb, kThreads, 0, s>>>(qbar, kbar, nb, p.hq, p.hkv, p.scale, p.sink_blocks, p.tau,
                                               p.max_blocks, counts, cols_tmp);
  } else {
    pool_kernel<64><<<pool_grid, kThreads, 0, s>>>(p.q, p.k, p.seqlen, p.hq, p.hkv, p.block_size, qbar, kbar);
    select_kernel<64><<<nb, kThreads, 0, s>>>(qbar, kbar, nb, p.hq, p.hkv, p.scale, p.sink_blocks, p.tau,
                                              p.max_blocks, counts, cols_tmp);
  }
  csr_kernel<<<nb, kThreads, 0, s>>>(counts, cols_tmp, nb, p.row_ptr, p.col_idx);
  return hipGetLastError();
}

}  // namespace flux
