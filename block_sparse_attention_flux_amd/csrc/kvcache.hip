// K/V cache writes for decode: the prompts' rows after prefill, and one new
// row per sequence at every decode step.
//
// The route is decided once at prefill and SA layers never read the rest of
// the history (technical summary on gist.science, section 2, deployment
// paragraph), so an SA layer's cache can hold just what its decode reads: the
// sink blocks and a ring of the last `local` blocks.  Compact layout per
// (sequence, kv head), block size B, s sink and w local blocks:
//   rows [0, s*B)            positions [0, s*B)        (sink)
//   rows [s*B, (s+w)*B)      position p >= s*B at s*B + p mod (w*B)   (ring)
// The decode mask row of a query at position N-1 covers blocks j < s and
// j >= (N-1)/B - w + 1, all within the last w*B positions or the sink, so no
// ring slot it needs has been overwritten.  A full cache keeps position p at
// row p.  Both kernels only move bytes (HBM-bound, 16-byte accesses).
#include "flux_device.h"
#include "flux_internal.h"

namespace flux {
namespace {

constexpr int kTokPerGroup = 32;  // prompt positions per workgroup (prefill store)

__device__ __forceinline__ int compact_row(int p, int B, int s, int w) {
  const int blk = p / B;
  return blk < s ? p : (s + blk % w) * B + p % B;
}

// Grid (ceil(max_seqlen / 32), n_req), 256 threads: the 32 positions of one
// request, every kv head, K then V; consecutive threads copy consecutive
// 16-byte chunks of a packed row.
__global__ __launch_bounds__(256) void kv_store_prefill_kernel(
    const u32x4* __restrict__ k, const u32x4* __restrict__ v, const int32_t* __restrict__ cu,
    int hkv, int ch, u32x4* __restrict__ kc, u32x4* __restrict__ vc, int cache_rows, int max_len,
    int compact, int B, int s, int w) {
  const int r = blockIdx.y;
  const int a = cu[r];
  const int S = cu[r + 1] - a;
  const int p0 = blockIdx.x * kTokPerGroup;
  if (p0 >= S) return;
  const int per_tok = hkv * ch;
  const int per_kv = kTokPerGroup * per_tok;
  const int keep_from = max(s * B, S - w * B);  // compact: first ring position kept
  for (int i = threadIdx.x; i < 2 * per_kv; i += blockDim.x) {
    const bool is_v = i >= per_kv;
    const int j = is_v ? i - per_kv : i;
    const int p = p0 + j / per_tok;
    const int g = (j % per_tok) / ch, c = j % ch;
    if (p >= S || p >= max_len) continue;
    int row = p;
    if (compact) {
      if (p >= s * B && p < keep_from) continue;  // overwritten before any decode reads it
      row = compact_row(p, B, s, w);
    }
    const size_t src = (static_cast<size_t>(a + p) * hkv + g) * ch + c;
    const size_t dst = ((static_cast<size_t>(r) * hkv + g) * cache_rows + row) * ch + c;
    if (is_v) vc[dst] = v[src]; else kc[dst] = k[src];
  }
}

// Grid (n_seq * hkv), 64 threads: row seqlens[b] - 1 of one (sequence, kv
// head), K by the first ch threads and V by the next ch.
__global__ __launch_bounds__(64) void kv_append_kernel(
    const u32x4* __restrict__ kn, const u32x4* __restrict__ vn, const int32_t* __restrict__ seqlens,
    int hkv, int ch, u32x4* __restrict__ kc, u32x4* __restrict__ vc, int cache_rows, int max_len,
    int compact, int B, int s, int w) {
  const int unit = blockIdx.x;
  const int p = seqlens[unit / hkv] - 1;
  if (p < 0 || p >= max_len) return;
  const int row = compact ? compact_row(p, B, s, w) : p;
  const size_t dst = (static_cast<size_t>(unit) * cache_rows + row) * ch;
  const size_t src = static_cast<size_t>(unit) * ch;
  const int t = threadIdx.x;
  if (t < ch) {
    kc[dst + t] = kn[src + t];
  } else if (t < 2 * ch) {
    vc[dst + t - ch] = vn[src + t - ch];
  }
}

}  // namespace

hipError_t launch_kv_store_prefill(const uint16_t* k, const uint16_t* v, const int32_t* cu_seqlens,
                                   int32_t n_req, int32_t max_seqlen, int32_t hkv, int32_t head_dim,
                                   uint16_t* k_cache, uint16_t* v_cache, int32_t cache_rows,
                                   int32_t max_len, int32_t compact, int32_t block_size,
                                   int32_t sink_blocks, int32_t local_blocks, hipStream_t s) {
  const dim3 grid((max_seqlen + kTokPerGroup - 1) / kTokPerGroup, n_req);
  kv_store_prefill_kernel<<<grid, 256, 0, s>>>(
      reinterpret_cast<const u32x4*>(k), reinterpret_cast<const u32x4*>(v), cu_seqlens, hkv,
      head_dim / 8, reinterpret_cast<u32x4*>(k_cache), reinterpret_cast<u32x4*>(v_cache), cache_rows,
      max_len, compact, block_size, sink_blocks, local_blocks);
  return hipGetLastError();
}

hipError_t launch_kv_append(const uint16_t* k_new, const uint16_t* v_new, const int32_t* seqlens,
                            int32_t n_seq, int32_t hkv, int32_t head_dim, uint16_t* k_cache,
                            uint16_t* v_cache, int32_t cache_rows, int32_t max_len, int32_t compact,
                            int32_t block_size, int32_t sink_blocks, int32_t local_blocks,
                            hipStream_t s) {
  kv_append_kernel<<<dim3(static_cast<uint32_t>(n_seq) * hkv), 64, 0, s>>>(
      reinterpret_cast<const u32x4*>(k_new), reinterpret_cast<const u32x4*>(v_new), seqlens, hkv,
      head_dim / 8, reinterpret_cast<u32x4*>(k_cache), reinterpret_cast<u32x4*>(v_cache), cache_rows,
      max_len, compact, block_size, sink_blocks, local_blocks);
  return hipGetLastError();
}

}  // namespace flux
