// extern "C" entry points of libflux: host-side validation, then dispatch to
// the kernels.  Declared and documented in include/flux.h.
#include "flux.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "flux_internal.h"

namespace {

bool sa_params_ok(const flux_sa_params& p) {
  return p.sink_blocks >= 0 && p.local_blocks >= 1;
}
bool block_supported(int32_t b) { return b == 64 || b == 128; }
bool head_dim_supported(int32_t d) { return d == 64 || d == 128; }

int64_t window_prefix(int64_t n, int64_t w) {
  return n <= w ? n * (n + 1) / 2 : w * (w + 1) / 2 + (n - w) * w;
}
int64_t sink_prefix(int64_t n, int64_t s, int64_t w) {
  const int64_t t = n - w;
  if (t <= 0 || s <= 0) return 0;
  return t <= s ? t * (t + 1) / 2 : s * (s + 1) / 2 + (t - s) * s;
}

flux_status from_hip(hipError_t e) { return e == hipSuccess ? FLUX_OK : FLUX_ERR_HIP; }

// Checks shared by prefill and decode.
flux_status check_attn_common(int32_t hq, int32_t hkv, int32_t head_dim, float scale,
                              const uint8_t* route, int32_t n_layers, int32_t layer,
                              const int32_t* row_ptr, const int32_t* col_idx,
                              int32_t mask_blocks, int32_t covered_len, flux_sa_params p) {
  if (route == nullptr || row_ptr == nullptr || col_idx == nullptr) return FLUX_ERR_INVALID_ARG;
  if (hq < 1 || hkv < 1 || hq % hkv != 0) return FLUX_ERR_INVALID_ARG;
  if (n_layers < 1 || layer < 0 || layer >= n_layers) return FLUX_ERR_INVALID_ARG;
  if (!(scale > 0.0f) || scale > 1e30f) return FLUX_ERR_INVALID_ARG;
  if (!sa_params_ok(p)) return FLUX_ERR_INVALID_ARG;
  if (!head_dim_supported(head_dim) || !block_supported(p.block_size)) return FLUX_ERR_UNSUPPORTED;
  if (hq / hkv > 16) return FLUX_ERR_UNSUPPORTED;
  const int64_t need = (static_cast<int64_t>(covered_len) + p.block_size - 1) / p.block_size;
  if (mask_blocks < need) return FLUX_ERR_INVALID_ARG;
  return FLUX_OK;
}

flux_status attn_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out,
                         const int32_t* cu_seqlens, int32_t n_req, int32_t max_seqlen, int32_t hq,
                         int32_t hkv, int32_t head_dim, float softmax_scale, const uint8_t* route,
                         int32_t n_layers, int32_t layer, const int32_t* mask_row_ptr,
                         const int32_t* mask_col_idx, int32_t mask_blocks, flux_sa_params p,
                         int32_t route_heads, const float* rsoft, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || cu_seqlens == nullptr)
    return FLUX_ERR_INVALID_ARG;
  if (workspace != nullptr &&
      (workspace_bytes < FLUX_PREFILL_WORKSPACE_BYTES || reinterpret_cast<uintptr_t>(workspace) % 16 != 0))
    return FLUX_ERR_WORKSPACE;
  if (out == q || out == k || out == v) return FLUX_ERR_INVALID_ARG;
  if (n_req < 1 || max_seqlen < 1) return FLUX_ERR_INVALID_ARG;
  const flux_status st = check_attn_common(hq, hkv, head_dim, softmax_scale, route, n_layers, layer,
                                           mask_row_ptr, mask_col_idx, mask_blocks, max_seqlen, p);
  if (st != FLUX_OK) return st;
  const int64_t n_qt = (static_cast<int64_t>(max_seqlen) + p.block_size - 1) / p.block_size;
  if (n_qt * hq * n_req > INT32_MAX) return FLUX_ERR_UNSUPPORTED;
  // K/V rows of one request are addressed with 32-bit byte offsets
  if (static_cast<int64_t>(max_seqlen) * hkv * head_dim * 2 > INT32_MAX) return FLUX_ERR_UNSUPPORTED;
  flux::PrefillParams pp{};
  pp.q = q; pp.k = k; pp.v = v; pp.out = out;
  pp.cu_seqlens = cu_seqlens; pp.route = route;
  pp.row_ptr = mask_row_ptr; pp.col_idx = mask_col_idx;
  pp.n_req = n_req; pp.max_seqlen = max_seqlen; pp.hq = hq; pp.hkv = hkv;
  pp.head_dim = head_dim; pp.n_layers = n_layers; pp.layer = layer;
  pp.mask_blocks = mask_blocks; pp.block_size = p.block_size;
  pp.sink_blocks = p.sink_blocks; pp.local_blocks = p.local_blocks;
  pp.scale = softmax_scale;
  pp.route_heads = route_heads;
  pp.rsoft = rsoft;
  // balanced order: one route decision per layer, whole XCD shares
  // (items % 8 == 0), at least one full round of the GPU's workgroups (768)
  // and room in a 32-bit grid for the extra items / 8
  const int64_t items = n_qt * hq * n_req;
  if (workspace != nullptr && route_heads == 1 && items % 8 == 0 && items >= 768 && items + items / 8 <= INT32_MAX)
    pp.wq = static_cast<int32_t*>(workspace);
  return from_hip(flux::launch_prefill(pp, static_cast<hipStream_t>(stream)));
}

// Work-item shape and workspace pointers of a decode call.  The workspace is
// needed (and checked) only when a call can have more items than units; it
// is sized for the largest item target, so it is checked before the device
// is queried for its own.  With use_scratch the device's scratch array stands
// in for the workspace (looked up only after every other check has passed).
flux_status decode_layout(int32_t n_seq, int32_t hq, int32_t hkv, int32_t head_dim, int32_t max_len,
                          void* workspace, size_t workspace_bytes, bool use_scratch, bool append,
                          void* stream, flux::DecodeParams* dp) {
  const flux::DecodeShape most = flux::decode_shape(n_seq, hkv, max_len, flux::kDecodeMaxItems);
  if (most.slots > INT32_MAX) return FLUX_ERR_UNSUPPORTED;
  const int64_t units = static_cast<int64_t>(n_seq) * hkv;
  const bool partials = most.slots > units;
  const size_t need = flux::decode_workspace_bytes(n_seq, hq, hkv, head_dim, max_len);
  if (use_scratch) {
    if (need > flux::kDecodeScratchBytes) return FLUX_ERR_WORKSPACE;
    workspace_bytes = flux::kDecodeScratchBytes;
    if (partials &&
        flux::decode_scratch(static_cast<hipStream_t>(stream), &workspace) != hipSuccess)
      return FLUX_ERR_HIP;
  }
  if (partials && (workspace == nullptr || workspace_bytes < need ||
                   reinterpret_cast<uintptr_t>(workspace) % 16 != 0))
    return FLUX_ERR_WORKSPACE;
  const int32_t target = flux::decode_target(static_cast<hipStream_t>(stream), head_dim, append);
  const flux::DecodeShape sh = flux::decode_shape(n_seq, hkv, max_len, target);
  const size_t n_part = static_cast<size_t>(most.slots) * (hq / hkv);
  float* ws = partials ? static_cast<float*>(workspace) : nullptr;
  dp->part_o = ws;
  dp->part_ml = ws != nullptr ? ws + n_part * head_dim : nullptr;
  dp->plan = ws != nullptr ? reinterpret_cast<int2*>(ws + n_part * (head_dim + 2)) : nullptr;
  dp->slots = static_cast<int32_t>(sh.slots);
  dp->balanced = sh.balanced;
  dp->target = target;
  return FLUX_OK;
}

flux_status attn_decode(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                        uint16_t* out, const int32_t* seqlens, int32_t n_seq, int32_t max_len,
                        int32_t hq, int32_t hkv, int32_t head_dim, float softmax_scale,
                        const uint8_t* route, int32_t n_layers, int32_t layer,
                        const int32_t* mask_row_ptr, const int32_t* mask_col_idx,
                        int32_t mask_blocks, flux_sa_params p, int32_t route_heads,
                        void* workspace, size_t workspace_bytes, void* stream,
                        bool use_scratch = false, const uint16_t* k_new = nullptr,
                        const uint16_t* v_new = nullptr, uint16_t* k_write = nullptr,
                        uint16_t* v_write = nullptr) {
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || out == nullptr ||
      seqlens == nullptr)
    return FLUX_ERR_INVALID_ARG;
  if (out == q) return FLUX_ERR_INVALID_ARG;
  if (n_seq < 1 || max_len < 1) return FLUX_ERR_INVALID_ARG;
  const flux_status st = check_attn_common(hq, hkv, head_dim, softmax_scale, route, n_layers, layer,
                                           mask_row_ptr, mask_col_idx, mask_blocks, max_len, p);
  if (st != FLUX_OK) return st;
  flux::DecodeParams dp{};
  const flux_status ws = decode_layout(n_seq, hq, hkv, head_dim, max_len, workspace,
                                       workspace_bytes, use_scratch, k_new != nullptr, stream, &dp);
  if (ws != FLUX_OK) return ws;
  dp.q = q; dp.k_cache = k_cache; dp.v_cache = v_cache; dp.out = out;
  dp.seqlens = seqlens; dp.route = route; dp.row_ptr = mask_row_ptr; dp.col_idx = mask_col_idx;
  dp.n_seq = n_seq; dp.max_len = max_len; dp.hq = hq; dp.hkv = hkv; dp.head_dim = head_dim;
  dp.n_layers = n_layers; dp.layer = layer; dp.mask_blocks = mask_blocks;
  dp.block_size = p.block_size; dp.scale = softmax_scale;
  dp.cache_rows = max_len; dp.compact = 0; dp.route_heads = route_heads;
  dp.sink_blocks = p.sink_blocks; dp.local_blocks = p.local_blocks;
  dp.k_new = k_new; dp.v_new = v_new; dp.k_write = k_write; dp.v_write = v_write;
  return from_hip(flux::launch_decode(dp, static_cast<hipStream_t>(stream)));
}

// Checks shared by the two cache writers; on success *rows is the cache's
// rows per (sequence, kv head).
flux_status check_cache(int32_t hkv, int32_t head_dim, int32_t max_len, int32_t compact,
                        flux_sa_params p, int32_t* rows) {
  if (hkv < 1 || max_len < 1 || (compact != 0 && compact != 1)) return FLUX_ERR_INVALID_ARG;
  if (!head_dim_supported(head_dim)) return FLUX_ERR_UNSUPPORTED;
  if (compact) {
    if (!sa_params_ok(p)) return FLUX_ERR_INVALID_ARG;
    if (!block_supported(p.block_size)) return FLUX_ERR_UNSUPPORTED;
    const int64_t r = flux::compact_rows(p.block_size, p.sink_blocks, p.local_blocks);
    if (r > INT32_MAX) return FLUX_ERR_UNSUPPORTED;
    *rows = static_cast<int32_t>(r);
  } else {
    *rows = max_len;
  }
  return FLUX_OK;
}

}  // namespace

extern "C" {

const char* flux_status_str(int32_t status) {
  switch (status) {
    case FLUX_OK: return "ok";
    case FLUX_ERR_INVALID_ARG: return "invalid argument";
    case FLUX_ERR_UNSUPPORTED: return "unsupported configuration";
    case FLUX_ERR_WORKSPACE: return "workspace missing or too small";
    case FLUX_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

size_t flux_route_workspace_size(int32_t n_req, int32_t d_in, int32_t h1) {
  if (n_req < 1 || d_in < 1 || h1 < 1) return 0;
  return flux::route_workspace_bytes(n_req, d_in, h1);
}

flux_status flux_route(const void* hidden, int32_t hidden_dtype, const int32_t* cu_seqlens,
                       int32_t n_req, int32_t d_in, const float* w1, const float* b1, int32_t h1,
                       const float* w2, const float* b2, int32_t n_layers, uint8_t* route_out,
                       float* logits_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (hidden == nullptr || cu_seqlens == nullptr || w1 == nullptr || b1 == nullptr ||
      w2 == nullptr || b2 == nullptr || route_out == nullptr)
    return FLUX_ERR_INVALID_ARG;
  if (hidden_dtype != FLUX_F32 && hidden_dtype != FLUX_BF16) return FLUX_ERR_INVALID_ARG;
  if (n_req < 1 || d_in < 1 || h1 < 1 || n_layers < 1) return FLUX_ERR_INVALID_ARG;
  if (d_in > 65536 || h1 > 65536 || n_layers > 65536) return FLUX_ERR_UNSUPPORTED;
  if (n_req > 65535) return FLUX_ERR_UNSUPPORTED;  // grid y dimension
  if (workspace == nullptr || workspace_bytes < flux::route_workspace_bytes(n_req, d_in, h1))
    return FLUX_ERR_WORKSPACE;
  return from_hip(flux::launch_route(hidden, hidden_dtype == FLUX_BF16, cu_seqlens, n_req, d_in,
                                     w1, b1, h1, w2, b2, n_layers, route_out, logits_out, workspace,
                                     static_cast<hipStream_t>(stream)));
}

int64_t flux_mask_blocks(int32_t seqlen, flux_sa_params p) {
  if (seqlen < 1 || p.block_size < 1) return FLUX_ERR_INVALID_ARG;
  return (static_cast<int64_t>(seqlen) + p.block_size - 1) / p.block_size;
}

int64_t flux_mask_nnz(int32_t seqlen, flux_sa_params p) {
  if (seqlen < 1 || p.block_size < 1 || !sa_params_ok(p)) return FLUX_ERR_INVALID_ARG;
  const int64_t nb = (static_cast<int64_t>(seqlen) + p.block_size - 1) / p.block_size;
  return window_prefix(nb, p.local_blocks) + sink_prefix(nb, p.sink_blocks, p.local_blocks);
}

flux_status flux_build_block_mask(int32_t seqlen, flux_sa_params p, uint8_t* mask_out,
                                  int32_t* row_ptr, int32_t* col_idx, void* stream) {
  if (row_ptr == nullptr || col_idx == nullptr) return FLUX_ERR_INVALID_ARG;
  if (seqlen < 1 || !sa_params_ok(p)) return FLUX_ERR_INVALID_ARG;
  if (!block_supported(p.block_size)) return FLUX_ERR_UNSUPPORTED;
  const int64_t nb = flux_mask_blocks(seqlen, p);
  if (nb > 65536) return FLUX_ERR_UNSUPPORTED;
  if (flux_mask_nnz(seqlen, p) > INT32_MAX) return FLUX_ERR_UNSUPPORTED;
  return from_hip(flux::launch_build_mask(static_cast<int32_t>(nb), p.sink_blocks, p.local_blocks,
                                          mask_out, row_ptr, col_idx,
                                          static_cast<hipStream_t>(stream)));
}

size_t flux_dynamic_mask_workspace_size(int32_t seqlen, int32_t hq, int32_t hkv, int32_t head_dim,
                                        int32_t block_size) {
  if (seqlen < 1 || hq < 1 || hkv < 1 || head_dim < 1 || block_size < 1) return 0;
  return flux::dynamic_mask_workspace_bytes(seqlen, hq, hkv, head_dim, block_size);
}

flux_status flux_build_block_mask_dynamic(const uint16_t* q, const uint16_t* k, int32_t seqlen,
                                          int32_t hq, int32_t hkv, int32_t head_dim,
                                          float softmax_scale, flux_dyn_params p, int32_t* row_ptr,
                                          int32_t* col_idx, int64_t col_capacity, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  if (q == nullptr || k == nullptr || row_ptr == nullptr || col_idx == nullptr)
    return FLUX_ERR_INVALID_ARG;
  if (seqlen < 1 || hq < 1 || hkv < 1 || hq % hkv != 0) return FLUX_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.0f) || softmax_scale > 1e30f) return FLUX_ERR_INVALID_ARG;
  if (!(p.tau >= 0.0f) || p.tau > 1e30f || p.sink_blocks < 0 || p.max_blocks < 0)
    return FLUX_ERR_INVALID_ARG;
  if (!head_dim_supported(head_dim) || !block_supported(p.block_size)) return FLUX_ERR_UNSUPPORTED;
  if (hq / hkv > 16) return FLUX_ERR_UNSUPPORTED;
  const int64_t nb = (static_cast<int64_t>(seqlen) + p.block_size - 1) / p.block_size;
  if (nb > flux::kMaxDynBlocks) return FLUX_ERR_UNSUPPORTED;
  if (col_capacity < nb * (nb + 1) / 2) return FLUX_ERR_INVALID_ARG;
  const size_t need = flux::dynamic_mask_workspace_bytes(seqlen, hq, hkv, head_dim, p.block_size);
  if (workspace == nullptr || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return FLUX_ERR_WORKSPACE;
  flux::DynMaskParams dp{};
  dp.q = q; dp.k = k; dp.seqlen = seqlen; dp.hq = hq; dp.hkv = hkv; dp.head_dim = head_dim;
  dp.block_size = p.block_size; dp.sink_blocks = p.sink_blocks; dp.max_blocks = p.max_blocks;
  dp.scale = softmax_scale; dp.tau = p.tau;
  dp.row_ptr = row_ptr; dp.col_idx = col_idx; dp.workspace = workspace;
  return from_hip(flux::launch_dynamic_mask(dp, static_cast<hipStream_t>(stream)));
}

flux_status flux_attn_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              uint16_t* out, const int32_t* cu_seqlens, int32_t n_req,
                              int32_t max_seqlen, int32_t hq, int32_t hkv, int32_t head_dim,
                              float softmax_scale, const uint8_t* route, int32_t n_layers,
                              int32_t layer, const int32_t* mask_row_ptr,
                              const int32_t* mask_col_idx, int32_t mask_blocks, flux_sa_params p,
                              void* workspace, size_t workspace_bytes, void* stream) {
  return attn_prefill(q, k, v, out, cu_seqlens, n_req, max_seqlen, hq, hkv, head_dim,
                      softmax_scale, route, n_layers, layer, mask_row_ptr, mask_col_idx,
                      mask_blocks, p, 1, nullptr, workspace, workspace_bytes, stream);
}

size_t flux_attn_prefill_workspace_size(void) { return FLUX_PREFILL_WORKSPACE_BYTES; }

flux_status flux_attn_prefill_heads(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                    uint16_t* out, const int32_t* cu_seqlens, int32_t n_req,
                                    int32_t max_seqlen, int32_t hq, int32_t hkv, int32_t head_dim,
                                    float softmax_scale, const uint8_t* route, int32_t n_layers,
                                    int32_t layer, const int32_t* mask_row_ptr,
                                    const int32_t* mask_col_idx, int32_t mask_blocks,
                                    flux_sa_params p, void* stream) {
  return attn_prefill(q, k, v, out, cu_seqlens, n_req, max_seqlen, hq, hkv, head_dim,
                      softmax_scale, route, n_layers, layer, mask_row_ptr, mask_col_idx,
                      mask_blocks, p, hkv, nullptr, nullptr, 0, stream);
}

flux_status flux_attn_prefill_soft(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   uint16_t* out, const int32_t* cu_seqlens, int32_t n_req,
                                   int32_t max_seqlen, int32_t hq, int32_t hkv, int32_t head_dim,
                                   float softmax_scale, const float* r_soft, int32_t n_layers,
                                   int32_t layer, const int32_t* mask_row_ptr,
                                   const int32_t* mask_col_idx, int32_t mask_blocks,
                                   flux_sa_params p, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  if (r_soft == nullptr) return FLUX_ERR_INVALID_ARG;
  // the weights take the route's place in the shared checks (the route itself is not read)
  return attn_prefill(q, k, v, out, cu_seqlens, n_req, max_seqlen, hq, hkv, head_dim,
                      softmax_scale, reinterpret_cast<const uint8_t*>(r_soft), n_layers, layer,
                      mask_row_ptr, mask_col_idx, mask_blocks, p, 1, r_soft, workspace,
                      workspace_bytes, stream);
}

size_t flux_attn_decode_workspace_size(int32_t n_seq, int32_t hq, int32_t hkv, int32_t head_dim,
                                       int32_t max_len) {
  if (n_seq < 1 || hq < 1 || hkv < 1 || head_dim < 1 || max_len < 1) return 0;
  if (hq % hkv != 0) return 0;
  return flux::decode_workspace_bytes(n_seq, hq, hkv, head_dim, max_len);
}

flux_status flux_attn_decode(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                             uint16_t* out, const int32_t* seqlens, int32_t n_seq,
                             int32_t max_len, int32_t hq, int32_t hkv, int32_t head_dim,
                             float softmax_scale, const uint8_t* route, int32_t n_layers,
                             int32_t layer, const int32_t* mask_row_ptr,
                             const int32_t* mask_col_idx, int32_t mask_blocks, flux_sa_params p,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return attn_decode(q, k_cache, v_cache, out, seqlens, n_seq, max_len, hq, hkv, head_dim,
                     softmax_scale, route, n_layers, layer, mask_row_ptr, mask_col_idx,
                     mask_blocks, p, 1, workspace, workspace_bytes, stream);
}

flux_status flux_attn_decode_noalloc(const uint16_t* q, const uint16_t* k_cache,
                                     const uint16_t* v_cache, uint16_t* out,
                                     const int32_t* seqlens, int32_t n_seq, int32_t max_len,
                                     int32_t hq, int32_t hkv, int32_t head_dim,
                                     float softmax_scale, const uint8_t* route, int32_t n_layers,
                                     int32_t layer, const int32_t* mask_row_ptr,
                                     const int32_t* mask_col_idx, int32_t mask_blocks,
                                     flux_sa_params p, void* stream) {
  // the device's scratch array stands in for the workspace; a call that needs
  // more than it holds returns FLUX_ERR_WORKSPACE
  return attn_decode(q, k_cache, v_cache, out, seqlens, n_seq, max_len, hq, hkv, head_dim,
                     softmax_scale, route, n_layers, layer, mask_row_ptr, mask_col_idx,
                     mask_blocks, p, 1, nullptr, 0, stream, true);
}

flux_status flux_attn_decode_append(const uint16_t* q, const uint16_t* k_new,
                                    const uint16_t* v_new, uint16_t* k_cache, uint16_t* v_cache,
                                    uint16_t* out, const int32_t* seqlens, int32_t n_seq,
                                    int32_t max_len, int32_t hq, int32_t hkv, int32_t head_dim,
                                    float softmax_scale, const uint8_t* route, int32_t n_layers,
                                    int32_t layer, const int32_t* mask_row_ptr,
                                    const int32_t* mask_col_idx, int32_t mask_blocks,
                                    flux_sa_params p, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  if (k_new == nullptr || v_new == nullptr) return FLUX_ERR_INVALID_ARG;
  if (k_new == k_cache || k_new == v_cache || v_new == k_cache || v_new == v_cache ||
      out == k_cache || out == v_cache || k_cache == v_cache)
    return FLUX_ERR_INVALID_ARG;
  return attn_decode(q, k_cache, v_cache, out, seqlens, n_seq, max_len, hq, hkv, head_dim,
                     softmax_scale, route, n_layers, layer, mask_row_ptr, mask_col_idx,
                     mask_blocks, p, 1, workspace, workspace_bytes, stream, false, k_new, v_new,
                     k_cache, v_cache);
}

flux_status flux_attn_decode_heads(const uint16_t* q, const uint16_t* k_cache,
                                   const uint16_t* v_cache, uint16_t* out, const int32_t* seqlens,
                                   int32_t n_seq, int32_t max_len, int32_t hq, int32_t hkv,
                                   int32_t head_dim, float softmax_scale, const uint8_t* route,
                                   int32_t n_layers, int32_t layer, const int32_t* mask_row_ptr,
                                   const int32_t* mask_col_idx, int32_t mask_blocks,
                                   flux_sa_params p, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  return attn_decode(q, k_cache, v_cache, out, seqlens, n_seq, max_len, hq, hkv, head_dim,
                     softmax_scale, route, n_layers, layer, mask_row_ptr, mask_col_idx,
                     mask_blocks, p, hkv, workspace, workspace_bytes, stream);
}

int64_t flux_kv_rows(int32_t max_len, flux_sa_params p, int32_t compact) {
  if (max_len < 1 || (compact != 0 && compact != 1)) return FLUX_ERR_INVALID_ARG;
  if (!compact) return max_len;
  if (!sa_params_ok(p) || p.block_size < 1) return FLUX_ERR_INVALID_ARG;
  return flux::compact_rows(p.block_size, p.sink_blocks, p.local_blocks);
}

flux_status flux_kv_store_prefill(const uint16_t* k, const uint16_t* v, const int32_t* cu_seqlens,
                                  int32_t n_req, int32_t max_seqlen, int32_t hkv, int32_t head_dim,
                                  uint16_t* k_cache, uint16_t* v_cache, int32_t max_len,
                                  int32_t compact, flux_sa_params p, void* stream) {
  if (k == nullptr || v == nullptr || cu_seqlens == nullptr || k_cache == nullptr ||
      v_cache == nullptr)
    return FLUX_ERR_INVALID_ARG;
  if (n_req < 1 || max_seqlen < 1 || max_seqlen > max_len) return FLUX_ERR_INVALID_ARG;
  int32_t rows = 0;
  const flux_status st = check_cache(hkv, head_dim, max_len, compact, p, &rows);
  if (st != FLUX_OK) return st;
  if (n_req > 65535) return FLUX_ERR_UNSUPPORTED;  // grid y dimension
  return from_hip(flux::launch_kv_store_prefill(k, v, cu_seqlens, n_req, max_seqlen, hkv, head_dim,
                                                k_cache, v_cache, rows, max_len, compact,
                                                p.block_size, p.sink_blocks, p.local_blocks,
                                                static_cast<hipStream_t>(stream)));
}

flux_status flux_kv_append(const uint16_t* k_new, const uint16_t* v_new, const int32_t* seqlens,
                           int32_t n_seq, int32_t hkv, int32_t head_dim, uint16_t* k_cache,
                           uint16_t* v_cache, int32_t max_len, int32_t compact, flux_sa_params p,
                           void* stream) {
  if (k_new == nullptr || v_new == nullptr || seqlens == nullptr || k_cache == nullptr ||
      v_cache == nullptr)
    return FLUX_ERR_INVALID_ARG;
  if (n_seq < 1) return FLUX_ERR_INVALID_ARG;
  int32_t rows = 0;
  const flux_status st = check_cache(hkv, head_dim, max_len, compact, p, &rows);
  if (st != FLUX_OK) return st;
  if (static_cast<int64_t>(n_seq) * hkv > INT32_MAX) return FLUX_ERR_UNSUPPORTED;
  return from_hip(flux::launch_kv_append(k_new, v_new, seqlens, n_seq, hkv, head_dim, k_cache,
                                         v_cache, rows, max_len, compact, p.block_size,
                                         p.sink_blocks, p.local_blocks,
                                         static_cast<hipStream_t>(stream)));
}

flux_status flux_attn_decode_sa_compact(const uint16_t* q, const uint16_t* k_cache,
                                        const uint16_t* v_cache, uint16_t* out,
                                        const int32_t* seqlens, int32_t n_seq, int32_t max_len,
                                        int32_t hq, int32_t hkv, int32_t head_dim,
                                        float softmax_scale, const int32_t* mask_row_ptr,
                                        const int32_t* mask_col_idx, int32_t mask_blocks,
                                        flux_sa_params p, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || out == nullptr ||
      seqlens == nullptr)
    return FLUX_ERR_INVALID_ARG;
  if (out == q) return FLUX_ERR_INVALID_ARG;
  if (n_seq < 1 || max_len < 1) return FLUX_ERR_INVALID_ARG;
  static const uint8_t kSa = 0;  // route placeholder for the shared checks (never read)
  const flux_status st = check_attn_common(hq, hkv, head_dim, softmax_scale, &kSa, 1, 0,
                                           mask_row_ptr, mask_col_idx, mask_blocks, max_len, p);
  if (st != FLUX_OK) return st;
  int32_t rows = 0;
  const flux_status sc = check_cache(hkv, head_dim, max_len, 1, p, &rows);
  if (sc != FLUX_OK) return sc;
  flux::DecodeParams dp{};
  const flux_status ws = decode_layout(n_seq, hq, hkv, head_dim, max_len, workspace,
                                       workspace_bytes, false, false, stream, &dp);
  if (ws != FLUX_OK) return ws;
  dp.q = q; dp.k_cache = k_cache; dp.v_cache = v_cache; dp.out = out;
  dp.seqlens = seqlens; dp.route = nullptr; dp.row_ptr = mask_row_ptr; dp.col_idx = mask_col_idx;
  dp.n_seq = n_seq; dp.max_len = max_len; dp.hq = hq; dp.hkv = hkv; dp.head_dim = head_dim;
  dp.n_layers = 1; dp.layer = 0; dp.mask_blocks = mask_blocks;
  dp.block_size = p.block_size; dp.scale = softmax_scale;
  dp.cache_rows = rows; dp.compact = 1; dp.route_heads = 1;
  dp.sink_blocks = p.sink_blocks; dp.local_blocks = p.local_blocks;
  return from_hip(flux::launch_decode(dp, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
