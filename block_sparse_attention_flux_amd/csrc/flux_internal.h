// Host-side launch entry points of the kernels (validated arguments only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace flux {

struct PrefillParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  const int32_t* cu_seqlens;
  const uint8_t* route;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  int32_t n_req, max_seqlen, hq, hkv, head_dim, n_layers, layer, mask_blocks;
  int32_t block_size, sink_blocks, local_blocks;
  int32_t route_heads;  // route decisions per (request, layer): 1, or hkv (one per kv head)
  const float* rsoft;   // non-null: soft-routed forward, weight of FA per (request, layer)
  float scale;
  int32_t* wq;          // non-null: balanced order, the caller's zeroed workspace (8 queue counters)
};

struct DecodeParams {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  uint16_t* out;
  const int32_t* seqlens;
  const uint8_t* route;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  float* part_o;   // [slots][hq / hkv][head_dim]  (partial of item slot, query column)
  float* part_ml;  // [slots][hq / hkv][2]         (its running max and sum)
  int2* plan;      // [n_seq * hkv]: (first slot, items) of each (sequence, kv head)
  int32_t n_seq, max_len, hq, hkv, head_dim, n_layers, layer, mask_blocks;
  int32_t block_size;
  int32_t slots;     // workgroups launched (work-item slots)
  int32_t balanced;  // 1: items sized by keys (decode_shape); 0: one item per unit
  int32_t target;    // items the plan aims at (decode_target)
  int32_t route_heads;                // route decisions per (sequence, layer): 1 or hkv
  int32_t cache_rows;                 // rows per (sequence, kv head) in the caches
  int32_t compact;                    // 1: SA cache of sink rows + a ring of window rows
  int32_t sink_blocks, local_blocks;  // the SA pattern (compact row mapping)
  float scale;
  // Append fused into the step (full caches only): the row of k_new/v_new
  // [n_seq][hkv][head_dim] goes to position seqlens[b] - 1 of k_write/v_write
  // (the caches), and the step reads that key from k_new/v_new.  Null: no append.
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_write;
  uint16_t* v_write;
};

// Route entry of (request r, layer, kv head g): route[r][layer] when one
// decision covers the layer, route[r][layer][g] when each kv head has its own.
__host__ __device__ inline int64_t route_index(int32_t r, int32_t n_layers, int32_t layer,
                                               int32_t route_heads, int32_t g) {
  return (static_cast<int64_t>(r) * n_layers + layer) * route_heads + (route_heads > 1 ? g : 0);
}

// Rows per (sequence, kv head) of a compact SA cache: sink + window blocks.
inline int64_t compact_rows(int32_t block_size, int32_t sink_blocks, int32_t local_blocks) {
  return static_cast<int64_t>(sink_blocks + local_blocks) * block_size;
}

// K/V cache writes (kvcache.hip).  Caches are [n_seq][hkv][cache_rows][d].
// store_prefill: rows of packed prompts k/v [T][hkv][d] (by cu_seqlens) at
// their positions; with compact set, only positions below sink*B and the
// last local*B positions of each prompt, at their compact rows.
hipError_t launch_kv_store_prefill(const uint16_t* k, const uint16_t* v, const int32_t* cu_seqlens,
                                   int32_t n_req, int32_t max_seqlen, int32_t hkv, int32_t head_dim,
                                   uint16_t* k_cache, uint16_t* v_cache, int32_t cache_rows,
                                   int32_t max_len, int32_t compact, int32_t block_size,
                                   int32_t sink_blocks, int32_t local_blocks, hipStream_t s);
// append: row of k_new/v_new [n_seq][hkv][d] at position seqlens[b] - 1.
hipError_t launch_kv_append(const uint16_t* k_new, const uint16_t* v_new, const int32_t* seqlens,
                            int32_t n_seq, int32_t hkv, int32_t head_dim, uint16_t* k_cache,
                            uint16_t* v_cache, int32_t cache_rows, int32_t max_len, int32_t compact,
                            int32_t block_size, int32_t sink_blocks, int32_t local_blocks,
                            hipStream_t s);

hipError_t launch_build_mask(int32_t nb, int32_t sink, int32_t local, uint8_t* mask,
                             int32_t* row_ptr, int32_t* col_idx, hipStream_t s);

// Content-aware mask (dynmask.hip): most key blocks per row (each thread of
// a 256-thread workgroup keeps up to 4 in registers, one probability per
// block in LDS).
constexpr int32_t kMaxDynBlocks = 1024;
struct DynMaskParams {
  const uint16_t* q;  // [seqlen][hq][d] bf16
  const uint16_t* k;  // [seqlen][hkv][d] bf16
  int32_t seqlen, hq, hkv, head_dim, block_size, sink_blocks, max_blocks;
  float scale, tau;
  int32_t* row_ptr;   // [nb + 1]
  int32_t* col_idx;   // capacity nb (nb + 1) / 2
  void* workspace;    // dynamic_mask_workspace_bytes
};
size_t dynamic_mask_workspace_bytes(int32_t seqlen, int32_t hq, int32_t hkv, int32_t head_dim,
                                    int32_t block_size);
hipError_t launch_dynamic_mask(const DynMaskParams& p, hipStream_t s);

// Workspace of the router: pooled vectors then hidden layers, fp32.
size_t route_workspace_bytes(int32_t n_req, int32_t d_in, int32_t h1);
hipError_t launch_route(const void* hidden, int32_t bf16, const int32_t* cu, int32_t n_req,
                        int32_t d_in, const float* w1, const float* b1, int32_t h1,
                        const float* w2, const float* b2, int32_t n_layers, uint8_t* route,
                        float* logits, void* workspace, hipStream_t s);

hipError_t launch_prefill(const PrefillParams& p, hipStream_t s);

// Decode work items.  Each (sequence, kv head) unit visits U keys (FA: the
// sequence's N keys; SA: its mask row's blocks); a call with at most
// kDecodePlanUnits units cuts them into about `target` items of equal size
// (at least kDecodeMinItemKeys keys each), planned on the device by every
// workgroup; larger calls take one item per unit.  The target is the number
// of split-kernel workgroups the GPU holds at once (one round), at most
// kDecodeMaxItems, which also sizes the workspace.
constexpr int32_t kDecodePlanUnits = 1024;
constexpr int32_t kDecodeMaxItems = 1024;
constexpr int32_t kDecodeMinItemKeys = 256;
struct DecodeShape {
  int64_t slots;     // workgroups to launch (an upper bound on the items)
  int32_t balanced;  // 1: keys-balanced items; 0: one item per unit
};
DecodeShape decode_shape(int32_t n_seq, int32_t hkv, int32_t max_len, int32_t target);
// Resident split-kernel workgroups on the device of `stream` (CUs times the
// kernel's occupancy), at most kDecodeMaxItems; queried once per device.
int32_t decode_target(hipStream_t stream, int32_t head_dim, bool append);
// Bytes of the decode workspace: partials of every slot, then the plan.
size_t decode_workspace_bytes(int32_t n_seq, int32_t hq, int32_t hkv, int32_t head_dim,
                              int32_t max_len);
hipError_t launch_decode(const DecodeParams& p, hipStream_t s);
// The decode scratch array of the device that `stream` belongs to (looked up
// once per device with hipGetSymbolAddress; allocates nothing).
constexpr size_t kDecodeScratchBytes = size_t(9) << 20;  // FLUX_DECODE_SCRATCH_BYTES
// The largest workspace a valid call needs: 1024 slots x 16 query heads per
// kv head x (128 + 2) floats, plus the plan of 1024 units.
static_assert(size_t(kDecodeMaxItems) * 16 * (128 + 2) * 4 + size_t(kDecodePlanUnits) * 8 <=
                  kDecodeScratchBytes,
              "the decode scratch must hold the largest workspace");
hipError_t decode_scratch(hipStream_t stream, void** ptr);

}  // namespace flux
