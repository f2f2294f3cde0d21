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
  float scale;
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
  float* part_o;   // [n_seq][hq][nsplit][head_dim]
  float* part_ml;  // [n_seq][hq][nsplit][2]
  int32_t n_seq, max_len, hq, hkv, head_dim, n_layers, layer, mask_blocks;
  int32_t block_size, nsplit;
  float scale;
};

hipError_t launch_build_mask(int32_t nb, int32_t sink, int32_t local, uint8_t* mask,
                             int32_t* row_ptr, int32_t* col_idx, hipStream_t s);

// Workspace of the router: pooled vectors then hidden layers, fp32.
size_t route_workspace_bytes(int32_t n_req, int32_t d_in, int32_t h1);
hipError_t launch_route(const void* hidden, int32_t bf16, const int32_t* cu, int32_t n_req,
                        int32_t d_in, const float* w1, const float* b1, int32_t h1,
                        const float* w2, const float* b2, int32_t n_layers, uint8_t* route,
                        float* logits, void* workspace, hipStream_t s);

hipError_t launch_prefill(const PrefillParams& p, hipStream_t s);

// Number of KV splits the decode kernel uses for these sizes.
int32_t decode_splits(int32_t n_seq, int32_t hkv, int32_t max_len);
hipError_t launch_decode(const DecodeParams& p, hipStream_t s);

}  // namespace flux
