// SA block mask builder: dense uint8 mask plus its CSR form, integer exact.
//
// Block (i, j) is active iff j <= i and (j < s or j >= i - w + 1): s sink
// blocks plus a causal window of w blocks ending at the diagonal.  The pages
// name block-sparse attention for SA layers (Flux Attention Qwen3-4B model
// card, "Sample Usage") and a minimal KV set that never touches the history
// (technical summary on gist.science, section 2); the sink + window pattern is
// the block pattern this library builds.
//
// One workgroup per mask row.  Row counts and row offsets come from closed
// forms, so rows are independent and no scan is needed.
#include "flux_device.h"
#include "flux_internal.h"

namespace flux {
namespace {

// Sum over rows i' < n of min(i'+1, w): the window part of the row counts.
__device__ __host__ inline int64_t window_prefix(int64_t n, int64_t w) {
  if (n <= w) return n * (n + 1) / 2;
  return w * (w + 1) / 2 + (n - w) * w;
}

// Sum over rows i' < n of max(0, min(s, i'-w+1)): sink blocks left of the window.
__device__ __host__ inline int64_t sink_prefix(int64_t n, int64_t s, int64_t w) {
  const int64_t t = n - w;  // rows whose window starts at block >= 1
  if (t <= 0 || s <= 0) return 0;
  if (t <= s) return t * (t + 1) / 2;
  return s * (s + 1) / 2 + (t - s) * s;
}

__global__ __launch_bounds__(256) void build_mask_kernel(int32_t nb, int32_t s, int32_t w,
                                                         uint8_t* __restrict__ mask,
                                                         int32_t* __restrict__ row_ptr,
                                                         int32_t* __restrict__ col_idx) {
  const int32_t i = blockIdx.x;
  const int32_t win_start = max(0, i - w + 1);
  const int32_t n_sink = max(0, min(s, i - w + 1));  // sink blocks outside the window
  const int32_t count = (i - win_start + 1) + n_sink;
  const int64_t base = window_prefix(i, w) + sink_prefix(i, s, w);
  if (threadIdx.x == 0) {
    row_ptr[i] = static_cast<int32_t>(base);
    if (i == nb - 1) row_ptr[nb] = static_cast<int32_t>(base + count);
  }
  for (int32_t e = threadIdx.x; e < count; e += blockDim.x) {
    const int32_t col = e < n_sink ? e : win_start + (e - n_sink);
    col_idx[base + e] = col;
  }
  if (mask != nullptr) {
    uint8_t* row = mask + static_cast<int64_t>(i) * nb;
    for (int32_t j = threadIdx.x; j < nb; j += blockDim.x) {
      const bool on = (j <= i) && (j < s || j >= i - w + 1);
      row[j] = on ? 1 : 0;
    }
  }
}

}  // namespace

hipError_t launch_build_mask(int32_t nb, int32_t sink, int32_t local, uint8_t* mask,
                             int32_t* row_ptr, int32_t* col_idx, hipStream_t s) {
  build_mask_kernel<<<dim3(nb), dim3(256), 0, s>>>(nb, sink, local, mask, row_ptr, col_idx);
  return hipGetLastError();
}

}  // namespace flux
