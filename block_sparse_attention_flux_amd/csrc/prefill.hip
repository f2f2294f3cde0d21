// Routed prefill attention for gfx950: one kernel serves Full Attention (FA)
// and block-Sparse Attention (SA) layers; the layer's mode is read from the
// route vector on the device (Flux Attention abstract: a router sends each
// layer to FA or SA; technical summary on gist.science, section 2).
//
// Work decomposition
//   One workgroup = one query block of BM rows (BM = the mask block size, 64
//   or 128) of one query head of one request; BM/32 waves of 32 rows each.
//   Key tiles of BN = 64 keys.  FA visits every tile up to the diagonal; SA
//   visits only the tiles of the blocks listed in the query block's CSR row,
//   so inactive K/V tiles are never loaded.
//
// Per key tile and wave (bf16 MFMA v_mfma_f32_32x32x16_bf16, fp32 accumulate):
//   S^T[key][q] = K Q^T      A = K tile from LDS, B = Q kept in registers
//   online softmax in the log2 domain, row max across the two lane halves
//   O^T[d][q] += V^T P^T     A = V^T from LDS (stored transposed), B = P
//   Computing the transposed products puts one query row in each lane
//   (q = lane % 32), so the softmax statistics and the O rescale are per-lane
//   scalars and P lands directly in the B-operand layout of the second MFMA.
//
// The running max is only moved when it grows by more than 2^8 (the final
// normalisation divides by a sum taken with the same stale max, so the result
// is unchanged in exact arithmetic), which skips almost every O rescale.
//
// Staging: K/V tiles go global -> registers -> LDS, double buffered, with the
// loads of tile n+1 in flight while tile n is computed (one barrier per tile).
// Workgroups are ordered so that each XCD (own L2) works through whole KV
// head groups, heaviest causal rows first.
#include "flux_device.h"
#include "flux_internal.h"

namespace flux {
namespace {

constexpr int BN = 64;                 // keys per tile
constexpr float kRescaleSlack = 8.0f;  // log2 units the stale max may lag

template <int D>
struct Lds {
  static constexpr int KPITCH = D * 2 + 16;   // bytes per K row (pad: conflict-free reads)
  static constexpr int VPITCH = BN * 2 + 16;  // bytes per V^T row
  static constexpr int KBYTES = BN * KPITCH;
  static constexpr int VBYTES = D * VPITCH;
  static constexpr int STAGE = KBYTES + VBYTES;
};

// Position (in 4-key quads) of key quad kq inside a V^T row.  The B operand
// slot i of lane half h in k-step ks holds key 16ks + 8(i/4) + 4h + i%4 (the
// row order of the S^T accumulator); this permutation puts those 8 keys next
// to each other so the A operand is one 16-byte read.
__device__ __forceinline__ int quad_slot(int kq) {
  return (kq & ~3) | ((kq & 1) << 1) | ((kq >> 1) & 1);
}
// XOR swizzle of quad positions by the d-chunk (keeps 16-byte pairs intact).
__device__ __forceinline__ int quad_swz(int d) { return ((d >> 3) & 7) << 1; }

// bf16 element e (0 = low half, 1 = high half) of dwords a and b, packed as
// (a.e, b.e): one column of two consecutive key rows.
__device__ __forceinline__ uint32_t pick_pair(uint32_t a, uint32_t b, int e) {
  return e ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
}

template <int D, int BM>
__global__ __launch_bounds__(BM * 2, 2) void prefill_kernel(const PrefillParams p) {
  constexpr int NT = BM * 2;          // threads
  constexpr int KS = D / 16;          // k-steps of K Q^T
  constexpr int DT = D / 32;          // 32-row tiles of O^T
  constexpr int TPB = BM / BN;        // key tiles per mask block
  constexpr int CH = D / 8;           // 16-byte chunks per row
  constexpr int KLOADS = BN * CH / NT;
  constexpr int NQC = (BN / 4) * CH;  // (key quad, chunk) pairs of a V tile
  constexpr int VLOADS = (NQC + NT - 1) / NT;
  using L = Lds<D>;
  static_assert(BN * CH % NT == 0, "K tile must split evenly over the threads");

  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * L::STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;

  // ---- work item: XCD-major, then (kv group, query block heaviest first, request, head)
  const int group = p.hq / p.hkv;
  const int n_qt = (p.max_seqlen + BM - 1) / BM;
  const int G = gridDim.x, bid = blockIdx.x;
  int w = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
  const int hi = w % group;
  w /= group;
  const int req = w % p.n_req;
  w /= p.n_req;
  const int t = n_qt - 1 - (w % n_qt);
  const int g = w / n_qt;
  const int head = g * group + hi;

  const int tok0 = p.cu_seqlens[req];
  const int S = p.cu_seqlens[req + 1] - tok0;
  const int q0 = t * BM;
  if (q0 >= S) return;
  const int q_end = min(q0 + BM, S);
  const bool fa = p.route[static_cast<int64_t>(req) * p.n_layers + p.layer] != 0;

  int rp0 = 0, n_tiles;
  const int mrow = min(t, p.mask_blocks - 1);
  if (fa) {
    n_tiles = (q_end + BN - 1) / BN;
  } else {
    rp0 = p.row_ptr[mrow];
    n_tiles = max(p.row_ptr[mrow + 1] - rp0, 0) * TPB;
  }
  auto tile_start = [&](int n) -> int {
    if (fa) return n * BN;
    const int blk = min(max(p.col_idx[rp0 + n / TPB], 0), t);
    return blk * BM + (n % TPB) * BN;
  };
  if (!fa) {
    while (n_tiles > 0 && tile_start(n_tiles - 1) >= q_end) --n_tiles;
  }

  const size_t kv_row = static_cast<size_t>(p.hkv) * D;  // elements per token in k/v
  const uint16_t* kbase = p.k + static_cast<size_t>(tok0) * kv_row + static_cast<size_t>(g) * D;
  const uint16_t* vbase = p.v + static_cast<size_t>(tok0) * kv_row + static_cast<size_t>(g) * D;

  // ---- Q^T operand, kept in registers for the whole key loop
  const int row = q0 + wave * 32 + l32;
  const bool row_ok = row < S;
  bf16x8 qreg[KS];
  {
    const uint16_t* qp =
        p.q + (static_cast<size_t>(tok0 + (row_ok ? row : 0)) * p.hq + head) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = row_ok ? ld16(qp + ks * 16) : u32x4{0, 0, 0, 0};
      qreg[ks] = as_bf16x8(v);
    }
  }

  // ---- staging registers
  u32x4 kreg[KLOADS];
  u32x4 vreg[VLOADS][4];

  auto load_tile = [&](int ks0) {
#pragma unroll
    for (int j = 0; j < KLOADS; ++j) {
      const int id = tid + NT * j;
      const int r = id / CH, c = id % CH;
      const int key = ks0 + r;
      kreg[j] = key < S ? ld16(kbase + static_cast<size_t>(key) * kv_row + c * 8)
                        : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < VLOADS; ++j) {
      const int id = tid + NT * j;
      if (NQC % NT == 0 || id < NQC) {
        const int c = id % CH, qd = id / CH;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int key = ks0 + qd * 4 + kk;
          vreg[j][kk] = key < S ? ld16(vbase + static_cast<size_t>(key) * kv_row + c * 8)
                                : u32x4{0, 0, 0, 0};
        }
      }
    }
  };

  auto store_tile = [&](int stage) {
    unsigned char* kl = lds + stage * L::STAGE;
    unsigned char* vl = kl + L::KBYTES;
#pragma unroll
    for (int j = 0; j < KLOADS; ++j) {
      const int id = tid + NT * j;
      const int r = id / CH, c = id % CH;
      *reinterpret_cast<u32x4*>(kl + r * L::KPITCH + c * 16) = kreg[j];
    }
#pragma unroll
    for (int j = 0; j < VLOADS; ++j) {
      const int id = tid + NT * j;
      if (NQC % NT == 0 || id < NQC) {
        const int c = id % CH, qd = id / CH;
        const int slot = quad_slot(qd);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int d = c * 8 + i;
          const int dw = i >> 1;
          const uint32_t lo = pick_pair(vreg[j][0][dw], vreg[j][1][dw], i & 1);
          const uint32_t hi2 = pick_pair(vreg[j][2][dw], vreg[j][3][dw], i & 1);
          *reinterpret_cast<u32x2*>(vl + d * L::VPITCH + ((slot ^ quad_swz(d)) * 8)) =
              u32x2{lo, hi2};
        }
      }
    }
  };

  // ---- per-wave softmax state and output accumulator
  const float cs = p.scale * kLog2e;  // scores -> log2 domain
  float m_run = kNegInf, l_run = 0.0f;
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};

  const int wrow0 = q0 + wave * 32;
  const bool wave_live = wrow0 < S;

  auto compute_tile = [&](int stage, int kst) {
    if (!wave_live || kst > wrow0 + 31) return;  // nothing visible to this wave
    const unsigned char* kl = lds + stage * L::STAGE;
    const unsigned char* vl = kl + L::KBYTES;

    f32x16 sacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      sacc[mt] = f32x16{};
      const unsigned char* kp = kl + (mt * 32 + l32) * L::KPITCH + half * 16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(kp + ks * 32));
        sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ks], sacc[mt], 0, 0, 0);
      }
    }

    if (kst + BN - 1 > wrow0) {  // tile crosses the diagonal: causal mask
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kst + mt * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
          if (key > row) sacc[mt][r] = kNegInf;
        }
    }

    float mx = kNegInf;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[mt][r]);
    mx = fmaxf(mx, xor32(mx));
    const float mxs = mx * cs;
    // Rows whose max grew past the slack move their max; every other row keeps
    // it and scales by exactly 1, so each row's result depends on its own data
    // only.  The multiply is skipped when no row of the wave moved.
    const bool grow = mxs > m_run + kRescaleSlack;
    if (__ballot(grow) != 0) {
      const float m_new = grow ? mxs : m_run;
      const float alpha = !grow ? 1.0f : (m_run == kNegInf) ? 0.0f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
      m_run = m_new;
    }
    const float mu = (m_run == kNegInf) ? 0.0f : m_run;

    uint32_t pk[16];
    float psum = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(sacc[mt][r], cs, -mu));
        const float p1 = fast_exp2(__builtin_fmaf(sacc[mt][r + 1], cs, -mu));
        psum += p0 + p1;
        pk[mt * 8 + r / 2] = pack_bf16x2(p0, p1);
      }
    l_run += psum;

#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = dt * 32 + l32;
      const unsigned char* vp = vl + d * L::VPITCH;
      const int swz = quad_swz(d);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int u = ks * 4 + half * 2;
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(vp + (u ^ swz) * 8));
        const bf16x8 b = as_bf16x8(u32x4{pk[ks * 4], pk[ks * 4 + 1], pk[ks * 4 + 2], pk[ks * 4 + 3]});
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, oacc[dt], 0, 0, 0);
      }
    }
  };

  // ---- key loop: tile n computed from LDS while tile n+1 is in flight
  if (n_tiles > 0) {
    int kst = tile_start(0);
    load_tile(kst);
    store_tile(0);
    __syncthreads();
    for (int n = 0; n < n_tiles; ++n) {
      const bool more = n + 1 < n_tiles;
      const int kst_next = more ? tile_start(n + 1) : 0;
      if (more) load_tile(kst_next);
      compute_tile(n & 1, kst);
      if (more) store_tile((n + 1) & 1);
      __syncthreads();
      kst = kst_next;
    }
  }

  // ---- epilogue: O = O^T / l, one query row per lane, 4 consecutive d per store
  const float lt = l_run + xor32(l_run);
  if (row_ok) {
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    uint16_t* op = p.out + (static_cast<size_t>(tok0 + row) * p.hq + head) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = dt * 32 + j * 8 + half * 4;
        const uint32_t lo = pack_bf16x2(oacc[dt][j * 4] * inv, oacc[dt][j * 4 + 1] * inv);
        const uint32_t hi2 = pack_bf16x2(oacc[dt][j * 4 + 2] * inv, oacc[dt][j * 4 + 3] * inv);
        *reinterpret_cast<u32x2*>(op + d0) = u32x2{lo, hi2};
      }
  }
}

template <int D, int BM>
hipError_t launch_typed(const PrefillParams& p, hipStream_t s) {
  const int n_qt = (p.max_seqlen + BM - 1) / BM;
  const int64_t grid = static_cast<int64_t>(n_qt) * p.hq * p.n_req;
  prefill_kernel<D, BM><<<dim3(static_cast<uint32_t>(grid)), dim3(BM * 2), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t s) {
  if (p.head_dim == 128) {
    return p.block_size == 128 ? launch_typed<128, 128>(p, s) : launch_typed<128, 64>(p, s);
  }
  return p.block_size == 128 ? launch_typed<64, 128>(p, s) : launch_typed<64, 64>(p, s);
}

}  // namespace flux
