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
//   S^T[key][q] = K Q^T      A = K rows from LDS, B = Q kept in registers
//   online softmax in the log2 domain, row max across the two lane halves
//   O^T[d][q] += V^T P^T     A = V^T via the LDS transpose read, B = P
//   The transposed products put one query row in each lane (q = lane % 32),
//   so softmax statistics and the O rescale are per-lane scalars and P lands
//   directly in the B-operand layout of the second MFMA.
//
// Data movement
//   K and V tiles go global -> LDS directly (global_load_lds_dwordx4, no
//   register staging), row-major with the 16-byte chunks of each row XOR
//   swizzled; every LDS read below is bank-conflict free.  V^T operands come
//   from ds_read_b64_tr_b16: within each 16-lane group, destination lane
//   4i+j receives element j of source lanes i, i+4, i+8, i+12, so four source
//   lanes pointing at four keys deliver those keys' values of one d column.
//   K is fetched two tiles ahead and V one tile ahead (two LDS buffers each),
//   which lets the wave issue tile n+1's K Q^T MFMAs while it runs tile n's
//   softmax on the VALU.  One barrier per tile.
//
// The running max is only moved when a row's max grows by more than 2^8 (the
// final normalisation divides by a sum taken with the same stale max, so the
// result is unchanged in exact arithmetic); rows that do not move scale by
// exactly 1, so each row depends on its own data only.
//
// Workgroups are ordered so that each XCD (own L2) works through whole KV
// head groups, heaviest causal rows first.
#include "flux_device.h"
#include "flux_internal.h"

namespace flux {
namespace {

constexpr int BN = 64;                 // keys per tile
constexpr float kRescaleSlack = 8.0f;  // log2 units the stale max may lag

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// XOR swizzle of a row's 16-byte chunks: rows r..r+7 map a fixed chunk to 8
// different bank groups, and rows {4h+m} map a chunk pair to 8 distinct ones.
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

template <int D, int BM>
__global__ __launch_bounds__(BM * 2, 2) void prefill_kernel(const PrefillParams p) {
  constexpr int NT = BM * 2;           // threads
  constexpr int KS = D / 16;           // k-steps of K Q^T
  constexpr int DT = D / 32;           // 32-row tiles of O^T
  constexpr int TPB = BM / BN;         // key tiles per mask block
  constexpr int CH = D / 8;            // 16-byte chunks per row
  constexpr int ROWB = D * 2;          // bytes per K/V row in LDS
  constexpr int TILEB = BN * ROWB;     // bytes per K or V tile
  constexpr int LOADS = TILEB / (NT * 16);
  static_assert(TILEB % (NT * 16) == 0, "tile must split into whole wave loads");
  __shared__ __attribute__((aligned(16))) unsigned char lds_raw[4 * TILEB];  // K0 K1 V0 V1
  lds_u8* lds = (lds_u8*)(lds_raw);  // the same array, addressed as LDS

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

  // ---- global -> LDS tile loads: thread slot s = j*NT + tid holds row s/CH,
  // chunk slot s%CH, which stores global chunk (s%CH) ^ swz(row).
  const size_t kv_row = static_cast<size_t>(p.hkv) * D;  // elements per token in k/v
  const uint16_t* kbase = p.k + static_cast<size_t>(tok0) * kv_row + static_cast<size_t>(g) * D;
  const uint16_t* vbase = p.v + static_cast<size_t>(tok0) * kv_row + static_cast<size_t>(g) * D;
  int ld_row[LOADS], ld_col[LOADS];
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int s = j * NT + tid;
    ld_row[j] = s / CH;
    ld_col[j] = ((s % CH) ^ swz(s / CH)) * 8;
  }
  auto issue_tile = [&](const uint16_t* base, int kst, int buf) {
    lds_u8* dst0 = lds + buf * TILEB + wave * 64 * 16;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int key = min(kst + ld_row[j], S - 1);  // rows past the end: any finite row, masked later
      const uint16_t* src = base + static_cast<size_t>(key) * kv_row + ld_col[j];
      __builtin_amdgcn_global_load_lds(src, reinterpret_cast<lds_void*>(dst0 + j * NT * 16), 16, 0, 0);
    }
  };

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

  // per-lane operand coordinates
  //   K A operand: row key = mt*32 + l32, chunk 2ks + half
  //   V^T A operand (transpose read): source lane s = lane%16 points at key
  //   16ks + 8a + 4*half + s/4 and d = 32dt + 16*((lane/16)%2) + 4*(s%4)
  const int vt_key0 = 4 * half + ((lane & 15) >> 2);          // + 16ks + 8a
  const int vt_d0 = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // + 32dt

  const float cs = p.scale * kLog2e;  // scores -> log2 domain
  float m_run = kNegInf, l_run = 0.0f;
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};

  const int wrow0 = q0 + wave * 32;
  // tiles this wave must see: every tile up to the last one starting at or before its last row
  int n_mine = 0;
  if (wrow0 < S) {
    n_mine = n_tiles;
    while (n_mine > 0 && tile_start(n_mine - 1) > wrow0 + 31) --n_mine;
  }

  auto qk = [&](int kbuf, f32x16 (&sacc)[2]) {
    const lds_u8* kl = lds + kbuf * TILEB;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      sacc[mt] = f32x16{};
      const int key = mt * 32 + l32;
      const lds_u8* kp = kl + key * ROWB;
      const int sw = swz(key);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 raw = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
            kp + (((2 * ks + half) ^ sw) << 4));
        sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(raw), qreg[ks], sacc[mt], 0, 0, 0);
      }
    }
  };

  // softmax of one S^T tile -> packed bf16 P (B operand layout), updates m/l/O
  auto softmax = [&](f32x16 (&sacc)[2], int kst, uint32_t (&pk)[16]) {
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
  };

  auto vt_read = [&](const lds_u8* vl, int key, int d) -> s16x4 {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4*>(
        const_cast<lds_u8*>(vl) + key * ROWB + ((((d >> 3) ^ swz(key)) << 4) | ((d & 7) << 1))));
  };

  auto pv = [&](int vbuf, const uint32_t (&pk)[16]) {
    const lds_u8* vl = lds + (2 + vbuf) * TILEB;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 b = as_bf16x8(u32x4{pk[ks * 4], pk[ks * 4 + 1], pk[ks * 4 + 2], pk[ks * 4 + 3]});
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = dt * 32 + vt_d0;
        const s16x4 lo = vt_read(vl, ks * 16 + vt_key0, d);
        const s16x4 hi4 = vt_read(vl, ks * 16 + 8 + vt_key0, d);
        const s16x8 a8 = __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a8), b, oacc[dt],
                                                           0, 0, 0);
      }
    }
  };

  // ---- key loop.  Iteration n: loads of K_{n+2}, V_{n+1} in flight; S_{n+1}
  // computed while tile n's softmax runs; then O += V_n P_n.
  if (n_tiles > 0) {
    const int kst0 = tile_start(0);
    int kst_nxt = n_tiles > 1 ? tile_start(1) : 0;
    issue_tile(kbase, kst0, 0);
    issue_tile(vbase, kst0, 2);
    if (n_tiles > 1) issue_tile(kbase, kst_nxt, 1);
    wait_vmem();
    __syncthreads();
    f32x16 s_cur[2], s_nxt[2];
    if (n_mine > 0) qk(0, s_cur);
    int kst_cur = kst0;
    for (int n = 0; n < n_tiles; ++n) {
      const int kst_n2 = n + 2 < n_tiles ? tile_start(n + 2) : 0;
      if (n + 2 < n_tiles) issue_tile(kbase, kst_n2, n & 1);
      if (n + 1 < n_tiles) issue_tile(vbase, kst_nxt, 2 + ((n + 1) & 1));
      if (n < n_mine) {
        uint32_t pk[16];
        if (n + 1 < n_mine) qk((n + 1) & 1, s_nxt);
        softmax(s_cur, kst_cur, pk);
        pv(n & 1, pk);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) s_cur[mt] = s_nxt[mt];
      }
      wait_vmem();
      __syncthreads();
      kst_cur = kst_nxt;
      kst_nxt = kst_n2;
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
