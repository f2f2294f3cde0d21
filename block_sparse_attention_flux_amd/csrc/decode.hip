// Routed split-KV decode attention for gfx950.
//
// One new token per sequence; the route fixed at prefill is reused, and SA
// layers read only the keys of their mask row (sink blocks + local window),
// never the rest of the history (technical summary on gist.science,
// section 2, deployment paragraph).  Decode is bound by HBM bandwidth, so the
// design streams K/V rows once, for all query heads of a GQA group at a time:
//
//   grid      = (sequence, kv head, split); the keys a layer must visit (all
//               N keys for FA, the mask row's blocks for SA) are cut into
//               `nsplit` contiguous ranges of 32-key chunks;
//   each wave streams its own chunks: K rows go straight from HBM into the A
//               operand of v_mfma_f32_16x16x32_bf16 (S^T = K Q^T, the group's
//               query heads padded to 16 columns), V rows are transposed
//               through a wave-private LDS slice into the A operand of
//               O^T += V^T P^T; the next chunk's loads are issued before the
//               current chunk is computed;
//   the 4 waves of a workgroup merge their (max, sum, O) through LDS, and a
//               second small kernel merges the splits with the log-sum-exp
//               rule  O = sum_s 2^(m_s - m) o_s / sum_s 2^(m_s - m) l_s.
#include "flux_device.h"
#include "flux_internal.h"

namespace flux {
namespace {

constexpr int kWaves = 4;
constexpr int kChunk = 32;                  // keys per wave iteration
constexpr float kRescaleSlack = 8.0f;       // log2 units the stale max may lag
constexpr int kVtPitch = kChunk * 2 + 16;   // bytes per V^T row in LDS

// Position (in quads) of key quad kq = 4a + u inside a V^T row: 2u + a.  The
// B operand slot i of lane quarter u holds key 16(i/4) + 4u + i%4 (row order
// of the 16x16 S^T accumulator), so each lane's 8 keys become contiguous.
__device__ __forceinline__ int dquad_slot(int kq) { return ((kq & 3) << 1) | (kq >> 2); }
__device__ __forceinline__ int dquad_swz(int d) { return ((d >> 3) & 3) << 1; }

__device__ __forceinline__ uint32_t pick_pair(uint32_t a, uint32_t b, int e) {
  return e ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D>
__global__ __launch_bounds__(kWaves * 64, 2) void decode_split_kernel(const DecodeParams p) {
  constexpr int KSTEPS = D / 32;      // k-steps of K Q^T
  constexpr int DT = D / 16;          // 16-row tiles of O^T
  constexpr int CH = D / 8;           // 16-byte chunks per K/V row
  constexpr int VQC = (kChunk / 4) * CH / 64;  // (quad, chunk) pairs per lane
  static_assert((kChunk / 4) * CH % 64 == 0, "V chunk must split over a wave");
  constexpr int VT_BYTES = D * kVtPitch;       // one wave's V^T slice
  constexpr int MERGE_BYTES = kWaves * (16 * D + 32) * 4;
  constexpr int LDS_BYTES = kWaves * VT_BYTES > MERGE_BYTES ? kWaves * VT_BYTES : MERGE_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, quarter = lane >> 4;

  const int split = blockIdx.x % p.nsplit;
  const int unit = blockIdx.x / p.nsplit;
  const int b = unit / p.hkv, g = unit % p.hkv;
  const int group = p.hq / p.hkv;

  // The sequence length and the route byte do not depend on each other and
  // are read together; only an SA layer then reads its mask row (bounds, then
  // the first 64 columns, lane i keeping column i), so an FA layer's first
  // K/V loads wait on one round trip and an SA layer's on three.
  // (one gathered load: lane 0 the length, lane 1 the route byte; a compact
  // cache only holds an SA layer's rows and comes without a route)
  int gv = 0;
  if (lane == 0)
    gv = p.seqlens[b];
  else if (lane == 1 && !p.compact)
    gv = p.route[route_index(b, p.n_layers, p.layer, p.route_heads, g)];
  const int n_raw = __builtin_amdgcn_readlane(gv, 0);
  const bool fa = !p.compact && __builtin_amdgcn_readlane(gv, 1) != 0;
  const int N = min(max(n_raw, 1), p.max_len);
  const int B = p.block_size;
  const int mrow = min((N - 1) / B, p.mask_blocks - 1);
  int rp0 = 0, n_blk = 0, col_lane = 0;
  if (!fa) {
    rp0 = p.row_ptr[mrow];
    n_blk = max(p.row_ptr[mrow + 1] - rp0, 0);
    col_lane = lane < n_blk ? min(max(p.col_idx[rp0 + lane], 0), mrow) : 0;
  }
  const int U = fa ? N : n_blk * B;
  // contiguous range of visited-key indices for this split, chunk aligned
  const int per = ((U + p.nsplit - 1) / p.nsplit + kChunk - 1) / kChunk * kChunk;
  const int u0 = split * per;
  const int u1 = min(U, u0 + per);

  const size_t cache_head = static_cast<size_t>(p.cache_rows) * D;
  const uint16_t* kc = p.k_cache + (static_cast<size_t>(b) * p.hkv + g) * cache_head;
  const uint16_t* vc = p.v_cache + (static_cast<size_t>(b) * p.hkv + g) * cache_head;

  // first key position of the chunk that starts at visited index u (wave-uniform)
  auto chunk_key = [&](int u) -> int {
    if (fa) return u;
    const int bi = u / B;
    const int blk = bi < 64 ? __builtin_amdgcn_readlane(col_lane, bi) : min(max(p.col_idx[rp0 + bi], 0), mrow);
    return blk * B + u % B;
  };
  // cache row of key position k: the position itself in a full cache; in a
  // compact cache the sink rows come first and every later block has its
  // ring slot (block j at rows sink*B + (j % local)*B).  A 32-key chunk never
  // crosses a block, so its rows are consecutive either way.
  auto cache_row = [&](int k) -> int {
    if (!p.compact) return k;
    const int blk = k / B;
    return blk < p.sink_blocks ? k : (p.sink_blocks + blk % p.local_blocks) * B + k % B;
  };

  // ---- Q^T operand: column n = l16 is query head g*group + l16 (zero beyond the group)
  bf16x8 qreg[KSTEPS];
  {
    const bool ok = l16 < group;
    const uint16_t* qp = p.q + (static_cast<size_t>(b) * p.hq + g * group + (ok ? l16 : 0)) * D +
                         quarter * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      qreg[ks] = as_bf16x8(ok ? ld16(qp + ks * 32) : u32x4{0, 0, 0, 0});
  }

  const float cs = p.scale * kLog2e;
  float m_run = kNegInf, l_run = 0.0f;
  f32x4 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4{};

  unsigned char* vt = lds + wave * VT_BYTES;

  // Two register buffers (A/B) of one 32-key chunk each: [16-key tile][k-step]
  // for K, [(quad, chunk) pair][key in quad] for V.
  using KRegs = u32x4[2][KSTEPS];
  using VRegs = u32x4[VQC][4];

  // Loads of the 32-key chunk whose first visited index is u.  Keys at or
  // beyond `limit` read as zero, so masked keys contribute exactly nothing.
  // Every K/V row is read once per step: streaming (non-temporal) loads keep
  // it from displacing anything in the caches (11 % faster per step than
  // plain loads).
  auto load_chunk = [&](int u, KRegs& kr, VRegs& vr, int& k0, int& limit) {
    k0 = chunk_key(u);
    limit = min(k0 + min(u1 - u, kChunk), N);
    const int row0 = cache_row(k0) - k0;  // row of key k is row0 + k within this chunk
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int key = k0 + mt * 16 + l16;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
        kr[mt][ks] = key < limit ? ld16_stream(kc + static_cast<size_t>(row0 + key) * D + ks * 32 + quarter * 8)
                                 : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < VQC; ++j) {
      const int id = lane + 64 * j;
      const int c = id % CH, qd = id / CH;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int key = k0 + qd * 4 + kk;
        vr[j][kk] = key < limit ? ld16_stream(vc + static_cast<size_t>(row0 + key) * D + c * 8)
                                : u32x4{0, 0, 0, 0};
      }
    }
  };

  auto compute_chunk = [&](const KRegs& kr, const VRegs& vr, int k0, int limit) {
    // V^T into this wave's LDS slice
#pragma unroll
    for (int j = 0; j < VQC; ++j) {
      const int id = lane + 64 * j;
      const int c = id % CH, qd = id / CH;
      const int slot = dquad_slot(qd);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int d = c * 8 + i;
        const int dw = i >> 1;
        const uint32_t lo = pick_pair(vr[j][0][dw], vr[j][1][dw], i & 1);
        const uint32_t hi2 = pick_pair(vr[j][2][dw], vr[j][3][dw], i & 1);
        *reinterpret_cast<u32x2*>(vt + d * kVtPitch + ((slot ^ dquad_swz(d)) * 8)) = u32x2{lo, hi2};
      }
    }
    // S^T = K Q^T for two 16-key tiles
    f32x4 sacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      sacc[mt] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
        sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[mt][ks]), qreg[ks],
                                                           sacc[mt], 0, 0, 0);
    }
    // mask keys beyond the split / the sequence; lane holds keys 16mt + 4*quarter + r
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (k0 + mt * 16 + quarter * 4 + r >= limit) sacc[mt][r] = kNegInf;

    float mx = kNegInf;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[mt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
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
    uint32_t pk[4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(sacc[mt][r], cs, -mu));
        const float p1 = fast_exp2(__builtin_fmaf(sacc[mt][r + 1], cs, -mu));
        l_run += p0 + p1;
        pk[mt * 2 + r / 2] = pack_bf16x2(p0, p1);
      }
    const bf16x8 pb = as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]});
    wave_lds_sync();
    // O^T += V^T P^T, 16 rows of d at a time
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = dt * 16 + l16;
      const bf16x8 a = as_bf16x8(
          *reinterpret_cast<const u32x4*>(vt + d * kVtPitch + (((2 * quarter) ^ dquad_swz(d)) * 8)));
      oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, oacc[dt], 0, 0, 0);
    }
    wave_lds_sync();
  };

  // ---- stream this wave's chunks u = u0 + 32 * (wave + 4 * it), ping-ponging
  // two register buffers so the next chunk's loads overlap this chunk's math.
  {
    KRegs kA, kB;
    VRegs vA, vB;
    int k0A = 0, limA = 0, k0B = 0, limB = 0;
    int u = u0 + kChunk * wave;
    constexpr int kStride = kChunk * kWaves;
    if (u < u1) load_chunk(u, kA, vA, k0A, limA);
    while (u < u1) {
      if (u + kStride < u1) load_chunk(u + kStride, kB, vB, k0B, limB);
      compute_chunk(kA, vA, k0A, limA);
      u += kStride;
      if (u >= u1) break;
      if (u + kStride < u1) load_chunk(u + kStride, kA, vA, k0A, limA);
      compute_chunk(kB, vB, k0B, limB);
      u += kStride;
    }
  }

  // ---- merge the 4 waves: per query column n = l16 (valid n < group)
  // l_run is a per-lane partial over this lane's keys; sum the 4 quarters.
  float lsum = l_run + __shfl_xor(l_run, 16);
  lsum += __shfl_xor(lsum, 32);
  __syncthreads();  // V^T slices are dead; reuse LDS for the merge
  float* mo = reinterpret_cast<float*>(lds);            // [wave][16 q][D]
  float* mm = mo + kWaves * 16 * D;                     // [wave][16] max
  float* ml = mm + kWaves * 16;                         // [wave][16] sum
  if (l16 < group) {  // the padding columns of the MFMA tile are never read
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4*>(mo + (wave * 16 + l16) * D + dt * 16 + quarter * 4) = oacc[dt];
    if (quarter == 0) {
      mm[wave * 16 + l16] = m_run;
      ml[wave * 16 + l16] = lsum;
    }
  }
  __syncthreads();

  const int qn = tid / D;     // query column handled by this thread (several passes)
  const int dd = tid % D;
  for (int n = qn; n < group; n += (kWaves * 64) / D) {
    float m = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) m = fmaxf(m, mm[w * 16 + n]);
    float o = 0.0f, l = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = mm[w * 16 + n];
      const float sc = (mw == kNegInf) ? 0.0f : fast_exp2(mw - m);
      o += sc * mo[(w * 16 + n) * D + dd];
      l += sc * ml[w * 16 + n];
    }
    const int head = g * group + n;
    const size_t slot = (static_cast<size_t>(b) * p.hq + head) * p.nsplit + split;
    if (p.nsplit == 1) {
      const float val = l > 0.0f ? o / l : 0.0f;
      const uint32_t bits = pack_bf16x2(val, 0.0f);
      p.out[(static_cast<size_t>(b) * p.hq + head) * D + dd] = static_cast<uint16_t>(bits & 0xffffu);
    } else {
      p.part_o[slot * D + dd] = o;
      if (dd == 0) {
        p.part_ml[slot * 2] = m;
        p.part_ml[slot * 2 + 1] = l;
      }
    }
  }
}

// Merge the nsplit partials of one (sequence, head): one thread per d.  Up
// to kCombineBatch splits are read with all their loads in flight together
// (one memory round trip); the sum runs over the splits in order either way.
constexpr int kCombineBatch = 16;

template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(const DecodeParams p) {
  const int sh = blockIdx.x;  // b * hq + head
  const int dd = threadIdx.x;
  const int ns = p.nsplit;
  const float* ml = p.part_ml + static_cast<size_t>(sh) * ns * 2;
  const float* po = p.part_o + static_cast<size_t>(sh) * ns * D;
  float m = kNegInf, o = 0.0f, l = 0.0f;
  if (ns <= kCombineBatch) {
    float mv[kCombineBatch], lv[kCombineBatch], ov[kCombineBatch];
#pragma unroll
    for (int s = 0; s < kCombineBatch; ++s) {
      const bool ok = s < ns;
      mv[s] = ok ? ml[s * 2] : kNegInf;
      lv[s] = ok ? ml[s * 2 + 1] : 0.0f;
      ov[s] = ok ? po[static_cast<size_t>(s) * D + dd] : 0.0f;
    }
#pragma unroll
    for (int s = 0; s < kCombineBatch; ++s) m = fmaxf(m, mv[s]);
#pragma unroll
    for (int s = 0; s < kCombineBatch; ++s) {
      if (s < ns) {
        const float sc = (mv[s] == kNegInf) ? 0.0f : fast_exp2(mv[s] - m);
        o += sc * ov[s];
        l += sc * lv[s];
      }
    }
  } else {
    for (int s = 0; s < ns; ++s) m = fmaxf(m, ml[s * 2]);
    for (int s = 0; s < ns; ++s) {
      const float ms = ml[s * 2];
      const float sc = (ms == kNegInf) ? 0.0f : fast_exp2(ms - m);
      o += sc * po[static_cast<size_t>(s) * D + dd];
      l += sc * ml[s * 2 + 1];
    }
  }
  const float val = l > 0.0f ? o / l : 0.0f;
  p.out[static_cast<size_t>(sh) * D + dd] = static_cast<uint16_t>(pack_bf16x2(val, 0.0f) & 0xffffu);
}

template <int D>
hipError_t launch_typed(const DecodeParams& p, hipStream_t s) {
  const int64_t grid = static_cast<int64_t>(p.n_seq) * p.hkv * p.nsplit;
  decode_split_kernel<D><<<dim3(static_cast<uint32_t>(grid)), dim3(kWaves * 64), 0, s>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  decode_combine_kernel<D><<<dim3(static_cast<uint32_t>(p.n_seq * p.hq)), dim3(D), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

int32_t decode_splits(int32_t n_seq, int32_t hkv, int32_t max_len) {
  // Aim at ~1024 workgroups (4 per CU over 256 CUs) but keep >= 256 keys per split.
  const int64_t units = static_cast<int64_t>(n_seq) * hkv;
  int64_t s = (1024 + units - 1) / units;
  const int64_t cap = (static_cast<int64_t>(max_len) + 255) / 256;
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  return static_cast<int32_t>(s);
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t s) {
  return p.head_dim == 128 ? launch_typed<128>(p, s) : launch_typed<64>(p, s);
}

}  // namespace flux
