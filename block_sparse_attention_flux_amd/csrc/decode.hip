// Routed split-KV decode attention for gfx950.
//
// One new token per sequence; the route fixed at prefill is reused, and SA
// layers read only the keys of their mask row (sink blocks + local window),
// never the rest of the history (technical summary on gist.science,
// section 2, deployment paragraph).  Decode is bound by HBM bandwidth, so the
// design streams K/V rows once, for all query heads of a GQA group at a time:
//
//   work list = every (sequence, kv head) unit visits U keys (all N keys for
//               FA, the mask row's blocks for SA); the units are cut into
//               work items of about the same number of keys (as many items
//               as the GPU holds split workgroups at once, at least 256 keys
//               each), so a long FA sequence beside short SA ones gets
//               proportionally more items.  Each
//               workgroup plans the whole call itself (every unit's U, its
//               share of the items, one block-wide prefix sum) and takes item
//               blockIdx.x: the plan costs no extra launch;
//   each wave streams its own chunks: K rows go straight from HBM into the A
//               operand of v_mfma_f32_16x16x32_bf16 (S^T = K Q^T, the group's
//               query heads padded to 16 columns), V rows are transposed
//               through a wave-private LDS slice into the A operand of
//               O^T += V^T P^T; the next chunk's loads are issued before the
//               current chunk is computed;
//   the 4 waves of a workgroup merge their (max, sum, O) through LDS, and a
//               second small kernel merges the splits with the log-sum-exp
//               rule  O = sum_s 2^(m_s - m) o_s / sum_s 2^(m_s - m) l_s.
#include <mutex>

#include "flux_device.h"
#include "flux_internal.h"

namespace flux {
namespace {

// Device-resident scratch of flux_attn_decode_noalloc: the same partials
// and plan as a caller's workspace, for callers that cannot allocate.  One
// copy per GPU, held until the process ends; its host-side name is not a
// device address, so host code uses only the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

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

// One work item: keys [u0, u1) of the visited-key list of unit (b, g), item
// j of the unit's s items (all values wave-uniform).
struct DecodeItem {
  int b, g, j, s, N, fa, mrow, rp0, n_blk, u0, u1;
  int app;  // a new row is appended at N - 1 (seqlens[b] in [1, max_len])
};

// The unit's length, route and mask row, clamped into range: N in
// [1, max_len], columns at most the row's own, at most mrow + 1 blocks.
struct UnitKeys {
  int N, fa, mrow, rp0, n_blk, U;
};

constexpr int kPlanPerThread = kDecodePlanUnits / (kWaves * 64);  // units per thread in the plan
static_assert(kPlanPerThread * kWaves * 64 == kDecodePlanUnits, "plan units must fill the workgroup");

// Balanced plan, computed by every workgroup for the whole call.  Thread t
// owns units [4t, 4t + 4) (unit u = b * hkv + g).  With `total` the keys of
// all units, `target` the split workgroups the GPU holds at once and
// T = ceil(total / (target - n_units / 2)), unit u gets
//   s_u = max(1, min(ceil(U_u / T), floor(U_u / 256)))
// items of about U_u / s_u <= T keys each (chunk aligned), in consecutive
// slots after those of the units before it: every item holds about the same
// number of keys, and a call of equal units has exactly `target` items (one
// round of the resident workgroups).  Returns false when no unit owns item
// blockIdx.x.  Workgroup 0 also records (first slot, items) per unit for the
// combine kernel.
__device__ bool plan_balanced(const DecodeParams& p, int tid, int lane, int wave, double* tot_sh,
                              int* cnt_sh, int* item_sh, DecodeItem& it) {
  constexpr int K = kPlanPerThread;
  const int n_units = p.n_seq * p.hkv;
  const int B = p.block_size;
  const int u_first = tid * K;
  // round trip 1: lengths and route bytes of this thread's units
  int nraw[K], rbyte[K];
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const int u = u_first + i;
    nraw[i] = 1;
    rbyte[i] = 0;
    if (u < n_units) {
      const int b = u / p.hkv, g = u - b * p.hkv;
      nraw[i] = p.seqlens[b];
      if (!p.compact) rbyte[i] = p.route[route_index(b, p.n_layers, p.layer, p.route_heads, g)];
    }
  }
  // round trip 2: mask row bounds of the SA units
  UnitKeys uk[K];
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const int u = u_first + i;
    uk[i].N = min(max(nraw[i], 1), p.max_len);
    uk[i].fa = !p.compact && rbyte[i] != 0;
    uk[i].mrow = min((uk[i].N - 1) / B, p.mask_blocks - 1);
    uk[i].rp0 = 0;
    uk[i].n_blk = 0;
    if (u < n_units && !uk[i].fa) {
      uk[i].rp0 = p.row_ptr[uk[i].mrow];
      uk[i].n_blk = p.row_ptr[uk[i].mrow + 1];
    }
  }
  double keys = 0.0;  // exact: fewer than 2^53 keys
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const int u = u_first + i;
    uk[i].n_blk = min(max(uk[i].n_blk - uk[i].rp0, 0), uk[i].mrow + 1);
    uk[i].U = u >= n_units ? 0 : uk[i].fa ? uk[i].N : uk[i].n_blk * B;
    keys += static_cast<double>(uk[i].U);
  }
  // all keys of the call
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) keys += __shfl_xor(keys, o);
  if (lane == 0) tot_sh[wave] = keys;
  if (tid == 0) item_sh[0] = -1;
  __syncthreads();
  double total = 0.0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) total += tot_sh[w];
  // items per unit when about `target` items share the keys: items of at
  // most T = ceil(total / target) keys, i.e. s_u = ceil(U_u / T) (at least
  // one, never below 256 keys each).  total / target is correctly rounded
  // and a non-integer quotient lies at least 1 / target >= 2^-10 from every
  // integer, while rounding moves it by at most 2^-12 (total < 2^41): the
  // ceiling of the double quotient is the exact ceiling.
  int sv[K];
  auto shares = [&](int target) {
    const double q = __builtin_ceil(total / static_cast<double>(target));
    const uint32_t T = q < 2147483647.0 ? max(static_cast<uint32_t>(q), 1u) : 2147483647u;
    int mine = 0;
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const int u = u_first + i;
      const uint32_t U = static_cast<uint32_t>(uk[i].U);
      const int by_size = static_cast<int>((U + T - 1) / T);
      sv[i] = u >= n_units ? 0 : max(1, min(by_size, uk[i].U / kDecodeMinItemKeys));
      mine += sv[i];
    }
    return mine;
  };
  // block-wide exclusive prefix of the item counts (threads in unit order);
  // returns the thread's first slot, `all` gets the call's item count
  auto prefix = [&](int mine, int* sh, int& all) {
    int x = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) sh[wave] = x;
    __syncthreads();
    int first = x - mine;
    all = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int c = sh[w];
      if (w < wave) first += c;
      all += c;
    }
    return first;
  };
  // Rounding each unit up adds half an item per unit on average, so the first
  // pass aims at target - n_units / 2 items.  If the count passes the grid
  // (p.slots workgroups, at least min(target, n_units + max keys / 256)), the
  // second pass aims at target - n_units: sum ceil(U_u / T) <= total / T +
  // n_units <= target.
  int all = 0;
  int first = prefix(shares(max(p.target - n_units / 2, 1)), cnt_sh, all);
  if (all > p.slots) first = prefix(shares(max(p.target - n_units, 1)), cnt_sh + kWaves, all);
  const int item = blockIdx.x;
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const int u = u_first + i;
    if (u < n_units) {
      if (item >= first && item < first + sv[i]) {
        const int b = u / p.hkv;
        item_sh[0] = b;
        item_sh[1] = u - b * p.hkv;
        item_sh[2] = item - first;
        item_sh[3] = sv[i];
        item_sh[4] = uk[i].N;
        item_sh[5] = uk[i].fa;
        item_sh[6] = uk[i].mrow;
        item_sh[7] = uk[i].rp0;
        item_sh[8] = uk[i].n_blk;
        item_sh[9] = uk[i].U;
        item_sh[10] = nraw[i] >= 1 && nraw[i] <= p.max_len;
      }
      if (blockIdx.x == 0 && p.plan != nullptr) p.plan[u] = int2{first, sv[i]};
    }
    first += sv[i];
  }
  __syncthreads();
  it.b = __builtin_amdgcn_readfirstlane(item_sh[0]);
  if (it.b < 0) return false;
  it.g = __builtin_amdgcn_readfirstlane(item_sh[1]);
  it.j = __builtin_amdgcn_readfirstlane(item_sh[2]);
  it.s = __builtin_amdgcn_readfirstlane(item_sh[3]);
  it.N = __builtin_amdgcn_readfirstlane(item_sh[4]);
  it.fa = __builtin_amdgcn_readfirstlane(item_sh[5]);
  it.mrow = __builtin_amdgcn_readfirstlane(item_sh[6]);
  it.rp0 = __builtin_amdgcn_readfirstlane(item_sh[7]);
  it.n_blk = __builtin_amdgcn_readfirstlane(item_sh[8]);
  const int U = __builtin_amdgcn_readfirstlane(item_sh[9]);
  it.app = p.k_new != nullptr && __builtin_amdgcn_readfirstlane(item_sh[10]) != 0;
  // contiguous, chunk-aligned range of the unit's visited keys
  const int per = ((U + it.s - 1) / it.s + kChunk - 1) / kChunk * kChunk;
  it.u0 = it.j * per;
  it.u1 = min(U, it.u0 + per);
  return true;
}

// One item per unit (calls with more units than the plan holds): the unit's
// length and route byte in one gathered load, then, for SA, its mask row.
__device__ __forceinline__ void plan_one_per_unit(const DecodeParams& p, int lane, DecodeItem& it) {
  const int unit = blockIdx.x;
  it.b = unit / p.hkv;
  it.g = unit - it.b * p.hkv;
  int gv = 0;
  if (lane == 0)
    gv = p.seqlens[it.b];
  else if (lane == 1 && !p.compact)
    gv = p.route[route_index(it.b, p.n_layers, p.layer, p.route_heads, it.g)];
  const int n_raw = __builtin_amdgcn_readlane(gv, 0);
  it.fa = !p.compact && __builtin_amdgcn_readlane(gv, 1) != 0;
  it.N = min(max(n_raw, 1), p.max_len);
  it.app = p.k_new != nullptr && n_raw >= 1 && n_raw <= p.max_len;
  it.mrow = min((it.N - 1) / p.block_size, p.mask_blocks - 1);
  it.rp0 = 0;
  it.n_blk = 0;
  if (!it.fa) {
    it.rp0 = p.row_ptr[it.mrow];
    it.n_blk = min(max(p.row_ptr[it.mrow + 1] - it.rp0, 0), it.mrow + 1);
  }
  it.j = 0;
  it.s = 1;
  it.u0 = 0;
  it.u1 = it.fa ? it.N : it.n_blk * p.block_size;
}

// APPEND: the step also appends the new K/V row (DecodeParams::k_new); a
// separate instantiation, so the plain decode carries none of its code.
template <int D, bool APPEND>
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
  const int group = p.hq / p.hkv;
  __shared__ double plan_keys[kWaves];  // the plan's per-wave key sums
  __shared__ int plan_cnt[2 * kWaves];  // ... and item counts (two passes at most)
  __shared__ int plan_item[11];         // the item this workgroup takes

  // The plan reads every unit's length and route byte in one round trip and
  // the SA units' mask-row bounds in a second; the item's SA columns (first
  // 64, lane i keeping column i) come in a third.  An item's first K/V loads
  // therefore wait on two or three round trips.  (A plan made by every wave
  // on its own, with no LDS or barrier, measured slower: 4 us per SA layer.)
  DecodeItem it;
  if (p.balanced) {
    if (!plan_balanced(p, tid, lane, wave, plan_keys, plan_cnt, plan_item, it)) return;
  } else {
    plan_one_per_unit(p, lane, it);
  }
  const int b = it.b, g = it.g;
  const bool fa = it.fa != 0;
  const int N = it.N;
  const int B = p.block_size;
  const int mrow = it.mrow;
  const int rp0 = it.rp0, n_blk = it.n_blk;
  const int col_lane = (!fa && lane < n_blk) ? min(max(p.col_idx[rp0 + lane], 0), mrow) : 0;
  const int u0 = it.u0, u1 = it.u1;

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

  // Fused append: the new row goes to cache row N - 1 before anything reads
  // it.  The one wave that visits key N - 1 (FA: visited index N - 1; SA:
  // inside the row's last block when that is the diagonal block) stores the
  // row and waits for its own store, so its later load of that row sees it
  // (no other item and no other wave reads row N - 1).  When no wave visits
  // it, wave 0 of the unit's last item stores it.
  if constexpr (APPEND) {
    if (it.app) {
      int vi = -1;  // visited index of key N - 1, or -1
      if (fa) {
        vi = N - 1;
      } else if (n_blk > 0) {
        const int last = (n_blk - 1) < 64 ? __builtin_amdgcn_readlane(col_lane, n_blk - 1)
                                          : min(max(p.col_idx[rp0 + n_blk - 1], 0), mrow);
        if (last == mrow) vi = (n_blk - 1) * B + (N - 1) % B;
      }
      const bool visit = vi >= u0 && vi < u1;
      const bool writer = visit ? wave == ((vi - u0) / kChunk) % kWaves
                                : vi < 0 && it.j == it.s - 1 && wave == 0;
      if (writer) {
        if (lane < 2 * CH) {
          const bool isv = lane >= CH;
          const int c = isv ? lane - CH : lane;
          const size_t nrow = (static_cast<size_t>(b) * p.hkv + g) * D + c * 8;
          const size_t dst = (static_cast<size_t>(b) * p.hkv + g) * cache_head + static_cast<size_t>(N - 1) * D + c * 8;
          st16((isv ? p.v_write : p.k_write) + dst, ld16((isv ? p.v_new : p.k_new) + nrow));
        }
        wait_vmem_all();
      }
    }
  }
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
    if (it.s == 1) {  // the unit's only item: the result itself
      const float val = l > 0.0f ? o / l : 0.0f;
      const uint32_t bits = pack_bf16x2(val, 0.0f);
      p.out[(static_cast<size_t>(b) * p.hq + head) * D + dd] = static_cast<uint16_t>(bits & 0xffffu);
    } else {  // partial of slot blockIdx.x, query column n
      const size_t slot = static_cast<size_t>(blockIdx.x) * group + n;
      p.part_o[slot * D + dd] = o;
      if (dd == 0) {
        p.part_ml[slot * 2] = m;
        p.part_ml[slot * 2 + 1] = l;
      }
    }
  }
}

// Merge the items' partials of one (sequence, head).  The unit's items
// occupy consecutive slots (first slot and count from the plan); lane l
// holds d = l + 64 k.  Up to kCombineBatch items: wave 0 alone reads them
// all with their loads in flight together and writes the result.  More:
// wave w merges items w, w + 4, w + 8, ... (kCombineBatch at a time, all
// loads in flight), then the 4 waves' results are merged through LDS in wave
// order.  Either way the sum has a fixed order, and up to 64 items cost one
// memory round trip.
constexpr int kCombineBatch = 16;
constexpr int kCombineWaves = 4;

template <int D>
__global__ __launch_bounds__(kCombineWaves * 64) void decode_combine_kernel(const DecodeParams p) {
  constexpr int DPL = D / 64;  // d values per lane
  __shared__ float wm[kCombineWaves], wl[kCombineWaves], wo[kCombineWaves][D];
  const int sh = blockIdx.x;  // b * hq + head
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int group = p.hq / p.hkv;
  const int b = sh / p.hq, head = sh - b * p.hq;
  const int u = b * p.hkv + head / group, n = head % group;
  const int2 pl = p.plan[u];
  const int first = pl.x, ns = pl.y;
  if (ns <= 1) return;  // the split kernel wrote the result itself
  const bool one_wave = ns <= kCombineBatch;
  if (one_wave && wave != 0) return;
  const int stride = one_wave ? 1 : kCombineWaves;
  float m = kNegInf, l = 0.0f, o[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) o[k] = 0.0f;
  for (int s0 = one_wave ? 0 : wave; s0 < ns; s0 += stride * kCombineBatch) {
    float mv[kCombineBatch], lv[kCombineBatch], ov[kCombineBatch][DPL];
#pragma unroll
    for (int t = 0; t < kCombineBatch; ++t) {
      const int si = s0 + stride * t;
      const bool ok = si < ns;
      const size_t slot = static_cast<size_t>(first + (ok ? si : 0)) * group + n;
      mv[t] = ok ? p.part_ml[slot * 2] : kNegInf;
      lv[t] = ok ? p.part_ml[slot * 2 + 1] : 0.0f;
#pragma unroll
      for (int k = 0; k < DPL; ++k) ov[t][k] = ok ? p.part_o[slot * D + lane + 64 * k] : 0.0f;
    }
    float mb = m;
#pragma unroll
    for (int t = 0; t < kCombineBatch; ++t) mb = fmaxf(mb, mv[t]);
    const float sc0 = (m == kNegInf) ? 0.0f : fast_exp2(m - mb);
    l *= sc0;
#pragma unroll
    for (int k = 0; k < DPL; ++k) o[k] *= sc0;
#pragma unroll
    for (int t = 0; t < kCombineBatch; ++t) {
      const float sc = (mv[t] == kNegInf) ? 0.0f : fast_exp2(mv[t] - mb);
      l += sc * lv[t];
#pragma unroll
      for (int k = 0; k < DPL; ++k) o[k] += sc * ov[t][k];
    }
    m = mb;
  }
  uint16_t* dst = p.out + static_cast<size_t>(sh) * D;
  if (one_wave) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
    for (int k = 0; k < DPL; ++k)
      dst[lane + 64 * k] = static_cast<uint16_t>(pack_bf16x2(o[k] * inv, 0.0f) & 0xffffu);
    return;
  }
  if (lane == 0) {
    wm[wave] = m;
    wl[wave] = l;
  }
#pragma unroll
  for (int k = 0; k < DPL; ++k) wo[wave][lane + 64 * k] = o[k];
  __syncthreads();
  const int dd = threadIdx.x;
  if (dd >= D) return;
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < kCombineWaves; ++w) M = fmaxf(M, wm[w]);
  float L = 0.0f, O = 0.0f;
#pragma unroll
  for (int w = 0; w < kCombineWaves; ++w) {
    const float sc = (wm[w] == kNegInf) ? 0.0f : fast_exp2(wm[w] - M);
    L += sc * wl[w];
    O += sc * wo[w][dd];
  }
  const float val = L > 0.0f ? O / L : 0.0f;
  dst[dd] = static_cast<uint16_t>(pack_bf16x2(val, 0.0f) & 0xffffu);
}

template <int D>
hipError_t launch_typed(const DecodeParams& p, hipStream_t s) {
  if (p.k_new != nullptr)
    decode_split_kernel<D, true><<<dim3(static_cast<uint32_t>(p.slots)), dim3(kWaves * 64), 0, s>>>(p);
  else
    decode_split_kernel<D, false><<<dim3(static_cast<uint32_t>(p.slots)), dim3(kWaves * 64), 0, s>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.slots <= p.n_seq * p.hkv) return e;  // one item per unit: no partials
  decode_combine_kernel<D><<<dim3(static_cast<uint32_t>(p.n_seq * p.hq)), dim3(kCombineWaves * 64), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

DecodeShape decode_shape(int32_t n_seq, int32_t hkv, int32_t max_len, int32_t target) {
  DecodeShape sh{};
  const int64_t units = static_cast<int64_t>(n_seq) * hkv;
  if (units > kDecodePlanUnits) {  // one item per unit
    sh.balanced = 0;
    sh.slots = units;
    return sh;
  }
  // A unit visits at most max_len keys (FA) or ceil(max_len / B) whole blocks
  // (SA), i.e. fewer than max_len + 128, in items of at least 256 keys.  The
  // plan keeps the count within max(units, min(target, units + most)).
  const int64_t most = units * (static_cast<int64_t>(max_len) + 127) / kDecodeMinItemKeys;
  const int64_t t = units + most < target ? units + most : target;
  sh.balanced = 1;
  sh.slots = t > units ? t : units;
  return sh;
}

size_t decode_workspace_bytes(int32_t n_seq, int32_t hq, int32_t hkv, int32_t head_dim,
                              int32_t max_len) {
  // sized for the largest target, so it does not depend on the device
  const DecodeShape sh = decode_shape(n_seq, hkv, max_len, kDecodeMaxItems);
  const size_t units = static_cast<size_t>(n_seq) * hkv;
  if (static_cast<size_t>(sh.slots) <= units) return 0;  // one item per unit: no partials
  const size_t partials = static_cast<size_t>(sh.slots) * (hq / hkv) * (head_dim + 2) * sizeof(float);
  return partials + units * sizeof(int2);
}

hipError_t decode_scratch(hipStream_t stream, void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

int32_t decode_target(hipStream_t stream, int32_t head_dim, bool append) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static int32_t cache[kMaxDevices][2][2] = {};
  int dev = 0;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 512;
  const int di = head_dim == 128 ? 1 : 0, ai = append ? 1 : 0;
  std::lock_guard<std::mutex> lock(mu);
  int32_t& t = cache[dev][di][ai];
  if (t == 0) {
    int cus = 0, per_cu = 0;
    const void* k = di ? (ai ? reinterpret_cast<const void*>(decode_split_kernel<128, true>)
                             : reinterpret_cast<const void*>(decode_split_kernel<128, false>))
                       : (ai ? reinterpret_cast<const void*>(decode_split_kernel<64, true>)
                             : reinterpret_cast<const void*>(decode_split_kernel<64, false>));
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kWaves * 64, 0) != hipSuccess ||
        cus < 1 || per_cu < 1) {
      t = 512;  // 256 CUs x 2 workgroups (head_dim 128)
    } else {
      t = cus * per_cu < kDecodeMaxItems ? cus * per_cu : kDecodeMaxItems;
    }
  }
  return t;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t s) {
  return p.head_dim == 128 ? launch_typed<128>(p, s) : launch_typed<64>(p, s);
}

}  // namespace flux
