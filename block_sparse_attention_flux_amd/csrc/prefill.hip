// Routed prefill attention for gfx950: one kernel family serves Full
// Attention (FA) and block-Sparse Attention (SA) layers; the layer's mode is
// read from the route vector on the device (Flux Attention abstract: a router
// sends each layer to FA or SA; technical summary on gist.science, section 2).
//
// Work decomposition
//   A workgroup owns one query block of BM rows (BM = the mask block size, 64
//   or 128) of one query head of one request; each of its BM/32 waves owns 32
//   query rows.  Keys are visited in tiles of BN = 32: FA visits every tile up
//   to the diagonal, SA only the tiles of the blocks in the query block's CSR
//   row, so inactive K/V tiles are never loaded.  A wave skips the tiles
//   that start past its last row (it still joins the block's barriers).
//
// Per key tile and wave (bf16 MFMA v_mfma_f32_16x16x32_bf16, fp32 accumulate):
//   S^T[key][q] = K Q^T      2 key halves x 2 row tiles of 16 x 16: four
//                            independent accumulators; A = K from LDS, B = Q
//                            kept in registers for the whole kernel
//   online softmax in the log2 domain; a row lives on 4 lanes (l%16 + 16g),
//   whose max and sum combine with v_permlane32_swap + v_permlane16_swap
//   O^T[d][q] += V^T P^T     d/16 x 2 tiles, one 32-key k-step each; A = V^T
//                            via the LDS transpose read, B = P
//   The transposed products leave P in the B-operand layout of the second
//   MFMA: its k index runs over the tile's keys in the order the S^T
//   accumulator holds them in a lane, and V^T is read in the same order.
//   The row sum is taken over the same bf16 P that the second product uses
//   (v_dot2c).
//
// Data movement
//   K and V tiles go global -> LDS directly (buffer_load_dwordx4 ... lds, no
//   register staging) through a buffer resource whose range ends at the last
//   key of the sequence, so a ragged last tile reads zeros.  K is row-major
//   with two 16-byte pad slots per row, V in 128-byte blocks of 4 keys x 16 d
//   with the d block XORed by the key quad's parity; every LDS read below is
//   bank-conflict free and addressed as a base register plus constant
//   offsets.  V^T operands come from ds_read_b64_tr_b16: within each 16-lane
//   group, destination lane 4i+j receives element j of source lanes i, i+4,
//   i+8, i+12, so four source lanes pointing at four keys deliver those keys'
//   values of one d column.  Two K and two V buffers live in four separate LDS
//   arrays: tile n is computed from one pair while tile n+1 loads into the
//   other.  With separate arrays the compiler can tell that the LDS reads
//   never alias the DMA in flight and does not make them wait for it.
//   A workgroup's scalars (sequence bounds, its mask row's CSR bounds, the
//   route byte) arrive in one gathered load; an SA row's first 64 columns
//   are held one per lane and picked with readlane, once per mask block.
//   O leaves through LDS (each wave stages its 32 rows in one of the tile
//   arrays after the last tile) so that the global stores are 16 bytes per
//   lane and cover whole rows.
//
// The running max is only moved when a row's max grows by more than 2^8 (the
// final normalisation divides by a sum taken with the same stale max, so the
// result is unchanged in exact arithmetic); rows that do not move scale by
// exactly 1, so each row depends on its own data only.
//
// Workgroups are ordered so that each XCD (own L2) works through whole KV
// head groups, heaviest causal rows first.  With a workspace, the last 20 % of
// each XCD's list is handed out at run time, so XCDs that run faster than
// the others take over part of their tails.
#include "flux_device.h"
#include "flux_internal.h"

namespace flux {
namespace {

constexpr int kBN = 32;                // keys per tile
constexpr int kOcc = 3;                // waves per SIMD the kernel is built for
constexpr float kRescaleSlack = 8.0f;  // log2 units the stale max may lag
constexpr float kSumLimit = 65536.0f;  // a lane's tile sum of P above this: retake the max
// Word 3 of a raw buffer resource on gfx9-family parts: 32-bit data format,
// no swizzle, no index stride (byte-addressed, range-checked per lane).
constexpr int kBufferFlags = 0x00020000;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) void lds_void;

// LDS layouts (64 banks of 4 bytes; an 8-byte read is served 32 lanes per
// pass):
//   K tile: row-major with rows CH + 2 slots of 16 bytes apart (two pad slots
//           per row), so a lane's reads for the k-steps are one base address
//           plus constant offsets.  For the K operand read (lane l: row l%16
//           of a 16-key half, chunk 4ks + l/16) this stride measured free of
//           bank conflicts on gfx950, where CH + 1 and CH + 3 cost 4 extra
//           cycles per read (SQ_LDS_BANK_CONFLICT).
//   V tile: 128-byte blocks of 4 keys x 16 d, inside a block key-major then
//           d; block (quad q = key/4, d block j) stored at block index
//           q * (D/16) + (j ^ (q & 1)).  A transpose read of one 16-lane group
//           covers exactly one block, and the two groups of a 32-lane pass
//           (quads 2i, 2i + 1, the same j) land 128 bytes apart modulo 256,
//           i.e. on disjoint halves of the banks.

// Loads of one K or V tile into LDS by NT threads.  Load j of thread tid
// fills LDS slot s = j*NT + tid (16 bytes, lane-linear per wave instruction);
// the global chunk it fetches is chosen so that the slot ends up where the
// layout wants it.  K: slot s is row s/KROW, chunk s%KROW (chunks CH and up
// are the pad: their loads are out of the buffer's range, so they fetch
// nothing and write zeros); the last K load covers only the first
// KSLOTS % NT threads.
// V: slot s is stored block s/8 = (key quad, d block ^ (quad & 1)), key
// 4*quad + (s%8)/2, chunk 2*dblk + s%2.
template <int D, int NT, int BN>
struct TileLoader {
  static constexpr int CH = D / 8;
  static constexpr int KROW = CH + 2;                      // 16-byte slots per K row
  static constexpr int KSLOTS = BN * KROW;
  static constexpr int KTILEB = KSLOTS * 16;
  static constexpr int KLOADS = (KSLOTS + NT - 1) / NT;
  static constexpr int KLAST = KSLOTS - (KLOADS - 1) * NT;  // threads in the last K load
  static constexpr int TILEB = BN * D * 2;                 // V tile
  static constexpr int LOADS = TILEB / (NT * 16);
  static_assert(TILEB % (NT * 16) == 0, "tile must split into whole wave loads");
  static constexpr uint32_t kNoFetch = 0x80000000u;        // past any tile's buffer range

  const unsigned char* kbase;
  const unsigned char* vbase;
  uint32_t row_bytes;
  int S, tid, wave_u;
  uint32_t koff[KLOADS], voff[LOADS];

  __device__ __forceinline__ uint32_t k_src(int j) const {
    const int s = j * NT + tid;
    const int r = s / KROW, c = s % KROW;
    return c >= CH ? kNoFetch : r * row_bytes + c * 16;
  }
  __device__ __forceinline__ void v_src(int j, int& r, int& c) const {
    const int s = j * NT + tid;
    const int blk = s / 8, kq = blk / (D / 16), dblk = (blk % (D / 16)) ^ (kq & 1);
    r = 4 * kq + (s % 8) / 2;
    c = 2 * dblk + (s % 2);
  }
  __device__ __forceinline__ void init(const uint16_t* k, const uint16_t* v, int tok0, int hkv, int g,
                                       int seqlen, int thread) {
    const size_t kv_row = static_cast<size_t>(hkv) * D;
    row_bytes = static_cast<uint32_t>(kv_row * 2);
    kbase = reinterpret_cast<const unsigned char*>(k + static_cast<size_t>(tok0) * kv_row +
                                                   static_cast<size_t>(g) * D);
    vbase = reinterpret_cast<const unsigned char*>(v + static_cast<size_t>(tok0) * kv_row +
                                                   static_cast<size_t>(g) * D);
    S = seqlen;
    tid = thread;
    wave_u = __builtin_amdgcn_readfirstlane(thread >> 6);
#pragma unroll
    for (int j = 0; j < KLOADS; ++j) koff[j] = k_src(j);
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      int r, c;
      v_src(j, r, c);
      voff[j] = r * row_bytes + c * 16;
    }
  }
  // Issue the loads of the tile starting at key kst into LDS at `dst`.  The
  // tile is read through a buffer resource whose range ends at the last key
  // of the sequence: rows at or past S come back as zeros from the hardware
  // range check, so a ragged last tile needs no separate path (its keys are
  // masked as causal, and zero V rows add nothing).
  __device__ __forceinline__ void issue(bool is_v, int kst, lds_u8* dst) const {
    const unsigned char* base = (is_v ? vbase : kbase) + static_cast<size_t>(kst) * row_bytes;
    const uint32_t rows = static_cast<uint32_t>(min(S - kst, BN));
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(base), 0, static_cast<int>(rows * row_bytes), kBufferFlags);
    lds_u8* dst0 = dst + wave_u * 64 * 16;
    if (is_v) {
#pragma unroll
      for (int j = 0; j < LOADS; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, reinterpret_cast<lds_void*>(dst0 + j * NT * 16), 16,
                                                 static_cast<int>(voff[j]), 0, 0, 0);
      return;
    }
#pragma unroll
    for (int j = 0; j < KLOADS - 1; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, reinterpret_cast<lds_void*>(dst0 + j * NT * 16), 16,
                                               static_cast<int>(koff[j]), 0, 0, 0);
    // last K load: only the threads whose slot is inside the tile (the LDS
    // array ends at the tile; the other lanes must not write)
    if (wave_u * 64 < KLAST && tid < KLAST)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc,
                                               reinterpret_cast<lds_void*>(dst0 + (KLOADS - 1) * NT * 16),
                                               16, static_cast<int>(koff[KLOADS - 1]), 0, 0, 0);
  }
};

// Per-wave state and math for 32 query rows of one head, on 16x16x32 MFMA
// tiles.  S^T = K Q^T is 2 key tiles x 2 row tiles of 16 x 16: lane l holds
// rows l%16 and 16 + l%16 (row tile c), keys 16kt + 4(l/16) + r (r = 0..3),
// so every row is spread over the 4 lanes l%16 + 16g.  O^T is D/16 d tiles x
// 2 row tiles.  Every MFMA of a tile is independent of the other chains: 4
// accumulators of K Q^T (4 dependent k-steps each for d 128), and each O^T
// tile takes one 32-key k-step.  One online-softmax state (O, running max,
// running sum) per row.
//
// The k index of the P V product runs over the tile's 32 keys in the order
// the S^T layout leaves them in a lane: k = 8g + e is key 16(e/4) + 4g + e%4,
// for P (the B operand, straight from the exponentials) and for V^T (the A
// operand, two transpose reads of 4 keys each) alike.
template <int D, int BN>
struct WaveAttn {
  static_assert(BN == 32, "one 32-key k-step of P V per tile");
  static constexpr int KS = D / 32;   // k-steps of K Q^T
  static constexpr int DT = D / 16;   // 16-row d tiles of O^T
  static constexpr int KROW = D / 8 + 2;
  static constexpr int VBLK = D / 16;  // 128-byte V blocks per key quad
  static constexpr int PK = 8;         // packed bf16 pairs of P per lane (2 rows x 4)

  bf16x8 qreg[2][KS];
  f32x4 oacc[2][DT];
  float m_run[2], l_run[2], cs;
  int l16, grp, wrow0, krd, vrd_e, vrd_o;

  __device__ __forceinline__ void init(const uint16_t* q, int tok0, int hq, int head, int q_row0,
                                       int S, float scale, int lane) {
    l16 = lane & 15;
    grp = lane >> 4;
    wrow0 = q_row0;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int row = q_row0 + 16 * c + l16;
      const bool row_ok = row < S;
      const uint16_t* qp =
          q + (static_cast<size_t>(tok0 + (row_ok ? row : 0)) * hq + head) * D + grp * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 v = row_ok ? ld16(qp + ks * 32) : u32x4{0, 0, 0, 0};
        qreg[c][ks] = as_bf16x8(v);
      }
    }
    cs = scale * kLog2e;  // scores -> log2 domain
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      m_run[c] = kNegInf;
      l_run[c] = 0.0f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[c][dt] = f32x4{};
    }
    // K operand: key row l%16 (+16 kt), chunk 4ks + g: one base, constant offsets
    krd = (l16 * KROW + grp) * 16;
    // V^T operand (transpose read): the 16 lanes of group g read the 128-byte
    // block of key quad 4kt + g and d block dt, stored at block index
    // quad * VBLK + (dt ^ (quad & 1)), byte 8 * (l%16).  g & 1 = quad & 1, so
    // even dt sit at +128 g&1 and odd dt at -128 g&1 from the plain position.
    const int h = grp & 1;
    vrd_e = grp * VBLK * 128 + h * 128 + l16 * 8;
    vrd_o = grp * VBLK * 128 - h * 128 + l16 * 8;
  }

  // S^T of the 32-key tile at kl
  __device__ __forceinline__ void qk(const lds_u8* kl, f32x4 (&s)[2][2]) const {
    u32x4 kop[2][KS];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kop[kt][ks] = *reinterpret_cast<const lds_u32x4*>(kl + krd + (kt * 16 * KROW + 4 * ks) * 16);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int c = 0; c < 2; ++c) s[kt][c] = f32x4{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          s[kt][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kop[kt][ks]), qreg[c][ks], s[kt][c],
                                                             0, 0, 0);
  }

  // P = 2^(S cs - mu) as packed bf16 pairs (pk[4c + j]: row tile c); ps[c] is
  // this lane's sum of the same bf16 P that the P V product uses
  __device__ __forceinline__ void exps(const f32x4 (&s)[2][2], const float (&mu)[2], uint32_t (&pk)[PK],
                                       float (&ps)[2]) const {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          const float p0 = fast_exp2(__builtin_fmaf(s[kt][c][r], cs, -mu[c]));
          const float p1 = fast_exp2(__builtin_fmaf(s[kt][c][r + 1], cs, -mu[c]));
          pk[4 * c + 2 * kt + r / 2] = pack_bf16x2(p0, p1);
        }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float a = add_bf16_pair(pk[4 * c], 0.0f);
#pragma unroll
      for (int j = 1; j < 4; ++j) a = add_bf16_pair(pk[4 * c + j], a);
      ps[c] = a;
    }
  }

  // Causal mask, exponentials against the running max, and the max update
  // only where it is needed.  The exponentials are taken first with the
  // current running max: as long as no P of this lane exceeds 2^16 (its
  // partial row sums stay below kSumLimit) the tile is done, and the running
  // max is left as it is (any P up to 2^16 is exact in fp32/bf16 range terms
  // and the final division uses the same reference).  Otherwise (and on the
  // first tile, when there is no reference yet) the tile's row max is taken,
  // rows whose max grew past the slack move their reference (rescaling their
  // O and sum), and the exponentials are redone; rows that did not move get
  // bit-identical P, so each row's result depends on its own data only.
  __device__ __forceinline__ void softmax(f32x4 (&s)[2][2], int kst, uint32_t (&pk)[PK]) {
    if (kst + BN - 1 > wrow0) {  // tile crosses the diagonal: causal mask
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = kst + 16 * kt + 4 * grp + r;
            if (key > wrow0 + 16 * c + l16) s[kt][c][r] = kNegInf;
          }
    }
    float ps[2] = {0.0f, 0.0f};
    bool slow = __ballot(m_run[0] == kNegInf || m_run[1] == kNegInf) != 0;  // wave-uniform
    if (!slow) {
      exps(s, m_run, pk, ps);
      slow = __ballot(!(ps[0] + ps[1] <= kSumLimit)) != 0;
    }
    if (slow) {
      bool grow[2];
      float mxs[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float mx = kNegInf;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kt][c][r]);
        mxs[c] = max_quarters(max_halves(mx)) * cs;
        grow[c] = mxs[c] > m_run[c] + kRescaleSlack;
      }
      if (__ballot(grow[0] || grow[1]) != 0) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const float m_new = grow[c] ? mxs[c] : m_run[c];
          const float alpha =
              !grow[c] ? 1.0f : (m_run[c] == kNegInf) ? 0.0f : fast_exp2(m_run[c] - m_new);
          l_run[c] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) oacc[c][dt] *= alpha;
          m_run[c] = m_new;
        }
      }
      const float mu[2] = {m_run[0] == kNegInf ? 0.0f : m_run[0],
                           m_run[1] == kNegInf ? 0.0f : m_run[1]};
      exps(s, mu, pk, ps);
    }
    l_run[0] += ps[0];
    l_run[1] += ps[1];
  }

  // 4 keys (quad 4kt + g) x 16 d (tile dt) of V^T, transposed: element e of
  // lane l is V[16kt + 4g + e][16dt + l%16]
  __device__ __forceinline__ s16x4 vt_read(const lds_u8* vl, int kt, int dt) const {
    const int off = ((dt & 1) ? vrd_o : vrd_e) + (kt * 4 * VBLK + dt) * 128;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4*>(const_cast<lds_u8*>(vl) + off));
  }

  // O^T += V^T P^T for the V tile at vl
  __device__ __forceinline__ void pv(const lds_u8* vl, const uint32_t (&pk)[PK]) {
    s16x8 vop[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      vop[dt] = __builtin_shufflevector(vt_read(vl, 0, dt), vt_read(vl, 1, dt), 0, 1, 2, 3, 4, 5, 6, 7);
    bf16x8 b[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) b[c] = as_bf16x8(u32x4{pk[4 * c], pk[4 * c + 1], pk[4 * c + 2], pk[4 * c + 3]});
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int c = 0; c < 2; ++c)
        oacc[c][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vop[dt]), b[c],
                                                                 oacc[c][dt], 0, 0, 0);
  }

  // Soft-routed forward: w O / l of this wave's rows (the weighted SA
  // output) parked in `out` as bf16, straight from the accumulator layout
  // (lane l: d 16dt + 4(l/16) .. +3 of rows 16c + l%16), 8 bytes per store;
  // unpark() reads the same bytes back into the same lanes.
  __device__ __forceinline__ uint16_t* parked_at(uint16_t* out, int tok0, int hq, int head, int c,
                                                 int dt) const {
    return out + (static_cast<size_t>(tok0 + wrow0 + 16 * c + l16) * hq + head) * D + 16 * dt + 4 * grp;
  }
  __device__ __forceinline__ void park(uint16_t* out, int tok0, int hq, int head, int S, float w) const {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const float lt = sum_quarters(sum_halves(l_run[c]));
      const float inv = (lt > 0.0f ? 1.0f / lt : 0.0f) * w;
      if (wrow0 + 16 * c + l16 < S) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          *reinterpret_cast<u32x2*>(parked_at(out, tok0, hq, head, c, dt)) =
              u32x2{pack_bf16x2(oacc[c][dt][0] * inv, oacc[c][dt][1] * inv),
                    pack_bf16x2(oacc[c][dt][2] * inv, oacc[c][dt][3] * inv)};
      }
    }
  }
  __device__ __forceinline__ void unpark(uint16_t* out, int tok0, int hq, int head, int S,
                                         u32x2 (&pk)[2][DT]) const {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bool ok = wrow0 + 16 * c + l16 < S;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        pk[c][dt] = ok ? *reinterpret_cast<const u32x2*>(parked_at(out, tok0, hq, head, c, dt)) : u32x2{0, 0};
    }
  }

  // O = w O / l (+ the parked values), staged through this wave's LDS slice
  // (32 rows of D bf16, free once the tile loop has ended) so that every
  // global store writes 16 bytes per lane and whole rows per instruction.
  // The slice is written in the accumulator layout (lane l: d 16dt + 4(l/16)
  // .. +3 of its two rows) and read row-major; the 16-byte chunks of a row
  // are XOR-swizzled by the row (D 128: row & 15; D 64: (row >> 1) & 7) so
  // both passes are free of bank conflicts.
  __device__ __forceinline__ void store(uint16_t* out, int tok0, int hq, int head, int S, lds_u8* stage,
                                        int lane, float w = 1.0f, const u32x2 (*parked)[DT] = nullptr) const {
    constexpr int CH = D / 8;  // 16-byte chunks per row
    auto swz = [](int r) { return CH == 16 ? (r & 15) : ((r >> 1) & 7); };
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const float lt = sum_quarters(sum_halves(l_run[c]));
      const float inv = (lt > 0.0f ? 1.0f / lt : 0.0f) * w;
      const int r = 16 * c + l16;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = oacc[c][dt][e] * inv;
        if (parked != nullptr) {
          const uint32_t a = parked[c][dt][0], b = parked[c][dt][1];
          o[0] += u32_as_f32(a << 16);
          o[1] += u32_as_f32(a & 0xffff0000u);
          o[2] += u32_as_f32(b << 16);
          o[3] += u32_as_f32(b & 0xffff0000u);
        }
        const int chunk = 2 * dt + (grp >> 1);
        *reinterpret_cast<lds_u32x2*>(stage + r * (D * 2) + ((chunk ^ swz(r)) * 16) + (grp & 1) * 8) =
            u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
      }
    }
    constexpr int RPI = 64 / CH;  // rows per 16-byte-per-lane instruction
    constexpr int NI = 32 / RPI, NB = NI > 4 ? 4 : NI;
    // LDS reads in batches of NB, each batch in flight together (read inside
    // the row check, every read waited for its own round trip)
#pragma unroll
    for (int i0 = 0; i0 < NI; i0 += NB) {
      u32x4 v[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int r = RPI * (i0 + i) + lane / CH, chunk = lane % CH;
        v[i] = *reinterpret_cast<const lds_u32x4*>(stage + r * (D * 2) + ((chunk ^ swz(r)) * 16));
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int r = RPI * (i0 + i) + lane / CH, chunk = lane % CH;
        if (wrow0 + r < S)  // streaming store: this kernel never reads O back
          __builtin_nontemporal_store(v[i], reinterpret_cast<u32x4*>(out + (static_cast<size_t>(tok0 + wrow0 + r) * hq + head) * D + chunk * 8));
      }
    }
  }
};

// Query block's key tiles: FA = every tile up to the diagonal, SA = the
// tiles of the blocks in the CSR row (columns clamped into [0, t]).  Each
// wave keeps the row's first 64 columns one per lane (read with one load,
// picked with readlane), so finding a tile's start needs no LDS and no
// barrier; later columns, rare, are read from memory.
//
// SA visits its diagonal block first when the row ends with it (the static
// and the content-aware masks always do): the first tile is then known from
// the block index alone, so its K/V loads leave with the Q loads instead of
// waiting for the row's columns; check_diag() then confirms the guess from
// the columns (otherwise the row is visited in its own order).  The order of
// the tiles does not change the result beyond rounding (online softmax).
template <int BM, int BN>
struct TileList {
  static constexpr int TPB = BM / BN;  // key tiles per mask block
  const int32_t* col_idx;
  int rp0, n_row, n_tiles, n_diag, t, col_lane;
  bool fa, diag_first;
  // rb, re: the mask row's CSR bounds (read by the caller beside the route);
  // q_end: one past the query block's last row
  __device__ __forceinline__ void init(const PrefillParams& p, int qt, bool is_fa, int rb, int re, int lane,
                                       int q_end) {
    fa = is_fa;
    t = qt;
    col_idx = p.col_idx;
    rp0 = rb;
    col_lane = 0;
    n_row = 0;
    diag_first = false;
    n_diag = min(TPB, (q_end - t * BM + BN - 1) / BN);  // tiles of the diagonal block before q_end
    if (fa) {
      n_tiles = (q_end + BN - 1) / BN;
      return;
    }
    n_row = max(re - rb, 0);
    col_lane = lane < n_row ? col_idx[rp0 + lane] : 0;  // clamped when read
    diag_first = n_row > 0;  // a guess until check_diag()
    n_tiles = diag_first ? (n_row - 1) * TPB + n_diag : 0;
  }
  __device__ __forceinline__ int col(int i) const {
    int c;
    if (i < 64) {
      c = __builtin_amdgcn_readlane(col_lane, i);
    } else {
      // made scalar inside the branch, so the wait for this load stays on
      // this (rare) path and never covers the tile loads in flight
      c = __builtin_amdgcn_readfirstlane(col_idx[rp0 + i]);
    }
    return min(max(c, 0), t);
  }
  // SA: keep the diagonal-first order if the row's last column is the
  // diagonal block; otherwise fall back to the row's order, without the
  // tiles that start past the block's last row.  Returns true if it changed.
  __device__ __forceinline__ bool check_diag() {
    if (fa || !diag_first || col(n_row - 1) == t) return false;
    diag_first = false;
    n_tiles = n_row * TPB;
    while (n_tiles > 0 && start(n_tiles - 1) >= t * BM + n_diag * BN) --n_tiles;
    return true;
  }
  __device__ __forceinline__ int start(int n) const {
    if (fa) return n * BN;
    if (diag_first) {
      if (n < n_diag) return t * BM + n * BN;
      n -= n_diag;  // then the row's other blocks, in order
    }
    return col(n / TPB) * BM + (n % TPB) * BN;
  }
  // start of tile n + 1 given that tile n starts at kst: the tiles of a block
  // are contiguous, so a column is looked up only at a block's first tile
  __device__ __forceinline__ int next_start(int n, int kst) const {
    const int k = n + 1 - (diag_first ? n_diag : 0);  // < 0: still inside the diagonal block
    return (fa || k < 0 || k % TPB != 0) ? kst + BN : start(n + 1);
  }
  // does the wave whose first row is wrow0 compute tile n (does it start at
  // or before the wave's last row)?
  __device__ __forceinline__ int visible_prefix(int wrow0, int S) const {  // sorted orders
    if (wrow0 >= S) return 0;
    int n = n_tiles;
    while (n > 0 && start(n - 1) > wrow0 + 31) --n;
    return n;
  }
};

// Tile order of the soft-routed forward: first the tiles of the blocks in the
// query block's CSR row (SA), then those of the other causal blocks 0 .. t in
// increasing order (what FA adds), so one softmax state yields SA after the
// first phase and FA after both.  The CSR row is trusted to be increasing;
// its columns are clamped into [0, t] as everywhere (repeats count once).
// start() must be called with n = 0, 1, 2, ... in order: the second phase
// walks the complement with a cursor into the row.
template <int BM, int BN>
struct SoftOrder {
  static constexpr int TPB = BM / BN;
  TileList<BM, BN> sa;
  int n_sa, n_tiles, n_row, t, cb, cp;
  __device__ __forceinline__ int col(int i) const { return sa.col(i); }  // clamped
  __device__ __forceinline__ void init(const PrefillParams& p, int qt, int rb, int re, int lane, int q_end) {
    t = qt;
    n_row = max(re - rb, 0);
    sa.init(p, qt, false, rb, re, lane, q_end);
    sa.check_diag();  // SA tiles in the diagonal-first order when the row allows it
    n_sa = sa.n_tiles;
    int distinct = 0, prev = -1;
    for (int i = 0; i < n_row; ++i) {
      const int c = col(i);
      distinct += c != prev;
      prev = c;
    }
    int comp = (t + 1 - distinct) * TPB;
    if (prev != t) comp -= TPB - (q_end - t * BM + BN - 1) / BN;  // block t is FA-only: trim it
    n_tiles = n_sa + comp;
    cb = -1;
    cp = 0;
  }
  __device__ __forceinline__ int start(int n) {
    if (n < n_sa) return sa.start(n);
    const int k = n - n_sa;
    if (k % TPB == 0) {  // next block that is not in the row
      int b = cb + 1;
      for (;;) {
        while (cp < n_row && col(cp) < b) ++cp;
        if (cp < n_row && col(cp) == b) {
          ++b;
          continue;
        }
        break;
      }
      cb = b;
    }
    return cb * BM + (k % TPB) * BN;
  }
};

// Workgroup -> (kv group, request, query block heaviest first, head slot).
// Workgroup ids are dealt to the 8 XCDs round-robin (id % 8).  With one route
// decision per layer the order is XCD-major: each XCD works through whole KV
// head groups, one request at a time, so the workgroups an XCD holds at once
// are the query heads of a few neighbouring query blocks of one request and
// share its K/V in the XCD's L2 (with the requests interleaved instead, a
// packed batch of long prompts spread them over every request's K/V).  With
// one decision per kv head the XCD-major order would leave the XCDs that drew
// FA groups running long after the others, so there each XCD's share cycles
// through all kv groups instead (heaviest query blocks still first).
//
// bid is the item's place in that order and G the number of items (equal to
// the grid, except in the balanced order below).
__device__ __forceinline__ void decode_work(int bid, int G, int n_slots, int n_req, int n_qt, int hkv, bool by_head,
                                            int& slot, int& req, int& t, int& g) {
  int w;
  if (by_head && G % (8 * hkv) == 0) {
    const int i = bid / 8;
    g = i % hkv;
    w = (i / hkv) * 8 + bid % 8;  // the other indices, heaviest blocks first
    slot = w % n_slots;
    w /= n_slots;
    req = w % n_req;
    w /= n_req;
    t = n_qt - 1 - w;
    return;
  }
  w = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
  slot = w % n_slots;
  w /= n_slots;
  t = n_qt - 1 - (w % n_qt);
  w /= n_qt;
  req = w % n_req;
  g = w / n_req;
}

// Balanced order (p.wq: a caller's zeroed workspace; the host sets it for
// layer-level routing when the items split into whole XCD shares and fill at
// least one round of the GPU's workgroups).  The eight XCDs finish equal
// static shares up to ~10 % apart, and which XCD is slow changes from run to
// run, so only the first 80 % of each XCD's list is static.  The rest of XCD
// x's list is queue x, counted by wq[x * kLine] (one counter per 128-byte
// line).  The grid has items / 8 more workgroups than items.  A tail
// workgroup whose blockIdx is below `items` first takes the next item of the
// queue of the XCD it runs on (hardware register XCC_ID); when that is empty,
// and for the extra workgroups, it reads all eight counters and tries only
// the queues that still had items, in order from its own.  Every taken index
// below the tail length is one item, so every item is taken at most once; a
// workgroup ends only when every queue has handed out all its items, and
// since there are at least as many tail workgroups as tail items, every item
// is taken.  The counters are set back to zero by a one-workgroup kernel
// launched after the attention kernel on the same stream, so the workspace
// is zero again when the call completes and no workgroup waits for another.
struct Balance {
  static constexpr int kTailPct = 20;
  static constexpr int kLine = 32;  // int32 counters 128 bytes apart
  int items, per, stat;             // items, items per XCD, static items per XCD
  __device__ __forceinline__ void init(int n_items) {
    items = n_items;
    per = n_items / 8;
    stat = per - static_cast<int>(static_cast<int64_t>(per) * kTailPct / 100);
  }
  __device__ __forceinline__ bool tail_wg(const PrefillParams& p) const {
    return p.wq != nullptr && static_cast<int>(gridDim.x) > items && static_cast<int>(blockIdx.x) >= 8 * stat;
  }
  // item of this tail workgroup in the XCD-major order, or -1 (thread 0)
  __device__ __forceinline__ int take(const PrefillParams& p) const {
    const int x = __builtin_amdgcn_s_getreg((31 << 11) | 20) & 7;  // hwreg(HW_REG_XCC_ID)
    const int tail = per - stat;
    if (static_cast<int>(blockIdx.x) < items) {
      const int i = atomicAdd(&p.wq[x * kLine], 1);
      if (i < tail) return (stat + i) * 8 + x;
    }
    int taken[8];
#pragma unroll
    for (int y = 0; y < 8; ++y)
      taken[y] = __hip_atomic_load(&p.wq[y * kLine], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int k = 0; k < 8; ++k) {
      const int y = (x + k) & 7;
      int ty = taken[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) ty = y == j ? taken[j] : ty;  // taken[y] without a dynamic index
      if (ty >= tail) continue;
      const int i = atomicAdd(&p.wq[y * kLine], 1);
      if (i < tail) return (stat + i) * 8 + y;
    }
    return -1;
  }
};

__global__ void balance_reset_kernel(int32_t* wq) {
  if (threadIdx.x < 8) wq[threadIdx.x * Balance::kLine] = 0;
}

// SOFT: the soft-routed forward, O = r FA + (1 - r) SA with r per (request,
// layer), with one softmax state (SoftOrder): the SA tiles come first; after
// the last of them every wave parks (1 - r) O / l of its rows in `out`; the
// same state then runs over FA's other causal tiles, and the result r O / l
// plus the parked value is written.  The SA blocks being a subset of FA's,
// this is FA's work alone, at the routed kernel's occupancy.
template <int D, int BM, int BN, int OCC, bool SOFT = false>
__global__ __launch_bounds__(BM * 2, OCC) void prefill_kernel(const PrefillParams p) {
  constexpr int NT = BM * 2;
  using Loader = TileLoader<D, NT, BN>;
  constexpr int TILEB = Loader::TILEB, KTILEB = Loader::KTILEB;
  // Four separate arrays: the compiler can then see that the LDS reads of
  // one buffer pair never alias the DMA still filling the other pair, and
  // does not make the reads wait for it.
  __shared__ __attribute__((aligned(16))) unsigned char k0_raw[KTILEB];
  __shared__ __attribute__((aligned(16))) unsigned char k1_raw[KTILEB];
  __shared__ __attribute__((aligned(16))) unsigned char v0_raw[TILEB];
  __shared__ __attribute__((aligned(16))) unsigned char v1_raw[TILEB];
  lds_u8* const k0 = (lds_u8*)(k0_raw);  // the same arrays, addressed as LDS
  lds_u8* const k1 = (lds_u8*)(k1_raw);
  lds_u8* const v0 = (lds_u8*)(v0_raw);
  lds_u8* const v1 = (lds_u8*)(v1_raw);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches below
  const int group = p.hq / p.hkv;
  const int n_qt = (p.max_seqlen + BM - 1) / BM;
  int hi, req, t, g;
  Balance bal;
  bal.init(n_qt * p.hq * p.n_req);
  int bid = blockIdx.x;
  if (bal.tail_wg(p)) {
    __shared__ int item_sh;
    if (tid == 0) item_sh = bal.take(p);
    __syncthreads();
    bid = __builtin_amdgcn_readfirstlane(item_sh);
    if (bid < 0) return;
  }
  decode_work(bid, p.wq != nullptr ? bal.items : static_cast<int>(gridDim.x), group, p.n_req, n_qt, p.hkv,
              p.route_heads > 1, hi, req, t, g);
  const int head = g * group + hi;

  // Sequence bounds, the mask row's CSR bounds and the route byte: one
  // gathered load (lanes 0-3 read a word each, lane 4 the byte), so the
  // workgroup pays a single memory round trip for all of them.
  const int mrow = min(t, p.mask_blocks - 1);
  const int32_t* src = lane == 0 ? p.cu_seqlens + req
                       : lane == 1 ? p.cu_seqlens + req + 1
                       : lane == 2 ? p.row_ptr + mrow
                                   : p.row_ptr + mrow + 1;
  int gv = 0;
  if (lane < 4)
    gv = *src;
  else if (lane == 4 && !SOFT)
    gv = p.route[route_index(req, p.n_layers, p.layer, p.route_heads, g)];
  const int tok0 = __builtin_amdgcn_readlane(gv, 0);
  const int S = min(__builtin_amdgcn_readlane(gv, 1) - tok0, p.max_seqlen);  // longer requests are cut
  const int rb = __builtin_amdgcn_readlane(gv, 2), re = __builtin_amdgcn_readlane(gv, 3);
  const int rbyte = __builtin_amdgcn_readlane(gv, 4);
  const int q0 = t * BM;
  if (q0 >= S) return;
  const bool fa = SOFT || rbyte != 0;
  const int q_end = min(q0 + BM, S);

  TileList<BM, BN> tiles;
  SoftOrder<BM, BN> soft;
  int n_tiles;
  if constexpr (SOFT) {
    soft.init(p, t, rb, re, lane, q_end);
    n_tiles = soft.n_tiles;
  } else {
    tiles.init(p, t, fa, rb, re, lane, q_end);
    n_tiles = tiles.n_tiles;
  }
  Loader ld;
  ld.init(p.k, p.v, tok0, p.hkv, g, S, tid);
  WaveAttn<D, BN> wa;
  const int wrow0 = q0 + wave * 32;
  wa.init(p.q, tok0, p.hq, head, wrow0, S, p.scale, lane);  // in flight with the first tile
  float r_fa = 1.0f;  // SOFT: the FA weight of this request and layer
  if constexpr (SOFT) r_fa = p.rsoft[static_cast<int64_t>(req) * p.n_layers + p.layer];

  // Step n computes tile n from one buffer pair while tile n+1 loads into the
  // other; the loop is unrolled by two so that each step names its buffers.
  // kst is the first key of tile n (looked up one step ahead, so no index
  // load waits behind the tile loads in flight).
  int kst = 0;
  // routed: this wave computes tile n iff n < n_mine or n >= n_lo (set below)
  int n_mine = 0, n_lo = 0;
  auto step = [&](int n, const lds_u8* kc, const lds_u8* vc, lds_u8* kn, lds_u8* vn) __attribute__((always_inline)) {
    int kst_next = 0;
    if (n + 1 < n_tiles) {
      if constexpr (SOFT) {
        kst_next = soft.start(n + 1);
      } else {
        kst_next = tiles.next_start(n, kst);
      }
      ld.issue(false, kst_next, kn);
      ld.issue(true, kst_next, vn);
    }
    // a wave computes the tiles that start at or before its last row (in the
    // routed kernel's sorted orders these are a prefix of the tiles)
    bool mine;
    if constexpr (SOFT) {
      mine = wrow0 < S && kst <= wrow0 + 31;
    } else {
      mine = n < n_mine || n >= n_lo;
    }
    if (mine) {
      f32x4 sacc[2][2];
      uint32_t pk[WaveAttn<D, BN>::PK];
      wa.qk(kc, sacc);
      wa.softmax(sacc, kst, pk);
      wa.pv(vc, pk);
    }
    kst = kst_next;
    wait_vmem_all();
    __syncthreads();
  };
  // tiles [n0, n1): tile n lives in buffer pair n & 1
  auto run = [&](int n0, int n1) __attribute__((always_inline)) {
    int n = n0;
    if (n < n1 && (n & 1)) step(n++, k1, v1, k0, v0);
    for (; n < n1; n += 2) {
      step(n, k0, v0, k1, v1);
      if (n + 1 >= n1) break;
      step(n + 1, k1, v1, k0, v0);
    }
  };
  if constexpr (SOFT) {
    if (n_tiles > 0) {
      kst = soft.start(0);
      ld.issue(false, kst, k0);
      ld.issue(true, kst, v0);
    }
  } else {
    if (n_tiles > 0) {  // SA: the diagonal block's first tile, before the columns are known
      kst = tiles.start(0);
      ld.issue(false, kst, k0);
      ld.issue(true, kst, v0);
    }
    if (tiles.check_diag()) {  // the row does not end with its diagonal block
      n_tiles = tiles.n_tiles;
      if (n_tiles > 0) {  // the earlier loads land first (in order); these replace them
        kst = tiles.start(0);
        ld.issue(false, kst, k0);
        ld.issue(true, kst, v0);
      }
    }
    if (tiles.diag_first) {  // the diagonal tiles up to the wave's last row, then every tile
      n_mine = wrow0 < S ? min(tiles.n_diag, (wrow0 + 31 - t * BM) / BN + 1) : 0;
      n_lo = wrow0 < S ? tiles.n_diag : n_tiles;
    } else {  // sorted: a prefix
      n_mine = tiles.visible_prefix(wrow0, S);
      n_lo = n_tiles;
    }
  }
  if (n_tiles > 0) {
    wait_vmem_all();
    __syncthreads();
  }
  if constexpr (SOFT) {
    run(0, soft.n_sa);                                         // SA's tiles
    wa.park(p.out, tok0, p.hq, head, S, 1.0f - r_fa);          // (1 - r) SA of these rows
    run(soft.n_sa, n_tiles);                                   // FA's other tiles
  } else {
    run(0, n_tiles);
  }
  // O goes out through LDS: wave w stages its rows in tile array w (every
  // wave has passed the loop's last barrier, so no tile is read any more)
  lds_u8* const stage = wave == 0 ? k0 : wave == 1 ? k1 : wave == 2 ? v0 : v1;
  if constexpr (SOFT) {
    // the parked SA part: written by this wave's own lanes at least one
    // vmcnt(0) wait ago (each step ends with one)
    u32x2 parked[2][WaveAttn<D, BN>::DT];
    wa.unpark(p.out, tok0, p.hq, head, S, parked);
    wa.store(p.out, tok0, p.hq, head, S, stage, lane, r_fa, parked);
  } else {
    wa.store(p.out, tok0, p.hq, head, S, stage, lane);
  }
}

template <int D, int BM>
hipError_t launch_typed(const PrefillParams& p, hipStream_t s) {
  const int n_qt = (p.max_seqlen + BM - 1) / BM;
  const int64_t items = static_cast<int64_t>(n_qt) * p.hq * p.n_req;
  const int64_t grid = p.wq != nullptr ? items + items / 8 : items;
  // 64-row blocks: 2-wave workgroups whose tiles hold LDS for 2 waves per SIMD
  constexpr int occ = BM == 128 ? kOcc : 2;
  if (p.rsoft != nullptr)
    prefill_kernel<D, BM, kBN, occ, true><<<dim3(static_cast<uint32_t>(grid)), dim3(BM * 2), 0, s>>>(p);
  else
    prefill_kernel<D, BM, kBN, occ><<<dim3(static_cast<uint32_t>(grid)), dim3(BM * 2), 0, s>>>(p);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && p.wq != nullptr) {
    balance_reset_kernel<<<1, 64, 0, s>>>(p.wq);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t s) {
  if (p.head_dim == 128) {
    return p.block_size == 128 ? launch_typed<128, 128>(p, s) : launch_typed<128, 64>(p, s);
  }
  return p.block_size == 128 ? launch_typed<64, 128>(p, s) : launch_typed<64, 64>(p, s);
}

}  // namespace flux
