// Split-KV partial attention for many query rows per sequence (128-row
// tiles): the compute-bound shapes of MLA decoding (many heads, several
// query tokens), written for gfx950.
//
// Same contract as the kernel in mla_decode.hip (topnet.top "Was ist
// FlashMLA?", "MLA-Decodierung ausfuehren"; sao.pub FlashMLA overview,
// 二、核心功能与架构): per query row, softmax attention over the 576-dim
// latent keys of its sequence (V = first 512 dims), out + natural-log lse,
// with causal / sparse-index masking and bf16 or 656-byte FP8 rows.
//
// Design for CDNA4:
//   * One workgroup = 8 waves = 4 wave pairs x 32 query rows.  Both waves
//     of a pair work on the same 32 rows; wave half h takes QK dims
//     288 h .. 288 h + 287 and V dims 256 h .. 256 h + 255.  Each wave then
//     needs only 128 VGPRs of O^T (256 dims x 32 rows, fp32) and 72 of Q^T,
//     so two waves share a SIMD with all MFMA accumulators in VGPRs, and
//     every MFMA is v_mfma_f32_32x32x16_bf16: a 1 KiB fragment from LDS feeds
//     32 K flops, twice the reuse of a 16-row tile, and its 32-key read
//     pattern hits all LDS banks once (K rows are XOR-swizzled, below).
//   * bf16 pages: the two groups of four waves (one wave of each group per
//     SIMD) run half a slice apart.  A slice is a QK half-step (K fragment
//     reads + 18 MFMAs, partial S^T to LDS) and a softmax + PV half-step;
//     while one group is in its QK half-step the other is in its softmax +
//     PV half-step, so each SIMD overlaps one wave's VALU softmax with the
//     other's MFMAs instead of running both waves through the same phase.
//     One workgroup barrier per half-step serves the pair exchange, the
//     arrival of the next slice and the release of a ring slot.  FP8 pages
//     keep both groups in step (the dequantised slice has a single buffer).
//   * S^T = K Q^T (32 keys x 32 rows) is contracted over each half's 288
//     dims; the two partial tiles are exchanged through LDS and added, so
//     both waves of a pair hold the same full S^T (the sum is commutative,
//     hence bitwise identical) and run the same online softmax.  The 32x32
//     result gives each lane one query row and 16 keys, which are exactly
//     the B operand P^T of O^T += V^T P^T for two 16-key k-steps, so P never
//     leaves registers.  V^T comes from ds_read_b64_tr_b16 (4 keys x 16 dims
//     transposed across a 16-lane group).
//   * Keys are staged in halves of 32 (a "slice": half of a 64-token page)
//     through a 3-slot LDS ring filled by global_load_lds (16 bytes per
//     lane, no VGPR round trip): two slices are in flight while the third
//     is computed.  A bf16 slice is stored chunk-group-major: the 72 16-byte
//     chunks of a key row form 9 groups of 8, and group G of all 32 keys is
//     one 4 KiB block (key t at 128 t), with the chunk index XOR-swizzled
//     within its group by a function of t, so that fragment reads of 32 keys
//     (K) or 4 keys x 32 dims (V) spread over all LDS banks.  In this layout
//     each lane of a copy always moves chunks of one key, so a copy address
//     is a per-lane constant plus a scalar base.  The copies are issued from asm, so the compiler does not
//     drain them before LDS reads; the ring waits for them itself
//     (s_waitcnt vmcnt before a barrier).
//   * Issuing a slice needs no vector-memory load whose wait would also
//     drain the copies in flight: dense pages come through the scalar cache,
//     and the pool rows of a sparse unit's index entries are resolved into
//     an LDS table when the unit starts.
//   * FP8 slices are copied raw into their own ring and dequantised (e4m3 ->
//     fp32, times the group scale, -> bf16) into a bf16 slice by all threads
//     before the MFMA work.
//   * Key slots nobody may see are loaded from a visible key of the same
//     slice (never from outside the sequence) and their probabilities are
//     forced to zero, so V never carries stale or poisoned memory.
#include "mla_slice.h"

namespace mla {
namespace wide {

using namespace slice;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerPair = 32;
constexpr int kRowsPerWg = kRowsPerPair * (kWaves / 2);   // 128
constexpr int kKSteps = kDqk / 2 / 16;                    // 18 k-steps of 16 dims per half
constexpr int kDimTiles = kDv / 2 / 32;                   // 8 tiles of 32 V dims per half
constexpr int kXchgBytes = 16 * 64 * 4;                   // one wave's S^T tile, fp32
constexpr float kRescaleSlack = 8.f;

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Per-format geometry: ring slot size, copy instructions (64 lanes x 16 B)
// per slice and per wave, and QL = k-steps of Q kept in LDS instead of
// VGPRs (LDS: bf16 3 x 36 KiB ring + 32 KiB exchange + 16 KiB Q (+ 4 KiB
// sparse table) = 160 KiB at most; FP8 3 x 21 KiB ring + 36 KiB slice + 32
// + 24 (+ 4) KiB).
template <int FMT>
struct Geo {
  static constexpr int kRingBytes = FMT == 0 ? kSliceBytes : kRawSlotBytes;
  static constexpr int kInst = kRingBytes / 1024;                 // 36 | 21
  static constexpr int kPerWave = (kInst + kWaves - 1) / kWaves;  // 5 | 3
  static constexpr int QL = FMT == 0 ? 2 : 3;
};

// Copy slice `sl` (entries 32 sl .. 32 sl + 31 of the unit's key list) into
// `dst` with global_load_lds.  bf16: wave w issues copy instructions
// inst = w + 8 i (chunk group (w >> 2) + 2 i of key octet w & 3, see
// bf16_copy_src), so its lanes keep one key for all i.  FP8: the 656-byte
// rows are copied linearly (chunk q = 64 inst + lane).  Masked slots load a
// visible row of the same slice (row 0 of the pool when the slice has none).
// Every wave issues exactly kPerWave loads (waves without a chunk left
// repeat their first one), also for a slice past the unit's range
// (active == false: row 0 of the pool, mask 0), so that every ring step
// waits with the same vmcnt (an empty pool issues none; the waits then pass
// at once).  Dense slices take their page from `page_in` (page_of of block
// sl / 2, loaded ahead by the caller).  Returns the mask of visible slots.
template <int FMT, bool SPARSE>
__device__ __forceinline__ uint32_t issue_slice(const DecodeParams& p, const int32_t* tab, int tab_base,
                                                uint8_t* dst, int sl, int L, bool active, int page_in) {
  const int ln = opaque_lane();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int kInst = Geo<FMT>::kInst;
  constexpr int kPer = Geo<FMT>::kPerWave;
  int first_row;
  const uint32_t mask = slice_mask<SPARSE>(tab, tab_base, sl, L, active, &first_row);
  if (p.num_pages == 0) return 0u;   // empty pool: no key exists, copy nothing
  if constexpr (FMT == 0) {
    const int k = wave & 3;
    const uint8_t* src =
        bf16_copy_src(p, slot_row<SPARSE>(tab, tab_base, sl, 8 * k + (ln >> 3), L, active, page_in, first_row), k);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      int inst = wave + kWaves * i;               // uniform
      if (inst >= kInst) inst = wave;             // repeat this wave's first load
      lds_dma16(src + 128 * (inst >> 2), dst + inst * 1024);
    }
  } else {
    constexpr int kCpr = kFp8RowBytes / 16;   // 41 chunks per row
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      int inst = wave + kWaves * i;
      if (inst >= kInst) inst = wave;
      int q = inst * 64 + ln;
      if (q >= kSlice * kCpr) q = kSlice * kCpr - 1;   // tail: stay in the slice
      const int t = q / kCpr;
      const int pc = q - t * kCpr;
      const int row = slot_row<SPARSE>(tab, tab_base, sl, t, L, active, page_in, first_row);
      lds_dma16(p.kcache + (size_t)row * kFp8RowBytes + pc * 16, dst + inst * 1024);
    }
  }
  return mask;
}

// A bf16 slice copy as single-instruction parts: prep_copy resolves the
// rows and returns the lane's source pointer; copy_part<i>() issues part i,
// copy instruction inst = wave + 8 i (chunk group (wave >> 2) + 2 i), if
// inst is within the slice: waves 0-3 issue 5 parts, waves 4-7 issue 4.
// Same rows and layout as issue_slice<0, false>.
struct SliceCopy {
  const uint8_t* src;   // lane's key row + its chunk within group (wave >> 2)
  uint8_t* dst;         // LDS: slot + 1 KiB x wave
  bool on;              // pool not empty
};
__device__ __forceinline__ SliceCopy prep_copy(const DecodeParams& p, uint8_t* slot, int sl, int L, bool active,
                                               int page_in) {
  const int ln = opaque_lane();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int k = wave & 3;
  const int row = slot_row<false>(nullptr, 0, sl, 8 * k + (ln >> 3), L, active, page_in, 0);
  SliceCopy c;
  c.src = bf16_copy_src(p, row, k) + 128 * (wave >> 2);
  c.dst = slot + 1024 * wave;
  c.on = p.num_pages != 0;
  return c;
}
template <int I>
__device__ __forceinline__ void copy_part(const SliceCopy& c) {
  constexpr int kInst = Geo<0>::kInst;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (!c.on) return;
  if (I + 1 < Geo<0>::kPerWave || wave + kWaves * I < kInst)
    lds_dma16(c.src + 256 * I, c.dst + kWaves * 1024 * I);   // group (wave >> 2) + 2 I
}
__device__ __forceinline__ void copy_all(const SliceCopy& c) {
  static_assert(Geo<0>::kPerWave == 5, "parts");
  copy_part<0>(c);
  copy_part<1>(c);
  copy_part<2>(c);
  copy_part<3>(c);
  copy_part<4>(c);
}



// ---- per-slice pieces shared by both kernels ------------------------------

// Partial S^T = K Q^T over this wave's 288 QK dims.  A = K: lane holds key
// l32, dims 288 hf + 16 ks + 8 g + 0..7, i.e. chunk c = 36 hf + 2 ks + g of
// its row, in group c / 8 = (hf ? 4 : 0) + (2 ks + 4 hf) / 8.  The swizzled
// position within the group repeats every 4 k-steps; four lane offsets carry
// it, the rest is an immediate.  B = Q^T from registers (k-steps < QR) or
// from this wave's LDS area.
template <int QR>
__device__ __forceinline__ f32x16 qk_partial(const uint8_t* kb, const bf16x8 (&qf)[QR], const uint8_t* qs_mine,
                                             int hf) {
  f32x16 s;
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = 0.f;
  const int ln = opaque_lane();
  const int t = ln & 31;
  const int gg = ln >> 5;
  const int sw = swz(t);
  int ko[4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
    ko[m] = t * 128 + (((4 * hf + 2 * m + gg) ^ sw) & 7) * 16 + hf * kGroupBytes * (4 + (m >= 2 ? 1 : 0));
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks) {
    const bf16x8 a = *(const bf16x8*)(kb + ko[ks & 3] + kGroupBytes * (ks >> 2));
    bf16x8 bq;
    if (ks < QR)
      bq = qf[ks < QR ? ks : 0];
    else
      bq = *(const bf16x8*)(qs_mine + ((ks - QR) * 64 + ln) * 16);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq, s, 0, 0, 0);
  }
  // Keep three fragment reads ahead of the MFMA chain.
  __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
  for (int i = 0; i < kKSteps - 1; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  return s;
}

// The pair exchange: each wave stores its partial tile (lane-major, 16 B per
// lane per quad) and adds its partner's after a barrier.
__device__ __forceinline__ void xchg_put(uint8_t* xs_mine, const f32x16& s, int lane) {
#pragma unroll
  for (int qd = 0; qd < 4; ++qd)
    *(f32x4*)(xs_mine + (qd * 64 + lane) * 16) = f32x4{s[4 * qd], s[4 * qd + 1], s[4 * qd + 2], s[4 * qd + 3]};
}
__device__ __forceinline__ void xchg_add(const uint8_t* xs_peer, f32x16& s, int lane) {
#pragma unroll
  for (int qd = 0; qd < 4; ++qd) {
    const f32x4 v = *(const f32x4*)(xs_peer + (qd * 64 + lane) * 16);
#pragma unroll
    for (int r = 0; r < 4; ++r) s[4 * qd + r] += v[r];
  }
}

// Mask + online softmax of the full S^T of one slice, then O^T += V^T P^T.
// Logits are sc * s with sc >= 0 (Q carries the sign of the scale), exp2
// domain.  Lane holds row l32 and keys 8 (r >> 2) + 4 g + (r & 3) of the
// slice, r = 0..15.  Only a slice that some row may not see entirely is
// masked (full == false).  The reference max m_run is only raised when a
// row's max exceeds it by more than kRescaleSlack: P then stays below
// 2^kRescaleSlack and O and the row sum always share one reference.
template <bool SPARSE>
__device__ __forceinline__ void softmax_pv(f32x16& s, f32x16 (&o)[kDimTiles], float& m_run, float& l_part,
                                           const uint8_t* kb, uint32_t vmask, bool full, int W, int key0,
                                           float sc, int hf, int g) {
  uint32_t okbits = 0xFFFFu;   // bit r: key of register r visible to this row
  if (!full) {
    const uint32_t lmask = vmask >> (4 * g);   // sparse: bit 8 (r >> 2) + (r & 3)
    const int klim = W - key0 - 4 * g;         // dense: visible iff 8 (r >> 2) + (r & 3) < klim
    okbits = 0u;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tl = 8 * (r >> 2) + (r & 3);
      const bool ok = SPARSE ? ((lmask >> tl) & 1u) != 0u : (tl < klim);
      okbits |= ok ? (1u << r) : 0u;
      s[r] = ok ? s[r] : -INFINITY;
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
  mx = fmaxf(mx, xor32(mx));
  mx = mx == -INFINITY ? -INFINITY : mx * sc;
  const bool raise = mx > m_run + kRescaleSlack;
  if (__any(raise)) {
    const float m_new = raise ? mx : m_run;
    const float alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new));
    m_run = m_new;
    l_part *= alpha;
#pragma unroll
    for (int d = 0; d < kDimTiles; ++d) o[d] *= alpha;
  }
  const float m_use = m_run == -INFINITY ? 0.f : m_run;
  bf16x8 pb[2];
  {
    float e[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) e[r] = fast_exp2(__builtin_fmaf(s[r], sc, -m_use));
    if (!full) {
#pragma unroll
      for (int r = 0; r < 16; ++r) e[r] = ((okbits >> r) & 1u) ? e[r] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) l_part += e[r];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      pb[kk] = __builtin_bit_cast(
          bf16x8, u32x4{pack_bf16x2(e[8 * kk + 0], e[8 * kk + 1]), pack_bf16x2(e[8 * kk + 2], e[8 * kk + 3]),
                        pack_bf16x2(e[8 * kk + 4], e[8 * kk + 5]), pack_bf16x2(e[8 * kk + 6], e[8 * kk + 7])});
  }

  // O^T += V^T P^T over two k-steps of 16 keys.  k-slot i of lane group g in
  // k-step kk is key 16 kk + 8 (i >> 2) + 4 g + (i & 3) (the lane's
  // e[8 kk + i]).  V^T rows come from two transposed reads of 4 keys each:
  // in 16-lane group G, source lane j supplies key 16 kk + 4 (G >> 1) +
  // (j >> 2) (+ 8 for the second read) and dims 4 (j & 3) .. +3 of the
  // group's 16-dim run 256 hf + 32 dt + 16 (G & 1), i.e. chunk
  // 32 hf + 4 dt + 2 (G & 1) + ((j >> 1) & 1), in group 4 hf + dt / 2.
  const int ln = opaque_lane();
  const int jj = ln & 15;
  const int gb = (ln >> 4) & 1;
  const int tA = 4 * (ln >> 5) + (jj >> 2);
  const int tB = tA + 8;
  const int sA = swz(tA), sB = swz(tB);
  const int cl0 = 2 * gb + ((jj >> 1) & 1);   // chunk within its group of 8, even dt
  const int lo = 4 * kGroupBytes * hf + 8 * (jj & 1);
  const int vA0 = tA * 128 + ((cl0 ^ sA) & 7) * 16 + lo;
  const int vA1 = tA * 128 + (((cl0 + 4) ^ sA) & 7) * 16 + lo;
  const int vB0 = tB * 128 + ((cl0 ^ sB) & 7) * 16 + lo;
  const int vB1 = tB * 128 + (((cl0 + 4) ^ sB) & 7) * 16 + lo;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int dt = 0; dt < kDimTiles; ++dt) {
      const int imm = kk * 16 * 128 + kGroupBytes * (dt >> 1);
      const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kb + ((dt & 1) ? vA1 : vA0) + imm));
      const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kb + ((dt & 1) ? vB1 : vB0) + imm));
      const u32x2 xa = __builtin_bit_cast(u32x2, va);
      const u32x2 xb = __builtin_bit_cast(u32x2, vb);
      const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{xa[0], xa[1], xb[0], xb[1]});
      o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[kk], o[dt], 0, 0, 0);
    }
  // Keep the reads of two fragments ahead of the MFMAs.
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int i = 0; i < 2 * kDimTiles - 2; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
}

// Per-unit setup shared by both kernels: loads this wave's Q^T (k-steps
// < QR into qf, the rest into its LDS area; negated when the scale is
// negative) and clears the accumulators.
// Lane-dependent values are derived from opaque_lane() here rather than
// passed in, so that they are not kept live across the slice loop.
template <int QR>
__device__ __forceinline__ void load_q(const DecodeParams& p, int u, int row_base, int hf, bool qneg,
                                       bf16x8 (&qf)[QR], uint8_t* qs_mine) {
  const int lane = opaque_lane();
  const int my_row = row_base + (lane & 31);
  const bool row_ok = my_row < p.R;
  const uint8_t* qrow = p.q + ((size_t)u * p.R + (row_ok ? my_row : 0)) * (2 * kDqk) + 576 * hf + 16 * (lane >> 5);
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks) {
    u32x4 v = *(const u32x4*)(qrow + 32 * ks);
    if (!row_ok) v = u32x4{0, 0, 0, 0};
    if (qneg) v ^= 0x80008000u;   // exact bf16 negation
    if (ks < QR)
      qf[ks < QR ? ks : 0] = __builtin_bit_cast(bf16x8, v);
    else
      *(u32x4*)(qs_mine + ((ks - QR) * 64 + lane) * 16) = v;
  }
}

// Epilogue of one unit: normalise and store O (bf16 out + lse when the unit
// has one split, else bf16 partials + fp32 lse into the split's workspace slot).
// Lane holds row l32, dims 256 hf + 32 dt + 8 (r >> 2) + 4 g + (r & 3); both
// halves hold the same row max, and each its own part of the row sum.
__device__ __forceinline__ void store_unit(const DecodeParams& p, const f32x16 (&o)[kDimTiles], float m_run,
                                           float l_sum, int u, int u0, int split0, int row_base, int hf) {
  const int lane = opaque_lane();
  const int my_row = row_base + (lane & 31);
  const bool row_ok = my_row < p.R;
  const int g = lane >> 5;
  const float inv = l_sum > 0.f ? 1.f / l_sum : 0.f;
  const float lse_nat =
      l_sum > 0.f ? ((m_run == -INFINITY ? 0.f : m_run) + fast_log2(l_sum)) * kLn2 : -INFINITY;
  const int k_u = p.num_splits[u + 1] - p.num_splits[u];
  const int split = p.num_splits[u] + (u == u0 ? split0 : 0);
  if (!row_ok) return;
  const size_t grow = (size_t)u * p.R + my_row;
  const int dbase = 256 * hf + 4 * g;
  if (k_u == 1) {
    uint16_t* orow = p.out + grow * kDv + dbase;
#pragma unroll
    for (int dt = 0; dt < kDimTiles; ++dt)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        *(u32x2*)(orow + 32 * dt + 8 * qd) = u32x2{pack_bf16x2(o[dt][4 * qd] * inv, o[dt][4 * qd + 1] * inv),
                                                  pack_bf16x2(o[dt][4 * qd + 2] * inv, o[dt][4 * qd + 3] * inv)};
    if (hf == 0 && g == 0) p.lse[grow] = lse_nat;
  } else {
    uint16_t* orow = p.ws_o + ((size_t)split * p.R + my_row) * kDv + dbase;
#pragma unroll
    for (int dt = 0; dt < kDimTiles; ++dt)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        *(u32x2*)(orow + 32 * dt + 8 * qd) = u32x2{pack_bf16x2(o[dt][4 * qd] * inv, o[dt][4 * qd + 1] * inv),
                                                  pack_bf16x2(o[dt][4 * qd + 2] * inv, o[dt][4 * qd + 3] * inv)};
    if (hf == 0 && g == 0) p.ws_lse[(size_t)split * p.R + my_row] = lse_nat;
  }
}

// Dense causal units: the block after the last key any row of 128-row
// tile rt may see (its last row has the widest window).  Blocks from there
// on are skipped; one block is always kept so that the unit still runs
// through its epilogue (its rows then see no key of this part).
__device__ __forceinline__ int causal_tile_end(const DecodeParams& p, int rt, int L, int jb, int je) {
  const int last_row = min(rt * kRowsPerWg + kRowsPerWg - 1, p.R - 1);
  const int W = min(max(L - p.s_q + 1 + last_row / p.h_q, 0), L);
  return min(je, max(jb + 1, (W + kPage - 1) / kPage));
}

// Work-item decode shared by both kernels (XCD-aware: consecutive block ids
// go to different XCDs, the row tiles of one part share an XCD and its L2).
struct Item {
  int part, rt, u0, j0, u1, j1, split0;
  const int32_t* unit_blocks;
};
__device__ __forceinline__ bool decode_item(const DecodeParams& p, Item& it) {
  work_item(blockIdx.x, p.num_parts, p.row_tiles, &it.part, &it.rt);
  if (it.part >= p.num_parts) return false;
  if (p.md[0] != p.num_parts || p.md[5] != kMagic || p.md[3] != p.units) return false;
  const int32_t* prow = p.md + kHeader + kPartRow * it.part;
  it.u0 = prow[0];
  it.j0 = prow[1];
  it.u1 = prow[2];
  it.j1 = prow[3];
  it.split0 = prow[4];
  it.unit_blocks = p.md + kHeader + kPartRow * p.num_parts;
  return it.u0 >= 0;
}

// ---- all eight waves in step (FP8 pages) ----------------------------------
template <int FMT, bool SPARSE>
__global__ __launch_bounds__(kThreads, 1) void wide_kernel(const DecodeParams p) {
  using G = Geo<FMT>;
  constexpr int QL = G::QL;
  constexpr int QR = kKSteps - QL;
  __shared__ __attribute__((aligned(1024))) uint8_t ring0[G::kRingBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t ring1[G::kRingBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t ring2[G::kRingBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t kbf[FMT == 1 ? kSliceBytes : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t xs[kWaves * kXchgBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t qs[kWaves * QL * 1024];
  __shared__ int32_t tab[SPARSE ? kTab : 1];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hf = wave & 1;    // dims half of this wave
  const int pr = wave >> 1;   // wave pair = 32-row group
  const int l32 = lane & 31;
  const int g = lane >> 5;
  Item it;
  if (!decode_item(p, it)) return;
  const int row_base = it.rt * kRowsPerWg + pr * kRowsPerPair;   // uniform
  const int my_row = row_base + l32;
  const bool row_ok = my_row < p.R;
  uint8_t* const qs_mine = qs + wave * QL * 1024;
  uint8_t* const xs_mine = xs + wave * kXchgBytes;
  const uint8_t* const xs_peer = xs + (wave ^ 1) * kXchgBytes;
  const float sc = fabsf(p.scale_log2);
  const bool qneg = p.scale_log2 < 0.f;

  for (int u = it.u0; u <= it.u1; ++u) {
    const int jb = (u == it.u0) ? it.j0 : 0;
    const int je_part = (u == it.u1) ? it.j1 : it.unit_blocks[u];
    const int b = SPARSE ? u / p.s_q : u;
    const int L = p.seqlens[b];
    const int je = (SPARSE || !p.causal) ? je_part : causal_tile_end(p, it.rt, L, jb, je_part);
    const int s_unit = SPARSE ? u % p.s_q : 0;
    const int s_row = SPARSE ? s_unit : (row_ok ? my_row / p.h_q : 0);
    const int W = p.causal ? min(max(L - p.s_q + 1 + s_row, 0), L) : L;
    const int Wunit = (SPARSE && p.causal) ? min(max(L - p.s_q + 1 + s_unit, 0), L) : L;
    const int W_lo = p.causal ? min(max(L - p.s_q + 1, 0), L) : L;   // every row sees keys < W_lo
    const int32_t* idx_row = SPARSE ? p.indices + (size_t)u * p.topk : nullptr;
    const int s_begin = 2 * jb;   // slices of this unit's blocks
    const int s_end = 2 * je;
    const int pos_end = kPage * je;   // sparse: index entries, resolved kTab at a time
    int tab_base = kPage * jb;
    if (SPARSE) fill_table<kThreads>(p, tab, b, tab_base, min(pos_end - tab_base, kTab), Wunit, idx_row);
    bf16x8 qf[QR];
    load_q(p, u, row_base, hf, qneg, qf, qs_mine);
    wait_vmem<0>();
    lds_barrier();   // tab complete

    float m_run = -INFINITY;
    float l_part = 0.f;
    f32x16 o[kDimTiles];
#pragma unroll
    for (int d = 0; d < kDimTiles; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[d][r] = 0.f;

    // Ring: slice s lives in slot (s - s_begin) % 3; two slices in flight.
    // A unit's block range is never empty, so it has at least two slices.
    uint32_t vis0 = issue_slice<FMT, SPARSE>(p, tab, tab_base, ring0, s_begin, L, true,
                                             SPARSE ? 0 : page_of(p, b, s_begin >> 1, L));
    uint32_t vis1 = issue_slice<FMT, SPARSE>(p, tab, tab_base, ring1, s_begin + 1, L, true,
                                             SPARSE ? 0 : page_of(p, b, (s_begin + 1) >> 1, L));
    uint32_t vis2 = 0u;

    int sl = s_begin;
    auto step = [&](auto slot) __attribute__((always_inline)) {
      constexpr int C = decltype(slot)::value;
      uint8_t* const rcur = C == 0 ? ring0 : (C == 1 ? ring1 : ring2);
      uint8_t* const rfree = C == 0 ? ring2 : (C == 1 ? ring0 : ring1);   // slot (C + 2) % 3
      uint32_t& vcur = C == 0 ? vis0 : (C == 1 ? vis1 : vis2);
      uint32_t& vfree = C == 0 ? vis2 : (C == 1 ? vis0 : vis1);
      // Slice sl must be in LDS; the copy of slice sl + 1 (the last
      // kPerWave loads of this wave) may still fly.
      wait_vmem<G::kPerWave>();
      lds_barrier();   // every wave is done with slice sl - 1 (slot rfree)
      const bool more = sl + 2 < s_end;
      if (SPARSE && more) {
        const int pos = kSlice * (sl + 2);
        if (pos - tab_base >= kTab) {   // the unit's range outgrew the table
          tab_base = pos;
          fill_table<kThreads>(p, tab, b, tab_base, min(pos_end - tab_base, kTab), Wunit, idx_row);
          lds_barrier();
        }
      }
      vfree = issue_slice<FMT, SPARSE>(p, tab, tab_base, rfree, sl + 2, L, more,
                                       (SPARSE || !more) ? 0 : page_of(p, b, (sl + 2) >> 1, L));
      const uint32_t vmask = vcur;
      const int key0 = sl * kSlice;
      ++sl;
      if (vmask == 0u) return;   // no visible key in this slice (uniform)
      const uint8_t* kb = rcur;
      if constexpr (FMT == 1) {
        dequant_slice<kThreads>(rcur, kbf);
        lds_barrier();
        kb = kbf;
      }
      f32x16 s = qk_partial<QR>(kb, qf, qs_mine, hf);
      xchg_put(xs_mine, s, lane);
      lds_barrier();
      xchg_add(xs_peer, s, lane);
      const bool full = SPARSE ? (vmask == 0xFFFFFFFFu) : (key0 + kSlice <= W_lo);
      softmax_pv<SPARSE>(s, o, m_run, l_part, kb, vmask, full, W, key0, sc, hf, g);
    };
    while (sl < s_end) {
      step(Slot<0>{});
      if (sl >= s_end) break;
      step(Slot<1>{});
      if (sl >= s_end) break;
      step(Slot<2>{});
    }
    store_unit(p, o, m_run, l_part + xor32(l_part), u, it.u0, it.split0, row_base, hf);
    wait_vmem<0>();
    lds_barrier();   // the next unit refills the table and the ring
  }
}

// ---- two wave groups half a slice apart (dense bf16 pages) -----------------
// Group 0 (waves 0-3) leads, group 1 (waves 4-7) trails by one half-step;
// every SIMD runs one wave of each.  Half-step k of a unit (k = 0, 1, ...)
// ends with a workgroup barrier; in it group 0 runs the QK half of slice
// k / 2 (k even) or the softmax + PV half of slice (k - 1) / 2 (k odd), and
// group 1 the same one half-step later, so that one group's VALU softmax
// overlaps the other's MFMAs.  Slice s is read in half-steps 2 s .. 2 s + 2.
// Each group copies its share of slice s + 2 at the end of its softmax + PV
// half of slice s (group 0: half-step 2 s + 1, group 1: 2 s + 2), into the
// slot of slice s - 1 (last read in 2 s), while the other group is in a QK
// half; both shares are waited for by the end of half-step 2 s + 3, before
// group 0 reads the slice.  Waves 0-3 copy 5 KiB of a slice, waves 4-7 4 KiB.
__global__ __launch_bounds__(kThreads, 1) void offset_kernel(const DecodeParams p) {
  using G = Geo<0>;
  constexpr int QL = G::QL;
  constexpr int QR = kKSteps - QL;
  __shared__ __attribute__((aligned(1024))) uint8_t ring0[G::kRingBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t ring1[G::kRingBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t ring2[G::kRingBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t xs[kWaves * kXchgBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t qs[kWaves * QL * 1024];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hf = wave & 1;
  const int pr = wave >> 1;
  const int grp = wave >> 2;   // 0 leads, 1 trails by half a slice
  const int g = lane >> 5;
  Item it;
  if (!decode_item(p, it)) return;
  const int row_base = it.rt * kRowsPerWg + pr * kRowsPerPair;   // uniform
  const int my_row = row_base + (lane & 31);
  const bool row_ok = my_row < p.R;
  uint8_t* const qs_mine = qs + wave * QL * 1024;
  uint8_t* const xs_mine = xs + wave * kXchgBytes;
  const uint8_t* const xs_peer = xs + (wave ^ 1) * kXchgBytes;
  const float sc = fabsf(p.scale_log2);
  const bool qneg = p.scale_log2 < 0.f;

  for (int u = it.u0; u <= it.u1; ++u) {
    const int jb = (u == it.u0) ? it.j0 : 0;
    const int je_part = (u == it.u1) ? it.j1 : it.unit_blocks[u];
    const int b = u;
    const int L = p.seqlens[b];
    const int je = p.causal ? causal_tile_end(p, it.rt, L, jb, je_part) : je_part;
    const int s_row = row_ok ? my_row / p.h_q : 0;
    const int W = p.causal ? min(max(L - p.s_q + 1 + s_row, 0), L) : L;
    const int W_lo = p.causal ? min(max(L - p.s_q + 1, 0), L) : L;
    const int s_begin = 2 * jb;
    const int s_end = 2 * je;   // at least s_begin + 2
    bf16x8 qf[QR];
    load_q(p, u, row_base, hf, qneg, qf, qs_mine);
    wait_vmem<0>();

    float m_run = -INFINITY;
    float l_part = 0.f;
    f32x16 o[kDimTiles];
#pragma unroll
    for (int d = 0; d < kDimTiles; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[d][r] = 0.f;

    // Slices s_begin and s_begin + 1, both groups' shares.
    copy_all(prep_copy(p, ring0, s_begin, L, true, page_of(p, b, s_begin >> 1, L)));
    copy_all(prep_copy(p, ring1, s_begin + 1, L, true, page_of(p, b, (s_begin + 1) >> 1, L)));
    int page_pf = page_of(p, b, min(s_begin + 2, s_end - 1) >> 1, L);
    wait_vmem<4>();               // slice s_begin (at most one slice of copies pending)
    lds_barrier();                // slice s_begin is in LDS
    if (grp == 1) lds_barrier();  // group 1 starts one half-step later

    int sl = s_begin;
    auto step = [&](auto slot) __attribute__((always_inline)) {
      constexpr int C = decltype(slot)::value;
      uint8_t* const rcur = C == 0 ? ring0 : (C == 1 ? ring1 : ring2);
      uint8_t* const rfree = C == 0 ? ring2 : (C == 1 ? ring0 : ring1);   // slot (C + 2) % 3
      const int key0 = sl * kSlice;
      const uint32_t vmask = key0 >= L ? 0u : (key0 + kSlice <= L ? 0xFFFFFFFFu : (1u << (L - key0)) - 1u);
      // QK half-step.
      f32x16 s;
      if (vmask != 0u) {
        s = qk_partial<QR>(rcur, qf, qs_mine, hf);
        xchg_put(xs_mine, s, lane);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
      }
      if (grp == 1) wait_vmem<0>();   // its share of slice sl + 1
      lds_barrier();
      // softmax + PV half-step, then this group's share of slice sl + 2.
      if (vmask != 0u) {
        xchg_add(xs_peer, s, lane);
        softmax_pv<false>(s, o, m_run, l_part, rcur, vmask, key0 + kSlice <= W_lo, W, key0, sc, hf, g);
      }
      copy_all(prep_copy(p, rfree, sl + 2, L, sl + 2 < s_end, page_pf));
      page_pf = page_of(p, b, min(sl + 3, s_end - 1) >> 1, L);
      if (grp == 0) wait_vmem<G::kPerWave>();   // its share of slice sl + 1
      lds_barrier();
      ++sl;
    };
    while (sl < s_end) {
      step(Slot<0>{});
      if (sl >= s_end) break;
      step(Slot<1>{});
      if (sl >= s_end) break;
      step(Slot<2>{});
    }
    if (grp == 0) lds_barrier();   // group 0 sits out group 1's last half-step
    store_unit(p, o, m_run, l_part + xor32(l_part), u, it.u0, it.split0, row_base, hf);
    wait_vmem<0>();
    lds_barrier();   // the next unit reuses the ring
  }
}

}  // namespace wide

hipError_t launch_wide(const DecodeParams& p, int kv_format, dim3 grid, hipStream_t stream) {
  const bool sparse = p.indices != nullptr;
  if (kv_format == 0) {
    if (sparse)
      hipLaunchKernelGGL((wide::wide_kernel<0, true>), grid, dim3(wide::kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((wide::offset_kernel), grid, dim3(wide::kThreads), 0, stream, p);
  } else {
    if (sparse)
      hipLaunchKernelGGL((wide::wide_kernel<1, true>), grid, dim3(wide::kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((wide::wide_kernel<1, false>), grid, dim3(wide::kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace mla
