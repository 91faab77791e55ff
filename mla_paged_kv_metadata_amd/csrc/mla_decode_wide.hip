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
//   * FP8 slices are copied raw into their own ring.  QK^T reads the raw
//     e4m3 codes on the fp8 MFMA (below); for PV the slice is dequantised
//     (e4m3 -> fp32, times the group scale, -> bf16) into a bf16 slice by
//     all threads.
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
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Per-format geometry: ring slot size, copy instructions (64 lanes x 16 B)
// per slice and per wave, and QL = k-steps of Q kept in LDS instead of
// VGPRs (LDS: bf16 3 x 36 KiB ring + 32 KiB exchange + 16 KiB Q (+ 4 KiB
// sparse table) = 160 KiB at most; FP8 3 x 21 KiB ring + 32 KiB V slice + 32
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
    if (!SPARSE && active && (sl + 1) * kSlice <= L) {
      // Every key of the slice is in the sequence: its 32 rows are
      // consecutive in one page, and chunk q of the slice (row q / 41,
      // chunk q % 41) sits at byte 16 q of that run, so the copy is linear:
      // instruction inst moves bytes 1024 inst .. + 1023 from a uniform
      // base; lanes past the slice's end re-read its last chunk.
      const uint8_t* const base = p.kcache + ((size_t)page_in * kPage + (sl & 1) * kSlice) * kFp8RowBytes;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        int inst = wave + kWaves * i;
        if (inst >= kInst) inst = wave;
        const uint32_t voff = (uint32_t)min(inst * 1024 + 16 * ln, kSlice * kFp8RowBytes - 16);
        lds_dma16_s(base, voff, dst + inst * 1024);
      }
      return mask;
    }
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

// The whole bf16 slice sl into `slot` by the four waves of the trailing
// group (waves 4-7): wave 4 + k issues copy instructions inst = 4 G + k,
// chunk group G = 0..8 of keys 8 k .. 8 k + 7 (as bf16_copy_src), nine per
// wave.  The slice's keys are consecutive rows of one page, so the page
// start is a uniform base and each lane adds its row within the page and
// its swizzled chunk; keys past the sequence take its last key, an inactive
// slice row 0 of the pool (as slot_row).  prep_slice_copy forms the
// addresses once; issue(G) sends instruction G, so that the nine can be
// spread between other instructions (the QK MFMAs).  Callers skip the copy
// for an empty pool.
struct SliceCopy {
  const uint8_t* base;
  uint32_t voff;
  uint8_t* slot;
  int k;
  __device__ __forceinline__ void issue(int G) const { lds_dma16_s(base + 128 * G, voff, slot + 1024 * (4 * G + k)); }
};
constexpr int kCopyInst = kSliceBytes / kGroupBytes;   // 9 per wave

__device__ __forceinline__ SliceCopy prep_slice_copy(const DecodeParams& p, uint8_t* slot, int sl, int L, bool active,
                                                     int page_in) {
  const int ln = opaque_lane();
  const int k = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & 3;
  const int t = 8 * k + (ln >> 3);
  const int lim = active ? max(L - 1 - (sl >> 1) * kPage, 0) : 0;   // last row of the page to read
  const int page = active ? page_in : 0;
  const int r = min((sl & 1) * kSlice + t, lim);
  SliceCopy c;
  c.voff = __umul24(r, kBf16RowBytes) + 16 * ((ln & 7) ^ swz(t));
  c.base = p.kcache + (size_t)page * (kPage * kBf16RowBytes);
  c.slot = slot;
  c.k = k;
  return c;
}

__device__ __forceinline__ void copy_slice_trailing(const DecodeParams& p, uint8_t* slot, int sl, int L, bool active,
                                                    int page_in) {
  if (p.num_pages == 0) return;
  const SliceCopy c = prep_slice_copy(p, slot, sl, L, active, page_in);
#pragma unroll
  for (int G = 0; G < kCopyInst; ++G) c.issue(G);
}

// ---- per-slice pieces shared by both kernels ------------------------------

// Per-lane LDS offsets of the bf16 slice reads of lane ln, packed into one
// register.  Bits 0..15: the K fragment of QK k-step 0 (key l32, chunk
// 36 hf + g; left 0 when QK is false).  Bits 16..31: the first V^T read of
// the PV product (key 4 (l >> 5) + (l & 15) / 4, chunk 32 hf + 2 ((l >> 4)
// & 1) + ((l >> 1) & 1), plus 8 bytes for odd lanes).  Every other fragment
// of a slice differs from these by an XOR of the swizzled chunk bits (bits
// 4..6) and an immediate, because stepping the chunk by 2 or 4 or the key by
// 8 flips single bits of the swizzled position.  The empty asm keeps the
// value as computed: with ln = threadIdx.x & 63 outside the slice loop it
// stays in one register, with opaque_lane() inside the loop it is rebuilt
// in every slice.
template <bool QK>
__device__ __forceinline__ int slice_lane_offsets(int ln, int hf) {
  const int t = ln & 31;
  const int qk0 = QK ? t * 128 + (((4 * hf + (ln >> 5)) ^ swz(t)) & 7) * 16 + 4 * kGroupBytes * hf : 0;
  const int jj = ln & 15;
  const int tA = 4 * (ln >> 5) + (jj >> 2);
  const int cl0 = 2 * ((ln >> 4) & 1) + ((jj >> 1) & 1);
  const int v0 = tA * 128 + ((cl0 ^ swz(tA)) & 7) * 16 + 4 * kGroupBytes * hf + 8 * (jj & 1);
  int packed = qk0 | (v0 << 16);
  asm volatile("" : "+v"(packed));
  return packed;
}

// Partial S^T = K Q^T over this wave's 288 QK dims.  A = K: lane holds key
// l32, dims 288 hf + 16 ks + 8 g + 0..7, i.e. chunk c = 36 hf + 2 ks + g of
// its row, in group c / 8 = (hf ? 4 : 0) + (2 ks + 4 hf) / 8.  The swizzled
// position within the group repeats every 4 k-steps: k-steps 4 i + m read
// at the k-step-0 offset XOR 32 m (m < 2), or XOR 32 m plus one group for
// wave half 1 (m >= 2), plus i groups.  B = Q^T from registers (k-steps
// < QR) or from this wave's LDS area.  With COPY the wave also issues the
// nine instructions of slice copy cp, one after every other MFMA of the
// chain, where their issue time is hidden behind it.
template <int QR, bool COPY = false>
__device__ __forceinline__ f32x16 qk_partial(const uint8_t* kb, const bf16x8 (&qf)[QR], const uint8_t* qs_mine,
                                             int hf, int lofs, const SliceCopy& cp = SliceCopy{}) {
  f32x16 s;
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = 0.f;
  const int ln = opaque_lane();
  int a = lofs & 0xFFFF;
  asm volatile("" : "+v"(a));   // the four offsets below are formed here, not kept live
  const uint8_t* const kp[4] = {kb + a, kb + (a ^ 32), kb + (a ^ 64) + hf * kGroupBytes,
                                kb + (a ^ 96) + hf * kGroupBytes};
  // Three fragment reads stay ahead of the MFMA chain.  The order is pinned
  // with scheduling barriers: left to itself the scheduler moves each read
  // next to its MFMA when the kernel is near its register limit, and every
  // MFMA then waits out a whole LDS round trip.
  auto frag = [&](int ks) -> bf16x8 { return *(const bf16x8*)(kp[ks & 3] + kGroupBytes * (ks >> 2)); };
  bf16x8 a0 = frag(0), a1 = frag(1), a2 = frag(2);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks) {
    bf16x8 bq;
    if (ks < QR)
      bq = qf[ks < QR ? ks : 0];
    else
      bq = *(const bf16x8*)(qs_mine + ((ks - QR) * 64 + ln) * 16);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bq, s, 0, 0, 0);
    a0 = a1;
    a1 = a2;
    if (ks + 3 < kKSteps) a2 = frag(ks + 3);
    if (COPY && (ks & 1) == 0 && (ks >> 1) < kCopyInst) cp.issue(ks >> 1);
    __builtin_amdgcn_sched_barrier(0);
  }
  return s;
}

// ---- FP8 pools: QK on the fp8 MFMA ----------------------------------------
// The 512 NoPE dims of the scores come from v_mfma_scale_f32_32x32x64_f8f6f4
// with the e4m3 codes of the raw slice as the A operand (exact, no
// conversion) and the query as the B operand in e4m3, per row and per wave
// half (dims 256 hf .. 256 hf + 255) scaled by a power of two 2^p: each
// bf16 query value x / 2^p is split into hi = e4m3(x / 2^p) and
// lo = e4m3(16 (x / 2^p - hi)), which is exact whenever the remainder's
// exponent stays within e4m3's range (a bf16 value has 8 significant bits,
// hi carries 4 and the remainder at most 4 more), and lo enters the MFMA
// with the operand scale 2^-4.  With `lo` dropped (QLO = false) the query is
// quantised to e4m3 per row half: half the MFMAs, with a relative error of
// up to 2^-4 per query value, and the row half's scale is 2^p * alpha
// with alpha = (x . x) / (x . hi) over its 256 dims (x = q / 2^p), which
// makes the rounding error orthogonal to the query (attention weights keys
// along q most, so this keeps the rounding from shifting all their scores
// together).  The RoPE dims stay bf16.  The four group
// scales of a key are applied to the partial sums (below), so no product
// code * scale is ever rounded.

// Per-slice scale table, written by the last wave: for wave half h and key
// t, groups 2 h and
// 2 h + 1: scl[32 (2 h) + t] and scl[32 (2 h + 1) + t] the scales, and
// scl[32 (4 + h) + t] their ratio (v_rcp_f32).  A group whose scale is 0
// gets its 128 codes zeroed in the raw slice and scale 1, which gives the
// same zeros (code * 0) and keeps the ratio finite.
__device__ __forceinline__ void fp8_scale_table(uint8_t* raw, float* scl) {
  const int w = (int)threadIdx.x - (kThreads - 64);
  if (w < 0) return;
  const int t = w & (kSlice - 1);
  const int h = w >> 5;
  uint8_t* row = raw + t * kFp8RowBytes;
  const f32x2 sv = *(const f32x2*)(row + kFp8ScaleOff + 8 * h);
  float s0 = sv[0], s1 = sv[1];
  if (s0 == 0.f || s1 == 0.f) {
#pragma unroll 1
    for (int i = 0; i < 16; ++i)
      if ((i < 8 ? s0 : s1) == 0.f) *(u32x4*)(row + 256 * h + 16 * i) = u32x4{0u, 0u, 0u, 0u};
    s0 = s0 == 0.f ? 1.f : s0;
    s1 = s1 == 0.f ? 1.f : s1;
  }
  scl[kSlice * (2 * h) + t] = s0;
  scl[kSlice * (2 * h + 1) + t] = s1;
  scl[kSlice * (4 + h) + t] = s0 * __builtin_amdgcn_rcpf(s1);
}

// The query of one unit for the fp8 path: lane l holds row row_base + l % 32
// and, for MFMA m = 0..3, NoPE dims 256 hf + 64 m + 32 (l / 32) .. + 31 in
// qh[m] (and ql[m]) as 32 e4m3 bytes; the RoPE k-steps j = 0, 1 (dims
// 512 + 32 hf + 16 j + 8 (l / 32) .. + 7) as bf16 in the wave's LDS area
// (1 KiB each, lane-major); *qsc = 2^p (times alpha without QLO).
// Rows past R are zero (p = 0).  A negative softmax scale negates q.
template <bool QLO>
__device__ __forceinline__ void load_q_fp8(const DecodeParams& p, int u, int row_base, int hf, bool qneg,
                                           i32x8 (&qh)[4], i32x8 (&ql)[QLO ? 4 : 1], uint8_t* qs_mine,
                                           float* qsc) {
  const int lane = opaque_lane();
  const int my_row = row_base + (lane & 31);
  const bool row_ok = my_row < p.R;
  const int hh = lane >> 5;
  const uint8_t* qrow = p.q + ((size_t)u * p.R + (row_ok ? my_row : 0)) * (2 * kDqk);
  const uint32_t neg = qneg ? 0x80008000u : 0u;
  // Rows past R read row 0 (in bounds) and are zeroed with a mask.  A select
  // on the loaded value would be turned into a branch around each load, and
  // the 18 loads would then wait out their memory round trips one by one.
  const uint32_t keep = row_ok ? 0xFFFFFFFFu : 0u;
  u32x4 v[4][4];   // [m][16-byte part]: 8 bf16 each
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const u32x4 x = *(const u32x4*)(qrow + 2 * (256 * hf + 64 * m + 32 * hh) + 16 * k);
      v[m][k] = (x ^ neg) & keep;
    }
#pragma unroll
  for (int j = 0; j < 2; ++j) {   // RoPE k-steps to the wave's LDS area
    const u32x4 x = *(const u32x4*)(qrow + 2 * (512 + 32 * hf + 16 * j + 8 * hh));
    *(u32x4*)(qs_mine + (j * 64 + lane) * 16) = (x ^ neg) & keep;
  }
  // Largest magnitude over the row's 256 dims of this half (both lanes of
  // the row), as bf16 bit patterns without sign.
  uint32_t amax = 0;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = v[m][k][e];
        amax = max(amax, max(w & 0x7FFFu, (w >> 16) & 0x7FFFu));
      }
  amax = max(amax, (uint32_t)__builtin_bit_cast(int, xor32(__builtin_bit_cast(float, (int)amax))));
  // 2^p with p = (exponent of amax) - 7, so every |x| / 2^p < 256 <= 448;
  // p = 0 for a zero row.  Scaling by powers of two is exact.
  const int e = (int)(amax >> 7);                       // biased bf16/fp32 exponent
  const int pe = amax == 0 ? 127 : max(e - 7, 1);       // biased exponent of 2^p
  const float two_p = __builtin_bit_cast(float, pe << 23);
  const float inv = __builtin_bit_cast(float, (254 - pe) << 23);   // 2^-p
  float xx = 0.f, xh = 0.f;   // x . x and x . hi (QLO = false)
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    int hi[8], lo[8];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {   // 4 values -> one dword of e4m3
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t w = v[m][k][2 * e2 + (i >> 1)];
          x[i] = __builtin_bit_cast(float, (i & 1) ? (w & 0xFFFF0000u) : (w << 16)) * inv;
        }
        int h = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
        h = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], h, true);
        hi[2 * k + e2] = h;
        const f32x2 b0 = __builtin_amdgcn_cvt_pk_f32_fp8(h, false);
        const f32x2 b1 = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
        if constexpr (QLO) {
          int l = __builtin_amdgcn_cvt_pk_fp8_f32(16.f * (x[0] - b0[0]), 16.f * (x[1] - b0[1]), 0, false);
          l = __builtin_amdgcn_cvt_pk_fp8_f32(16.f * (x[2] - b1[0]), 16.f * (x[3] - b1[1]), l, true);
          lo[2 * k + e2] = l;
        } else {
          xx += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
          xh += x[0] * b0[0] + x[1] * b0[1] + x[2] * b1[0] + x[3] * b1[1];
        }
      }
#pragma unroll
    for (int i = 0; i < 8; ++i) qh[m][i] = hi[i];
    if constexpr (QLO) {
#pragma unroll
      for (int i = 0; i < 8; ++i) ql[QLO ? m : 0][i] = lo[i];
    }
  }
  if constexpr (QLO) {
    *qsc = two_p;
  } else {
    xx += xor32(xx);
    xh += xor32(xh);
    *qsc = two_p * (xh > 0.f ? xx / xh : 1.f);
  }
}

// Partial S^T of this wave's half for FP8 pools: NoPE groups A = 2 hf (fp8
// MFMAs m = 0, 1) and B = 2 hf + 1 (m = 2, 3) in one accumulator,
// s = ((sum_A * scA / scB) + sum_B) * scB * qsc (qsc = 2^p, times alpha
// without the low part), then the two RoPE k-steps (bf16, read from the raw
// rows as stored).  Output register r holds key 8 (r >> 2) + 4 (l / 32) +
// (r & 3) of the slice for query row l % 32.
template <bool QLO>
__device__ __forceinline__ f32x16 qk_fp8(const uint8_t* raw, const float* scl, const i32x8 (&qh)[4],
                                         const i32x8 (&ql)[QLO ? 4 : 1], const uint8_t* qs_mine, float qsc,
                                         int hf) {
  const int ln = opaque_lane();
  const int t = ln & 31;
  const int hh = ln >> 5;
  const uint8_t* krow = raw + t * kFp8RowBytes + 256 * hf + 32 * hh;
  f32x16 s;
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = 0.f;
  auto frag = [&](int m) -> i32x8 {
    const u32x4 a0 = *(const u32x4*)(krow + 64 * m);
    const u32x4 a1 = *(const u32x4*)(krow + 64 * m + 16);
    return __builtin_bit_cast(i32x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  const float* rA = scl + kSlice * (4 + hf) + 4 * hh;
  const float* sB = scl + kSlice * (2 * hf + 1) + 4 * hh;
  if constexpr (QLO) {
    // Two MFMAs per A operand; one A operand (8 registers) in flight at a
    // time: this variant has no registers to spare for more.
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (m == 2) {   // group A done: s *= scA / scB
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 r4 = *(const f32x4*)(rA + 8 * j);
#pragma unroll
          for (int i = 0; i < 4; ++i) s[4 * j + i] *= r4[i];
        }
      }
      const i32x8 a = frag(m);
      s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qh[m], s, 0, 0, 0, 127, 0, 127);
      s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, ql[QLO ? m : 0], s, 0, 0, 0, 127, 0, 123);
      asm volatile("" ::: "memory");
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 b4 = *(const f32x4*)(sB + 8 * j);
#pragma unroll
      for (int i = 0; i < 4; ++i) s[4 * j + i] *= b4[i] * qsc;
    }
  } else {
    // One MFMA per A operand: the next A operand is read while the current
    // one's MFMA runs, and each fold's scales while the MFMA before it runs
    // (order pinned by scheduling barriers).
    i32x8 acur = frag(0);
    f32x4 sc4[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (m == 2) {   // group A done: s *= scA / scB
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[4 * j + i] *= sc4[j][i];
      }
      const i32x8 a = acur;
      if (m < 3) acur = frag(m + 1);
      s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qh[m], s, 0, 0, 0, 127, 0, 127);
      if (m == 1 || m == 3) {
        const float* src = m == 1 ? rA : sB;
#pragma unroll
        for (int j = 0; j < 4; ++j) sc4[j] = *(const f32x4*)(src + 8 * j);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) s[4 * j + i] *= sc4[j][i] * qsc;
  }
  // RoPE dims 512 + 32 hf + 16 j + 8 hh .. + 7, bf16 as stored in the raw row.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const bf16x8 a = *(const bf16x8*)(raw + t * kFp8RowBytes + kFp8RopeOff + 2 * (32 * hf + 16 * j + 8 * hh));
    const bf16x8 b = *(const bf16x8*)(qs_mine + (j * 64 + ln) * 16);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, s, 0, 0, 0);
  }
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
// AHEAD V^T fragments are read ahead of the PV MFMAs (measured: 3 in the
// lock-step kernel, 2 in offset_kernel, where a third was not faster).
template <bool SPARSE, int AHEAD>
__device__ __forceinline__ void softmax_pv(f32x16& s, f32x16 (&o)[kDimTiles], float& m_run, float& l_part,
                                           const uint8_t* kb, uint32_t vmask, bool full, int W, int key0,
                                           float sc, int hf, int g, int lofs) {
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
  // Odd dt moves the chunk by 4 (XOR 64 on the swizzled offset); the
  // second read's key + 8 moves 1024 bytes and flips swizzle bit 0 (XOR 16).
  int v0 = lofs >> 16;
  asm volatile("" : "+v"(v0));   // as in qk_partial
  const uint8_t* const pA0 = kb + v0;
  const uint8_t* const pA1 = kb + (v0 ^ 64);
  const uint8_t* const pB0 = kb + (v0 ^ 16) + 1024;
  const uint8_t* const pB1 = kb + (v0 ^ 80) + 1024;
  // MFMA i = 8 kk + dt reads its V^T fragment AHEAD MFMAs earlier; the
  // order is pinned with scheduling barriers (as in qk_partial): left to
  // the scheduler, the lock-step kernels kept fewer reads in flight.
  auto vfrag = [&](int i) -> bf16x8 {
    const int kk = i / kDimTiles, dt = i % kDimTiles;
    const int imm = kk * 16 * 128 + kGroupBytes * (dt >> 1);
    const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(((dt & 1) ? pA1 : pA0) + imm));
    const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(((dt & 1) ? pB1 : pB0) + imm));
    const u32x2 xa = __builtin_bit_cast(u32x2, va);
    const u32x2 xb = __builtin_bit_cast(u32x2, vb);
    return __builtin_bit_cast(bf16x8, u32x4{xa[0], xa[1], xb[0], xb[1]});
  };
  bf16x8 f[AHEAD];
#pragma unroll
  for (int j = 0; j < AHEAD; ++j) f[j] = vfrag(j);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 2 * kDimTiles; ++i) {
    const int kk = i / kDimTiles, dt = i % kDimTiles;
    o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[0], pb[kk], o[dt], 0, 0, 0);
#pragma unroll
    for (int j = 0; j + 1 < AHEAD; ++j) f[j] = f[j + 1];
    if (i + AHEAD < 2 * kDimTiles) f[AHEAD - 1] = vfrag(i + AHEAD);
    __builtin_amdgcn_sched_barrier(0);
  }
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
  int L0, n0;   // length and block count of the first unit (from the part row)
  const int32_t* unit_blocks;
};
// A schedule header that does not match the call gives every row out = 0
// and lse = NaN (fill_mismatch) and no work item.
// A uniform int32 the kernel never writes, through the scalar cache (waited
// for by lgkmcnt, so vector-memory waits do not cover it and it does not
// hold up the copies in flight).
__device__ __forceinline__ int scalar_ld(const int32_t* base, int i) {
  return ((const __attribute__((address_space(4))) int32_t*)base)[i];
}

// The header and the part row are read together (one round trip);
// workgroups past the last part read the last part's row and then stop.
__device__ __forceinline__ bool decode_item(const DecodeParams& p, Item& it) {
  work_item(blockIdx.x, p.num_parts, p.row_tiles, &it.part, &it.rt);
  const int32_t* prow = p.md + kHeader + kPartRow * min(it.part, p.num_parts - 1);
  const int h0 = p.md[0], h3 = p.md[3], h5 = p.md[5];
  it.u0 = prow[0];
  it.j0 = prow[1];
  it.u1 = prow[2];
  it.j1 = prow[3];
  it.split0 = prow[4];
  it.L0 = prow[5];
  it.n0 = prow[6];
  if (!header_ok(p, h0, h3, h5)) {
    fill_mismatch<kThreads>(p);
    return false;
  }
  if (it.part >= p.num_parts) return false;
  it.unit_blocks = p.md + kHeader + kPartRow * p.num_parts;
  return it.u0 >= 0;
}

// ---- all eight waves in step (FP8 pages) ----------------------------------
// QLO (FP8): the query's e4m3 remainder part is used (exact products);
// without it, the query is quantised to e4m3 per row half.
template <int FMT, bool SPARSE, bool QLO = true>
__global__ __launch_bounds__(kThreads, 1) void wide_kernel(const DecodeParams p) {
  using G = Geo<FMT>;
  constexpr int QL = FMT == 1 ? 2 : G::QL;   // FP8: the RoPE query in LDS, the rest in registers
  constexpr int QR = FMT == 1 ? 1 : kKSteps - QL;
  __shared__ __attribute__((aligned(1024))) uint8_t ring0[G::kRingBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t ring1[G::kRingBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t ring2[G::kRingBytes];
  // FP8: the slice's V dims (512) dequantised to bf16, chunk groups 0-7 of
  // the slice layout (the RoPE group is read from the raw rows).
  __shared__ __attribute__((aligned(1024))) uint8_t kbf[FMT == 1 ? 8 * kGroupBytes : 16];
  static_assert(kSlice * 32 / kThreads == 2, "two dequantisation items per thread and slice");
  __shared__ __attribute__((aligned(1024))) uint8_t xs[kWaves * kXchgBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t qs[kWaves * QL * 1024];
  __shared__ int32_t tab[SPARSE ? kTab : 1];
  __shared__ __attribute__((aligned(16))) float scl[FMT == 1 ? 6 * kSlice : 4];   // FP8 scales, ratios

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hf = wave & 1;    // dims half of this wave
  const int pr = wave >> 1;   // wave pair = 32-row group
  const int l32 = lane & 31;
  const int g = lane >> 5;
  Item it;
  if (!decode_item(p, it)) return;
  // The packed slice-read offsets stay in a register for the whole kernel,
  // except in the exact dense FP8 variant, which is at its register limit
  // and rebuilds them in every slice (measured: holding them there spills
  // inside the slice loop and costs 10 %).
  constexpr bool kLofsHeld = !(FMT == 1 && !SPARSE && QLO);
  const int lofs_held = kLofsHeld ? slice_lane_offsets<FMT == 0>(lane, hf) : 0;
  const int row_base = it.rt * kRowsPerWg + pr * kRowsPerPair;   // uniform
  const int my_row = row_base + l32;
  const bool row_ok = my_row < p.R;
  uint8_t* const qs_mine = qs + wave * QL * 1024;
  uint8_t* const xs_mine = xs + wave * kXchgBytes;
  const uint8_t* const xs_peer = xs + (wave ^ 1) * kXchgBytes;
  const float sc = fabsf(p.scale_log2);
  const bool qneg = p.scale_log2 < 0.f;

  // Length and block count of the current unit: the part row carries them
  // for the first unit; those of the next are loaded at each unit start and
  // waited for with the unit's own loads.
  int L_nx = it.L0, n_nx = it.n0;
  for (int u = it.u0; u <= it.u1; ++u) {
    const int jb = (u == it.u0) ? it.j0 : 0;
    const int je_part = (u == it.u1) ? it.j1 : n_nx;
    const int b = SPARSE ? u / p.s_q : u;
    const int L = L_nx;
    if (u < it.u1) {
      n_nx = scalar_ld(it.unit_blocks, u + 1);
      L_nx = scalar_ld(p.seqlens, SPARSE ? (u + 1) / p.s_q : u + 1);
    }
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
    // Sparse: the index entries are loaded first, and the query loads go
    // out behind them (one round trip for both); the block-table lookups
    // follow once the query is in registers.
    static_assert(kTab <= 2 * kThreads, "two table entries per thread");
    const int tab_count = SPARSE ? min(pos_end - tab_base, kTab) : 0;
    int2 tix = make_int2(-1, -1);
    if (SPARSE) tix = fill_table_issue<kThreads>(p, tab_base, tab_count, idx_row);
    bf16x8 qf[QR];
    i32x8 qh[FMT == 1 ? 4 : 1], ql[FMT == 1 && QLO ? 4 : 1];
    float qsc = 1.f;
    if constexpr (FMT == 1)
      load_q_fp8<QLO>(p, u, row_base, hf, qneg, qh, ql, qs_mine, &qsc);
    else
      load_q(p, u, row_base, hf, qneg, qf, qs_mine);
    if (SPARSE) fill_table_finish<kThreads>(p, tab, b, tab_count, Wunit, tix);
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
          fill_table<kThreads, kTab / kThreads>(p, tab, b, tab_base, min(pos_end - tab_base, kTab), Wunit, idx_row);
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
      const int lofs = kLofsHeld ? lofs_held : slice_lane_offsets<FMT == 0>(opaque_lane(), hf);
      f32x16 s;
      if constexpr (FMT == 1) {
        // QK^T reads the raw slice; V is dequantised into kbf (scaled
        // bf16).  Dequantising after QK^T (published by the exchange barrier
        // below) lets each wave start its MFMAs one dequantisation earlier;
        // the exact sparse variant keeps the dequantisation first, where the
        // other order spills more registers (measured slower).
        constexpr bool kDequantFirst = SPARSE && QLO;
        if constexpr (kDequantFirst) {
#pragma unroll 1
          for (int i = 0; i < 2; ++i) dequant_item<kThreads>(rcur, kbf, i);
        }
        fp8_scale_table(rcur, scl);
        lds_barrier();
        s = qk_fp8<QLO>(rcur, scl, qh, ql, qs_mine, qsc, hf);
        if constexpr (!kDequantFirst) {
          dequant_item<kThreads>(rcur, kbf, 0);
          dequant_item<kThreads>(rcur, kbf, 1);
        }
        kb = kbf;
      } else {
        s = qk_partial<QR>(kb, qf, qs_mine, hf, lofs);
      }
      xchg_put(xs_mine, s, lane);
      lds_barrier();
      xchg_add(xs_peer, s, lane);
      const bool full = SPARSE ? (vmask == 0xFFFFFFFFu) : (key0 + kSlice <= W_lo);
      softmax_pv<SPARSE, 3>(s, o, m_run, l_part, kb, vmask, full, W, key0, sc, hf, g, lofs);
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
// Group 1 issues every copy: in its QK half of slice s (half-step 2 s + 1)
// it copies slice s + 2 into the slot of slice s - 1 (last read in
// half-step 2 s), nine instructions per wave, one after every other of
// its 18 QK MFMAs, and at the end of that half-step it waits for slice
// s + 1 (issued one step earlier), which group 0 reads next.  The copy
// issue, which can stall while the compute unit's misses are in flight,
// thus stays off the softmax group's critical path (measured: MTP and dense
// prefill 2 % faster than with each group issuing its share at the end of
// its softmax half) and hides behind the MFMA chain (dense prefill 2 %
// faster than issuing all nine before the chain; spread over the whole
// chain instead of after its first nine MFMAs, MTP 0.9 % and dense prefill
// 0.8 % faster, means of five A/B runs).
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
  const int g = lane >> 5;
  Item it;
  if (!decode_item(p, it)) return;
  const int lofs = slice_lane_offsets<true>(lane, hf);   // held for the whole kernel
  const int row_base = it.rt * kRowsPerWg + pr * kRowsPerPair;   // uniform
  const int my_row = row_base + (lane & 31);
  const bool row_ok = my_row < p.R;
  uint8_t* const qs_mine = qs + wave * QL * 1024;
  uint8_t* const xs_mine = xs + wave * kXchgBytes;
  const uint8_t* const xs_peer = xs + (wave ^ 1) * kXchgBytes;
  const float sc = fabsf(p.scale_log2);
  const bool qneg = p.scale_log2 < 0.f;

  // Each group runs its own copy of the unit loop, with grp a compile-time
  // constant: the register allocator then handles the two groups' half-steps
  // separately instead of merging them at every branch on the group
  // (measured: MTP and dense prefill split-KV 1.4-1.6 % faster than one
  // shared loop with run-time branches, same instructions per group).
  auto units = [&](auto grp_c) __attribute__((always_inline)) {
    constexpr int grp = decltype(grp_c)::value;   // 0 leads, 1 trails by half a slice
    int L_nx = it.L0, n_nx = it.n0;   // as in wide_kernel
    for (int u = it.u0; u <= it.u1; ++u) {
      const int jb = (u == it.u0) ? it.j0 : 0;
      const int je_part = (u == it.u1) ? it.j1 : n_nx;
      const int b = u;
      const int L = L_nx;
      if (u < it.u1) {
        n_nx = scalar_ld(it.unit_blocks, u + 1);
        L_nx = scalar_ld(p.seqlens, u + 1);
      }
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
      // All copies are issued by the trailing group, at the start of its QK
      // half-steps, off the softmax group's critical path.
      if (grp == 1) {
        copy_slice_trailing(p, ring0, s_begin, L, true, page_of(p, b, s_begin >> 1, L));
        copy_slice_trailing(p, ring1, s_begin + 1, L, true, page_of(p, b, (s_begin + 1) >> 1, L));
        wait_vmem<9>();             // slice s_begin (slice s_begin + 1 may fly)
      }
      int page_pf = page_of(p, b, min(s_begin + 2, s_end - 1) >> 1, L);
      lds_barrier();                // slice s_begin is in LDS
      if (grp == 1) lds_barrier();  // group 1 starts one half-step later

      int sl = s_begin;
      auto step = [&](auto slot) __attribute__((always_inline)) {
        constexpr int C = decltype(slot)::value;
        uint8_t* const rcur = C == 0 ? ring0 : (C == 1 ? ring1 : ring2);
        uint8_t* const rfree = C == 0 ? ring2 : (C == 1 ? ring0 : ring1);   // slot (C + 2) % 3
        const int key0 = sl * kSlice;
        const uint32_t vmask = key0 >= L ? 0u : (key0 + kSlice <= L ? 0xFFFFFFFFu : (1u << (L - key0)) - 1u);
        // QK half-step.  The trailing group refills the free slot (slice
        // sl - 1's, last read in the half-step before) with slice sl + 2,
        // its copy instructions spread over the QK MFMAs.  QK^T also runs on
        // a slice with no visible key (at most the last slice of a unit,
        // whose slot then holds stale rows): its scores are never read, and
        // skipping it would cost a zeroed tile every slice.
        f32x16 s;
        if (grp == 1 && p.num_pages != 0) {
          const SliceCopy c = prep_slice_copy(p, rfree, sl + 2, L, sl + 2 < s_end, page_pf);
          s = qk_partial<QR, true>(rcur, qf, qs_mine, hf, lofs, c);
        } else {
          s = qk_partial<QR>(rcur, qf, qs_mine, hf, lofs);
        }
        if (grp == 1) page_pf = page_of(p, b, min(sl + 3, s_end - 1) >> 1, L);
        xchg_put(xs_mine, s, lane);
        if (grp == 1) wait_vmem<9>();   // slice sl + 1 (issued one step earlier)
        lds_barrier();
        // softmax + PV half-step.
        if (vmask != 0u) {
          xchg_add(xs_peer, s, lane);
          softmax_pv<false, 2>(s, o, m_run, l_part, rcur, vmask, key0 + kSlice <= W_lo, W, key0, sc, hf, g, lofs);
        }
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
  };
  if (wave >> 2)
    units(Slot<1>{});
  else
    units(Slot<0>{});
}

}  // namespace wide

hipError_t launch_wide(const DecodeParams& p, int kv_format, dim3 grid, hipStream_t stream) {
  const bool sparse = p.indices != nullptr;
  if (kv_format == 0) {
    if (sparse)
      hipLaunchKernelGGL((wide::wide_kernel<0, true>), grid, dim3(wide::kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((wide::offset_kernel), grid, dim3(wide::kThreads), 0, stream, p);
  } else if (p.qk8) {
    if (sparse)
      hipLaunchKernelGGL((wide::wide_kernel<1, true, false>), grid, dim3(wide::kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((wide::wide_kernel<1, false, false>), grid, dim3(wide::kThreads), 0, stream, p);
  } else {
    if (sparse)
      hipLaunchKernelGGL((wide::wide_kernel<1, true, true>), grid, dim3(wide::kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((wide::wide_kernel<1, false, true>), grid, dim3(wide::kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace mla
