// Split-KV partial attention for few query rows per sequence (16-row tiles):
// the memory-bound shapes of MLA decoding (one or two query tokens, up to
// 32 heads), written for gfx950.
//
// Same contract as the 128-row kernel (topnet.top "Was ist FlashMLA?",
// "MLA-Decodierung ausfuehren"; sao.pub FlashMLA overview, 二、核心功能与
// 架构): per query row, softmax attention over the 576-dim latent keys of its
// sequence (V = first 512 dims), out + natural-log lse, with causal /
// sparse-index masking and bf16 or 656-byte FP8 rows.
//
// Design for CDNA4, where these shapes only have to stream the cache:
//   * One workgroup = 4 waves = 16 query rows.  Keys stream through an LDS
//     ring of 32-key slices filled by global_load_lds (no VGPR round trip);
//     with bf16 pages the ring has 4 slots, three slices (108 KiB) in flight
//     while the fourth is computed, enough to cover the HBM latency at full
//     bandwidth with one workgroup per CU (3 slots when a sparse index table
//     also needs LDS).
//   * The 16 rows x 32 keys of a slice are split over the waves by the
//     contraction dims: wave w computes the partial S^T over its share of
//     the 18 QK k-steps (32 dims each; 5, 5, 4, 4) with
//     v_mfma_f32_16x16x32_bf16, the four partial tiles are summed through
//     LDS in a fixed order (so every wave holds the same S^T), every wave
//     runs the same online softmax, and wave w accumulates O^T for V dims
//     128 w .. 128 w + 127.  One barrier per slice serves the exchange, the
//     arrival of the next slice and the release of the oldest slot; the
//     exchange buffer alternates between two halves by slice parity, so a
//     wave that runs ahead never overwrites tiles still being read.
//   * The 16x16 S^T tiles give each lane one row and 8 keys, which are the
//     B operand P^T of the 16x16x32 PV product (the k order of V^T follows
//     them), so P never leaves registers; V^T comes from ds_read_b64_tr_b16.
//   * FP8 slices are copied raw and dequantised into one bf16 slice by all
//     threads before their QK (two more barriers per slice).
//   * Key slots nobody may see are loaded from a visible key of the same
//     slice and their probabilities forced to zero.
#include "mla_slice.h"

namespace mla {
namespace narrow {

using namespace slice;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 16;
constexpr int kQKSteps = 5;                   // QK k-steps per wave (the last two waves: 4 + a zero step)
constexpr int kDimTiles = kDv / 16 / kWaves;  // 8 tiles of 16 V dims per wave
constexpr int kXchgBytes = 8 * 64 * 4;        // one wave's partial S^T: 2 tiles x 4 fp32 per lane
constexpr float kRescaleSlack = 8.f;

// LDS: bf16 dense 4 x 36 KiB + 2 x 8 KiB exchange = 160 KiB; bf16 sparse
// 3 slots + 16 KiB + 4 KiB table; FP8 4 x 21 KiB raw + 36 KiB dequantised
// slice + 16 + 4 KiB.
template <int FMT>
struct Geo {
  static constexpr int kRingBytes = FMT == 0 ? kSliceBytes : kRawSlotBytes;
  static constexpr int kInst = kRingBytes / 1024;                 // 36 | 21
  static constexpr int kPerWave = kInst / kWaves;                 // 9 | 5 (wave 0 of FP8: 6)
  static constexpr int kMaxPerWave = (kInst + kWaves - 1) / kWaves;
};

// First QK k-step of wave w (18 = 5 + 5 + 4 + 4); ks_begin(4) = 18.
__device__ __forceinline__ int ks_begin(int w) { return w <= 2 ? 5 * w : (w == 3 ? 14 : 18); }

// Copy slice sl of the unit into slot dst (this wave's share).  bf16: wave
// w issues instructions w + 4 i, i.e. key octet w, chunk group i.  FP8:
// rows copied linearly, chunk q = 64 inst + lane.  Returns the slice's
// visible-slot mask (uniform).
template <int FMT, bool SPARSE>
__device__ __forceinline__ uint32_t copy_slice(const DecodeParams& p, const int32_t* tab, int tab_base,
                                               uint8_t* dst, int sl, int L, bool active, int page) {
  const int ln = opaque_lane();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int first_row;
  const uint32_t mask = slice_mask<SPARSE>(tab, tab_base, sl, L, active, &first_row);
  if (p.num_pages == 0) return 0u;   // empty pool: no key exists, copy nothing
  if constexpr (FMT == 0) {
    const uint8_t* src =
        bf16_copy_src(p, slot_row<SPARSE>(tab, tab_base, sl, 8 * wave + (ln >> 3), L, active, page, first_row),
                      wave);
#pragma unroll
    for (int i = 0; i < Geo<0>::kPerWave; ++i) lds_dma16(src + 128 * i, dst + 1024 * (wave + kWaves * i));
  } else {
    constexpr int kCpr = kFp8RowBytes / 16;   // 41 chunks per row
#pragma unroll
    for (int i = 0; i < Geo<1>::kMaxPerWave; ++i) {
      const int inst = wave + kWaves * i;
      if (inst < Geo<1>::kInst) {
        int q = inst * 64 + ln;
        if (q >= kSlice * kCpr) q = kSlice * kCpr - 1;   // tail: stay in the slice
        const int t = q / kCpr;
        const int pc = q - t * kCpr;
        const int row = slot_row<SPARSE>(tab, tab_base, sl, t, L, active, page, first_row);
        lds_dma16(p.kcache + (size_t)row * kFp8RowBytes + pc * 16, dst + inst * 1024);
      }
    }
  }
  return mask;
}

template <int FMT, bool SPARSE>
__global__ __launch_bounds__(kThreads, 1) void narrow_kernel(const DecodeParams p) {
  using G = Geo<FMT>;
  constexpr int NS = (FMT == 0 && SPARSE) ? 3 : 4;   // ring slots
  __shared__ __attribute__((aligned(1024))) uint8_t ring0[G::kRingBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t ring1[G::kRingBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t ring2[G::kRingBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t ring3[NS == 4 ? G::kRingBytes : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t kbf[FMT == 1 ? kSliceBytes : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t xs[2 * kWaves * kXchgBytes];
  __shared__ int32_t tab[SPARSE ? kTab : 1];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;   // 16-lane group: keys 4 g .. 4 g + 3 of each key tile

  // Work item: XCD-aware (consecutive block ids go to different XCDs, the
  // row tiles of one part share an XCD and its L2).
  const int bid = blockIdx.x;
  const int rest = bid >> 3;
  const int rt = rest % p.row_tiles;
  const int part = (rest / p.row_tiles) * 8 + (bid & 7);
  if (part >= p.num_parts) return;
  if (p.md[0] != p.num_parts || p.md[5] != kMagic || p.md[3] != p.units) return;
  const int32_t* prow = p.md + kHeader + kPartRow * part;
  const int u0 = prow[0], j0 = prow[1], u1 = prow[2], j1 = prow[3], split0 = prow[4];
  if (u0 < 0) return;
  const int32_t* unit_blocks = p.md + kHeader + kPartRow * p.num_parts;

  const int row_base = rt * kRows;   // uniform
  const int my_row = row_base + (lane & 15);
  const bool row_ok = my_row < p.R;
  const float sc = fabsf(p.scale_log2);
  const bool qneg = p.scale_log2 < 0.f;   // the sign goes into Q
  const int ks0 = ks_begin(wave);
  const int nks = ks_begin(wave + 1) - ks0;   // 5 or 4

  for (int u = u0; u <= u1; ++u) {
    const int jb = (u == u0) ? j0 : 0;
    const int je = (u == u1) ? j1 : unit_blocks[u];
    const int b = SPARSE ? u / p.s_q : u;
    const int L = p.seqlens[b];
    const int s_unit = SPARSE ? u % p.s_q : 0;
    const int s_row = SPARSE ? s_unit : (row_ok ? my_row / p.h_q : 0);
    const int W = p.causal ? min(max(L - p.s_q + 1 + s_row, 0), L) : L;
    const int Wunit = (SPARSE && p.causal) ? min(max(L - p.s_q + 1 + s_unit, 0), L) : L;
    const int W_lo = p.causal ? min(max(L - p.s_q + 1, 0), L) : L;   // every row sees keys < W_lo
    const int32_t* idx_row = SPARSE ? p.indices + (size_t)u * p.topk : nullptr;
    const int s_begin = 2 * jb;
    const int s_end = 2 * je;   // at least s_begin + 2
    const int pos_end = kPage * je;
    int tab_base = kPage * jb;
    if (SPARSE) fill_table<kThreads>(p, tab, b, tab_base, min(pos_end - tab_base, kTab), Wunit, idx_row);

    // Q^T for this wave's k-steps: lane holds row l % 16, dims
    // 32 ks + 8 (l / 16) .. + 7; a missing fifth k-step is zero.
    bf16x8 qf[kQKSteps];
    {
      const int ln = opaque_lane();
      const int r = row_base + (ln & 15);
      const uint8_t* qrow = p.q + ((size_t)u * p.R + (r < p.R ? r : 0)) * (2 * kDqk) + 16 * (ln >> 4);
#pragma unroll
      for (int i = 0; i < kQKSteps; ++i) {
        u32x4 v = *(const u32x4*)(qrow + 64 * (ks0 + min(i, nks - 1)));
        if (r >= p.R || i >= nks) v = u32x4{0, 0, 0, 0};
        if (qneg) v ^= 0x80008000u;   // exact bf16 negation
        qf[i] = __builtin_bit_cast(bf16x8, v);
      }
    }
    wait_vmem<0>();
    lds_barrier();   // tab complete

    float m_run = -INFINITY;
    float l_part = 0.f;
    f32x4 o[kDimTiles];
#pragma unroll
    for (int d = 0; d < kDimTiles; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Slices s_begin .. s_begin + NS - 2 (slice s in slot (s - s_begin) % NS).
    uint32_t vis[4];
    vis[0] = copy_slice<FMT, SPARSE>(p, tab, tab_base, ring0, s_begin, L, true,
                                     SPARSE ? 0 : page_of(p, b, s_begin >> 1, L));
    vis[1] = copy_slice<FMT, SPARSE>(p, tab, tab_base, ring1, s_begin + 1, L, true,
                                     SPARSE ? 0 : page_of(p, b, (s_begin + 1) >> 1, L));
    vis[2] = 0u;
    vis[3] = 0u;
    if (NS == 4)
      vis[2] = copy_slice<FMT, SPARSE>(p, tab, tab_base, ring2, s_begin + 2, L, s_begin + 2 < s_end,
                                       SPARSE ? 0 : page_of(p, b, min(s_begin + 2, s_end - 1) >> 1, L));
    int page_pf = SPARSE ? 0 : page_of(p, b, min(s_begin + NS - 1, s_end - 1) >> 1, L);
    wait_vmem<(NS - 2) * G::kPerWave>();   // slice s_begin
    lds_barrier();

    int sl = s_begin;
    auto step = [&](auto slot) __attribute__((always_inline)) {
      constexpr int C = decltype(slot)::value;
      constexpr int F = (C + NS - 1) % NS;   // slot of slice sl - 1
      uint8_t* const rcur = C == 0 ? ring0 : (C == 1 ? ring1 : (C == 2 ? ring2 : ring3));
      uint8_t* const rfree = F == 0 ? ring0 : (F == 1 ? ring1 : (F == 2 ? ring2 : ring3));
      const uint32_t vmask = vis[C];
      const int key0 = sl * kSlice;
      uint8_t* const xcur = xs + (sl & 1) * (kWaves * kXchgBytes);
      const uint8_t* kb = rcur;
      if constexpr (FMT == 1) {
        lds_barrier();   // every wave is done with the previous slice in kbf
        if (vmask != 0u) dequant_slice<kThreads>(rcur, kbf);
        lds_barrier();   // kbf holds slice sl
        kb = kbf;
      }
      // ---- partial S^T = K Q^T over this wave's k-steps; tile kt covers
      // keys 16 kt + 0..15: lane holds key 16 kt + l % 16 (A) and row
      // l % 16 (B), dims 32 ks + 8 (l / 16) .. + 7.
      f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = f32x4{0.f, 0.f, 0.f, 0.f};
      if (vmask != 0u) {
        const int ln = opaque_lane();
        const int t0 = ln & 15;
        const int gg = ln >> 4;
#pragma unroll
        for (int i = 0; i < kQKSteps; ++i) {
          const int c = 4 * (ks0 + min(i, nks - 1)) + gg;   // chunk (a zero Q step re-reads the last one)
          const bf16x8 a0 = *(const bf16x8*)(kb + slice_off(t0, c));
          const bf16x8 a1 = *(const bf16x8*)(kb + slice_off(16 + t0, c));
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[i], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[i], s1, 0, 0, 0);
        }
        *(f32x4*)(xcur + wave * kXchgBytes + lane * 16) = s0;
        *(f32x4*)(xcur + wave * kXchgBytes + 1024 + lane * 16) = s1;
      }
      wait_vmem<(NS - 3) * G::kPerWave>();   // this wave's share of slice sl + 1
      lds_barrier();   // partial tiles and slice sl + 1 visible; slot of sl - 1 free
      // ---- copy slice sl + NS - 1 into the slot of slice sl - 1.
      {
        const bool more = sl + NS - 1 < s_end;
        if (SPARSE && more) {
          const int pos = kSlice * (sl + NS - 1);
          if (pos - tab_base >= kTab) {   // the unit's range outgrew the table
            tab_base = pos;
            fill_table<kThreads>(p, tab, b, tab_base, min(pos_end - tab_base, kTab), Wunit, idx_row);
            lds_barrier();
          }
        }
        vis[F] = copy_slice<FMT, SPARSE>(p, tab, tab_base, rfree, sl + NS - 1, L, more, page_pf);
        if (!SPARSE) page_pf = page_of(p, b, min(sl + NS, s_end - 1) >> 1, L);
      }
      const int cur_sl = sl;
      ++sl;
      if (vmask == 0u) return;
      // ---- S^T = sum of the four partial tiles, in wave order.
      float sv[8];
      {
        f32x4 a0 = *(const f32x4*)(xcur + lane * 16);
        f32x4 a1 = *(const f32x4*)(xcur + 1024 + lane * 16);
#pragma unroll
        for (int w = 1; w < kWaves; ++w) {
          a0 += *(const f32x4*)(xcur + w * kXchgBytes + lane * 16);
          a1 += *(const f32x4*)(xcur + w * kXchgBytes + 1024 + lane * 16);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sv[r] = a0[r];
          sv[4 + r] = a1[r];
        }
      }
      // ---- mask + online softmax (exp2 domain, logit = sc * s).  Lane
      // holds row l % 16 and keys 16 (i >> 2) + 4 g + (i & 3), i = 0..7.
      const bool full = SPARSE ? (vmask == 0xFFFFFFFFu) : (cur_sl * kSlice + kSlice <= W_lo);
      uint32_t okbits = 0xFFu;
      if (!full) {
        okbits = 0u;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int tl = 16 * (i >> 2) + 4 * g + (i & 3);
          const bool ok = SPARSE ? ((vmask >> tl) & 1u) != 0u : (key0 + tl < W);
          okbits |= ok ? (1u << i) : 0u;
          sv[i] = ok ? sv[i] : -INFINITY;
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 8; ++i) mx = fmaxf(mx, sv[i]);
      mx = fmaxf(mx, xor16(mx));
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
      float e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) e[i] = fast_exp2(__builtin_fmaf(sv[i], sc, -m_use));
      if (!full) {
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = ((okbits >> i) & 1u) ? e[i] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) l_part += e[i];
      const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]),
                                                         pack_bf16x2(e[4], e[5]), pack_bf16x2(e[6], e[7])});
      // ---- O^T += V^T P^T for V dims 128 wave + 16 dt .. + 15.  k-slot i
      // of lane group g is key 4 g + i (i < 4) or 16 + 4 g + i - 4; the
      // transposed read of 16-lane group G takes keys 4 G + (j >> 2) (+ 16
      // for the second read) and dims 4 (j & 3) .. + 3 of the tile, i.e.
      // chunk 16 wave + 2 dt + ((j >> 1) & 1).
      {
        const int ln = opaque_lane();
        const int jj = ln & 15;
        const int tA = 4 * (ln >> 4) + (jj >> 2);
        const int tB = tA + 16;
        const int xo = 8 * (jj & 1);
#pragma unroll
        for (int dt = 0; dt < kDimTiles; ++dt) {
          const int c = 16 * wave + 2 * dt + ((jj >> 1) & 1);
          const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kb + slice_off(tA, c) + xo));
          const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kb + slice_off(tB, c) + xo));
          const u32x2 xa = __builtin_bit_cast(u32x2, va);
          const u32x2 xb = __builtin_bit_cast(u32x2, vb);
          const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{xa[0], xa[1], xb[0], xb[1]});
          o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb, o[dt], 0, 0, 0);
        }
      }
    };
    while (sl < s_end) {
      step(Slot<0>{});
      if (sl >= s_end) break;
      step(Slot<1>{});
      if (sl >= s_end) break;
      step(Slot<2>{});
      if constexpr (NS == 4) {
        if (sl >= s_end) break;
        step(Slot<3>{});
      }
    }

    // ---- epilogue: lane holds row l % 16, dims 128 wave + 16 dt + 4 g +
    // (0..3); the row sum is spread over the four lane groups.
    float l_sum = l_part + xor16(l_part);
    l_sum += xor32(l_sum);
    {
      const int ln = opaque_lane();
      const int r = row_base + (ln & 15);
      const int gg = ln >> 4;
      const float inv = l_sum > 0.f ? 1.f / l_sum : 0.f;
      const float lse_nat =
          l_sum > 0.f ? ((m_run == -INFINITY ? 0.f : m_run) + fast_log2(l_sum)) * kLn2 : -INFINITY;
      const int k_u = p.num_splits[u + 1] - p.num_splits[u];
      const int split = p.num_splits[u] + (u == u0 ? split0 : 0);
      if (r < p.R) {
        const size_t grow = (size_t)u * p.R + r;
        const int dbase = 128 * wave + 4 * gg;
        if (k_u == 1) {
          uint16_t* orow = p.out + grow * kDv + dbase;
#pragma unroll
          for (int dt = 0; dt < kDimTiles; ++dt)
            *(u32x2*)(orow + 16 * dt) = u32x2{pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv),
                                              pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv)};
          if (wave == 0 && gg == 0) p.lse[grow] = lse_nat;
        } else {
          float* orow = p.ws_o + ((size_t)split * p.R + r) * kDv + dbase;
#pragma unroll
          for (int dt = 0; dt < kDimTiles; ++dt) *(f32x4*)(orow + 16 * dt) = o[dt] * inv;
          if (wave == 0 && gg == 0) p.ws_lse[(size_t)split * p.R + r] = lse_nat;
        }
      }
    }
    wait_vmem<0>();
    lds_barrier();   // the next unit refills the table and the ring
  }
}

}  // namespace narrow

hipError_t launch_narrow(const DecodeParams& p, int kv_format, dim3 grid, hipStream_t stream) {
  const bool sparse = p.indices != nullptr;
  if (kv_format == 0) {
    if (sparse)
      hipLaunchKernelGGL((narrow::narrow_kernel<0, true>), grid, dim3(narrow::kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((narrow::narrow_kernel<0, false>), grid, dim3(narrow::kThreads), 0, stream, p);
  } else {
    if (sparse)
      hipLaunchKernelGGL((narrow::narrow_kernel<1, true>), grid, dim3(narrow::kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((narrow::narrow_kernel<1, false>), grid, dim3(narrow::kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace mla
