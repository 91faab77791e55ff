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
// Design for CDNA4, where these shapes only have to stream the cache and
// the one wave per SIMD that the LDS ring leaves room for has no other wave
// to hide its latencies behind, so every step is built to be short:
//   * One workgroup = 4 waves = 16 query rows, one step = one 64-token page.
//     Pages stream through two LDS page slots filled by global_load_lds (no
//     VGPR round trip).  Page p + 2 is requested as soon as every wave is
//     done with page p (its slot), so while page p + 1 is awaited two pages
//     are in flight; a unit's first two pages are requested together.
//   * QK: wave w computes the full S^T tile of keys 16 w .. 16 w + 15 over
//     all 576 dims (18 v_mfma_f32_16x16x32_bf16, Q^T kept in registers for
//     the whole unit), so there are no partial sums to reduce; the four 1 KiB
//     tiles are exchanged through LDS once per page, after which every wave
//     holds the whole 16 x 64 S^T and runs the same online softmax.
//   * The 16x16 S^T tiles give each lane one row and 16 keys, which are the
//     B operand P^T of the 16x16x32 PV products (the k order of V^T follows
//     them), so P never leaves registers; wave w accumulates O^T for V dims
//     128 w .. 128 w + 127 from ds_read_b64_tr_b16 reads of V^T.
//   * Three barriers per page: the page's arrival, the S^T exchange, and
//     the release of its slot for page p + 2.
//   * FP8 pages are copied raw and dequantised into one bf16 page by all
//     threads after the arrival barrier (one more barrier per page).
//   * Page numbers of a dense unit are held one per lane and read with
//     v_readlane, so issuing a copy needs no memory access of its own.
//   * Key slots nobody may see are loaded from a visible key of the same
//     half page and their probabilities forced to zero.
#include "mla_slice.h"

namespace mla {
namespace narrow {

using namespace slice;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 16;
constexpr int kKSteps = kDqk / 32;            // 18 QK k-steps of 32 dims
constexpr int kDimTiles = kDv / 16 / kWaves;  // 8 tiles of 16 V dims per wave
constexpr int kPageBf16 = 2 * kSliceBytes;    // 73,728
constexpr int kRawPage = kPage * kFp8RowBytes;  // 41,984 = 41 x 1 KiB
constexpr int kRawInst = kRawPage / 1024;       // 41
constexpr int kXchgBytes = kWaves * 1024;       // four 16 x 16 fp32 tiles
constexpr float kRescaleSlack = 8.f;

// LDS: bf16 2 x 72 KiB + 4 KiB exchange (+ 4 KiB sparse table); FP8 2 x 41 KiB
// raw + 72 KiB dequantised page + 4 KiB (+ 2 KiB table): at most 160 KiB.
template <int FMT, bool SPARSE>
struct Geo {
  static constexpr int kSlotBytes = FMT == 0 ? kPageBf16 : kRawPage;
  static constexpr int kTabN = (FMT == 1 && SPARSE) ? 512 : kTab;
};

// Copy page j of the unit's key list into an LDS slot (this wave's share)
// and return its visible-key mask (bit 32 h + t: key t of half h).  bf16:
// per half, wave w issues instructions w + 4 i (key octet w, chunk group i).
// FP8: the 64 raw rows are copied linearly, 16-byte chunk q = 64 inst + lane.
template <int FMT, bool SPARSE>
__device__ __forceinline__ uint64_t copy_page(const DecodeParams& p, const int32_t* tab, int tab_base, uint8_t* dst,
                                              int j, int L, int page) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int fr0, fr1;
  const uint32_t m0 = slice_mask<SPARSE>(tab, tab_base, 2 * j, L, true, &fr0);
  const uint32_t m1 = slice_mask<SPARSE>(tab, tab_base, 2 * j + 1, L, true, &fr1);
  const uint64_t mask = (uint64_t)m0 | ((uint64_t)m1 << 32);
  // A half without a visible key still goes through PV (with zero
  // probabilities): it loads the other half's first visible row.
  if (m0 == 0u) fr0 = fr1;
  if (m1 == 0u) fr1 = fr0;
  if (p.num_pages == 0) return 0u;   // empty pool: no key exists, copy nothing
  if constexpr (FMT == 0) {
    const int ln = opaque_lane();
    const int t = 8 * wave + (ln >> 3);
    const uint8_t* s0 = bf16_copy_src(p, slot_row<SPARSE>(tab, tab_base, 2 * j, t, L, true, page, fr0), wave);
    const uint8_t* s1 = bf16_copy_src(p, slot_row<SPARSE>(tab, tab_base, 2 * j + 1, t, L, true, page, fr1), wave);
#pragma unroll
    for (int i = 0; i < 9; ++i) lds_dma16(s0 + 128 * i, dst + 1024 * (wave + kWaves * i));
#pragma unroll
    for (int i = 0; i < 9; ++i) lds_dma16(s1 + 128 * i, dst + kSliceBytes + 1024 * (wave + kWaves * i));
  } else {
    constexpr int kCpr = kFp8RowBytes / 16;   // 41 chunks per row
    const int ln = opaque_lane();
#pragma unroll
    for (int i = 0; i < (kRawInst + kWaves - 1) / kWaves; ++i) {
      const int inst = wave + kWaves * i;
      if (inst < kRawInst) {
        const int q = inst * 64 + ln;
        const int t = q / kCpr;   // row of the page, 0..63
        const int pc = q - t * kCpr;
        const int h = t >> 5;
        const int row = slot_row<SPARSE>(tab, tab_base, 2 * j + h, t & 31, L, true, page, h ? fr1 : fr0);
        lds_dma16(p.kcache + (size_t)row * kFp8RowBytes + pc * 16, dst + inst * 1024);
      }
    }
  }
  return mask;
}

template <int FMT, bool SPARSE>
__global__ __launch_bounds__(kThreads, 1) void narrow_kernel(const DecodeParams p) {
  using G = Geo<FMT, SPARSE>;
  // Copy instructions of one page that every wave issues at least (bf16:
  // 18 each; FP8: 41 over four waves, at least 10 each).
  constexpr int kFirstWait = FMT == 0 ? 18 : kRawInst / kWaves;
  __shared__ __attribute__((aligned(1024))) uint8_t slot0[G::kSlotBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t slot1[G::kSlotBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t kbf[FMT == 1 ? kPageBf16 : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t xs[kXchgBytes];
  __shared__ int32_t tab[SPARSE ? G::kTabN : 1];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;   // 16-lane group: keys 4 g .. 4 g + 3 of each key tile

  // Work item: XCD-aware (consecutive block ids go to different XCDs, the
  // row tiles of one part share an XCD and its L2).
  int part, rt;
  work_item(blockIdx.x, p.num_parts, p.row_tiles, &part, &rt);
  // Header and part row are read together (one round trip); workgroups
  // past the last part read the last part's row and then stop.
  const int32_t* prow = p.md + kHeader + kPartRow * min(part, p.num_parts - 1);
  const int h0 = p.md[0], h3 = p.md[3], h5 = p.md[5];
  const int u0 = prow[0], j0 = prow[1], u1 = prow[2], j1 = prow[3], split0 = prow[4];
  if (!header_ok(p, h0, h3, h5)) {
    fill_mismatch<kThreads>(p);
    return;
  }
  if (part >= p.num_parts || u0 < 0) return;
  const int32_t* unit_blocks = p.md + kHeader + kPartRow * p.num_parts;

  const int row_base = rt * kRows;   // uniform
  const int my_row = row_base + (lane & 15);
  const bool row_ok = my_row < p.R;
  const float sc = fabsf(p.scale_log2);
  const bool qneg = p.scale_log2 < 0.f;   // the sign goes into Q

  // Length and block count of the current unit: the part row carries them
  // for the first unit; those of the next are prefetched at each unit start.
  int L_nx = prow[5], n_nx = prow[6];
  for (int u = u0; u <= u1; ++u) {
    const int jb = (u == u0) ? j0 : 0;
    const int je = (u == u1) ? j1 : n_nx;
    const int b = SPARSE ? u / p.s_q : u;
    const int L = L_nx;
    const int s_unit = SPARSE ? u % p.s_q : 0;
    const int s_row = SPARSE ? s_unit : (row_ok ? my_row / p.h_q : 0);
    const int W = p.causal ? min(max(L - p.s_q + 1 + s_row, 0), L) : L;
    const int Wunit = (SPARSE && p.causal) ? min(max(L - p.s_q + 1 + s_unit, 0), L) : L;
    const int W_lo = p.causal ? min(max(L - p.s_q + 1, 0), L) : L;   // every row sees keys < W_lo
    const int32_t* idx_row = SPARSE ? p.indices + (size_t)u * p.topk : nullptr;
    const int pos_end = kPage * je;
    int tab_base = kPage * jb;

    // Q^T for all 18 k-steps: lane holds row l % 16, dims 32 ks + 8 (l / 16)
    // .. + 7.  Issued first: it depends on u only.
    bf16x8 qf[kKSteps];
    {
      const int ln = opaque_lane();
      const int r = row_base + (ln & 15);
      const uint8_t* qrow = p.q + ((size_t)u * p.R + (r < p.R ? r : 0)) * (2 * kDqk) + 16 * (ln >> 4);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        u32x4 v = *(const u32x4*)(qrow + 64 * ks);
        if (r >= p.R) v = u32x4{0, 0, 0, 0};
        if (qneg) v ^= 0x80008000u;   // exact bf16 negation
        qf[ks] = __builtin_bit_cast(bf16x8, v);
      }
    }
    if (SPARSE) fill_table<kThreads, G::kTabN / kThreads>(p, tab, b, tab_base, min(pos_end - tab_base, G::kTabN), Wunit, idx_row);
    // Dense: lane i holds the page of block pb + i.
    int pb = jb;
    int pages_v = 0;
    if (!SPARSE) {
      const int jl = jb + lane;
      pages_v = (jl < je && jl * kPage < L) ? p.block_table[(size_t)b * p.max_blocks + jl] : 0;
    }
    // The next unit's length and blocks, through the scalar cache; the
    // barrier below waits for them with everything else.
    if (u < u1) {
      n_nx = unit_blocks[u + 1];
      L_nx = p.seqlens[SPARSE ? (u + 1) / p.s_q : u + 1];
    }
    wait_vmem<0>();
    lds_barrier();   // Q, page list and tab complete

    // The unit's first page.
    auto page_at = [&](int j) -> int {
      if (SPARSE) return 0;
      if (j - pb >= 64) {   // past the lanes' page list: reload it
        pb = j;
        const int jl = pb + lane;
        pages_v = (jl < je && jl * kPage < L) ? p.block_table[(size_t)b * p.max_blocks + jl] : 0;
      }
      return __builtin_amdgcn_readlane(pages_v, j - pb);
    };
    // Both slots are free at the unit's start: its first two pages are
    // requested together, so the second does not wait for the first to land.
    uint64_t vis[2];   // visible-key mask of the page in each slot
    vis[0] = copy_page<FMT, SPARSE>(p, tab, tab_base, slot0, jb, L, page_at(jb));
    vis[1] = 0u;
    if (jb + 1 < je) vis[1] = copy_page<FMT, SPARSE>(p, tab, tab_base, slot1, jb + 1, L, page_at(jb + 1));

    float m_run = -INFINITY;
    float l_part = 0.f;
    f32x4 o[kDimTiles];
#pragma unroll
    for (int d = 0; d < kDimTiles; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto step = [&](auto slot_c, int j) __attribute__((always_inline)) {
      constexpr int C = decltype(slot_c)::value;
      uint8_t* const rcur = C == 0 ? slot0 : slot1;
      // Page j must be in LDS; page j + 1's copies (requested after page
      // j - 1 was done, or at the unit's start) may still fly: at least
      // kFirstWait instructions of this wave.
      if (j + 1 < je)
        wait_vmem<kFirstWait>();
      else
        wait_vmem<0>();
      lds_barrier();   // page j visible
      const uint64_t vmask = vis[C];
      const uint8_t* kb = rcur;
      if constexpr (FMT == 1) {
        if (vmask != 0u) {
          dequant_codes<kThreads>(rcur, kbf);
          dequant_codes<kThreads>(rcur + kSlice * kFp8RowBytes, kbf + kSliceBytes);
        }
        lds_barrier();   // kbf holds page j
        kb = kbf;
      }
      if (vmask != 0u) {
        // ---- S^T tile of keys 16 wave .. + 15 (half wave >> 1 of the page,
        // keys 16 (wave & 1) + l % 16) over all 18 k-steps.
        {
          const uint8_t* kh = kb + (wave >> 1) * kSliceBytes;
          const int ln = opaque_lane();
          const int t = 16 * (wave & 1) + (ln & 15);
          const int gg = ln >> 4;
          f32x4 sres;
          if constexpr (FMT == 1) {
            // Exact codes: k-steps 4 G .. 4 G + 3 are NoPE group G, 16 and 17
            // RoPE.  Each group's partial sums are multiplied by that group's
            // scale of their key (the lane's output keys 16 (wave & 1) + 4 g
            // + i of half wave >> 1: raw rows 32 (wave >> 1) + ...).
            f32x4 sc4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) sc4[i] = fp8_scales(rcur, 32 * (wave >> 1) + 16 * (wave & 1) + 4 * gg + i);
            f32x4 sr = f32x4{0.f, 0.f, 0.f, 0.f};
            sr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(kh + slice_off(t, 64 + gg)), qf[16], sr,
                                                         0, 0, 0);
            sr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(kh + slice_off(t, 68 + gg)), qf[17], sr,
                                                         0, 0, 0);
#pragma unroll
            for (int G = 0; G < 4; ++G) {
              f32x4 ta = f32x4{0.f, 0.f, 0.f, 0.f}, tb = ta;
#pragma unroll
              for (int kk = 0; kk < 4; kk += 2) {
                const int ks = 4 * G + kk;
                const bf16x8 a0 = *(const bf16x8*)(kh + slice_off(t, 4 * ks + gg));
                const bf16x8 a1 = *(const bf16x8*)(kh + slice_off(t, 4 * ks + 4 + gg));
                ta = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[ks], ta, 0, 0, 0);
                tb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[ks + 1], tb, 0, 0, 0);
              }
              const f32x4 tg = ta + tb;
#pragma unroll
              for (int i = 0; i < 4; ++i) sr[i] = __builtin_fmaf(tg[i], sc4[i][G], sr[i]);
            }
            sres = sr;
          } else {
            f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f}, sb = sa;
#pragma unroll
            for (int ks = 0; ks < kKSteps; ks += 2) {
              const bf16x8 a0 = *(const bf16x8*)(kh + slice_off(t, 4 * ks + gg));
              const bf16x8 a1 = *(const bf16x8*)(kh + slice_off(t, 4 * ks + 4 + gg));
              sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[ks], sa, 0, 0, 0);
              sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[ks + 1], sb, 0, 0, 0);
            }
            sres = sa + sb;
          }
          *(f32x4*)(xs + wave * 1024 + lane * 16) = sres;
        }
        lds_barrier();   // all four S^T tiles visible
        // ---- lane holds row l % 16 and keys 16 w + 4 g + i (i < 4) for w < 4.
        float sv[16];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const f32x4 a = *(const f32x4*)(xs + w * 1024 + lane * 16);
#pragma unroll
          for (int i = 0; i < 4; ++i) sv[4 * w + i] = a[i];
        }
        // ---- mask + online softmax (exp2 domain, logit = sc * s).
        const int key0 = kPage * j;
        const bool full = SPARSE ? (vmask == ~0ull) : (key0 + kPage <= W_lo);
        uint32_t okbits = 0xFFFFu;
        if (!full) {
          okbits = 0u;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int tl = 16 * (i >> 2) + 4 * g + (i & 3);
            const bool ok = SPARSE ? ((vmask >> tl) & 1u) != 0u : (key0 + tl < W);
            okbits |= ok ? (1u << i) : 0u;
            sv[i] = ok ? sv[i] : -INFINITY;
          }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sv[i]);
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
        float e[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) e[i] = fast_exp2(__builtin_fmaf(sv[i], sc, -m_use));
        if (!full) {
#pragma unroll
          for (int i = 0; i < 16; ++i) e[i] = ((okbits >> i) & 1u) ? e[i] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) l_part += e[i];
        // ---- O^T += V^T P^T over the two halves of the page.  PV k-step h
        // covers key tiles 2 h and 2 h + 1: k-slot i of lane group g is key
        // 4 g + i of tile 2 h (i < 4) or of tile 2 h + 1 (i >= 4); the
        // transposed read of 16-lane group G takes keys 4 G + (j >> 2) (+ 16
        // for the second read) and dims 4 (j & 3) .. + 3 of the dim tile, i.e.
        // chunk 16 wave + 2 dt + ((j >> 1) & 1) of the half.
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          // FP8: wave w's V dims are NoPE group w; the probabilities times
          // that group's scale of their key (page key 32 h + 16 (i >> 2) +
          // 4 g + (i & 3) for e[8 h + i]).
          float ev[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            ev[i] = e[8 * h + i];
            if constexpr (FMT == 1)
              ev[i] *= *(const float*)(rcur + (32 * h + 16 * (i >> 2) + 4 * g + (i & 3)) * kFp8RowBytes +
                                       kFp8ScaleOff + 4 * wave);
          }
          const bf16x8 pb = __builtin_bit_cast(
              bf16x8, u32x4{pack_bf16x2(ev[0], ev[1]), pack_bf16x2(ev[2], ev[3]), pack_bf16x2(ev[4], ev[5]),
                            pack_bf16x2(ev[6], ev[7])});
          const uint8_t* vh = kb + h * kSliceBytes;
          const int ln = opaque_lane();
          const int jj = ln & 15;
          const int tA = 4 * (ln >> 4) + (jj >> 2);
          const int tB = tA + 16;
          const int xo = 8 * (jj & 1);
#pragma unroll
          for (int dt = 0; dt < kDimTiles; ++dt) {
            const int c = 16 * wave + 2 * dt + ((jj >> 1) & 1);
            const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vh + slice_off(tA, c) + xo));
            const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vh + slice_off(tB, c) + xo));
            const u32x2 xa = __builtin_bit_cast(u32x2, va);
            const u32x2 xb = __builtin_bit_cast(u32x2, vb);
            const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{xa[0], xa[1], xb[0], xb[1]});
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb, o[dt], 0, 0, 0);
          }
        }
      }
      // ---- page j's slot is free once every wave is past its PV: page
      // j + 2 goes into it now, so that it flies while page j + 1 is awaited.
      if (j + 2 < je) {
        lds_barrier();
        if (SPARSE) {
          const int pos = kPage * (j + 2);
          if (pos + kPage - tab_base > G::kTabN) {   // the unit's range outgrew the table
            tab_base = pos;
            fill_table<kThreads, G::kTabN / kThreads>(p, tab, b, tab_base, min(pos_end - tab_base, G::kTabN), Wunit, idx_row);
            wait_vmem<0>();
            lds_barrier();
          }
        }
        vis[C] = copy_page<FMT, SPARSE>(p, tab, tab_base, rcur, j + 2, L, page_at(j + 2));
      }
    };
    int j = jb;
    while (j < je) {
      step(Slot<0>{}, j);
      if (++j >= je) break;
      step(Slot<1>{}, j);
      ++j;
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
          uint16_t* orow = p.ws_o + ((size_t)split * p.R + r) * kDv + dbase;
#pragma unroll
          for (int dt = 0; dt < kDimTiles; ++dt)
            *(u32x2*)(orow + 16 * dt) = u32x2{pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv),
                                              pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv)};
          if (wave == 0 && gg == 0) p.ws_lse[(size_t)split * p.R + r] = lse_nat;
        }
      }
    }
    wait_vmem<0>();
    lds_barrier();   // the next unit refills the table and the slots
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
