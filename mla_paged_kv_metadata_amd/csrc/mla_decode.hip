// Split-KV partial attention and log-sum-exp combine for MLA decoding over a
// 64-token paged KV cache, written for gfx950 (CDNA4, wave64, bf16 MFMA).
//
// What is computed (topnet.top "Was ist FlashMLA?", "MLA-Decodierung
// ausfuehren"; sao.pub FlashMLA overview, 二、核心功能与架构): for every query
// row (576 dims = 512 NoPE + 64 RoPE), softmax attention over the keys of its
// sequence, each key being one shared latent row whose first 512 dims are
// also V; the result out (bf16) and its log-sum-exp (natural log, fp32).
// Keys may be restricted by a causal window or by a list of token indices,
// and may be stored as bf16 rows or as 656-byte FP8 rows.
//
// Kernel structure (one workgroup = 4 waves = 256 threads per (part, row
// tile)):
//   * The schedule assigns each part a run of 64-key blocks (see
//     mla_metadata.hip).  Row tiles of 16/32/64 query rows split the rows of
//     a unit; their workgroups for one part are given block ids that land on
//     the same XCD (ids are dealt round-robin over the 8 XCDs), so the
//     repeated reads of a KV block are served by that XCD's L2.
//   * Each 64-key block is staged HBM -> registers -> LDS by all 256 threads
//     with 16-byte coalesced loads (the next block's loads are in flight
//     while the current block is computed).  FP8 rows are dequantised while
//     staging (e4m3 -> fp32, times the group's fp32 scale, -> bf16).  Key
//     slots that no query may see (beyond the sequence, masked indices) are
//     staged as zeros so that the PV product never touches stale memory.
//   * Wave w owns 16 query rows (row block w % NRB) and 64/TG keys of each
//     block (token group w / NRB, TG = 4 / NRB).  S^T = K Q^T runs on
//     v_mfma_f32_16x16x32_bf16 with K read from LDS and Q held in registers
//     for the whole unit; the 16x16 result puts one query row in each lane
//     and four keys per lane, which is exactly the B-operand layout the PV
//     product O^T += V^T P^T needs, so P never leaves registers.
//   * Online softmax in the exp2 domain: the row max is a 4-way cross-lane
//     reduction per block; the row sum stays per lane until the end.
//   * Token groups of one row block are merged in LDS at the end of a unit;
//     a unit covered by one part writes out/lse directly, otherwise its
//     normalised partial O and partial lse go to the workspace and the
//     combine kernel merges them.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

constexpr int kLdsRow = kDqk * 2 + 16;          // padded LDS row of one key (bytes)
constexpr int kLdsBuf = kPage * kLdsRow;        // one staged block
constexpr int kOStride = kDv + 4;               // padded fp32 row for the epilogue
constexpr int kThreads = 256;
constexpr float kRescaleSlack = 8.f;     // see the online softmax step

// ---------------------------------------------------------------------------
// Staging of one 64-key block: HBM -> registers -> LDS.
// ---------------------------------------------------------------------------
template <int FMT, bool SPARSE>
struct Stager;

// Resolve key slot `tok` of block j to a row pointer, or null if masked.
template <bool SPARSE>
__device__ __forceinline__ const uint8_t* key_row(const DecodeParams& p, int b, int j, int tok,
                                                  int L, int Wunit, const int32_t* idx_row,
                                                  int row_bytes, int dense_page, int* tpos) {
  if (!SPARSE) {
    const int t = j * kPage + tok;
    *tpos = t;
    if (t >= L || dense_page < 0) return nullptr;
    return p.kcache + ((size_t)dense_page * kPage + tok) * row_bytes;
  } else {
    const int e = j * kPage + tok;
    const int t = e < p.topk ? idx_row[e] : -1;
    const bool ok = t >= 0 && t < Wunit;
    *tpos = ok ? t : -1;
    if (!ok) return nullptr;
    const int page = p.block_table[(size_t)b * p.max_blocks + (t >> 6)];
    return p.kcache + ((size_t)page * kPage + (t & (kPage - 1))) * row_bytes;
  }
}

template <bool SPARSE>
struct Stager<0, SPARSE> {
  static constexpr int kChunksPerRow = kBf16RowBytes / 16;            // 72
  static constexpr int kN = kPage * kChunksPerRow / kThreads;         // 18
  u32x4 r[kN];
  int tp[kN];

  __device__ __forceinline__ void load(const DecodeParams& p, int b, int j, int L, int Wunit,
                                       const int32_t* idx_row) {
    const int tid = threadIdx.x;
    int dense_page = -1;
    if (!SPARSE && j * kPage < L) dense_page = p.block_table[(size_t)b * p.max_blocks + j];
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int c = tid + kThreads * i;
      const int tok = c / kChunksPerRow;
      const int col = c - tok * kChunksPerRow;
      const uint8_t* row =
          key_row<SPARSE>(p, b, j, tok, L, Wunit, idx_row, kBf16RowBytes, dense_page, &tp[i]);
      if (row)
        r[i] = *(const u32x4*)(row + col * 16);
      else
        r[i] = u32x4{0, 0, 0, 0};
    }
  }

  __device__ __forceinline__ void store(uint8_t* kb, int* tokpos) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int c = tid + kThreads * i;
      const int tok = c / kChunksPerRow;
      const int col = c - tok * kChunksPerRow;
      *(u32x4*)(kb + tok * kLdsRow + col * 16) = r[i];
      if (SPARSE && col == 0) tokpos[tok] = tp[i];
    }
  }
};

template <bool SPARSE>
struct Stager<1, SPARSE> {
  static constexpr int kChunksPerRow = kFp8RowBytes / 16;             // 41
  static constexpr int kTotal = kPage * kChunksPerRow;                // 2624
  static constexpr int kN = (kTotal + kThreads - 1) / kThreads;       // 11
  u32x4 r[kN];
  float sc[kN];
  int tp[kN];

  __device__ __forceinline__ void load(const DecodeParams& p, int b, int j, int L, int Wunit,
                                       const int32_t* idx_row) {
    const int tid = threadIdx.x;
    int dense_page = -1;
    if (!SPARSE && j * kPage < L) dense_page = p.block_table[(size_t)b * p.max_blocks + j];
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int c = tid + kThreads * i;
      const int tok = c / kChunksPerRow;
      const int col = c - tok * kChunksPerRow;
      r[i] = u32x4{0, 0, 0, 0};
      sc[i] = 0.f;
      tp[i] = -1;
      if (c < kTotal && col != 32) {
        const uint8_t* row =
            key_row<SPARSE>(p, b, j, tok, L, Wunit, idx_row, kFp8RowBytes, dense_page, &tp[i]);
        if (row) {
          r[i] = *(const u32x4*)(row + col * 16);
          if (col < 32) sc[i] = *(const float*)(row + kFp8ScaleOff + 4 * (col >> 3));
        }
      }
    }
  }

  __device__ __forceinline__ void store(uint8_t* kb, int* tokpos) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int c = tid + kThreads * i;
      if (c >= kTotal) continue;
      const int tok = c / kChunksPerRow;
      const int col = c - tok * kChunksPerRow;
      uint8_t* dst = kb + tok * kLdsRow;
      if (col < 32) {
        // 16 e4m3 codes of NoPE group col/8 -> 16 bf16 at dims [16 col, 16 col + 16)
        u32x4 lo, hi;
        const float s = sc[i];
        uint32_t w[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)r[i][q], false);
          const f32x2 bq = __builtin_amdgcn_cvt_pk_f32_fp8((int)r[i][q], true);
          w[2 * q] = pack_bf16x2(a[0] * s, a[1] * s);
          w[2 * q + 1] = pack_bf16x2(bq[0] * s, bq[1] * s);
        }
        lo = u32x4{w[0], w[1], w[2], w[3]};
        hi = u32x4{w[4], w[5], w[6], w[7]};
        *(u32x4*)(dst + col * 32) = lo;
        *(u32x4*)(dst + col * 32 + 16) = hi;
      } else if (col > 32) {
        // 8 bf16 RoPE values -> dims [512 + 8 (col - 33), +8)
        *(u32x4*)(dst + 2 * kDnope + (col - 33) * 16) = r[i];
      }
      if (SPARSE && col == 0) tokpos[tok] = tp[i];
    }
  }
};

// ---------------------------------------------------------------------------
// The split-KV kernel.
// ---------------------------------------------------------------------------
template <int FMT, bool SPARSE, int NRB>
__global__ __launch_bounds__(kThreads, 1) void splitkv_kernel(const DecodeParams p) {
  constexpr int TG = 4 / NRB;         // token groups sharing one row block
  constexpr int TPW = kPage / TG;     // keys per wave per block
  constexpr int NSUB = TPW / 16;      // 16-key sub-blocks per wave per block
  constexpr int RT = 16 * NRB;        // rows per workgroup

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kLdsBuf];
  __shared__ int tokpos[2][kPage];
  __shared__ float red_m[4][16];
  __shared__ float red_l[4][16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rb = wave % NRB;
  const int tg = wave / NRB;
  const int l16 = lane & 15;
  const int lg = lane >> 4;

  // Block id -> (part, row tile): the row tiles of one part share an XCD.
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

  const int row0 = rt * RT;
  const int my_row = row0 + rb * 16 + l16;   // the query row this lane tracks
  const bool row_ok = my_row < p.R;

  for (int u = u0; u <= u1; ++u) {
    const int jb = (u == u0) ? j0 : 0;
    const int je = (u == u1) ? j1 : unit_blocks[u];
    const int b = SPARSE ? u / p.s_q : u;
    const int L = p.seqlens[b];
    const int s_unit = SPARSE ? u % p.s_q : 0;
    const int s_row = SPARSE ? s_unit : (row_ok ? my_row / p.h_q : 0);
    int W = L;
    if (p.causal) W = min(max(L - p.s_q + 1 + s_row, 0), L);
    int Wunit = L;
    if (SPARSE && p.causal) Wunit = min(max(L - p.s_q + 1 + s_unit, 0), L);
    const int32_t* idx_row = SPARSE ? p.indices + (size_t)u * p.topk : nullptr;

    // Q fragments (B operand of S^T = K Q^T), held for the whole unit.
    bf16x8 qf[kDqk / 32];
    {
      const uint8_t* qrow = p.q + ((size_t)u * p.R + (row_ok ? my_row : 0)) * (2 * kDqk);
#pragma unroll
      for (int i = 0; i < kDqk / 32; ++i) {
        u32x4 v = *(const u32x4*)(qrow + (32 * i + 8 * lg) * 2);
        if (!row_ok) v = u32x4{0, 0, 0, 0};
        qf[i] = __builtin_bit_cast(bf16x8, v);
      }
    }

    float m_run = -INFINITY;
    float l_part = 0.f;
    f32x4 o[kDv / 16];
#pragma unroll
    for (int d = 0; d < kDv / 16; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};

    Stager<FMT, SPARSE> st;
    if (jb < je) st.load(p, b, jb, L, Wunit, idx_row);

    for (int j = jb; j < je; ++j) {
      const int buf = (j - jb) & 1;
      uint8_t* kb = smem + buf * kLdsBuf;
      st.store(kb, tokpos[buf]);
      if (j + 1 < je) st.load(p, b, j + 1, L, Wunit, idx_row);
      __syncthreads();

      // ---- scores S^T for this wave's keys
      float sv[NSUB][4];
#pragma unroll
      for (int sb = 0; sb < NSUB; ++sb) {
        const int tok_base = tg * TPW + sb * 16;
        const uint8_t* arow = kb + (tok_base + l16) * kLdsRow + lg * 16;
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < kDqk / 32; ++i) {
          const bf16x8 a = *(const bf16x8*)(arow + i * 64);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[i], acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tl = tok_base + 4 * lg + r;
          bool ok;
          if (SPARSE)
            ok = tokpos[buf][tl] >= 0;
          else
            ok = j * kPage + tl < W;
          sv[sb][r] = ok ? acc[r] * p.scale_log2 : -INFINITY;
        }
      }

      // ---- online softmax (exp2 domain).  The reference max m_run is only
      // raised when a row's block max exceeds it by more than kRescaleSlack
      // (log2 units): P values then stay below 2^kRescaleSlack, and O and
      // the row sum always share one reference, so out = O / l is unchanged
      // while the O accumulators are rescaled only rarely.
      float mx = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < NSUB; ++sb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sv[sb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const bool raise = mx > m_run + kRescaleSlack;
      if (__any(raise)) {
        const float m_new = raise ? mx : m_run;
        const float alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new));
        m_run = m_new;
        l_part *= alpha;
        // (not force-unrolled: that makes the scheduler lift every
        // accumulator read at once and spill other live registers)
        for (int d = 0; d < kDv / 16; ++d) o[d] *= alpha;
      }
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
      float psum = 0.f;
#pragma unroll
      for (int sb = 0; sb < NSUB; ++sb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sv[sb][r] = fast_exp2(sv[sb][r] - m_use);
          psum += sv[sb][r];
        }
      l_part += psum;

      // ---- O^T += V^T P^T
      if constexpr (NSUB == 1) {
        const int tok_base = tg * TPW;
        s16x4 pb;
#pragma unroll
        for (int r = 0; r < 4; ++r) pb[r] = (short)bf16_rne_bits(sv[0][r]);
        const uint8_t* vcol = kb + (tok_base + 4 * lg) * kLdsRow + l16 * 2;
#pragma unroll
        for (int d = 0; d < kDv / 16; ++d) {
          s16x4 va;
#pragma unroll
          for (int r = 0; r < 4; ++r) va[r] = *(const short*)(vcol + r * kLdsRow + d * 32);
          o[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, o[d], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int pr = 0; pr < NSUB / 2; ++pr) {
          const int tb0 = tg * TPW + (2 * pr) * 16;
          const int tb1 = tb0 + 16;
          u32x4 pw;
          pw[0] = pack_bf16x2(sv[2 * pr][0], sv[2 * pr][1]);
          pw[1] = pack_bf16x2(sv[2 * pr][2], sv[2 * pr][3]);
          pw[2] = pack_bf16x2(sv[2 * pr + 1][0], sv[2 * pr + 1][1]);
          pw[3] = pack_bf16x2(sv[2 * pr + 1][2], sv[2 * pr + 1][3]);
          const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
          const uint8_t* v0 = kb + (tb0 + 4 * lg) * kLdsRow + l16 * 2;
          const uint8_t* v1 = kb + (tb1 + 4 * lg) * kLdsRow + l16 * 2;
#pragma unroll
          for (int d = 0; d < kDv / 16; ++d) {
            uint32_t w[4];
#pragma unroll
            for (int r = 0; r < 2; ++r) {
              const uint32_t a0 = *(const uint16_t*)(v0 + (2 * r) * kLdsRow + d * 32);
              const uint32_t a1 = *(const uint16_t*)(v0 + (2 * r + 1) * kLdsRow + d * 32);
              w[r] = a0 | (a1 << 16);
              const uint32_t c0 = *(const uint16_t*)(v1 + (2 * r) * kLdsRow + d * 32);
              const uint32_t c1 = *(const uint16_t*)(v1 + (2 * r + 1) * kLdsRow + d * 32);
              w[2 + r] = c0 | (c1 << 16);
            }
            const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
            o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[d], 0, 0, 0);
          }
        }
      }
    }

    // ---- end of this unit's blocks: merge token groups, normalise, write
    float l_row = l_part + __shfl_xor(l_part, 16);
    l_row += __shfl_xor(l_row, 32);
    __syncthreads();   // every wave is done with the staged blocks
    if (lane < 16) {
      red_m[wave][lane] = m_run;
      red_l[wave][lane] = l_row;
    }
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int g = 0; g < TG; ++g) M = fmaxf(M, red_m[g * NRB + rb][l16]);
    const float M_use = M == -INFINITY ? 0.f : M;
    const float f = fast_exp2(m_run - M_use);
    float* ob = (float*)smem + wave * 16 * kOStride;
#pragma unroll
    for (int d = 0; d < kDv / 16; ++d)
      *(f32x4*)(ob + l16 * kOStride + 16 * d + 4 * lg) = o[d] * f;
    __syncthreads();

    const int k_u = p.num_splits[u + 1] - p.num_splits[u];
    const int slot = p.num_splits[u] + (u == u0 ? split0 : 0);
    constexpr int RPW = 16 / TG;   // rows each wave finalises
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
      const int rr = tg * RPW + q;               // row within the row block
      const int r = row0 + rb * 16 + rr;
      if (r >= p.R) continue;
      float Mr = -INFINITY;
#pragma unroll
      for (int g = 0; g < TG; ++g) Mr = fmaxf(Mr, red_m[g * NRB + rb][rr]);
      const float Mr_use = Mr == -INFINITY ? 0.f : Mr;
      float Lr = 0.f;
#pragma unroll
      for (int g = 0; g < TG; ++g)
        Lr += red_l[g * NRB + rb][rr] * fast_exp2(red_m[g * NRB + rb][rr] - Mr_use);
      f32x4 a0 = f32x4{0.f, 0.f, 0.f, 0.f}, a1 = a0;
#pragma unroll
      for (int g = 0; g < TG; ++g) {
        const float* src = (const float*)smem + (g * NRB + rb) * 16 * kOStride + rr * kOStride + 8 * lane;
        a0 += *(const f32x4*)src;
        a1 += *(const f32x4*)(src + 4);
      }
      const float inv = Lr > 0.f ? 1.f / Lr : 0.f;
      a0 *= inv;
      a1 *= inv;
      const float lse_nat = Lr > 0.f ? (Mr_use + fast_log2(Lr)) * kLn2 : -INFINITY;
      const size_t grow = (size_t)u * p.R + r;
      if (k_u == 1) {
        u32x4 w;
        w[0] = pack_bf16x2(a0[0], a0[1]);
        w[1] = pack_bf16x2(a0[2], a0[3]);
        w[2] = pack_bf16x2(a1[0], a1[1]);
        w[3] = pack_bf16x2(a1[2], a1[3]);
        *(u32x4*)(p.out + grow * kDv + 8 * lane) = w;
        if (lane == 0) p.lse[grow] = lse_nat;
      } else {
        float* dst = p.ws_o + ((size_t)slot * p.R + r) * kDv + 8 * lane;
        *(f32x4*)dst = a0;
        *(f32x4*)(dst + 4) = a1;
        if (lane == 0) p.ws_lse[(size_t)slot * p.R + r] = lse_nat;
      }
    }
    __syncthreads();   // LDS is reused by the next unit's staging
  }
}

// ---------------------------------------------------------------------------
// Combine: merge the k_u partial results of every split unit.
//   lse = log sum_i exp(lse_i);  out = sum_i exp(lse_i - lse) * O_i
// One wave per query row; lanes own 8 output dims each.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(const int32_t* __restrict__ num_splits,
                                                      const float* __restrict__ ws_o,
                                                      const float* __restrict__ ws_lse,
                                                      uint16_t* __restrict__ out,
                                                      float* __restrict__ lse, int R) {
  const int u = blockIdx.x;
  const int base = num_splits[u];
  const int k = num_splits[u + 1] - base;
  if (k <= 1) return;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  float M = -INFINITY;
  for (int i = lane; i < k; i += 64) M = fmaxf(M, ws_lse[(size_t)(base + i) * R + r]);
  M = wave_max(M);
  const size_t grow = (size_t)u * R + r;
  if (M == -INFINITY) {
    *(u32x4*)(out + grow * kDv + 8 * lane) = u32x4{0, 0, 0, 0};
    if (lane == 0) lse[grow] = -INFINITY;
    return;
  }
  float S = 0.f;
  for (int i = lane; i < k; i += 64) S += fast_exp2((ws_lse[(size_t)(base + i) * R + r] - M) * kLog2e);
  S = wave_sum(S);
  const float lse_r = M + fast_log2(S) * kLn2;
  f32x4 a0 = f32x4{0.f, 0.f, 0.f, 0.f}, a1 = a0;
  for (int i = 0; i < k; ++i) {
    const float w = fast_exp2((ws_lse[(size_t)(base + i) * R + r] - lse_r) * kLog2e);
    const float* src = ws_o + ((size_t)(base + i) * R + r) * kDv + 8 * lane;
    a0 += w * *(const f32x4*)src;
    a1 += w * *(const f32x4*)(src + 4);
  }
  u32x4 wv;
  wv[0] = pack_bf16x2(a0[0], a0[1]);
  wv[1] = pack_bf16x2(a0[2], a0[3]);
  wv[2] = pack_bf16x2(a1[0], a1[1]);
  wv[3] = pack_bf16x2(a1[2], a1[3]);
  *(u32x4*)(out + grow * kDv + 8 * lane) = wv;
  if (lane == 0) lse[grow] = lse_r;
}

int rows_per_workgroup(int rows_per_unit) {
  if (rows_per_unit <= 16) return 16;
  if (rows_per_unit <= 32) return 32;
  return 128;   // mla_decode_wide.hip
}

template <int FMT, bool SPARSE>
static void launch_variant(const DecodeParams& p, dim3 grid, hipStream_t stream) {
  const int rt = rows_per_workgroup(p.R);
  if (rt == 16)
    hipLaunchKernelGGL((splitkv_kernel<FMT, SPARSE, 1>), grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((splitkv_kernel<FMT, SPARSE, 2>), grid, dim3(kThreads), 0, stream, p);
}

hipError_t launch_decode(const DecodeParams& p, int kv_format, int which, hipStream_t stream) {
  if (which & 1) {
    const int parts8 = (p.num_parts + 7) / 8 * 8;
    const dim3 grid(parts8 * p.row_tiles);
    const bool sparse = p.indices != nullptr;
    if (rows_per_workgroup(p.R) == 128) {
      hipError_t e = launch_wide(p, kv_format, grid, stream);
      if (e != hipSuccess) return e;
    } else if (kv_format == 0) {
      if (sparse)
        launch_variant<0, true>(p, grid, stream);
      else
        launch_variant<0, false>(p, grid, stream);
    } else {
      if (sparse)
        launch_variant<1, true>(p, grid, stream);
      else
        launch_variant<1, false>(p, grid, stream);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (which & 2) {
    const dim3 cgrid(p.units, (p.R + 3) / 4);
    hipLaunchKernelGGL(combine_kernel, cgrid, dim3(256), 0, stream, p.num_splits, p.ws_o, p.ws_lse,
                       p.out, p.lse, p.R);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace mla
