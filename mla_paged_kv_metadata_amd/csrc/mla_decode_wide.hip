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
//   * One workgroup = 8 waves = 128 query rows; wave w owns 16 rows and all
//     64 keys of every block, so each wave's softmax is self-contained and
//     waves only meet at the block barrier.  Two waves share a SIMD, so
//     every MFMA keeps its accumulators in VGPRs: O^T (16 rows x 512 dims,
//     fp32, 128 VGPRs) and the Q^T fragments (72 VGPRs) fit beside the
//     working set.
//   * Both products run on v_mfma_f32_16x16x32_bf16.  S^T = K Q^T with K
//     (16 keys x 32 dims) from LDS and Q^T held in registers for the whole
//     sequence; the 16x16 result gives each lane one query row and 4 keys,
//     so two key tiles make exactly the 8-key B operand of O^T += V^T P^T
//     and P never leaves registers.  V^T comes from ds_read_b64_tr_b16,
//     which transposes 4 keys x 16 dims across a 16-lane group.
//   * Pages are copied HBM -> LDS with global_load_lds (16 bytes per lane,
//     no VGPR round trip), double buffered.  The 16-byte chunks of each key
//     row are XOR-swizzled (chunk c of key t sits at c ^ swz(t) within its
//     group of 8) so that the fragment reads spread over the LDS banks.
//   * FP8 rows are copied raw into LDS, then dequantised (e4m3 -> fp32,
//     times the group scale, -> bf16) into the swizzled bf16 block by all
//     threads before the MFMA work.
//   * Key slots nobody may see are loaded from a visible key of the same
//     block (never from outside the sequence) and their probabilities are
//     forced to zero, so V never carries stale or poisoned memory.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace wide {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 16;
constexpr int kRowsPerWg = kRowsPerWave * kWaves;   // 128
constexpr int kChunks = kBf16RowBytes / 16;            // 72 16-byte chunks per key row
constexpr int kBlockBytes = kPage * kBf16RowBytes;     // 73,728
constexpr int kRawBytes = kPage * kFp8RowBytes;        // 41,984
constexpr int kKSteps = kDqk / 32;                     // 18
constexpr float kRescaleSlack = 8.f;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Bank swizzle of the 16-byte chunk index within its aligned group of 8.
// Bits of t: s = 4*(t1^t0) + 2*t2 + (t3^t0).  Makes the 32-key x 1-chunk
// fragment reads conflict-free and spreads the transposed 4-key reads.
__device__ __forceinline__ int swz(int t) {
  return ((((t >> 1) ^ t) & 1) << 2) | (((t >> 2) & 1) << 1) | (((t >> 3) ^ t) & 1);
}
__device__ __forceinline__ int phys_chunk(int t, int c) { return (c & ~7) | ((c ^ swz(t)) & 7); }

__device__ __forceinline__ void lds_dma16(const void* gsrc, void* lds_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)gsrc,
                                   (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// The lane id behind an empty asm: values derived from it inside a loop are
// recomputed there (a few ALU ops) instead of being hoisted out of the loop
// and kept live in registers, which would crowd out the Q fragments.
__device__ __forceinline__ int opaque_lane() {
  int l = threadIdx.x & 63;
  asm volatile("" : "+v"(l));
  return l;
}

// Resolve the 64 key slots of block j: lane t returns the pool row index
// (page * 64 + slot) to load for slot t, and whether slot t is visible.
// Masked slots get the row of a visible slot of the same block.  *mask
// receives the wave-uniform bitmask of visible slots.
template <bool SPARSE>
__device__ __forceinline__ int resolve_slot(const DecodeParams& p, int b, int j, int L, int Wunit,
                                            const int32_t* idx_row, int lane,
                                            unsigned long long* mask) {
  int row = 0;
  bool ok;
  if (!SPARSE) {
    const int t = j * kPage + lane;
    ok = t < L;
    const int page = j * kPage < L ? p.block_table[(size_t)b * p.max_blocks + j] : 0;
    const int last = min(L - 1 - j * kPage, kPage - 1);
    row = page * kPage + (ok ? lane : max(last, 0));
  } else {
    const int e = j * kPage + lane;
    const int t = e < p.topk ? idx_row[e] : -1;
    ok = t >= 0 && t < Wunit;
    if (ok) row = p.block_table[(size_t)b * p.max_blocks + (t >> 6)] * kPage + (t & (kPage - 1));
    const unsigned long long m = __ballot(ok);
    const int first = m ? __builtin_ctzll(m) : 0;
    const int first_row = __shfl(row, first);
    if (!ok) row = first_row;
  }
  *mask = __ballot(ok);
  return row;
}

// Copy block j into `dst` (bf16 rows, swizzled) or `raw` (FP8 rows, linear)
// with global_load_lds; returns the visible-slot mask (0: nothing copied).
template <int FMT, bool SPARSE>
__device__ __forceinline__ unsigned long long issue_block(const DecodeParams& p, uint8_t* dst, int b,
                                                          int j, int L, int Wunit,
                                                          const int32_t* idx_row) {
  const int ln = opaque_lane();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  unsigned long long mask;
  const int row = resolve_slot<SPARSE>(p, b, j, L, Wunit, idx_row, ln, &mask);
  if (mask == 0ull) return 0ull;
  if constexpr (FMT == 0) {
    int dense_base = 0, dense_last = 0;
    if (!SPARSE) {
      dense_base = p.block_table[(size_t)b * p.max_blocks + j] * kPage;
      dense_last = min(L - 1 - j * kPage, kPage - 1);
    }
#pragma unroll
    for (int i = 0; i < 72 / kWaves; ++i) {
      const int inst = wave * (72 / kWaves) + i;
      const int q = inst * 64 + ln;
      const int t = q / kChunks;
      const int pc = q - t * kChunks;
      const int c = phys_chunk(t, pc);
      const int trow = SPARSE ? __shfl(row, t) : dense_base + min(t, dense_last);
      lds_dma16(p.kcache + (size_t)trow * kBf16RowBytes + c * 16, dst + inst * 1024);
    }
  } else {
    for (int inst = wave; inst < 41; inst += kWaves) {
      const int q = inst * 64 + ln;
      const int t = q / 41;
      const int cc = q - t * 41;
      const int trow = __shfl(row, t);
      lds_dma16(p.kcache + (size_t)trow * kFp8RowBytes + cc * 16, dst + inst * 1024);
    }
  }
  return mask;
}

// Dequantise a raw FP8 block into the swizzled bf16 block (all threads).
__device__ __forceinline__ void dequant_block(const uint8_t* raw, uint8_t* dst) {
  for (int w = threadIdx.x; w < kPage * 40; w += kThreads) {
    const int t = w / 40;
    const int k = w - t * 40;
    const uint8_t* rrow = raw + t * kFp8RowBytes;
    uint8_t* drow = dst + t * kBf16RowBytes;
    if (k < 32) {
      const u32x4 codes = *(const u32x4*)(rrow + 16 * k);
      const float s = *(const float*)(rrow + kFp8ScaleOff + 4 * (k >> 3));
      uint32_t wv[8];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes[qq], false);
        const f32x2 c2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes[qq], true);
        wv[2 * qq] = pack_bf16x2(a[0] * s, a[1] * s);
        wv[2 * qq + 1] = pack_bf16x2(c2[0] * s, c2[1] * s);
      }
      *(u32x4*)(drow + phys_chunk(t, 2 * k) * 16) = u32x4{wv[0], wv[1], wv[2], wv[3]};
      *(u32x4*)(drow + phys_chunk(t, 2 * k + 1) * 16) = u32x4{wv[4], wv[5], wv[6], wv[7]};
    } else {
      const int rc = k - 32;
      *(u32x4*)(drow + phys_chunk(t, 64 + rc) * 16) = *(const u32x4*)(rrow + kFp8RopeOff + 16 * rc);
    }
  }
}


template <int FMT>
struct Smem;
template <>
struct Smem<0> {
  uint8_t kb[2][kBlockBytes];     // double-buffered bf16 blocks
  __device__ uint8_t* copy_target(int buf) { return kb[buf]; }
};
template <>
struct Smem<1> {
  uint8_t raw[2][kRawBytes];      // double-buffered FP8 rows as stored
  uint8_t kb[1][kBlockBytes];     // the block being computed, dequantised
  __device__ uint8_t* copy_target(int buf) { return raw[buf]; }
};

template <int FMT, bool SPARSE>
__global__ __launch_bounds__(kThreads, 1) void wide_kernel(const DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) Smem<FMT> sm;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15;
  const int lg = lane >> 4;

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

  const int my_row = rt * kRowsPerWg + wave * kRowsPerWave + l16;
  const bool row_ok = my_row < p.R;

  for (int u = u0; u <= u1; ++u) {
    const int jb = (u == u0) ? j0 : 0;
    const int je = (u == u1) ? j1 : unit_blocks[u];
    const int b = SPARSE ? u / p.s_q : u;
    const int L = p.seqlens[b];
    const int s_unit = SPARSE ? u % p.s_q : 0;
    const int s_row = SPARSE ? s_unit : (row_ok ? my_row / p.h_q : 0);
    const int W = p.causal ? min(max(L - p.s_q + 1 + s_row, 0), L) : L;
    const int Wunit = (SPARSE && p.causal) ? min(max(L - p.s_q + 1 + s_unit, 0), L) : L;
    const int32_t* idx_row = SPARSE ? p.indices + (size_t)u * p.topk : nullptr;

    // Q^T fragments (B operand): lane holds row l16, dims 32 ks + 8 lg + 0..7.
    bf16x8 qf[kKSteps];
    {
      const uint8_t* qrow = p.q + ((size_t)u * p.R + (row_ok ? my_row : 0)) * (2 * kDqk);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        u32x4 v = *(const u32x4*)(qrow + 64 * ks + 16 * lg);
        if (!row_ok) v = u32x4{0, 0, 0, 0};
        qf[ks] = __builtin_bit_cast(bf16x8, v);
      }
    }

    float m_run = -INFINITY;
    float l_part = 0.f;
    f32x4 o[kDv / 16];
#pragma unroll
    for (int d = 0; d < kDv / 16; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};

    unsigned long long vis[2];
    vis[0] = issue_block<FMT, SPARSE>(p, sm.copy_target(0), b, jb, L, Wunit, idx_row);
    vis[1] = 0ull;
    for (int j = jb; j < je; ++j) {
      const int buf = (j - jb) & 1;
      wait_vmem();
      __syncthreads();   // block j is in LDS; every wave is done with block j-1
      if (j + 1 < je)
        vis[buf ^ 1] = issue_block<FMT, SPARSE>(p, sm.copy_target(buf ^ 1), b, j + 1, L, Wunit, idx_row);
      const unsigned long long vmask = vis[buf];
      if (vmask == 0ull) continue;   // no visible key in block j (uniform)
      const uint8_t* kb;
      if constexpr (FMT == 0) {
        kb = sm.kb[buf];
      } else {
        dequant_block(sm.copy_target(buf), sm.kb[0]);
        __syncthreads();
        kb = sm.kb[0];
      }

      // ---- S^T = K Q^T: tile kt covers keys 16 kt + 0..15; lane holds row
      // l16 and keys 16 kt + 4 lg + r.  The swizzle repeats every 2 k-steps
      // (8 chunks), so two lane offsets per tile are live.
      f32x4 sacc[4];
      {
        const int ln = opaque_lane();
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const int t = 16 * kt + (ln & 15);
          const int sw = swz(t);
          const int ko0 = t * kBf16RowBytes + (((ln >> 4) ^ sw) & 7) * 16;
          const int ko1 = t * kBf16RowBytes + (((4 + (ln >> 4)) ^ sw) & 7) * 16;
          f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < kKSteps; ++ks) {
            const bf16x8 a = *(const bf16x8*)(kb + ((ks & 1) ? ko1 : ko0) + (ks >> 1) * 128);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[ks], acc, 0, 0, 0);
          }
          sacc[kt] = acc;
        }
      }

      // ---- mask + online softmax (exp2 domain).  The reference max m_run is
      // only raised when a row's block max exceeds it by more than
      // kRescaleSlack: P then stays below 2^kRescaleSlack and O and the row
      // sum always share one reference.
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tl = 16 * kt + 4 * lg + r;
          const bool ok = SPARSE ? ((vmask >> tl) & 1ull) != 0ull : (j * kPage + tl < W);
          sacc[kt][r] = ok ? sacc[kt][r] * p.scale_log2 : -INFINITY;
          mx = fmaxf(mx, sacc[kt][r]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const bool raise = mx > m_run + kRescaleSlack;
      if (__any(raise)) {
        const float m_new = raise ? mx : m_run;
        const float alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new));
        m_run = m_new;
        l_part *= alpha;
#pragma unroll
        for (int d = 0; d < kDv / 16; ++d) o[d] *= alpha;
      }
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
      u32x4 pw[2];   // B operands of the two PV MFMA groups (key tiles 0+1, 2+3)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        float e[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          e[r] = fast_exp2(sacc[2 * pp][r] - m_use);
          e[4 + r] = fast_exp2(sacc[2 * pp + 1][r] - m_use);
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) l_part += e[r];
        pw[pp] = u32x4{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]), pack_bf16x2(e[4], e[5]),
                       pack_bf16x2(e[6], e[7])};
      }

      // ---- O^T += V^T P^T.  Group pp covers key tiles 2pp and 2pp+1; k-slot
      // i of lane group lg is key 16 (2pp + (i >> 2)) + 4 lg + (i & 3).  The
      // transposed read of 16-lane group lg takes 4 keys x 16 dims; source
      // lane jj supplies key (jj >> 2) of the run and dims 4 (jj & 3) .. +3.
      {
        const int ln = opaque_lane();
        const int G = ln >> 4;
        const int jj = ln & 15;
        const int boff = (jj & 1) * 8;              // dims 4 (jj & 3): byte 8 within a chunk
        const int csub = (jj & 3) >> 1;             // chunk within a 16-dim tile
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const bf16x8 pb = __builtin_bit_cast(bf16x8, pw[pp]);
          const int tA = 32 * pp + 4 * G + (jj >> 2);
          const int tB = tA + 16;
          const int sA = swz(tA), sB = swz(tB);
          int voA[4], voB[4];
#pragma unroll
          for (int dq = 0; dq < 4; ++dq) {   // swizzle period: 4 dim tiles (8 chunks)
            voA[dq] = tA * kBf16RowBytes + (((2 * dq + csub) ^ sA) & 7) * 16 + boff;
            voB[dq] = tB * kBf16RowBytes + (((2 * dq + csub) ^ sB) & 7) * 16 + boff;
          }
#pragma unroll
          for (int dt = 0; dt < kDv / 16; ++dt) {
            const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(kb + voA[dt & 3] + (dt >> 2) * 128));
            const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(kb + voB[dt & 3] + (dt >> 2) * 128));
            const u32x2 xa = __builtin_bit_cast(u32x2, va);
            const u32x2 xb = __builtin_bit_cast(u32x2, vb);
            const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{xa[0], xa[1], xb[0], xb[1]});
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb, o[dt], 0, 0, 0);
          }
        }
      }
    }

    // ---- epilogue: lane holds row l16, dims 16 dt + 4 lg + (0..3)
    float l_row = l_part + __shfl_xor(l_part, 16);
    l_row += __shfl_xor(l_row, 32);
    const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
    const float lse_nat =
        l_row > 0.f ? ((m_run == -INFINITY ? 0.f : m_run) + fast_log2(l_row)) * kLn2 : -INFINITY;
    const int k_u = p.num_splits[u + 1] - p.num_splits[u];
    const int slot = p.num_splits[u] + (u == u0 ? split0 : 0);
    if (row_ok) {
      const size_t grow = (size_t)u * p.R + my_row;
      if (k_u == 1) {
        uint16_t* orow = p.out + grow * kDv;
#pragma unroll
        for (int dt = 0; dt < kDv / 16; ++dt)
          *(u32x2*)(orow + 16 * dt + 4 * lg) = u32x2{pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv),
                                                    pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv)};
        if (lg == 0) p.lse[grow] = lse_nat;
      } else {
        float* orow = p.ws_o + ((size_t)slot * p.R + my_row) * kDv;
#pragma unroll
        for (int dt = 0; dt < kDv / 16; ++dt) *(f32x4*)(orow + 16 * dt + 4 * lg) = o[dt] * inv;
        if (lg == 0) p.ws_lse[(size_t)slot * p.R + my_row] = lse_nat;
      }
    }
    __syncthreads();   // the next unit's first copy reuses the buffers
  }
}

}  // namespace wide

hipError_t launch_wide(const DecodeParams& p, int kv_format, dim3 grid, hipStream_t stream) {
  const bool sparse = p.indices != nullptr;
  if (kv_format == 0) {
    if (sparse)
      hipLaunchKernelGGL((wide::wide_kernel<0, true>), grid, dim3(wide::kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((wide::wide_kernel<0, false>), grid, dim3(wide::kThreads), 0, stream, p);
  } else {
    if (sparse)
      hipLaunchKernelGGL((wide::wide_kernel<1, true>), grid, dim3(wide::kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((wide::wide_kernel<1, false>), grid, dim3(wide::kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace mla
