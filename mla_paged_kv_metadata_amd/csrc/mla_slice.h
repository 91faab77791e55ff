// Staging of 32-key "slices" (half a 64-token page) in LDS for the gfx950
// decode kernels: LDS layout, copies straight from global memory into LDS,
// the waits and barriers around them, and small cross-lane helpers.
//
// A bf16 slice (32 keys x 576 dims) is stored chunk-group-major: the 72
// 16-byte chunks of a key row form 9 groups of 8, and group G of all 32 keys
// is one 4 KiB block (key t at 128 t), with the chunk index XOR-swizzled
// within its group by a function of t.  Fragment reads of 16 or 32 keys at
// one chunk (K operands) or of 4 keys x 32 dims (transposed V operands) then
// hit every LDS bank once, and each lane of a copy moves chunks of a single
// key, so a copy's address is a per-lane constant plus a scalar base.
// An FP8 slice is copied as stored (32 rows of 656 bytes) and dequantised
// into a bf16 slice in LDS.
#pragma once

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace slice {

constexpr int kSlice = 32;                              // keys per slice
constexpr int kSliceBytes = kSlice * kBf16RowBytes;     // 36,864
constexpr int kRawSliceBytes = kSlice * kFp8RowBytes;   // 20,992
constexpr int kRawSlotBytes = 21 * 1024;                // FP8 slot, whole 1 KiB copies
constexpr int kGroupBytes = kSlice * 128;               // 8 chunks of all 32 keys: 4 KiB
constexpr int kTab = 1024;                              // sparse: resolved rows per table fill

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Bank swizzle of the 16-byte chunk index within its group of 8, for key t
// of the slice.  Bits of t: s = 4*(t1^t0) + 2*t2 + (t3^t0).
__device__ __forceinline__ int swz(int t) {
  return ((((t >> 1) ^ t) & 1) << 2) | (((t >> 2) & 1) << 1) | (((t >> 3) ^ t) & 1);
}
// Byte offset of chunk c (dims 8 c .. 8 c + 7) of key t in a bf16 slice.
__device__ __forceinline__ int slice_off(int t, int c) {
  return (c >> 3) * kGroupBytes + t * 128 + 16 * ((c ^ swz(t)) & 7);
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes
// land at lds_base + 16 l (global_load_lds_dwordx4; M0 holds the LDS base).
// No instruction offset is used: it would move the LDS destination as well.
// Written as asm, so the compiler neither tracks these copies nor inserts
// waits for them; the callers order them against LDS reads with barriers
// and wait for them with wait_vmem.  The asm has no output registers; its
// address operands are consumed at issue.  It has no memory clobber, so
// MFMAs and LDS reads of other buffers may be scheduled around it; volatile
// asm keeps its order against the barriers.
__device__ __forceinline__ void lds_dma16(const void* gsrc, void* lds_base) {
  const uint32_t m0 = (uint32_t)(uintptr_t)lds_base;
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gsrc), "{m0}"(m0));
}

// As lds_dma16, with the source split into a uniform 64-bit base (SGPRs)
// and a 32-bit per-lane byte offset (the saddr form): the steps between the
// instructions of one copy are then scalar adds to the base.
__device__ __forceinline__ void lds_dma16_s(const void* sbase, uint32_t voff, void* lds_base) {
  const uint32_t m0 = (uint32_t)(uintptr_t)lds_base;
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(m0));
}

// Wait until at most N vector-memory operations of this wave are pending
// (s_waitcnt with expcnt and lgkmcnt left at their no-wait maxima; vmcnt is
// split over bits 3:0 and 15:14).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier that waits only for this wave's own LDS operations
// (lgkmcnt), with compiler memory barriers on both sides.  (__syncthreads
// would also drain the copies into LDS still in flight.)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt: no wait
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The lane id behind an empty asm: values derived from it inside a loop are
// recomputed there (a few ALU ops) instead of being hoisted out of the loop
// and kept live in registers.
__device__ __forceinline__ int opaque_lane() {
  int l = threadIdx.x & 63;
  asm volatile("" : "+v"(l));
  return l;
}

// Value of lane l ^ 32 (v_permlane32_swap: no LDS round trip).
__device__ __forceinline__ float xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return (threadIdx.x & 32) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}
// Value of lane l ^ 16 (v_permlane16_swap).
__device__ __forceinline__ float xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return (threadIdx.x & 16) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}

// Sparse: resolve entries base .. base + count - 1 of the unit's index list
// into tab (all THREADS threads): the pool row of the indexed key, or -1
// when the entry is out of range or not visible to the unit.
// Entries are resolved in three batches, so that a fill costs two memory
// round trips whatever its size: every index entry is loaded, then every
// block-table entry (unconditionally: a masked entry reads entry 0 of the
// sequence's row, always in bounds, and is masked to -1 with bit
// operations, because a select on a loaded value becomes a branch and a
// wait around each load), then the table is written.
__device__ __forceinline__ int resolve_row(int page, int t, bool ok) {
  return (page * kPage + (t & (kPage - 1))) | (ok ? 0 : -1);
}

template <int THREADS, int MAXN>
__device__ __forceinline__ void fill_table(const DecodeParams& p, int32_t* tab, int b, int base, int count,
                                           int Wunit, const int32_t* idx_row) {
  int t[MAXN];
#pragma unroll
  for (int i = 0; i < MAXN; ++i) {
    const int k = (int)threadIdx.x + THREADS * i;
    t[i] = -1;
    if (k < count && base + k < p.topk) t[i] = idx_row[base + k];
  }
  const int32_t* bt = p.block_table + (size_t)b * p.max_blocks;
  int pg[MAXN];
#pragma unroll
  for (int i = 0; i < MAXN; ++i) pg[i] = bt[(t[i] >= 0 && t[i] < Wunit) ? (t[i] >> 6) : 0];
#pragma unroll
  for (int i = 0; i < MAXN; ++i) {
    const int k = (int)threadIdx.x + THREADS * i;
    if (k < count) tab[k] = resolve_row(pg[i], t[i], t[i] >= 0 && t[i] < Wunit);
  }
}

// The same fill in two halves, for a table of at most 2 THREADS entries:
// fill_table_issue loads the thread's index entries (a unit's start issues
// its query loads right after them, so both share one round trip);
// fill_table_finish resolves them through the block table and writes tab.
template <int THREADS>
__device__ __forceinline__ int2 fill_table_issue(const DecodeParams& p, int base, int count,
                                                 const int32_t* idx_row) {
  int2 t = make_int2(-1, -1);
  const int i0 = threadIdx.x, i1 = threadIdx.x + THREADS;
  if (i0 < count && base + i0 < p.topk) t.x = idx_row[base + i0];
  if (i1 < count && base + i1 < p.topk) t.y = idx_row[base + i1];
  return t;
}
template <int THREADS>
__device__ __forceinline__ void fill_table_finish(const DecodeParams& p, int32_t* tab, int b, int count, int Wunit,
                                                  int2 t) {
  const int i0 = threadIdx.x, i1 = threadIdx.x + THREADS;
  const int32_t* bt = p.block_table + (size_t)b * p.max_blocks;
  const bool ok0 = t.x >= 0 && t.x < Wunit, ok1 = t.y >= 0 && t.y < Wunit;
  const int pg0 = bt[ok0 ? (t.x >> 6) : 0];
  const int pg1 = bt[ok1 ? (t.y >> 6) : 0];
  if (i0 < count) tab[i0] = resolve_row(pg0, t.x, ok0);
  if (i1 < count) tab[i1] = resolve_row(pg1, t.y, ok1);
}

// Dense: the page of block j of sequence b (0 past the end of the
// sequence), read through the scalar cache.  Scalar loads are counted by
// lgkmcnt, so waiting for one leaves the copies into LDS in flight.
__device__ __forceinline__ int page_of(const DecodeParams& p, int b, int j, int L) {
  const __attribute__((address_space(4))) int32_t* bt =
      (const __attribute__((address_space(4))) int32_t*)p.block_table;
  const int page = bt[(size_t)b * p.max_blocks + j];
  return j * kPage < L ? page : 0;
}

// Pool row to load for slot t of slice sl of a unit: dense keys past the
// sequence take its last key of the same page; sparse masked entries take
// the slice's first visible row (first_row).  Inactive slices (past the
// unit's range) load row 0 of the pool.
template <bool SPARSE>
__device__ __forceinline__ int slot_row(const int32_t* tab, int tab_base, int sl, int t, int L, bool active,
                                        int page, int first_row) {
  if (!active) return 0;
  if (!SPARSE) {
    const int j = sl >> 1;
    const int tt = sl * kSlice + t;
    return page * kPage + max(min(tt, L - 1) - j * kPage, 0);
  }
  const int v = tab[sl * kSlice + t - tab_base];
  return v >= 0 ? v : first_row;
}

// Visible-slot mask of slice sl (bit t: slot t may be seen by some row of
// the unit) and, for sparse units, the slice's first visible row.  Uniform.
template <bool SPARSE>
__device__ __forceinline__ uint32_t slice_mask(const int32_t* tab, int tab_base, int sl, int L, bool active,
                                               int* first_row) {
  *first_row = 0;
  if (!active) return 0u;
  if (!SPARSE) {
    const int key0 = sl * kSlice;
    return key0 >= L ? 0u : (key0 + kSlice <= L ? 0xFFFFFFFFu : (1u << (L - key0)) - 1u);
  }
  const int v_own = tab[sl * kSlice + (opaque_lane() & (kSlice - 1)) - tab_base];
  const uint32_t mask = (uint32_t)__ballot(v_own >= 0);
  if (mask) *first_row = __builtin_amdgcn_readlane(v_own, __builtin_ctz(mask));
  return mask;
}

// Copy of a bf16 slice as 36 instructions of 64 lanes x 16 B: instruction
// inst = 4 G + k moves chunk group G of keys 8 k .. 8 k + 7 (lane l: key
// 8 k + l / 8, stored chunk 8 G + l % 8, which holds logical chunk
// 8 G + ((l % 8) ^ swz)).  Lane source for key octet k:
__device__ __forceinline__ const uint8_t* bf16_copy_src(const DecodeParams& p, int row, int k) {
  const int ln = opaque_lane();
  const int t = 8 * k + (ln >> 3);
  return p.kcache + (size_t)row * kBf16RowBytes + 16 * ((ln & 7) ^ swz(t));
}

// Decode a raw FP8 slice for the MFMAs with the scales left out (all
// THREADS threads): the 512 e4m3 NoPE codes of each key become bf16 values
// equal to the codes themselves (every e4m3 value is exact in bf16;
// v_cvt_scalef32_pk_bf16_fp8 with scale 1.0), the 64 bf16 RoPE values are
// copied, all into a bf16 slice `dst`.  The group scales stay in the raw
// rows (fp8_scales) and are applied after the MFMAs: to the score partial
// sums of each 128-dim group, and to the probabilities of each V group, so
// that no product code * scale is ever rounded.
template <int THREADS>
__device__ __forceinline__ void dequant_codes(const uint8_t* raw, uint8_t* dst) {
  static_assert((kSlice * 32) % THREADS == 0 && THREADS % 64 == 0, "whole items per thread");
  // NoPE: item w is 16-code chunk k = w / 32 of key t = w % 32, so that a
  // wave's lanes read 32 rows at one offset (the 656-byte row stride puts
  // 16 lanes on 64 distinct banks) and write one chunk of 32 keys (the
  // pattern the swizzle keeps conflict-free).  Every thread takes the same
  // number of items and no lane branches.  One item at a time: the callers
  // hold all their accumulators across this.
#pragma unroll 1
  for (int i = 0; i < kSlice * 32 / THREADS; ++i) {
    const int w = threadIdx.x + THREADS * i;
    const int t = w & (kSlice - 1);
    const int k = w >> 5;
    const u32x4 codes = *(const u32x4*)(raw + t * kFp8RowBytes + 16 * k);
    uint32_t wv[8];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      wv[2 * qq] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)codes[qq], 1.0f, false));
      wv[2 * qq + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)codes[qq], 1.0f, true));
    }
    *(u32x4*)(dst + slice_off(t, 2 * k)) = u32x4{wv[0], wv[1], wv[2], wv[3]};
    *(u32x4*)(dst + slice_off(t, 2 * k + 1)) = u32x4{wv[4], wv[5], wv[6], wv[7]};
  }
  // RoPE: 8 chunks of 8 bf16 per key, copied; item w is chunk w / 32 of key
  // w % 32 (whole waves take part or skip).
  for (int w = threadIdx.x; w < kSlice * 8; w += THREADS) {
    const int t = w & (kSlice - 1);
    const int rc = w >> 5;
    *(u32x4*)(dst + slice_off(t, 64 + rc)) = *(const u32x4*)(raw + t * kFp8RowBytes + kFp8RopeOff + 16 * rc);
  }
}

// Item i (< kSlice * 32 / THREADS) of the dequantisation of a raw FP8
// slice's 512 NoPE dims into a bf16 slice (the V operand), all THREADS
// threads: item w = threadIdx.x + THREADS i is 16-code chunk k = w / 32 of
// key t = w % 32, so that a wave's lanes read 32 rows at one offset (the
// 656-byte row stride puts 16 lanes on 64 distinct banks) and write one
// chunk of 32 keys (the pattern the swizzle keeps conflict-free).  Every
// thread takes the same number of items and no lane branches; the caller
// issues the items one at a time (it holds all its accumulators across
// them).  Each value is fp32(code) * scale rounded to bf16.
template <int THREADS>
__device__ __forceinline__ void dequant_item(const uint8_t* raw, uint8_t* dst, int i) {
  static_assert((kSlice * 32) % THREADS == 0 && THREADS % 64 == 0, "whole items per thread");
  const int w = (int)threadIdx.x + THREADS * i;
  const int t = w & (kSlice - 1);
  const int k = w >> 5;
  const uint8_t* rrow = raw + t * kFp8RowBytes;
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
  *(u32x4*)(dst + slice_off(t, 2 * k)) = u32x4{wv[0], wv[1], wv[2], wv[3]};
  *(u32x4*)(dst + slice_off(t, 2 * k + 1)) = u32x4{wv[4], wv[5], wv[6], wv[7]};
}

// The four group scales of key t of a raw FP8 slice (group g in element g).
__device__ __forceinline__ f32x4 fp8_scales(const uint8_t* raw, int t) {
  return *(const f32x4*)(raw + t * kFp8RowBytes + kFp8ScaleOff);
}

// The schedule's header does not match the call (built for another part or
// unit count, or not by the schedule kernel): nothing in it can be trusted,
// so no key is read.  Every workgroup of the grid writes out = 0 and
// lse = NaN for its share of all query rows (one row per wave at a time,
// strided by the grid), so that no row keeps stale memory.
template <int THREADS>
__device__ __forceinline__ void fill_mismatch(const DecodeParams& p) {
  constexpr int kW = THREADS / 64;
  const int lane = threadIdx.x & 63;
  const long long total = (long long)p.units * p.R;
  for (long long r = (long long)blockIdx.x * kW + (threadIdx.x >> 6); r < total;
       r += (long long)gridDim.x * kW) {
    *(u32x4*)(p.out + r * kDv + 8 * lane) = u32x4{0u, 0u, 0u, 0u};
    if (lane == 0) p.lse[r] = __builtin_nanf("");
  }
}

// True when the header of the schedule matches the call.
__device__ __forceinline__ bool header_ok(const DecodeParams& p, int h0, int h3, int h5) {
  return h0 == p.num_parts && h5 == kMagic && h3 == p.units;
}

template <int C>
struct Slot {
  static constexpr int value = C;
};

}  // namespace slice
}  // namespace mla
