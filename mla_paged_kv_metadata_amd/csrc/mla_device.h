// Device-side constants, vector types and small helpers shared by the
// gfx950 (CDNA4) kernels of the MLA paged-KV decode library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Geometry fixed by the method: 64-token pages (topnet.top "Was ist
// FlashMLA?", Hauptmerkmale), 576-dim query/key rows of 512 latent NoPE dims
// plus 64 RoPE dims, V = the first 512 dims, and the 656-byte FP8 row of
// 512 e4m3 codes, 4 fp32 scales and 64 bf16 RoPE values (sao.pub FlashMLA
// overview, 二、核心功能与架构).
constexpr int kPage = 64;
constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kDnope = 512;
constexpr int kBf16RowBytes = 2 * kDqk;  // 1152
constexpr int kFp8RowBytes = 656;
constexpr int kFp8ScaleOff = 512;
constexpr int kFp8RopeOff = 528;

// Schedule array layout (tile_metadata).
constexpr int kHeader = 8;
constexpr int kPartRow = 8;
constexpr int kMagic = 0x4D4C4131;
constexpr int kUnitOverhead = 2;  // c0: cost of one (unit, part) piece, in blocks
constexpr int kMaxParts = 2048;   // part rows the schedule kernel assembles in LDS

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 -> packed bf16 (lo in bits 0..15), round to nearest even, in one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// 2^x via v_exp_f32; exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) via v_log_f32.
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

// Work item (part, row tile) of workgroup bid.  With eight or more parts
// the grid holds the parts rounded up to a multiple of 8 times the row
// tiles, and consecutive block ids (which go to different XCDs) take
// consecutive parts, the row tiles of one part sharing an XCD and its L2:
// part = (rest / row_tiles) * 8 + (bid & 7), tile = rest % row_tiles with
// rest = bid / 8.  With fewer parts (row tiles alone fill the device) the
// grid is parts * row_tiles and bid = tile * parts + part.
__device__ __forceinline__ void work_item(int bid, int num_parts, int row_tiles, int* part, int* tile) {
  if (num_parts >= 8) {
    const int rest = bid >> 3;
    *tile = rest % row_tiles;
    *part = (rest / row_tiles) * 8 + (bid & 7);
  } else {
    *tile = bid / num_parts;
    *part = bid - *tile * num_parts;
  }
}

// Grid size for the mapping above.
inline int decode_grid(int num_parts, int row_tiles) {
  return (num_parts >= 8 ? (num_parts + 7) / 8 * 8 : num_parts) * row_tiles;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

}  // namespace mla
