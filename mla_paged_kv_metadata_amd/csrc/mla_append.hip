// Writing new tokens into the paged KV pool (the cache update that precedes
// a decode step), for gfx950.
//
// Row formats are those the decode reads (sao.pub FlashMLA overview,
// 二、核心功能与架构): a bf16 row is the token's 576 values; a 656-byte FP8
// row is 512 float8_e4m3fn NoPE codes (四、进阶玩法 names the type), 4 fp32
// scales (one per 128 NoPE values) and the 64 bf16 RoPE values.  The pages
// give the layout, not how the scales are chosen; here each group of 128
// values gets scale = amax / 448 (448 = the largest e4m3fn magnitude) and
// each code is x / scale rounded to the nearest e4m3fn value, ties to even,
// after clamping to +-448; a group of zeros gets scale 0 and codes 0.  Both
// divisions are correctly rounded fp32.  NoPE inputs are taken to be
// finite.
//
// One wave per token, four tokens per 256-thread workgroup.  FP8: lane l
// holds NoPE values 8 l .. 8 l + 7 (one 16-byte load), the group maximum
// is reduced over the 16 lanes of its group, the quotients are rounded to
// e4m3fn codes by v_cvt_pk_fp8_f32 (round to nearest even, two per
// instruction) and the lane writes its eight codes as one 8-byte store;
// lanes 0..7 copy the RoPE values.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__global__ __launch_bounds__(256) void append_kernel(const uint8_t* __restrict__ rows,
                                                     const int32_t* __restrict__ slots, int n, int fmt,
                                                     uint8_t* __restrict__ kcache, long long pool_rows) {
  const int lane = threadIdx.x & 63;
  const long long t = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= n) return;
  const int slot = slots[t];
  if (slot < 0 || slot >= pool_rows) return;   // nothing to write
  const uint8_t* src = rows + t * kBf16RowBytes;
  if (fmt == 0) {
    uint8_t* dst = kcache + (size_t)slot * kBf16RowBytes;
    *(u32x4*)(dst + 16 * lane) = *(const u32x4*)(src + 16 * lane);
    if (lane < 8) *(u32x4*)(dst + 1024 + 16 * lane) = *(const u32x4*)(src + 1024 + 16 * lane);
    return;
  }
  uint8_t* dst = kcache + (size_t)slot * kFp8RowBytes;
  const u32x4 w = *(const u32x4*)(src + 16 * lane);
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_lo(w[i]);
    x[2 * i + 1] = bf16_hi(w[i]);
  }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[i]));
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) m = fmaxf(m, __shfl_xor(m, d));
  const float scale = m / 448.f;
  // x / scale, correctly rounded, from the correctly rounded reciprocal y:
  // q0 = x * y is within one ulp of x / scale, the residual x - scale * q0
  // is exact in an FMA, and q0 + residual * y rounds to the correctly
  // rounded quotient (Markstein's theorem).  A subnormal scale, whose
  // reciprocal could overflow, divides directly.
  const bool normal_scale = scale >= 0x1p-126f;
  const float y = normal_scale ? 1.f / scale : 0.f;
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (normal_scale) {
      const float q0 = x[i] * y;
      // the correction of an exact zero adds +0: the quotient keeps x's sign
      q[i] = copysignf(fmaf(fmaf(-scale, q0, x[i]), y, q0), x[i]);
    } else {
      q[i] = scale > 0.f ? x[i] / scale : 0.f;
    }
    q[i] = fminf(fmaxf(q[i], -448.f), 448.f);
  }
  // v_cvt_pk_fp8_f32: two fp32 values to two e4m3fn codes, round to
  // nearest even (the inputs are already within +-448).
  u32x2 codes;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * h], q[4 * h + 1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * h + 2], q[4 * h + 3], w, true);
    codes[h] = scale > 0.f ? (uint32_t)w : 0u;
  }
  *(u32x2*)(dst + 8 * lane) = codes;
  if ((lane & 15) == 0) *(float*)(dst + 512 + 4 * (lane >> 4)) = scale;
  if (lane < 8) *(u32x4*)(dst + 528 + 16 * lane) = *(const u32x4*)(src + 1024 + 16 * lane);
}

}  // namespace

hipError_t launch_append(const void* rows, const int32_t* slots, int n, int kv_format, void* kcache,
                         long long pool_rows, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 3) / 4));
  hipLaunchKernelGGL(append_kernel, grid, dim3(256), 0, stream, (const uint8_t*)rows, slots, n, kv_format,
                     (uint8_t*)kcache, pool_rows);
  return hipGetLastError();
}

}  // namespace mla
