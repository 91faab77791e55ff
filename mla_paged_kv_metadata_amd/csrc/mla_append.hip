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
// is reduced over the 16 lanes of its group, and the lane writes its eight
// codes as one 8-byte store; lanes 0..7 copy the RoPE values.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

// fp32 in [-448, 448] -> e4m3fn code, round to nearest, ties to even.
// Normal codes (|v| >= 2^-6) keep the top three mantissa bits of the fp32
// value, rounded at bit 20 with the usual add-and-carry (a carry out of the
// mantissa raises the exponent, as it should); the exponent is rebiased
// from 127 to 7.  Below 2^-6 the codes are the multiples of 2^-9: v * 512
// is exact and rint rounds it to the nearest even integer (8 is the
// smallest normal, code 0x08).
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t bits = __float_as_uint(v);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t a = bits & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x3C800000u) {
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    code = (r >> 20) - (120u << 3);
  } else {
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.f);
  }
  return sign | code;
}

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
  uint32_t c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float q = scale > 0.f ? fminf(fmaxf(x[i] / scale, -448.f), 448.f) : 0.f;
    c[i] = scale > 0.f ? e4m3_rne(q) : 0u;
  }
  *(u32x2*)(dst + 8 * lane) = u32x2{c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                                    c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)};
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
