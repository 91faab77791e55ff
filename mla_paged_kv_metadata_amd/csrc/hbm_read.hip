// Read-bandwidth reference for the benchmark (libmla_bw.so, not part of the
// decode ABI): one pass over a device buffer with 16-byte loads, eight in
// flight per lane, every byte read once and folded into an XOR that is
// written per wave, so that the loads cannot be dropped.  The decode
// kernels' HBM rates are compared with what this plain streaming read
// reaches on the same part.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr size_t kChunkBytes = (size_t)16 * kThreads * kUnroll;   // 32 KiB per workgroup step

// Chunk c of the buffer (kChunkBytes each) is read by workgroup c % grid;
// lane t reads 16-byte words t, t + 256, ... of it.  n16 is a multiple of
// kThreads * kUnroll, so every index stays below n16.
__global__ __launch_bounds__(kThreads) void read_kernel(const uint4* __restrict__ src, size_t n16,
                                                         uint32_t* __restrict__ sink) {
  const size_t step = (size_t)gridDim.x * kThreads * kUnroll;
  uint32_t acc = 0;
  for (size_t base = (size_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < n16; base += step) {
    uint4 v[kUnroll];
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) v[i] = src[base + (size_t)i * kThreads];
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) sink[(size_t)blockIdx.x * (kThreads / 64) + threadIdx.x / 64] = acc;
}

}  // namespace

// Reads `bytes` bytes at `src` (device memory, 16-byte aligned, a multiple
// of 32 KiB) with `blocks` workgroups on `stream`; writes blocks * 4 words
// to `sink`.  Returns 0 when the launch was accepted, -1 on a bad argument,
// else the HIP error code.
extern "C" __attribute__((visibility("default"))) int mla_bw_read(const void* src, size_t bytes, uint32_t* sink,
                                                                   int blocks, void* stream) {
  if (!src || !sink || blocks < 1 || bytes == 0 || bytes % kChunkBytes != 0 || ((uintptr_t)src & 15) != 0)
    return -1;
  hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream, (const uint4*)src,
                     bytes / 16, sink);
  return (int)hipGetLastError();
}
