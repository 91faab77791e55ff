// Internal interface between the C ABI (mla_api.cpp) and the kernel
// launchers (mla_metadata.hip, mla_decode.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

struct DecodeParams {
  const uint8_t* q;            // bf16 [units*R, 576]
  const uint8_t* kcache;       // page pool
  const int32_t* block_table;  // [batch, max_blocks]
  const int32_t* seqlens;      // [batch]
  const int32_t* indices;      // [batch, s_q, topk] or null
  const int32_t* md;           // tile_metadata
  const int32_t* num_splits;   // [units + 1]
  uint16_t* out;               // bf16 [units*R, 512]
  float* lse;                  // [units*R]
  uint16_t* ws_o;              // [slots, R, 512] bf16 partial outputs
  float* ws_lse;               // [slots, R]
  int batch, s_q, h_q;
  int R;                       // query rows per unit
  int units;
  int max_blocks, topk, num_parts, row_tiles;
  int num_pages;               // pages in the pool (0: no key can be read)
  int causal;
  float scale_log2;            // softmax_scale * log2(e)
  int qk8;                     // FP8 pools: query quantised to e4m3 (one fp8 MFMA per 64 dims)
};

// Rows one decode workgroup covers for a given number of rows per unit.
int rows_per_workgroup(int rows_per_unit);

// The schedule (mla_metadata.hip); num_parts in [1, kMaxParts].
hipError_t launch_metadata(const int32_t* seqlens, const int32_t* indices, int s_q, int topk,
                           int units, int num_parts, int32_t* md, int32_t* num_splits,
                           hipStream_t stream);
// The 128-row-tile kernels (mla_decode_wide.hip).
hipError_t launch_wide(const DecodeParams& p, int kv_format, dim3 grid, hipStream_t stream);
// The 16-row-tile kernels (mla_decode_narrow.hip).
hipError_t launch_narrow(const DecodeParams& p, int kv_format, dim3 grid, hipStream_t stream);
// which: 1 = split-KV attention kernel, 2 = combine kernel, 3 = both.
hipError_t launch_decode(const DecodeParams& p, int kv_format, int which, hipStream_t stream);
// The device address and size of the library's scratch array on the
// current device (mla_decode.hip; looked up once per device).
hipError_t scratch_for_current_device(void** ptr, size_t* bytes);
// Writing tokens into the pool (mla_append.hip): row i to pool row
// slots[i] unless it lies outside [0, pool_rows).
hipError_t launch_append(const void* rows, const int32_t* slots, int n, int kv_format, void* kcache,
                         long long pool_rows, hipStream_t stream);

}  // namespace mla
