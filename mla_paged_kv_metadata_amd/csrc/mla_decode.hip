// Log-sum-exp combine of split-KV partial results and the launch routing of
// the decode kernels, for MLA decoding over a 64-token paged KV cache on
// gfx950.
//
// What is computed (topnet.top "Was ist FlashMLA?", "MLA-Decodierung
// ausfuehren"; sao.pub FlashMLA overview, 二、核心功能与架构): for every query
// row (576 dims = 512 NoPE + 64 RoPE), softmax attention over the keys of its
// sequence, each key being one shared latent row whose first 512 dims are
// also V; the result out (bf16) and its log-sum-exp (natural log, fp32).
// The split-KV schedule (mla_metadata.hip) cuts long units into pieces
// handled by different workgroups; each piece's kernel writes its
// normalised partial O and partial lse, and the combine kernel below merges
// the pieces of a unit.  The partial-attention kernels are chosen by the
// number of query rows per unit: 16-row tiles (mla_decode_narrow.hip) for
// up to 32 rows, 128-row tiles (mla_decode_wide.hip) above.
#include <mutex>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

// ---------------------------------------------------------------------------
// Device scratch of mla_decode_kvcache_noalloc, for callers that cannot
// allocate: the split partials of one decode call, kScratchBytes at most.
// Every device the library runs on holds its own copy until the process
// ends; each call on a device overwrites it (calls that overlap on one
// device race).  Host code never uses the array's name as an address: its
// device address is looked up once per device (scratch_for_current_device).
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)96 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kScratchDevices] = {};
}  // namespace

hipError_t scratch_for_current_device(void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  *bytes = kScratchBytes;
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Combine: merge the k_u partial results of every split unit.
//   lse = log sum_i exp(lse_i);  out = sum_i exp(lse_i - lse) * O_i
// One wave per query row; lanes own 8 output dims each, i.e. one 16-byte
// load of bf16 partial values per partial row.  The partial lses are loaded
// by the lanes in parallel (64 at a time), together with the first eight
// partial rows (which do not depend on the weights); the weights are formed
// in-lane and further partial rows are summed eight at a time.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void acc_bf16x8(f32x4& a0, f32x4& a1, float w, const u32x4& v) {
  a0[0] += w * __builtin_bit_cast(float, v[0] << 16);
  a0[1] += w * __builtin_bit_cast(float, v[0] & 0xFFFF0000u);
  a0[2] += w * __builtin_bit_cast(float, v[1] << 16);
  a0[3] += w * __builtin_bit_cast(float, v[1] & 0xFFFF0000u);
  a1[0] += w * __builtin_bit_cast(float, v[2] << 16);
  a1[1] += w * __builtin_bit_cast(float, v[2] & 0xFFFF0000u);
  a1[2] += w * __builtin_bit_cast(float, v[3] << 16);
  a1[3] += w * __builtin_bit_cast(float, v[3] & 0xFFFF0000u);
}

__global__ __launch_bounds__(256) void combine_kernel(const int32_t* __restrict__ md,
                                                      const int32_t* __restrict__ num_splits,
                                                      const uint16_t* __restrict__ ws_o,
                                                      const float* __restrict__ ws_lse,
                                                      uint16_t* __restrict__ out,
                                                      float* __restrict__ lse, int R, int num_parts,
                                                      int units) {
  // Workgroup = (unit, four rows), flattened so that any row count fits.
  const int quads = (R + 3) / 4;
  const int u = blockIdx.x / quads;
  // The header and the unit's split range are read together (one round
  // trip; the checks below do not short-circuit the loads).
  const int h0 = md[0], h3 = md[3], h5 = md[5];
  const int base = num_splits[u];
  const int k = num_splits[u + 1] - base;
  // A schedule that does not match the call: the split-KV kernel has
  // already given every row out = 0 and lse = NaN; nothing to merge.
  if ((h0 != num_parts) | (h5 != kMagic) | (h3 != units)) return;
  if (k <= 1) return;
  const int lane = threadIdx.x & 63;
  const int r = (blockIdx.x - u * quads) * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  const float* lrow = ws_lse + (size_t)base * R + r;
  // Lane i keeps lse_i of the first 64 splits.
  const float own = lane < k ? lrow[(size_t)lane * R] : -INFINITY;
  constexpr int kPre = 8;
  const uint16_t* src = ws_o + ((size_t)base * R + r) * kDv + 8 * lane;
  const size_t stride = (size_t)R * kDv;
  // The first kPre partial rows, loaded unconditionally (rows past the
  // unit's last split repeat that split and get weight 0), so that all of
  // them are in flight at once.
  u32x4 pre[kPre];
#pragma unroll
  for (int j = 0; j < kPre; ++j) pre[j] = *(const u32x4*)(src + (size_t)min(j, k - 1) * stride);
  float M = own;
  for (int i = 64 + lane; i < k; i += 64) M = fmaxf(M, lrow[(size_t)i * R]);
  M = wave_max(M);
  const size_t grow = (size_t)u * R + r;
  if (M == -INFINITY) {
    *(u32x4*)(out + grow * kDv + 8 * lane) = u32x4{0, 0, 0, 0};
    if (lane == 0) lse[grow] = -INFINITY;
    return;
  }
  float S = fast_exp2((own - M) * kLog2e);
  for (int i = 64 + lane; i < k; i += 64) S += fast_exp2((lrow[(size_t)i * R] - M) * kLog2e);
  S = wave_sum(S);
  const float lse_r = M + fast_log2(S) * kLn2;
  const float w_own = fast_exp2((own - lse_r) * kLog2e);
  auto weight = [&](int s) -> float {
    return s < 64 ? __shfl(w_own, s) : fast_exp2((lrow[(size_t)s * R] - lse_r) * kLog2e);
  };
  f32x4 a0 = f32x4{0.f, 0.f, 0.f, 0.f}, a1 = a0;
#pragma unroll
  for (int j = 0; j < kPre; ++j) acc_bf16x8(a0, a1, j < k ? __shfl(w_own, j) : 0.f, pre[j]);
  int i = kPre;
  for (; i + 8 <= k; i += 8) {
    u32x4 x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = *(const u32x4*)(src + (i + j) * stride);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc_bf16x8(a0, a1, weight(i + j), x[j]);
  }
  for (; i < k; ++i) acc_bf16x8(a0, a1, weight(i), *(const u32x4*)(src + i * stride));
  u32x4 wv;
  wv[0] = pack_bf16x2(a0[0], a0[1]);
  wv[1] = pack_bf16x2(a0[2], a0[3]);
  wv[2] = pack_bf16x2(a1[0], a1[1]);
  wv[3] = pack_bf16x2(a1[2], a1[3]);
  *(u32x4*)(out + grow * kDv + 8 * lane) = wv;
  if (lane == 0) lse[grow] = lse_r;
}

// Up to 32 rows per unit: 16-row tiles (one or two per unit), else 128.
int rows_per_workgroup(int rows_per_unit) { return rows_per_unit <= 32 ? 16 : 128; }

hipError_t launch_decode(const DecodeParams& p, int kv_format, int which, hipStream_t stream) {
  if (which & 1) {
    const dim3 grid(decode_grid(p.num_parts, p.row_tiles));
    const hipError_t e = rows_per_workgroup(p.R) == 128 ? launch_wide(p, kv_format, grid, stream)
                                                         : launch_narrow(p, kv_format, grid, stream);
    if (e != hipSuccess) return e;
  }
  // With a single part no unit is split: there is nothing to combine.
  if ((which & 2) && p.num_parts > 1) {
    const dim3 cgrid((unsigned)((size_t)p.units * ((p.R + 3) / 4)));
    hipLaunchKernelGGL(combine_kernel, cgrid, dim3(256), 0, stream, p.md, p.num_splits, p.ws_o, p.ws_lse,
                       p.out, p.lse, p.R, p.num_parts, p.units);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace mla
