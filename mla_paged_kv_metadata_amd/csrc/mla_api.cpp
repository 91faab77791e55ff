// C ABI of libmla.so: argument checks, schedule/workspace sizing and kernel
// launches.  Declarations and contracts are in include/mla.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "mla.h"
#include "mla_device.h"
#include "mla_internal.h"

#define MLA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return MLA_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_cu_mutex;
int g_cu_count[kMaxDevices] = {0};

// Compute units of the current device (cached per device).
int current_cu_count(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MLA_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return fail(MLA_ERR_HIP, "device id %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_cu_mutex);
  if (g_cu_count[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return fail(MLA_ERR_HIP, "cannot read the compute-unit count of device %d", dev);
    g_cu_count[dev] = n;
  }
  *cus = g_cu_count[dev];
  return MLA_OK;
}

int units_of(int batch, int s_q, int topk) { return topk > 0 ? batch * s_q : batch; }

int rows_per_unit(int s_q, int h_q, int topk) { return topk > 0 ? h_q : s_q * h_q; }

// One decode workgroup per compute unit: P * row_tiles ~= #CUs, P a
// multiple of 8 (whole XCD groups), at least 8.
int auto_parts(int rows, int cus) {
  const int rt = mla::rows_per_workgroup(rows);
  const int tiles = (rows + rt - 1) / rt;
  int p = cus / tiles;
  p = p / 8 * 8;
  return p < 8 ? 8 : p;
}

size_t md_elems(int units, int parts) {
  return (size_t)mla::kHeader + (size_t)mla::kPartRow * parts + (size_t)units;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace: partial O [slots, R, 512] fp32 then partial lse [slots, R].
// Every part boundary splits at most one unit, so slots <= units + parts.
void workspace_layout(int units, int parts, int R, size_t* o_bytes, size_t* total) {
  const size_t slots = (size_t)units + (size_t)parts;
  *o_bytes = align_up(slots * (size_t)R * mla::kDv * sizeof(float), 256);
  *total = *o_bytes + align_up(slots * (size_t)R * sizeof(float), 256);
}

// Shape and option checks (no pointers): enough for workspace sizing.
int check_decode_shape(const mla_decode_args* a) {
  if (!a) return fail(MLA_ERR_INVALID_ARGUMENT, "args is NULL");
  if (a->h_kv != 1) return fail(MLA_ERR_UNSUPPORTED, "h_kv must be 1 (got %d)", a->h_kv);
  if (a->d_qk != mla::kDqk || a->d_v != mla::kDv)
    return fail(MLA_ERR_UNSUPPORTED, "d_qk/d_v must be 576/512 (got %d/%d)", a->d_qk, a->d_v);
  if (a->page_size != mla::kPage)
    return fail(MLA_ERR_UNSUPPORTED, "page_size must be 64 (got %d)", a->page_size);
  if (a->kv_format != MLA_KV_BF16 && a->kv_format != MLA_KV_FP8_656)
    return fail(MLA_ERR_UNSUPPORTED, "unknown kv_format %d", a->kv_format);
  if (a->batch < 0 || a->s_q < 1 || a->h_q < 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "bad batch/s_q/h_q (%d/%d/%d)", a->batch, a->s_q, a->h_q);
  if (a->num_pages < 0 || a->max_blocks_per_seq < 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "bad num_pages/max_blocks_per_seq (%d/%d)", a->num_pages,
                a->max_blocks_per_seq);
  if (a->topk < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "topk must be >= 0");
  if (a->topk == 0 && a->indices != nullptr)
    return fail(MLA_ERR_INVALID_ARGUMENT, "indices must be NULL when topk is 0");
  if (a->num_parts < 1 || a->num_parts > mla::kMaxParts)
    return fail(MLA_ERR_INVALID_ARGUMENT, "num_parts must be in [1, %d]", mla::kMaxParts);
  if (!std::isfinite(a->softmax_scale))
    return fail(MLA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite");
  if ((long long)a->batch * a->s_q * a->h_q > (1LL << 31) / mla::kDqk)
    return fail(MLA_ERR_INVALID_ARGUMENT, "too many query rows");
  return MLA_OK;
}

int check_decode_args(const mla_decode_args* a) {
  int st = check_decode_shape(a);
  if (st != MLA_OK) return st;
  if (a->topk > 0 && !a->indices) return fail(MLA_ERR_INVALID_ARGUMENT, "indices is NULL");
  if (a->batch > 0) {
    if (!a->q || !a->kcache || !a->block_table || !a->cache_seqlens || !a->tile_metadata ||
        !a->num_splits || !a->out || !a->lse)
      return fail(MLA_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  }
  return MLA_OK;
}

}  // namespace

MLA_EXPORT int mla_version(void) { return 1; }

MLA_EXPORT const char* mla_last_error(void) { return g_last_error.c_str(); }

MLA_EXPORT int mla_metadata_size_for_parts(int batch, int s_q, int topk, int num_parts,
                                           size_t* tile_metadata_elems, size_t* num_splits_elems) {
  if (batch < 0 || s_q < 1 || topk < 0 || num_parts < 1 || num_parts > mla::kMaxParts)
    return fail(MLA_ERR_INVALID_ARGUMENT, "bad batch/s_q/topk/num_parts (%d/%d/%d/%d)", batch, s_q,
                topk, num_parts);
  if (!tile_metadata_elems || !num_splits_elems)
    return fail(MLA_ERR_INVALID_ARGUMENT, "output pointer is NULL");
  const int units = units_of(batch, s_q, topk);
  *tile_metadata_elems = md_elems(units, num_parts);
  *num_splits_elems = (size_t)units + 1;
  return ok();
}

MLA_EXPORT int mla_metadata_size(int batch, int s_q, int q_rows_per_kv_head, int h_kv, int topk,
                                 int* num_parts, size_t* tile_metadata_elems,
                                 size_t* num_splits_elems) {
  if (h_kv != 1) return fail(MLA_ERR_UNSUPPORTED, "h_kv must be 1 (got %d)", h_kv);
  if (s_q < 1 || q_rows_per_kv_head < 1 || q_rows_per_kv_head % s_q != 0)
    return fail(MLA_ERR_INVALID_ARGUMENT,
                "q_rows_per_kv_head (%d) must be a positive multiple of s_q (%d)",
                q_rows_per_kv_head, s_q);
  if (!num_parts) return fail(MLA_ERR_INVALID_ARGUMENT, "num_parts is NULL");
  int cus = 0;
  int st = current_cu_count(&cus);
  if (st != MLA_OK) return st;
  const int h_q = q_rows_per_kv_head / s_q;
  *num_parts = auto_parts(rows_per_unit(s_q, h_q, topk), cus);
  return mla_metadata_size_for_parts(batch, s_q, topk, *num_parts, tile_metadata_elems,
                                     num_splits_elems);
}

MLA_EXPORT int mla_get_metadata(const int32_t* cache_seqlens, const int32_t* indices, int batch,
                                int s_q, int q_rows_per_kv_head, int h_kv, int topk, int num_parts,
                                int32_t* tile_metadata, int32_t* num_splits, void* stream) {
  if (h_kv != 1) return fail(MLA_ERR_UNSUPPORTED, "h_kv must be 1 (got %d)", h_kv);
  if (batch < 0 || s_q < 1 || topk < 0 || num_parts < 1 || num_parts > mla::kMaxParts ||
      q_rows_per_kv_head < 1 || q_rows_per_kv_head % s_q != 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "bad batch/s_q/rows/topk/num_parts");
  if ((topk > 0) != (indices != nullptr))
    return fail(MLA_ERR_INVALID_ARGUMENT, "indices must be non-NULL exactly when topk > 0");
  if (!tile_metadata || !num_splits || (batch > 0 && !cache_seqlens))
    return fail(MLA_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  const int units = units_of(batch, s_q, topk);
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = mla::launch_metadata(cache_seqlens, indices, s_q, topk, units, num_parts,
                                            tile_metadata, num_splits, s);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "schedule launch: %s", hipGetErrorString(e));
  return ok();
}

MLA_EXPORT int mla_workspace_size(const mla_decode_args* args, size_t* bytes) {
  int st = check_decode_shape(args);
  if (st != MLA_OK) return st;
  if (!bytes) return fail(MLA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  size_t ob;
  workspace_layout(units_of(args->batch, args->s_q, args->topk), args->num_parts,
                   rows_per_unit(args->s_q, args->h_q, args->topk), &ob, bytes);
  return ok();
}

namespace {

int decode_impl(const mla_decode_args* a, void* stream, int which) {
  int st = check_decode_args(a);
  if (st != MLA_OK) return st;
  if (a->batch == 0) return ok();
  const int units = units_of(a->batch, a->s_q, a->topk);
  const int R = rows_per_unit(a->s_q, a->h_q, a->topk);
  size_t ob, need;
  workspace_layout(units, a->num_parts, R, &ob, &need);
  if (a->workspace_bytes < need || (!a->workspace && need > 0))
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes is smaller than the %zu needed",
                a->workspace_bytes, need);
  mla::DecodeParams p;
  p.q = (const uint8_t*)a->q;
  p.kcache = (const uint8_t*)a->kcache;
  p.block_table = a->block_table;
  p.seqlens = a->cache_seqlens;
  p.indices = a->topk > 0 ? a->indices : nullptr;
  p.md = a->tile_metadata;
  p.num_splits = a->num_splits;
  p.out = (uint16_t*)a->out;
  p.lse = a->lse;
  p.ws_o = (float*)a->workspace;
  p.ws_lse = (float*)((uint8_t*)a->workspace + ob);
  p.batch = a->batch;
  p.s_q = a->s_q;
  p.h_q = a->h_q;
  p.R = R;
  p.units = units;
  p.max_blocks = a->max_blocks_per_seq;
  p.topk = a->topk;
  p.num_parts = a->num_parts;
  const int rt = mla::rows_per_workgroup(R);
  p.row_tiles = (R + rt - 1) / rt;
  p.causal = a->causal ? 1 : 0;
  p.num_pages = a->num_pages;
  p.scale_log2 = a->softmax_scale * mla::kLog2e;
  hipError_t e = mla::launch_decode(p, a->kv_format, which, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

MLA_EXPORT int mla_decode_kvcache(const mla_decode_args* a, void* stream) {
  return decode_impl(a, stream, 3);
}

MLA_EXPORT int mla_decode_partial(const mla_decode_args* a, void* stream) {
  return decode_impl(a, stream, 1);
}

MLA_EXPORT int mla_decode_combine(const mla_decode_args* a, void* stream) {
  return decode_impl(a, stream, 2);
}
