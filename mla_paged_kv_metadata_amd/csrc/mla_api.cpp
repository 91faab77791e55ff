// C ABI of libmla.so: argument checks, schedule/workspace sizing and kernel
// launches.  Declarations and contracts are in include/mla.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "mla.h"
#include "mla_device.h"
#include "mla_internal.h"

#define MLA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

mla_status fail(mla_status status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

mla_status ok() {
  g_last_error.clear();
  return MLA_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_cu_mutex;
int g_cu_count[kMaxDevices] = {0};

// Compute units of the current device (cached per device).
mla_status current_cu_count(int* cus) {
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

// Sparse units are (sequence, query token) pairs; their count is an int.
bool units_fit(int batch, int s_q, int topk) { return topk == 0 || (long long)batch * s_q <= 0x7FFFFFFFLL; }

int rows_per_unit(int s_q, int h_q, int topk) { return topk > 0 ? h_q : s_q * h_q; }

// One decode workgroup per compute unit: P * row_tiles ~= #CUs, P a
// multiple of 8 (whole XCD groups) when that leaves at least 8 parts.
// With more row tiles than that (many query rows per sequence, e.g. a
// prefill) the tiles fill the device by themselves: fewer parts, down to
// 1 (no key splits at all) once there is a tile per compute unit.
int auto_parts(int rows, int cus) {
  const int rt = mla::rows_per_workgroup(rows);
  const int tiles = (rows + rt - 1) / rt;
  const int p = cus / tiles;
  if (p >= 8) return p / 8 * 8;
  return p < 1 ? 1 : p;
}

size_t md_elems(int units, int parts) {
  return (size_t)mla::kHeader + (size_t)mla::kPartRow * parts + (size_t)units;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace: partial O [slots, R, 512] bf16 then partial lse [slots, R]
// fp32.  Every part boundary splits at most one unit, so slots <= units +
// parts.
void workspace_layout(int units, int parts, int R, size_t* o_bytes, size_t* total) {
  const size_t slots = (size_t)units + (size_t)parts;
  *o_bytes = align_up(slots * (size_t)R * mla::kDv * sizeof(uint16_t), 256);
  *total = *o_bytes + align_up(slots * (size_t)R * sizeof(float), 256);
}

// Shape and option checks (no pointers): enough for workspace sizing.
mla_status check_decode_shape(const mla_decode_args* a) {
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
  if (a->qk_fp8 != 0 && a->qk_fp8 != 1) return fail(MLA_ERR_INVALID_ARGUMENT, "qk_fp8 must be 0 or 1");
  if (a->qk_fp8 && (a->kv_format != MLA_KV_FP8_656 || rows_per_unit(a->s_q, a->h_q, a->topk) <= 32))
    return fail(MLA_ERR_UNSUPPORTED,
                "qk_fp8 needs an FP8 pool and more than 32 query rows per unit (the 16-row kernel "
                "of the memory-bound shapes has no fp8 query path)");
  // Row counts are 32-bit in the kernels (every memory offset is 64-bit).
  if ((long long)std::max(a->batch, 1) * a->s_q * a->h_q > 0x7FFFFFFFLL)
    return fail(MLA_ERR_INVALID_ARGUMENT, "too many query rows (batch * s_q * h_q must be below 2^31)");
  {
    // One workgroup per (part, row tile); the grid is one-dimensional.
    const int R = rows_per_unit(a->s_q, a->h_q, a->topk);
    const int rt = mla::rows_per_workgroup(R);
    const long long tiles = (R + rt - 1) / rt;
    const long long parts = a->num_parts >= 8 ? (a->num_parts + 7) / 8 * 8 : a->num_parts;
    if (parts * tiles > 0x7FFFFFFFLL)
      return fail(MLA_ERR_INVALID_ARGUMENT, "num_parts * row tiles (%lld) exceeds the grid limit",
                  parts * tiles);
  }
  return MLA_OK;
}

mla_status check_decode_args(const mla_decode_args* a) {
  mla_status st = check_decode_shape(a);
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

MLA_EXPORT int mla_version(void) { return 2; }

MLA_EXPORT const char* mla_last_error(void) { return g_last_error.c_str(); }

MLA_EXPORT mla_status mla_metadata_size_for_parts(int batch, int s_q, int topk, int num_parts,
                                           size_t* tile_metadata_elems, size_t* num_splits_elems) {
  if (batch < 0 || s_q < 1 || topk < 0 || num_parts < 1 || num_parts > mla::kMaxParts)
    return fail(MLA_ERR_INVALID_ARGUMENT, "bad batch/s_q/topk/num_parts (%d/%d/%d/%d)", batch, s_q,
                topk, num_parts);
  if (!tile_metadata_elems || !num_splits_elems)
    return fail(MLA_ERR_INVALID_ARGUMENT, "output pointer is NULL");
  if (!units_fit(batch, s_q, topk)) return fail(MLA_ERR_INVALID_ARGUMENT, "batch * s_q must be below 2^31");
  const int units = units_of(batch, s_q, topk);
  *tile_metadata_elems = md_elems(units, num_parts);
  *num_splits_elems = (size_t)units + 1;
  return ok();
}

MLA_EXPORT mla_status mla_metadata_size(int batch, int s_q, int q_rows_per_kv_head, int h_kv, int topk,
                                 int* num_parts, size_t* tile_metadata_elems,
                                 size_t* num_splits_elems) {
  if (h_kv != 1) return fail(MLA_ERR_UNSUPPORTED, "h_kv must be 1 (got %d)", h_kv);
  if (s_q < 1 || q_rows_per_kv_head < 1 || q_rows_per_kv_head % s_q != 0)
    return fail(MLA_ERR_INVALID_ARGUMENT,
                "q_rows_per_kv_head (%d) must be a positive multiple of s_q (%d)",
                q_rows_per_kv_head, s_q);
  if (!num_parts) return fail(MLA_ERR_INVALID_ARGUMENT, "num_parts is NULL");
  int cus = 0;
  mla_status st = current_cu_count(&cus);
  if (st != MLA_OK) return st;
  const int h_q = q_rows_per_kv_head / s_q;
  *num_parts = auto_parts(rows_per_unit(s_q, h_q, topk), cus);
  return mla_metadata_size_for_parts(batch, s_q, topk, *num_parts, tile_metadata_elems,
                                     num_splits_elems);
}

MLA_EXPORT mla_status mla_get_metadata(const int32_t* cache_seqlens, const int32_t* indices, int batch,
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
  if (!units_fit(batch, s_q, topk)) return fail(MLA_ERR_INVALID_ARGUMENT, "batch * s_q must be below 2^31");
  const int units = units_of(batch, s_q, topk);
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = mla::launch_metadata(cache_seqlens, indices, s_q, topk, units, num_parts,
                                            tile_metadata, num_splits, s);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "schedule launch: %s", hipGetErrorString(e));
  return ok();
}

MLA_EXPORT mla_status mla_workspace_size(const mla_decode_args* args, size_t* bytes) {
  mla_status st = check_decode_shape(args);
  if (st != MLA_OK) return st;
  if (!bytes) return fail(MLA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  size_t ob;
  workspace_layout(units_of(args->batch, args->s_q, args->topk), args->num_parts,
                   rows_per_unit(args->s_q, args->h_q, args->topk), &ob, bytes);
  return ok();
}

namespace {

// Workspace present and large enough; *o_bytes = offset of the partial lse.
mla_status check_workspace(const mla_decode_args* a, size_t* o_bytes) {
  size_t need;
  workspace_layout(units_of(a->batch, a->s_q, a->topk), a->num_parts,
                   rows_per_unit(a->s_q, a->h_q, a->topk), o_bytes, &need);
  if (a->workspace_bytes < need || (!a->workspace && need > 0))
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes is smaller than the %zu needed",
                a->workspace_bytes, need);
  return MLA_OK;
}

mla_status decode_impl(const mla_decode_args* a, void* stream, int which) {
  mla_status st = check_decode_args(a);
  if (st != MLA_OK) return st;
  if (a->batch == 0) return ok();
  const int units = units_of(a->batch, a->s_q, a->topk);
  const int R = rows_per_unit(a->s_q, a->h_q, a->topk);
  size_t ob;
  st = check_workspace(a, &ob);
  if (st != MLA_OK) return st;
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
  p.ws_o = (uint16_t*)a->workspace;
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
  p.qk8 = a->qk_fp8;
  hipError_t e = mla::launch_decode(p, a->kv_format, which, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

MLA_EXPORT mla_status mla_decode_kvcache(const mla_decode_args* a, void* stream) {
  return decode_impl(a, stream, 3);
}

// mla_decode_kvcache with the library's own device scratch in place of the
// caller's workspace: no allocation anywhere on this path.
MLA_EXPORT mla_status mla_decode_kvcache_noalloc(const mla_decode_args* a, void* stream) {
  mla_status st = check_decode_args(a);
  if (st != MLA_OK) return st;
  if (a->batch == 0) return ok();
  size_t ob, need;
  workspace_layout(units_of(a->batch, a->s_q, a->topk), a->num_parts,
                   rows_per_unit(a->s_q, a->h_q, a->topk), &ob, &need);
  void* ws = nullptr;
  size_t cap = 0;
  const hipError_t e = mla::scratch_for_current_device(&ws, &cap);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "device scratch lookup: %s", hipGetErrorString(e));
  if (need > cap)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL,
                "this call needs %zu bytes of scratch; the library's device scratch holds %zu "
                "(use mla_decode_kvcache with a workspace)", need, cap);
  mla_decode_args b = *a;
  b.workspace = ws;
  b.workspace_bytes = cap;
  return decode_impl(&b, stream, 3);
}

MLA_EXPORT mla_status mla_decode_partial(const mla_decode_args* a, void* stream) {
  return decode_impl(a, stream, 1);
}

MLA_EXPORT mla_status mla_decode_combine(const mla_decode_args* a, void* stream) {
  return decode_impl(a, stream, 2);
}

namespace {

template <typename T>
mla_status copy_to_host(std::vector<T>* dst, const void* src, size_t n, hipStream_t s, const char* what) {
  dst->resize(n);
  if (n == 0) return MLA_OK;
  const hipError_t e = hipMemcpyAsync(dst->data(), src, n * sizeof(T), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "copying %s to the host: %s", what, hipGetErrorString(e));
  return MLA_OK;
}

// Keys of query token s of a sequence of length L that any row may see.
int window_of(const mla_decode_args* a, int L, int s) {
  if (!a->causal) return L;
  const int w = L - a->s_q + 1 + s;
  return w < 0 ? 0 : (w > L ? L : w);
}

}  // namespace

namespace {

// The audit's checks on host copies of the buffers a decode call reads: L
// [batch], bt [batch * max_blocks_per_seq], idx [units * topk] (NULL when
// dense), md [the schedule's elements for the call's part and unit counts;
// only the header is read if those do not match], ns [units + 1].
mla_status audit_host(const mla_decode_args* a, const int32_t* L, const int32_t* bt, const int32_t* idx,
                      const int32_t* md, const int32_t* ns) {
  if (a->num_pages < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "num_pages must be >= 1");
  const bool sparse = a->topk > 0;
  const int B = a->batch, U = units_of(a->batch, a->s_q, a->topk), P = a->num_parts;
  const size_t mb = (size_t)a->max_blocks_per_seq;
  if (md[5] != mla::kMagic)
    return fail(MLA_ERR_INVALID_ARGUMENT, "tile_metadata was not written by mla_get_metadata");
  if (md[0] != P || md[3] != U)
    return fail(MLA_ERR_INVALID_ARGUMENT,
                "tile_metadata is for %d parts and %d units, the call has %d and %d", md[0], md[3],
                P, U);
  // Sequence lengths, and the pool page of every block a visible key lies in.
  for (int b = 0; b < B; ++b) {
    if (L[b] < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "cache_seqlens[%d] = %d is negative", b, L[b]);
    const long long nb = ((long long)L[b] + mla::kPage - 1) / mla::kPage;
    if (nb > (long long)mb)
      return fail(MLA_ERR_INVALID_ARGUMENT,
                  "cache_seqlens[%d] = %d needs %lld blocks, more than max_blocks_per_seq %zu", b,
                  L[b], nb, mb);
    auto bad_page = [&](long long j) {
      const int32_t pg = bt[b * mb + j];
      return fail(MLA_ERR_INVALID_ARGUMENT,
                  "block_table[%d][%lld] = %d is outside the pool [0, %d)", b, j, pg, a->num_pages);
    };
    if (!sparse) {
      for (long long j = 0; j < nb; ++j) {
        const int32_t pg = bt[b * mb + j];
        if (pg < 0 || pg >= a->num_pages) return bad_page(j);
      }
      continue;
    }
    for (int q = 0; q < a->s_q; ++q) {
      const int W = window_of(a, L[b], q);
      const int32_t* row = &idx[((size_t)b * a->s_q + q) * a->topk];
      for (int i = 0; i < a->topk; ++i) {
        if (row[i] < 0 || row[i] >= W) continue;   // masked: no page is read for it
        const int32_t pg = bt[b * mb + (row[i] >> 6)];
        if (pg < 0 || pg >= a->num_pages) return bad_page(row[i] >> 6);
      }
    }
  }

  // The schedule must be the one mla_get_metadata builds for these lengths
  // (and indices): header, blocks per unit, and parts that cover every
  // (unit, block) once, in order, with split indices counted by num_splits.
  const int32_t* hdr = md;
  const int32_t* nblk = md + mla::kHeader + (size_t)mla::kPartRow * P;
  long long total = 0;
  for (int u = 0; u < U; ++u) {
    int want;
    if (!sparse) {
      want = (int)(((long long)L[u] + mla::kPage - 1) / mla::kPage);
    } else {
      // Blocks up to the last entry that indexes the sequence.
      const int Lb = L[u / a->s_q];
      const int32_t* row = &idx[(size_t)u * a->topk];
      int end = 0;
      for (int i = 0; i < a->topk; ++i)
        if (row[i] >= 0 && row[i] < Lb) end = i + 1;
      want = (end + mla::kPage - 1) / mla::kPage;
    }
    if (want < 1) want = 1;
    if (nblk[u] != want)
      return fail(MLA_ERR_INVALID_ARGUMENT,
                  "tile_metadata is stale: unit %d spans %d blocks there, %d for these inputs", u,
                  nblk[u], want);
    total += want;
  }
  if (hdr[4] != total)
    return fail(MLA_ERR_INVALID_ARGUMENT, "tile_metadata total blocks %d, expected %lld", hdr[4], total);
  if (ns[0] != 0) return fail(MLA_ERR_INVALID_ARGUMENT, "num_splits[0] = %d, expected 0", ns[0]);
  int cu = 0, cj = 0;   // next (unit, block) to be covered
  int last_u = -1, next_split = 0;
  for (int p = 0; p < P; ++p) {
    const int32_t* r = md + mla::kHeader + (size_t)mla::kPartRow * p;
    if (r[0] < 0) continue;
    const int u0 = r[0], j0 = r[1], u1 = r[2], j1 = r[3];
    if (u0 != cu || j0 != cj || u1 < u0 || u1 >= U || j1 < 1 || j1 > nblk[u1] ||
        (u1 == u0 && j1 <= j0))
      return fail(MLA_ERR_INVALID_ARGUMENT, "tile_metadata part %d {%d, %d, %d, %d} does not continue "
                  "the schedule at unit %d block %d", p, u0, j0, u1, j1, cu, cj);
    if (r[5] != L[sparse ? u0 / a->s_q : u0] || r[6] != nblk[u0])
      return fail(MLA_ERR_INVALID_ARGUMENT, "tile_metadata part %d has a stale length or block count", p);
    // Split index of u0 in this part: one past the previous part's if that
    // one also held u0, else 0.
    const int split = (u0 == last_u) ? next_split : 0;
    if (r[4] != split)
      return fail(MLA_ERR_INVALID_ARGUMENT, "tile_metadata part %d: split index %d, expected %d", p,
                  r[4], split);
    for (int u = u0; u <= u1; ++u) {
      const int k = (u == u0) ? split + 1 : 1;   // splits of u seen so far
      const bool ends = (u < u1) || (j1 == nblk[u1]);
      if (ends && ns[u + 1] - ns[u] != k)
        return fail(MLA_ERR_INVALID_ARGUMENT, "num_splits: unit %d has %d splits, the parts give %d", u,
                    ns[u + 1] - ns[u], k);
    }
    last_u = u1;
    next_split = (u1 == u0) ? split + 1 : 1;
    if (j1 == nblk[u1]) {
      cu = u1 + 1;
      cj = 0;
    } else {
      cu = u1;
      cj = j1;
    }
  }
  if (cu != U)
    return fail(MLA_ERR_INVALID_ARGUMENT, "tile_metadata parts stop at unit %d block %d of %d units", cu,
                cj, U);
  return ok();
}

}  // namespace

// Host-side audit of the device-resident values the kernels trust.  Every
// buffer is copied to the host once; audit_host checks them there.
MLA_EXPORT mla_status mla_validate_inputs(const mla_decode_args* a, void* stream) {
  mla_status st = check_decode_args(a);
  if (st != MLA_OK) return st;
  if (a->batch == 0) return ok();
  size_t ob;
  st = check_workspace(a, &ob);
  if (st != MLA_OK) return st;
  if (a->num_pages < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "num_pages must be >= 1");
  const bool sparse = a->topk > 0;
  const int B = a->batch, U = units_of(a->batch, a->s_q, a->topk), P = a->num_parts;
  const size_t mb = (size_t)a->max_blocks_per_seq;
  hipStream_t s = (hipStream_t)stream;
  auto sync = [&]() {
    const hipError_t e = hipStreamSynchronize(s);
    return e == hipSuccess ? MLA_OK : fail(MLA_ERR_HIP, "hipStreamSynchronize: %s", hipGetErrorString(e));
  };
  // The schedule's header first: a schedule built for another part or unit
  // count has another size, so nothing past the header is read before the
  // counts are known to match.
  std::vector<int32_t> L, bt, idx, md, ns;
  if ((st = copy_to_host(&md, a->tile_metadata, mla::kHeader, s, "tile_metadata")) != MLA_OK ||
      (st = sync()) != MLA_OK)
    return st;
  if (md[5] != mla::kMagic || md[0] != P || md[3] != U) return audit_host(a, nullptr, nullptr, nullptr, md.data(), nullptr);
  if ((st = copy_to_host(&L, a->cache_seqlens, B, s, "cache_seqlens")) != MLA_OK ||
      (st = copy_to_host(&bt, a->block_table, (size_t)B * mb, s, "block_table")) != MLA_OK ||
      (st = copy_to_host(&idx, a->indices, sparse ? (size_t)U * a->topk : 0, s, "indices")) != MLA_OK ||
      (st = copy_to_host(&md, a->tile_metadata, md_elems(U, P), s, "tile_metadata")) != MLA_OK ||
      (st = copy_to_host(&ns, a->num_splits, (size_t)U + 1, s, "num_splits")) != MLA_OK ||
      (st = sync()) != MLA_OK)
    return st;
  return audit_host(a, L.data(), bt.data(), sparse ? idx.data() : nullptr, md.data(), ns.data());
}

// The same audit on buffers the caller already holds in host memory.
MLA_EXPORT mla_status mla_validate_host_inputs(const mla_decode_args* a, const int32_t* cache_seqlens,
                                               const int32_t* block_table, const int32_t* indices,
                                               const int32_t* tile_metadata, const int32_t* num_splits) {
  mla_status st = check_decode_shape(a);
  if (st != MLA_OK) return st;
  if (a->batch == 0) return ok();
  if (!cache_seqlens || !block_table || !tile_metadata || !num_splits || (a->topk > 0 && !indices))
    return fail(MLA_ERR_INVALID_ARGUMENT, "a required host pointer is NULL");
  return audit_host(a, cache_seqlens, block_table, a->topk > 0 ? indices : nullptr, tile_metadata, num_splits);
}

MLA_EXPORT mla_status mla_append_kv(const void* rows, const int32_t* slots, int n, int kv_format, void* kcache,
                             int num_pages, void* stream) {
  if (n < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "n must be >= 0 (got %d)", n);
  if (kv_format != MLA_KV_BF16 && kv_format != MLA_KV_FP8_656)
    return fail(MLA_ERR_UNSUPPORTED, "unknown kv_format %d", kv_format);
  if (num_pages < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "num_pages must be >= 0 (got %d)", num_pages);
  if (n == 0) return ok();
  if (!rows || !slots || (!kcache && num_pages > 0))
    return fail(MLA_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if (((uintptr_t)rows & 15) != 0 || ((uintptr_t)kcache & 15) != 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "rows and kcache must be 16-byte aligned");
  const hipError_t e = mla::launch_append(rows, slots, n, kv_format, kcache,
                                          (long long)num_pages * mla::kPage, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "append launch: %s", hipGetErrorString(e));
  return ok();
}
