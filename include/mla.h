/*
 * mla.h - C ABI of the MI355X (gfx950) MLA paged-KV decode library, libmla.so.
 *
 * Multi-head latent attention (MLA) decoding: every query row of 576 dims
 * (512 latent "NoPE" dims followed by 64 RoPE dims) attends over one shared
 * latent KV row per token; the first 512 dims of that row also serve as V.
 * Tokens live in 64-token pages of a shared pool, found through a per-
 * sequence block table.  Sources: geoz.com.cn "FlashMLA: DeepSeek's
 * high-performance decoding kernel for Hopper GPUs" (Introduction: MLA
 * decoding over a paged KV cache for variable-length sequences);
 * topnet.top "Was ist FlashMLA?" (Hauptmerkmale: BF16, page size 64;
 * "MLA-Metadaten abrufen" and "MLA-Decodierung ausfuehren": the two-call
 * interface, metadata computed once and reused by every layer, output plus
 * log-sum-exp, causal flag); sao.pub FlashMLA overview (二、核心功能与架构:
 * sparse `indices` and the FP8 cache row of 512 FP8 NoPE values, 4 FP32
 * scales and 64 BF16 RoPE values).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers of the current HIP device,
 *     owned by the caller.  The library allocates no device memory and keeps
 *     no per-call state; it caches only the device's compute-unit count.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously on it; nothing synchronises.
 *   - Every function returns an mla_status.  Host-checkable problems are
 *     reported before anything is launched; nothing aborts or throws.  The
 *     message for the last non-OK status of the calling thread is returned
 *     by mla_last_error().
 *   - Values inside device buffers are not validated on the hot path:
 *     sparse indices outside [0, window) are masked (treated as absent);
 *     block_table entries for needed blocks must lie in [0, num_pages).
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MLA_OK = 0,
    MLA_ERR_INVALID_ARGUMENT = -1,   /* null pointer, bad size or mismatch */
    MLA_ERR_UNSUPPORTED = -2,        /* h_kv != 1, dims != 576/512, page != 64 */
    MLA_ERR_WORKSPACE_TOO_SMALL = -3,
    MLA_ERR_HIP = -4                 /* a HIP runtime call or launch failed */
} mla_status;

typedef enum {
    /* [num_pages, 64, 1, 576] bf16, one 1152-byte row per token */
    MLA_KV_BF16 = 0,
    /* [num_pages, 64, 1, 656] bytes per token: 512 e4m3fn NoPE codes, then
     * 4 little-endian fp32 scales (scale g applies to NoPE dims
     * [128g, 128g+128)), then 64 little-endian bf16 RoPE values */
    MLA_KV_FP8_656 = 1
} mla_kv_format;

/* Arguments of one decode call (one layer). */
typedef struct {
    int batch;               /* number of sequences b */
    int s_q;                 /* query tokens per sequence (>= 1) */
    int h_q;                 /* query heads */
    int h_kv;                /* KV heads; must be 1 */
    int d_qk;                /* must be 576 */
    int d_v;                 /* must be 512 (the "dv" argument of the pages) */
    int page_size;           /* must be 64 */
    int num_pages;           /* pages in the pool */
    int max_blocks_per_seq;  /* row stride of block_table, in elements */
    int topk;                /* 0: dense; > 0: indices is [batch, s_q, topk] */
    int kv_format;           /* an mla_kv_format */
    float softmax_scale;     /* multiplies q.k; the usual value is 576^-0.5 */
    int causal;              /* 1: query s of s_q sees the first
                                L - s_q + 1 + s keys (clamped to [0, L]) */
    int num_parts;           /* the value mla_metadata_size returned (or the
                                one passed to mla_get_metadata) */
    const void *q;           /* [batch, s_q, h_q, 576] bf16, contiguous */
    const void *kcache;      /* page pool, layout per kv_format */
    const int32_t *block_table;    /* [batch, max_blocks_per_seq]; entry j is
                                      the pool page of tokens [64j, 64j+64) */
    const int32_t *cache_seqlens;  /* [batch], L_b >= 0 */
    const int32_t *indices;        /* NULL, or [batch, s_q, topk] logical
                                      token positions; -1 / out of range =
                                      masked */
    const int32_t *tile_metadata;  /* from mla_get_metadata */
    const int32_t *num_splits;     /* from mla_get_metadata */
    void *workspace;               /* scratch for split partials */
    size_t workspace_bytes;
    void *out;               /* [batch, s_q, h_q, 512] bf16 (written) */
    float *lse;              /* [batch, s_q, h_q] fp32 natural-log
                                log-sum-exp of the scaled scores (written);
                                -inf and out = 0 where no key is visible */
    int qk_fp8;              /* FP8 pools only.  0 (default): QK^T uses the
                                query exactly (its e4m3 hi and remainder
                                parts on the fp8 MFMA; products of codes
                                and query values are exact).  1: the query
                                is quantised to e4m3 per row and per half
                                of its 512 NoPE dims, at a power-of-two
                                scale 2^p with 2^(p+7) <= max |q| <
                                2^(p+8), nearest value, ties to even (RoPE
                                dims stay bf16), and QK^T runs on the fp8
                                MFMA with half the operations (sao.pub
                                FlashMLA overview, 一、项目速览: the FP8 cache
                                and its sparse-decode throughput).  Needs an
                                FP8 pool and more than 32 query rows per
                                unit (s_q * h_q dense, h_q sparse), else
                                MLA_ERR_UNSUPPORTED. */
} mla_decode_args;

/*
 * Sizes of the schedule arrays (topnet.top "Was ist FlashMLA?",
 * "MLA-Metadaten abrufen": get_mla_metadata(cache_seqlens,
 * s_q * h_q // h_kv, h_kv) returns tile_scheduler_metadata and num_splits).
 * The pages pass no s_q and return no part count; here the caller passes
 * s_q (sparse schedules have one unit per query token) and gets back the
 * part count, which every later call of the step takes.
 *
 *   q_rows_per_kv_head = s_q * h_q / h_kv; topk = 0 for dense.
 *   *num_parts (out): the part count the library picks for this device and
 *     row count: about (compute units) / (row tiles of one unit) parts,
 *     rounded down to a multiple of 8 when that leaves at least 8 (whole
 *     XCD groups), otherwise 1..7 (the row tiles alone nearly fill the
 *     device, e.g. a prefill).
 *   *tile_metadata_elems, *num_splits_elems (out): int32 element counts to
 *     allocate, for the picked part count.  Use
 *     mla_metadata_size_for_parts to size for a forced count.
 * Errors: MLA_ERR_UNSUPPORTED for h_kv != 1; MLA_ERR_INVALID_ARGUMENT for a
 * bad count or a NULL output; MLA_ERR_HIP if the device cannot be queried.
 */
mla_status mla_metadata_size(int batch, int s_q, int q_rows_per_kv_head, int h_kv, int topk,
                             int *num_parts, size_t *tile_metadata_elems, size_t *num_splits_elems);

/* Same sizes for an explicit part count (1 <= num_parts <= 2048); same
 * passage.  Host only, launches nothing. */
mla_status mla_metadata_size_for_parts(int batch, int s_q, int topk, int num_parts,
                                       size_t *tile_metadata_elems, size_t *num_splits_elems);

/*
 * Build the split-KV schedule on the device (same passage as above).
 *
 *   cache_seqlens [batch] int32 (device); indices NULL (dense) or
 *   [batch, s_q, topk] int32 (device).
 *   num_parts: normally the value mla_metadata_size returned; any value
 *   in [1, 2048] gives a valid (if slower) schedule and must then be passed to the
 *   decode unchanged.
 *   tile_metadata, num_splits: device int32 arrays of the sizes above
 *   (written).  Layout of tile_metadata:
 *     [0..7]   header {num_parts, T, c0, units, total_blocks, 0x4D4C4131, 0, 0}
 *     [8 + 8p .. 8 + 8p + 7] part p: {u_first, j_first, u_last, j_end,
 *              split index of u_first, cache_seqlens of u_first's sequence,
 *              blocks of u_first, 0}; an empty part has u_first -1
 *     [8 + 8P + u] blocks of 64 keys that unit u spans
 *   where a unit is a sequence (dense) or a (sequence, query token) pair
 *   (sparse).  num_splits[u+1] - num_splits[u] is the number of parts unit u
 *   is spread over (num_splits[0] = 0).
 * The result depends only on cache_seqlens (and indices); compute it once
 * per decode step and reuse it for every layer.
 */
mla_status mla_get_metadata(const int32_t *cache_seqlens, const int32_t *indices, int batch, int s_q,
                            int q_rows_per_kv_head, int h_kv, int topk, int num_parts,
                            int32_t *tile_metadata, int32_t *num_splits, void *stream);

/* Bytes of device workspace mla_decode_kvcache needs for these arguments:
 * the partial results of sequences whose keys the schedule splits over
 * several parts (topnet.top "Was ist FlashMLA?", "MLA-Metadaten abrufen":
 * num_splits counts those pieces per sequence), as bf16 partial outputs,
 * each normalised by its own row sum, and fp32 partial log-sum-exps.  The
 * contents need no initialisation.  Host only; errors as for the decode's
 * shape checks (the pointers in args are not read).
 * Layout, with R query rows per unit (s_q * h_q dense, h_q sparse) and
 * slots = units + num_parts: partial outputs [slots, R, 512] bf16 at byte 0,
 * then partial log-sum-exps [slots, R] fp32 at byte
 * align256(slots * R * 1024); piece i of unit u (0 <= i < num_splits[u+1] -
 * num_splits[u]) is slot num_splits[u] + i. */
mla_status mla_workspace_size(const mla_decode_args *args, size_t *bytes);

/*
 * Decode one layer: out and lse for every (sequence, query token, head)
 * (topnet.top "Was ist FlashMLA?", "MLA-Decodierung ausfuehren":
 * flash_mla_with_kvcache(q, kvcache, block_table, cache_seqlens, dv,
 * tile_scheduler_metadata, num_splits, causal) -> (o, lse); sao.pub,
 * 二、核心功能与架构: with `indices`, only the listed tokens are attended).
 *
 * Enqueues the split-KV attention kernel and the log-sum-exp combine kernel
 * on `stream`.  The metadata must come from mla_get_metadata with the same
 * batch, s_q, h_q * s_q, topk, cache_seqlens, indices and num_parts.  The
 * kernels check the schedule's header on the device: if it was built for
 * another part or unit count (or is not a schedule), no key is read and
 * every row gets out = 0 and lse = NaN (the call itself cannot see this
 * and returns MLA_OK; mla_validate_inputs names the problem).  The header
 * is read together with the part row of each workgroup, so tile_metadata
 * must span the tile_metadata_elems that mla_metadata_size gives for this
 * call's num_parts even when it holds a schedule for fewer parts.
 * Limits (MLA_ERR_INVALID_ARGUMENT beyond them): batch * s_q * h_q below
 * 2^31 query rows, and num_parts (rounded up to a multiple of 8 when >= 8)
 * times the row tiles of one unit below 2^31 workgroups.
 */
mla_status mla_decode_kvcache(const mla_decode_args *args, void *stream);

/*
 * mla_decode_kvcache for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): args->workspace and args->workspace_bytes are ignored and the
 * split partials go to the library's own device scratch, a static array of
 * 96 MiB (100,663,296 bytes) that each device the library runs on holds
 * until the process ends.  Calls whose workspace (mla_workspace_size) would
 * exceed it return MLA_ERR_WORKSPACE_TOO_SMALL before launching anything.
 * Allocates nothing.  All calls on one device share that device's scratch:
 * calls that overlap in time on one device (other streams or threads) race
 * and must not be issued.  Same arguments, results and other errors as
 * mla_decode_kvcache.
 */
mla_status mla_decode_kvcache_noalloc(const mla_decode_args *args, void *stream);

/*
 * The two halves of mla_decode_kvcache (same passages: the per-layer decode
 * of topnet.top "Was ist FlashMLA?", "MLA-Decodierung ausfuehren", and the
 * merge of the num_splits pieces of "MLA-Metadaten abrufen"), for callers
 * that schedule them separately (e.g. to time each kernel, or to overlap the combine with
 * other work).  mla_decode_partial enqueues only the split-KV attention
 * kernel: sequences covered by one part get their final out/lse, split
 * sequences leave partial results in the workspace.  mla_decode_combine
 * enqueues only the merge of those partials (log-sum-exp weighting:
 * lse = log sum_i exp(lse_i), out = sum_i exp(lse_i - lse) * out_i) into
 * out/lse (with num_parts = 1 no sequence is split and nothing is
 * enqueued); it must follow mla_decode_partial on the same arguments and
 * workspace.  Same arguments and errors as mla_decode_kvcache.
 */
mla_status mla_decode_partial(const mla_decode_args *args, void *stream);
mla_status mla_decode_combine(const mla_decode_args *args, void *stream);

/*
 * Debug audit of the values a decode call reads from device memory, which
 * the kernels take on trust for speed (sao.pub FlashMLA overview, 三、动手实践,
 * pitfall 3: the sparse kernel does no input checking, so a malformed
 * `indices` gives silently wrong results).  SYNCHRONOUS and slow: it copies
 * cache_seqlens, block_table, indices, tile_metadata and num_splits to host
 * memory on `stream`, waits for the stream, and checks there that
 *   - every check of mla_decode_kvcache passes (shapes, pointers, workspace);
 *   - num_pages >= 1 and every L_b >= 0 with ceil(L_b / 64) blocks fitting
 *     in max_blocks_per_seq;
 *   - block_table holds a page in [0, num_pages) for every block a visible
 *     key lies in (dense: all blocks of the sequence; sparse: the blocks of
 *     the unmasked indices);
 *   - tile_metadata and num_splits are the schedule mla_get_metadata builds
 *     for these cache_seqlens / indices and num_parts (not stale): header,
 *     blocks per unit, parts covering every (unit, block) once in order,
 *     split indices and split counts.
 * Launches nothing and writes no device memory.  Returns MLA_OK, or
 * MLA_ERR_INVALID_ARGUMENT with mla_last_error() naming the first problem
 * (MLA_ERR_HIP if a copy or the wait fails).  Not capturable in a graph.
 */
mla_status mla_validate_inputs(const mla_decode_args *args, void *stream);

/*
 * The same audit (same passage) on copies the caller already holds in HOST
 * memory: cache_seqlens [batch], block_table [batch * max_blocks_per_seq],
 * indices [batch * s_q * topk] (ignored when topk = 0), tile_metadata (the
 * element count mla_metadata_size_for_parts gives for args->num_parts; only
 * its 8-int header is read when the header names other part or unit
 * counts) and num_splits [units + 1].  The device pointers in args are not
 * read; the shape checks of the decode apply.  Synchronous, touches no
 * device.  Returns MLA_OK or MLA_ERR_INVALID_ARGUMENT naming the first
 * problem.
 */
mla_status mla_validate_host_inputs(const mla_decode_args *args, const int32_t *cache_seqlens,
                                    const int32_t *block_table, const int32_t *indices,
                                    const int32_t *tile_metadata, const int32_t *num_splits);

/*
 * Write new tokens' latent rows into the page pool: the cache update that
 * precedes a decode step.  Row formats are the decode's (sao.pub FlashMLA
 * overview, 二、核心功能与架构: 512 FP8 NoPE values, 4 FP32 scales, one per
 * 128 values, and 64 BF16 RoPE values; 四、进阶玩法: float8_e4m3fn).
 *
 *   rows:   [n, 576] bf16 (device, 16-byte aligned, contiguous): the tokens'
 *           latent rows, RoPE already applied to dims 512..575.
 *   slots:  [n] int32 (device): token i goes to pool row slots[i] =
 *           page * 64 + position in page; a slot outside [0, num_pages * 64)
 *           (e.g. -1) writes nothing.  Slots must be distinct: two tokens
 *           with the same slot leave that row unspecified (their stores may
 *           interleave, e.g. one token's codes with the other's scales).
 *   kv_format: MLA_KV_BF16 copies the 1152-byte row.  MLA_KV_FP8_656
 *           quantises: per group of 128 NoPE values scale = amax / 448 (fp32;
 *           448 is the largest e4m3fn magnitude), code = x / scale rounded
 *           to the nearest e4m3fn value, ties to even, after clamping to
 *           +-448; an all-zero group gets scale 0 and codes 0; the RoPE
 *           values are copied bit for bit.  NoPE inputs must be finite.
 *   kcache: the pool (device, 16-byte aligned), num_pages pages in kv_format.
 * Enqueued on `stream`; n = 0 is a no-op.  The pool rows of other slots are
 * not touched.
 */
mla_status mla_append_kv(const void *rows, const int32_t *slots, int n, int kv_format, void *kcache,
                         int num_pages, void *stream);

/* Message for the calling thread's last non-OK status ("" if none). */
const char *mla_last_error(void);

/* Library ABI version (increments on incompatible changes). */
int mla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
