/*
 * MLA paged-KV decode: plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * loads this file; only the tests, the package's smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code with the HIP path.
 *
 * What it computes is the plain definition of softmax attention for one
 * shared latent KV head (multi-head latent attention decoding), with the
 * keys read through a paged cache:
 *
 *   for every sequence b, query token s, head h:
 *     W  = L_b                          (non-causal)
 *     W  = clamp(L_b - s_q + 1 + s, 0, L_b)   (causal, aligned to the end)
 *     candidates C = 0..L_b-1           (dense)
 *                  = indices[b, s, :]   (sparse; kept in order, repeats count)
 *     K = { t in C : 0 <= t < W }
 *     row(t) = 576 values of token t, found in page block_table[b][t / 64]
 *              at slot t % 64
 *     x_t = sigma * sum_d q[d] * row(t)[d]
 *     lse = log(sum_t exp(x_t))   (natural log, computed as m + log sum exp(x - m))
 *     out = sum_t exp(x_t - lse) * row(t)[0:512]
 *   K empty -> out = 0, lse = -inf.
 *
 * Passages followed:
 *   - geoz.com.cn "FlashMLA: DeepSeek's high-performance decoding kernel for
 *     Hopper GPUs", Introduction: an MLA decoding kernel over a paged KV
 *     cache for variable-length sequences.
 *   - topnet.top "Was ist FlashMLA?", Hauptmerkmale: page (block) size 64,
 *     BF16; "MLA-Decodierung ausfuehren": the call takes q, the KV cache,
 *     block_table, cache_seqlens, the output dimension dv and a causal flag,
 *     and returns the output together with its log-sum-exp.
 *   - sao.pub FlashMLA overview, 二、核心功能与架构: a sparse `indices`
 *     tensor makes the kernel attend only to the listed tokens; the FP8 cache
 *     row is 512 FP8 NoPE values, 4 FP32 scales (one per 128 values) and 64
 *     BF16 RoPE values kept unquantised.  Section 四、进阶玩法 names the FP8
 *     type as float8_e4m3fn.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   576 = 512 NoPE + 64 RoPE query/key dims, V = first 512 dims of the same
 *   row; causal masks are bottom-right aligned; sparse indices are logical
 *   token positions of sequence b, and any value < 0 or >= W is masked; the
 *   656-byte FP8 row stores its three parts in the order listed above, all
 *   little-endian; e4m3fn follows the OCP 8-bit floating point spec (bias 7,
 *   no infinities, S.1111.111 is NaN, max 448); RoPE is already applied to q
 *   and k; the scale sigma is given as an fp32 value and widened exactly.
 *
 * Precision: every product and sum is fp64; bf16 and e4m3 inputs are widened
 * exactly; the fp32 scale factors of the FP8 rows are widened exactly and
 * multiplied in fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_PAGE 64
#define ORC_DQK 576
#define ORC_DV 512
#define ORC_DNOPE 512
#define ORC_DROPE 64
#define ORC_FP8_ROW 656
#define ORC_BF16_ROW 1152

/* bf16 is the upper half of an IEEE binary32: widen by a 16-bit shift. */
double oracle_bf16_to_double(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP 8-bit floating point, E4M3 ("fn": finite, no infinities).
 * sign = bit 7, exponent = bits 6..3 with bias 7, mantissa = bits 2..0.
 * exponent 0: subnormal, value = (-1)^s * (m / 8) * 2^(1-7)
 * exponent 15 and mantissa 7: NaN
 * otherwise: (-1)^s * (1 + m / 8) * 2^(e - 7)                               */
double oracle_e4m3_to_double(uint8_t code)
{
    int s = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double v;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, 1 - 7);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

static float read_f32_le(const uint8_t *p)
{
    uint32_t u = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint16_t read_u16_le(const uint8_t *p)
{
    return (uint16_t)(p[0] | (p[1] << 8));
}

/* Decode one stored token row into 576 fp64 values.
 * fmt 0: 576 little-endian bf16.
 * fmt 1: bytes [0,512) e4m3 codes, [512,528) four fp32 scales,
 *        [528,656) 64 bf16; NoPE[i] = e4m3(code_i) * scale[i / 128].       */
void oracle_decode_row(const uint8_t *row, int fmt, double *dst)
{
    if (fmt == 0) {
        for (int d = 0; d < ORC_DQK; ++d)
            dst[d] = oracle_bf16_to_double(read_u16_le(row + 2 * d));
        return;
    }
    double scale[4];
    for (int g = 0; g < 4; ++g)
        scale[g] = (double)read_f32_le(row + ORC_DNOPE + 4 * g);
    for (int i = 0; i < ORC_DNOPE; ++i)
        dst[i] = oracle_e4m3_to_double(row[i]) * scale[i / 128];
    for (int j = 0; j < ORC_DROPE; ++j)
        dst[ORC_DNOPE + j] = oracle_bf16_to_double(read_u16_le(row + ORC_DNOPE + 16 + 2 * j));
}

/*
 * Compute out/lse for a set of query rows.
 *
 *   q            [batch, s_q, h_q, 576] bf16 bits
 *   kcache       [num_pages, 64, 1, row_bytes] bytes (row_bytes 1152 or 656)
 *   block_table  [batch, max_blocks] int32
 *   seqlens      [batch] int32
 *   indices      NULL (dense) or [batch, s_q, topk] int32
 *   sel          NULL = every row in order; else n_sel flat row ids
 *                ((b * s_q + s) * h_q + h)
 *   out          [n_rows, 512] fp64, lse [n_rows] fp64
 *   q_f64        NULL, or the query as fp64 values [batch, s_q, h_q, 576]
 *                used in place of q (e.g. a quantised query that is not a
 *                bf16 value)
 *
 * Returns 0, or -1 if a needed block_table entry is outside [0, num_pages),
 * -2 on a bad argument, -3 if memory runs out.
 */
int oracle_mla_decode(const uint16_t *q, const uint8_t *kcache, int fmt, int num_pages,
                      const int32_t *block_table, int max_blocks, const int32_t *seqlens,
                      const int32_t *indices, int topk, int batch, int s_q, int h_q,
                      float softmax_scale, int causal, int n_sel, const int32_t *sel,
                      double *out, double *lse, int num_threads, const double *q_f64)
{
    if ((!q && !q_f64) || !kcache || !block_table || !seqlens || !out || !lse)
        return -2;
    if (fmt != 0 && fmt != 1)
        return -2;
    if (batch < 0 || s_q <= 0 || h_q <= 0 || max_blocks <= 0)
        return -2;
    if (indices && topk <= 0)
        return -2;
    const size_t row_bytes = fmt == 0 ? ORC_BF16_ROW : ORC_FP8_ROW;
    const long n_rows = sel ? (long)n_sel : (long)batch * s_q * h_q;
    const double sigma = (double)softmax_scale;
    int max_keys = 0;
    for (int b = 0; b < batch; ++b) {
        int L = seqlens[b];
        if (L < 0 || (L + ORC_PAGE - 1) / ORC_PAGE > max_blocks)
            return -2;
        if (L > max_keys)
            max_keys = L;
    }
    if (indices && topk > max_keys)
        max_keys = topk;
    int status = 0;

#ifdef _OPENMP
    if (num_threads > 0)
        omp_set_num_threads(num_threads);
#pragma omp parallel
#endif
    {
        double *x = (double *)malloc(sizeof(double) * (size_t)(max_keys > 0 ? max_keys : 1));
        int32_t *tok = (int32_t *)malloc(sizeof(int32_t) * (size_t)(max_keys > 0 ? max_keys : 1));
        double *krow = (double *)malloc(sizeof(double) * ORC_DQK);
        double *qrow = (double *)malloc(sizeof(double) * ORC_DQK);
        double *acc = (double *)malloc(sizeof(double) * ORC_DV);
        if (!x || !tok || !krow || !qrow || !acc) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            status = -3;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
            for (long i = 0; i < n_rows; ++i) {
                long flat = sel ? (long)sel[i] : i;
                int h = (int)(flat % h_q);
                int s = (int)((flat / h_q) % s_q);
                int b = (int)(flat / ((long)h_q * s_q));
                int L = seqlens[b];
                int W = L;
                if (causal) {
                    W = L - s_q + 1 + s;
                    if (W < 0) W = 0;
                    if (W > L) W = L;
                }
                /* key set, in candidate order */
                int n = 0;
                if (!indices) {
                    for (int t = 0; t < W; ++t)
                        tok[n++] = t;
                } else {
                    const int32_t *idx = indices + ((long)b * s_q + s) * topk;
                    for (int j = 0; j < topk; ++j)
                        if (idx[j] >= 0 && idx[j] < W)
                            tok[n++] = idx[j];
                }
                double *o = out + i * ORC_DV;
                if (n == 0) {
                    for (int d = 0; d < ORC_DV; ++d)
                        o[d] = 0.0;
                    lse[i] = -INFINITY;
                    continue;
                }
                if (q_f64) {
                    for (int d = 0; d < ORC_DQK; ++d)
                        qrow[d] = q_f64[flat * ORC_DQK + d];
                } else {
                    const uint16_t *qp = q + flat * ORC_DQK;
                    for (int d = 0; d < ORC_DQK; ++d)
                        qrow[d] = oracle_bf16_to_double(qp[d]);
                }
                /* pass 1: every score */
                int bad = 0;
                for (int k = 0; k < n; ++k) {
                    int t = tok[k];
                    int page = block_table[(long)b * max_blocks + t / ORC_PAGE];
                    if (page < 0 || page >= num_pages) { bad = 1; break; }
                    const uint8_t *row = kcache + ((size_t)page * ORC_PAGE + (size_t)(t % ORC_PAGE)) * row_bytes;
                    oracle_decode_row(row, fmt, krow);
                    double dot = 0.0;
                    for (int d = 0; d < ORC_DQK; ++d)
                        dot += qrow[d] * krow[d];
                    x[k] = sigma * dot;
                }
                if (bad) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
                    status = -1;
                    continue;
                }
                double m = x[0];
                for (int k = 1; k < n; ++k)
                    if (x[k] > m) m = x[k];
                double z = 0.0;
                for (int k = 0; k < n; ++k)
                    z += exp(x[k] - m);
                double l = m + log(z);
                lse[i] = l;
                /* pass 2: weighted sum of the V rows */
                for (int d = 0; d < ORC_DV; ++d)
                    acc[d] = 0.0;
                for (int k = 0; k < n; ++k) {
                    int t = tok[k];
                    int page = block_table[(long)b * max_blocks + t / ORC_PAGE];
                    const uint8_t *row = kcache + ((size_t)page * ORC_PAGE + (size_t)(t % ORC_PAGE)) * row_bytes;
                    oracle_decode_row(row, fmt, krow);
                    double w = exp(x[k] - l);
                    for (int d = 0; d < ORC_DV; ++d)
                        acc[d] += w * krow[d];
                }
                for (int d = 0; d < ORC_DV; ++d)
                    o[d] = acc[d];
            }
        }
        free(x);
        free(tok);
        free(krow);
        free(qrow);
        free(acc);
    }
    return status;
}

/* Number of threads the OpenMP runtime would use (1 without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
