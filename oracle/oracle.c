/*
 * fp64 CPU oracle for the attention hot path.  TEST INFRASTRUCTURE ONLY: nothing in the product path
 * (the HIP library and its Python binding) may include, link, load or call this file; only the tests,
 * the smoke check and the CPU-baseline leg of the benchmark use it.  It shares no code, header, table or
 * constant with the HIP kernels.
 *
 * What it computes (the pages' subject is FlashAttention-style attention; the plain definition that the
 * tiled kernels reach up to rounding is mask-based softmax attention, "SkyRL: Add cuDNN flash attention",
 * Summary and Changes, which keeps mask-based attention as the reference path):
 *
 *   s_j  = scale * sum_d q_d k_jd                       over the keys j the row may see
 *   p_j  = exp(s_j - m) / sum_j' exp(s_j' - m),  m = max_j s_j
 *   o    = sum_j p_j v_j,   lse = m + log(sum_j exp(s_j - m))
 *   a row that sees no key gives o = 0 and lse = -inf
 *
 * Three modes per row:
 *   MODE_DENSE  the definition above, no tiles.
 *   MODE_SKIP   skip-softmax ("TensorRT-LLM: Skip Softmax Attention", Description; "Model-Optimizer:
 *               Add split-k decode kernel for skip softmax", What does this PR do): key tiles of `tile`
 *               keys aligned to key 0 are visited in ascending order with online softmax; a tile whose
 *               max logit tmax satisfies exp(tmax - m) < thr, m the running max before the tile, is
 *               skipped whole (no exp, no P.V, no rescale).  The first visited tile is never skipped
 *               (m = -inf), and thr = 0 never skips.  A replay map may impose the decisions instead.
 *               Map codes: 0 processed, 1 skipped, 2 not visited (no visible key in the tile).
 *   MODE_SPLIT  split-K ("Model-Optimizer: Add split-k decode kernel for skip softmax", the 32-split,
 *               128-token schedule): ntiles = ceil(n / tile), c = ceil(ntiles / S); split s takes tiles
 *               [s c, (s+1) c) and is attended densely to (o_s, lse_s); then
 *               lse = log sum_{finite} exp(lse_s) and o = sum_s exp(lse_s - lse) o_s.
 *
 * NVFP4 fake quantization of P and V under skip-softmax in the one-token decode (orc_decode_qdq_rows,
 * with the quantizer itself exported as orc_nvfp4_qdq and orc_fp_round) follows the plain reading of the
 * format stated at nvfp4_block; its rounding decisions are taken in fp32, the precision the format is
 * defined in.
 * Plus multi-token paged decode (orc_paged_multi_rows), the backward of the dense prefill
 * (orc_prefill_bwd) and of the small-seq cross-attention from its stored attention weights
 * (orc_smallseq_bwd), at the end of this file.
 *
 * Inputs are read as the exact bytes the GPU reads (fp32, or bf16 widened exactly to fp64); all
 * arithmetic is in fp64.
 *
 * Paged layout: k_cache / v_cache are [num_pages, Hkv, page, D]; key j of batch row b lives in page
 * block_table[b * max_pages + j / page], slot j % page.  GQA: query head h reads KV head h / (Hq / Hkv).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1 };
enum { MODE_DENSE = 0, MODE_SKIP = 1, MODE_SPLIT = 2 };
enum { MAP_DONE = 0, MAP_SKIPPED = 1, MAP_UNVISITED = 2 };

static double widen(const void *base, int dtype, size_t idx)
{
    if (dtype == ORC_F32)
        return (double)((const float *)base)[idx];
    uint32_t u = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double dot(const double *a, const double *b, int D)
{
    double s = 0.0;
    for (int d = 0; d < D; ++d)
        s += a[d] * b[d];
    return s;
}

/*
 * NVFP4 fake quantization (quantize, then dequantize), "Model-Optimizer: Add split-k decode kernel for
 * skip softmax", What does this PR do and Usage (P and V quantized to NVFP4 in the one-token decode,
 * each with an amax).  The pages name the format but print no recipe; this is the format's published
 * definition, read plainly:
 *   - a tensor is cut into blocks of 16 consecutive values along its last dimension;
 *   - each element is an E2M1 code: sign, 2 exponent bits (bias 1), 1 mantissa bit, subnormals,
 *     magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6};
 *   - each block has one E4M3 scale code: 4 exponent bits (bias 7), 3 mantissa bits, subnormals,
 *     largest finite 448 (the all-ones pattern is NaN);
 *   - one fp32 scale per tensor, from amax, maps amax to the largest element times the largest scale,
 *     6 * 448 = 2688.
 * In fp32, each rounding to the nearest grid value, ties to the even code, saturating at the top:
 *   enc = 448 / amax, dec = amax / 2688
 *   scale code c_b = e4m3(max_i |x_i| * enc),  block scale s_b = c_b * dec
 *   x^_i = sign(x_i) * e2m1(|x_i| * (1 / s_b)) * s_b,   and x^_i = 0 when s_b = 0.
 * The grids are enumerated code by code, so that each rounding is a plain nearest-point search.
 */
enum { ORC_E2M1 = 0, ORC_E4M3 = 1 };

/* Non-negative value of code c (ascending with c) of a minifloat with eb exponent bits (bias b) and mb
 * mantissa bits, subnormals at exponent field 0. */
static double minifloat_value(int c, int mb, int bias)
{
    int e = c >> mb, m = c & ((1 << mb) - 1);
    double frac = (double)m / (double)(1 << mb);
    return e == 0 ? ldexp(frac, 1 - bias) : ldexp(1.0 + frac, e - bias);
}

/* Nearest grid value to y >= 0 (ties to the even code, values above the top go to the top). */
static float fp_round(int fmt, float y)
{
    int mb = fmt == ORC_E2M1 ? 1 : 3, bias = fmt == ORC_E2M1 ? 1 : 7;
    int ncodes = fmt == ORC_E2M1 ? 8 : 127; /* E4M3 codes 0..126; 127 (exponent and mantissa all ones) is NaN */
    if ((double)y >= minifloat_value(ncodes - 1, mb, bias)) /* saturate (far above the top the distances */
        return (float)minifloat_value(ncodes - 1, mb, bias); /* to the top codes round to a false tie) */
    int best = 0;
    double bd = fabs((double)y);
    for (int c = 1; c < ncodes; ++c) {
        double d = fabs((double)y - minifloat_value(c, mb, bias));
        if (d < bd || (d == bd && (c & 1) == 0)) {
            bd = d;
            best = c;
        }
    }
    return (float)minifloat_value(best, mb, bias);
}

/* Quantize-dequantize n <= 16 values that form one block, in place. */
static void nvfp4_block(float *x, int n, float amax)
{
    float enc = 448.0f / amax, dec = amax / 2688.0f;
    float bmax = 0.0f;
    for (int i = 0; i < n; ++i)
        if (fabsf(x[i]) > bmax)
            bmax = fabsf(x[i]);
    float sb = fp_round(ORC_E4M3, bmax * enc) * dec;
    float inv = sb > 0.0f ? 1.0f / sb : 0.0f;
    for (int i = 0; i < n; ++i) {
        float mag = fp_round(ORC_E2M1, fabsf(x[i]) * inv) * sb;
        x[i] = x[i] < 0.0f ? -mag : mag;
    }
}

/* Round to the nearest bf16 (ties to even): the dtype a bf16 tensor's fake quantization returns. */
static float round_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Exported for the tests: y[i] rounded to the grid of fmt (ORC_E2M1 or ORC_E4M3), y[i] >= 0. */
int orc_fp_round(int fmt, const float *y, float *out, size_t n)
{
    if (fmt != ORC_E2M1 && fmt != ORC_E4M3)
        return -1;
    for (size_t i = 0; i < n; ++i) {
        if (!(y[i] >= 0.0f))
            return -1;
        out[i] = fp_round(fmt, y[i]);
    }
    return 0;
}

/* Exported for the tests: NVFP4 fake quantization of rows x [rows, len] (blocks of 16 along each row,
 * the last one ragged), in fp32, into out. */
int orc_nvfp4_qdq(const float *x, size_t rows, int len, float amax, float *out)
{
    if (len <= 0 || !(amax > 0.0f) || isinf(amax))
        return -1;
    memcpy(out, x, sizeof(float) * rows * (size_t)len);
    for (size_t r = 0; r < rows; ++r)
        for (int b0 = 0; b0 < len; b0 += 16)
            nvfp4_block(out + r * (size_t)len + b0, len - b0 < 16 ? len - b0 : 16, amax);
    return 0;
}

/* The plain definition.  K, V: n rows of D.  p (nullable) receives the n probabilities. */
static void dense_row(const double *q, const double *K, const double *V, int n, int D, double scale,
                      double *o, double *lse, double *p)
{
    for (int d = 0; d < D; ++d)
        o[d] = 0.0;
    if (n == 0) {
        *lse = -INFINITY;
        return;
    }
    double *s = malloc(sizeof(double) * (size_t)n);
    double m = -INFINITY;
    for (int j = 0; j < n; ++j) {
        s[j] = scale * dot(q, K + (size_t)j * D, D);
        if (s[j] > m)
            m = s[j];
    }
    double sum = 0.0;
    for (int j = 0; j < n; ++j)
        sum += exp(s[j] - m);
    for (int j = 0; j < n; ++j) {
        double pj = exp(s[j] - m) / sum;
        if (p)
            p[j] = pj;
        for (int d = 0; d < D; ++d)
            o[d] += pj * V[(size_t)j * D + d];
    }
    *lse = m + log(sum);
    free(s);
}

/* Skip-softmax over `tile`-key tiles in ascending order.  map: one code per tile slot (width stride);
 * replay (nullable): decisions to impose, 1 = skip, 0 = process.  Returns 0, or -1 on a bad replay.
 * p_amax > 0 fake-quantizes P to NVFP4 before P.V: the unnormalized probabilities exp(s_j - m) of a
 * processed tile, m the running max including the tile (so that P lies in [0, 1]), are rounded to fp32
 * and quantized in blocks of 16 consecutive keys counted from key 0 (tile must be a multiple of 16);
 * the row sum l takes the unquantized values.  Returns -1 if tile is not a multiple of 16 then. */
static int skip_row(const double *q, const double *K, const double *V, int n, int D, double scale,
                    int tile, double thr, const uint8_t *replay, int stride, float p_amax, double *o,
                    double *lse, uint8_t *map)
{
    int ntiles = (n + tile - 1) / tile;
    if (ntiles > stride || (p_amax > 0.0f && tile % 16))
        return -1;
    if (map)
        for (int t = 0; t < stride; ++t)
            map[t] = MAP_UNVISITED;
    double m = -INFINITY, l = 0.0;
    double *acc = calloc((size_t)D, sizeof(double));
    double *s = malloc(sizeof(double) * (size_t)tile);
    int rc = 0;
    for (int t = 0; t < ntiles; ++t) {
        int j0 = t * tile, j1 = j0 + tile < n ? j0 + tile : n;
        double tmax = -INFINITY;
        for (int j = j0; j < j1; ++j) {
            s[j - j0] = scale * dot(q, K + (size_t)j * D, D);
            if (s[j - j0] > tmax)
                tmax = s[j - j0];
        }
        int skip;
        if (replay) {
            if (replay[t] > 1) {
                rc = -1;
                break;
            }
            skip = replay[t] == 1;
        } else {
            skip = thr > 0.0 && m > -INFINITY && exp(tmax - m) < thr;
        }
        if (map)
            map[t] = skip ? MAP_SKIPPED : MAP_DONE;
        if (skip)
            continue;
        double m_new = tmax > m ? tmax : m;
        double alpha = m == -INFINITY ? 0.0 : exp(m - m_new);
        l *= alpha;
        for (int d = 0; d < D; ++d)
            acc[d] *= alpha;
        for (int j = j0; j < j1; ++j) {
            s[j - j0] = exp(s[j - j0] - m_new); /* s now holds P of the tile */
            l += s[j - j0];
        }
        if (p_amax > 0.0f)
            for (int b0 = j0; b0 < j1; b0 += 16) {
                float blk[16];
                int cnt = j1 - b0 < 16 ? j1 - b0 : 16;
                for (int i = 0; i < cnt; ++i)
                    blk[i] = (float)s[b0 - j0 + i];
                nvfp4_block(blk, cnt, p_amax);
                for (int i = 0; i < cnt; ++i)
                    s[b0 - j0 + i] = blk[i];
            }
        for (int j = j0; j < j1; ++j)
            for (int d = 0; d < D; ++d)
                acc[d] += s[j - j0] * V[(size_t)j * D + d];
        m = m_new;
    }
    if (rc == 0) {
        for (int d = 0; d < D; ++d)
            o[d] = l > 0.0 ? acc[d] / l : 0.0;
        *lse = l > 0.0 ? m + log(l) : -INFINITY;
    }
    free(acc);
    free(s);
    return rc;
}

/* Split-K: dense attention per contiguous chunk of tiles, then the log-sum-exp merge. */
static void split_row(const double *q, const double *K, const double *V, int n, int D, double scale,
                      int tile, int S, double *o, double *lse)
{
    int ntiles = (n + tile - 1) / tile;
    int c = (ntiles + S - 1) / S;
    double *os = malloc(sizeof(double) * (size_t)S * D);
    double *ls = malloc(sizeof(double) * (size_t)S);
    for (int sp = 0; sp < S; ++sp) {
        long j0 = (long)sp * c * tile, j1 = (long)(sp + 1) * c * tile;
        if (j0 > n)
            j0 = n;
        if (j1 > n)
            j1 = n;
        dense_row(q, K + j0 * D, V + j0 * D, (int)(j1 - j0), D, scale, os + (size_t)sp * D, ls + sp, NULL);
    }
    double mx = -INFINITY;
    for (int sp = 0; sp < S; ++sp)
        if (ls[sp] > mx)
            mx = ls[sp];
    for (int d = 0; d < D; ++d)
        o[d] = 0.0;
    if (mx == -INFINITY) {
        *lse = -INFINITY;
    } else {
        double sum = 0.0;
        for (int sp = 0; sp < S; ++sp)
            if (ls[sp] > -INFINITY)
                sum += exp(ls[sp] - mx);
        *lse = mx + log(sum);
        for (int sp = 0; sp < S; ++sp) {
            if (ls[sp] == -INFINITY)
                continue;
            double w = exp(ls[sp] - *lse);
            for (int d = 0; d < D; ++d)
                o[d] += w * os[(size_t)sp * D + d];
        }
    }
    free(os);
    free(ls);
}

static int run_mode(int mode, const double *q, const double *K, const double *V, int n, int D,
                    double scale, int tile, double thr, int splits, const uint8_t *replay, int stride,
                    float p_amax, double *o, double *lse, uint8_t *map)
{
    if (p_amax != 0.0f && mode != MODE_SKIP)
        return -1;
    switch (mode) {
    case MODE_DENSE:
        dense_row(q, K, V, n, D, scale, o, lse, NULL);
        return 0;
    case MODE_SKIP:
        return skip_row(q, K, V, n, D, scale, tile, thr, replay, stride, p_amax, o, lse, map);
    case MODE_SPLIT:
        if (splits < 1)
            return -1;
        split_row(q, K, V, n, D, scale, tile, splits, o, lse);
        return 0;
    }
    return -1;
}

/*
 * Varlen (THD) attention, "Model-Optimizer: Add Triton unified attention kernel" (variable-length
 * batching, GQA, causal and non-causal) with sequences packed by cu_seqlens ("ROCm TransformerEngine:
 * Integrate CK varlen cross attention", THD with cu_seqlens).
 * q [tq, Hq, D], k/v [tk, Hkv, D]; rows: n_rows pairs (token, head).  Query row i of sequence b sees keys
 * j < Lk when non-causal and j <= i + (Lk - Lq) when causal (bottom-right aligned).
 * Outputs per requested row: o [n_rows, D], lse [n_rows], map [n_rows, stride] (MODE_SKIP, nullable).
 */
int orc_prefill_rows(int dtype, const void *q, const void *k, const void *v, const int32_t *cu_q,
                     const int32_t *cu_k, int B, int Hq, int Hkv, int D, double scale, int causal,
                     int mode, double thr, int tile, int splits, const int32_t *rows, int n_rows,
                     const uint8_t *replay, int stride, double *o, double *lse, uint8_t *map)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || D <= 0 || (mode != MODE_DENSE && tile <= 0))
        return -1;
    int G = Hq / Hkv, bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int r = 0; r < n_rows; ++r) {
        int t = rows[2 * r], h = rows[2 * r + 1];
        int b = -1;
        for (int bb = 0; bb < B; ++bb)
            if (cu_q[bb] <= t && t < cu_q[bb + 1]) {
                b = bb;
                break;
            }
        if (b < 0 || h < 0 || h >= Hq) {
            bad = 1;
            continue;
        }
        int Lq = cu_q[b + 1] - cu_q[b], Lk = cu_k[b + 1] - cu_k[b], i = t - cu_q[b], g = h / G;
        int n = Lk;
        if (causal) {
            n = i + 1 + (Lk - Lq);
            if (n < 0)
                n = 0;
            if (n > Lk)
                n = Lk;
        }
        double *qd = malloc(sizeof(double) * D);
        double *K = malloc(sizeof(double) * ((size_t)n * D + 1));
        double *V = malloc(sizeof(double) * ((size_t)n * D + 1));
        for (int d = 0; d < D; ++d)
            qd[d] = widen(q, dtype, ((size_t)t * Hq + h) * D + d);
        for (int j = 0; j < n; ++j)
            for (int d = 0; d < D; ++d) {
                size_t src = ((size_t)(cu_k[b] + j) * Hkv + g) * D + d;
                K[(size_t)j * D + d] = widen(k, dtype, src);
                V[(size_t)j * D + d] = widen(v, dtype, src);
            }
        if (run_mode(mode, qd, K, V, n, D, scale, tile, thr, splits, replay ? replay + (size_t)r * stride : NULL,
                     stride, 0.0f, o + (size_t)r * D, lse + r, map ? map + (size_t)r * stride : NULL))
            bad = 1;
        free(qd);
        free(K);
        free(V);
    }
    return bad ? -1 : 0;
}

/*
 * One-token paged decode, "Model-Optimizer: Add split-k decode kernel for skip softmax", Usage
 * (query, key_cache, value_cache, block_table, sequence_lengths): the single query token of batch row b
 * sees all seq_lens[b] cached keys.  q [B, Hq, D] bf16; caches [num_pages, Hkv, page, D] bf16.
 * rows: n_rows pairs (b, head).  Outputs as for orc_prefill_rows.
 */
static int decode_rows(const void *q, const void *kc, const void *vc, const int32_t *block_table,
                       const int32_t *seq_lens, int B, int Hq, int Hkv, int D, int page, int max_pages,
                       double scale, int mode, double thr, int tile, int splits, const int32_t *rows,
                       int n_rows, const uint8_t *replay, int stride, float p_amax, float v_amax, double *o,
                       double *lse, uint8_t *map)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || D <= 0 || page <= 0 || (mode != MODE_DENSE && tile <= 0))
        return -1;
    int G = Hq / Hkv, bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int r = 0; r < n_rows; ++r) {
        int b = rows[2 * r], h = rows[2 * r + 1];
        if (b < 0 || b >= B || h < 0 || h >= Hq || seq_lens[b] < 0 || seq_lens[b] > max_pages * page) {
            bad = 1;
            continue;
        }
        int n = seq_lens[b], g = h / G;
        double *qd = malloc(sizeof(double) * D);
        double *K = malloc(sizeof(double) * ((size_t)n * D + 1));
        double *V = malloc(sizeof(double) * ((size_t)n * D + 1));
        for (int d = 0; d < D; ++d)
            qd[d] = widen(q, ORC_BF16, ((size_t)b * Hq + h) * D + d);
        for (int j = 0; j < n; ++j) {
            int pg = block_table[(size_t)b * max_pages + j / page];
            for (int d = 0; d < D; ++d) {
                size_t src = (((size_t)pg * Hkv + g) * page + j % page) * D + d;
                K[(size_t)j * D + d] = widen(kc, ORC_BF16, src);
                V[(size_t)j * D + d] = widen(vc, ORC_BF16, src);
            }
            if (v_amax > 0.0f) /* V [n, D] in blocks of 16 along D, back to bf16 */
                for (int d0 = 0; d0 < D; d0 += 16) {
                    float blk[16];
                    int cnt = D - d0 < 16 ? D - d0 : 16;
                    for (int i = 0; i < cnt; ++i)
                        blk[i] = (float)V[(size_t)j * D + d0 + i];
                    nvfp4_block(blk, cnt, v_amax);
                    for (int i = 0; i < cnt; ++i)
                        V[(size_t)j * D + d0 + i] = round_bf16(blk[i]);
                }
        }
        if (run_mode(mode, qd, K, V, n, D, scale, tile, thr, splits, replay ? replay + (size_t)r * stride : NULL,
                     stride, p_amax, o + (size_t)r * D, lse + r, map ? map + (size_t)r * stride : NULL))
            bad = 1;
        free(qd);
        free(K);
        free(V);
    }
    return bad ? -1 : 0;
}

int orc_decode_rows(const void *q, const void *kc, const void *vc, const int32_t *block_table,
                    const int32_t *seq_lens, int B, int Hq, int Hkv, int D, int page, int max_pages,
                    double scale, int mode, double thr, int tile, int splits, const int32_t *rows,
                    int n_rows, const uint8_t *replay, int stride, double *o, double *lse, uint8_t *map)
{
    return decode_rows(q, kc, vc, block_table, seq_lens, B, Hq, Hkv, D, page, max_pages, scale, mode, thr, tile,
                       splits, rows, n_rows, replay, stride, 0.0f, 0.0f, o, lse, map);
}

/*
 * One-token paged decode with NVFP4 fake quantization of P and V ("Model-Optimizer: Add split-k decode
 * kernel for skip softmax", What does this PR do: skip-softmax together with NVFP4 P/V QDQ, in the one
 * sequential split of 32-key tiles; Usage: p_qdq / v_qdq with their amax).  The sequential skip pass of
 * skip_row with tile = 32 and threshold thr (thr = 0 skips nothing), where
 *   - V, when v_amax > 0, is replaced by its fake quantization: every key's D values in blocks of 16,
 *     the result rounded back to bf16, the cache's dtype;
 *   - P, when p_amax > 0, is fake-quantized per tile as skip_row describes.
 * amax = 0 leaves that side unquantized.  replay (nullable, [n_rows, stride]) imposes the skip decisions
 * as in skip_row.  Arguments and outputs as for orc_decode_rows.
 */
int orc_decode_qdq_rows(const void *q, const void *kc, const void *vc, const int32_t *block_table,
                        const int32_t *seq_lens, int B, int Hq, int Hkv, int D, int page, int max_pages,
                        double scale, double thr, float p_amax, float v_amax, const int32_t *rows, int n_rows,
                        const uint8_t *replay, int stride, double *o, double *lse, uint8_t *map)
{
    if (!(p_amax >= 0.0f) || !(v_amax >= 0.0f) || isinf(p_amax) || isinf(v_amax))
        return -1;
    return decode_rows(q, kc, vc, block_table, seq_lens, B, Hq, Hkv, D, page, max_pages, scale, MODE_SKIP, thr, 32,
                       1, rows, n_rows, replay, stride, p_amax, v_amax, o, lse, map);
}

/*
 * Small-seq cross-attention, "ROCm TransformerEngine: Integrate CK varlen cross attention for small-seq
 * (s_q=1, s_kv<=16)": one query token per sequence, s_kv = cu_kv[b+1] - cu_kv[b] keys, non-causal,
 * H query heads = H KV heads.  Besides o it returns the attention weights w[b, h, 0, j] = p_j for
 * j < s_kv and 0 for s_kv <= j < max_s.  q [B, H, D], k/v [total_kv, H, D] (dtype).
 * rows: n_rows pairs (b, head); o [n_rows, D], w [n_rows, max_s], lse (nullable) [n_rows]: the row's
 * natural-log log-sum-exp of its logits (-inf with no key).
 */
int orc_smallseq_rows(int dtype, const void *q, const void *k, const void *v, const int32_t *cu_kv, int B,
                      int H, int D, int max_s, double scale, const int32_t *rows, int n_rows, double *o,
                      double *w, double *lse_out)
{
    if (B < 0 || H <= 0 || D <= 0 || max_s < 0)
        return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : bad)
    for (int r = 0; r < n_rows; ++r) {
        int b = rows[2 * r], h = rows[2 * r + 1];
        if (b < 0 || b >= B || h < 0 || h >= H) {
            bad = 1;
            continue;
        }
        int n = cu_kv[b + 1] - cu_kv[b];
        if (n < 0 || n > max_s) {
            bad = 1;
            continue;
        }
        double *qd = malloc(sizeof(double) * D);
        double *K = malloc(sizeof(double) * ((size_t)n * D + 1));
        double *V = malloc(sizeof(double) * ((size_t)n * D + 1));
        double *p = malloc(sizeof(double) * ((size_t)n + 1)), lse;
        for (int d = 0; d < D; ++d)
            qd[d] = widen(q, dtype, ((size_t)b * H + h) * D + d);
        for (int j = 0; j < n; ++j)
            for (int d = 0; d < D; ++d) {
                size_t src = ((size_t)(cu_kv[b] + j) * H + h) * D + d;
                K[(size_t)j * D + d] = widen(k, dtype, src);
                V[(size_t)j * D + d] = widen(v, dtype, src);
            }
        dense_row(qd, K, V, n, D, scale, o + (size_t)r * D, &lse, p);
        for (int j = 0; j < max_s; ++j)
            w[(size_t)r * max_s + j] = j < n ? p[j] : 0.0;
        if (lse_out)
            lse_out[r] = lse;
        free(qd);
        free(K);
        free(V);
        free(p);
    }
    return bad ? -1 : 0;
}

/*
 * Backward of the dense varlen prefill (the gradients of the masked-softmax definition above); the
 * Triton kernel of "Model-Optimizer: Add Triton unified attention kernel with HuggingFace integration"
 * (summary) has an autograd backward beside its forward.  With p_j = exp(s_j - lse), s_j = scale q.k_j
 * over the visible keys of a row and dO the output gradient:
 *   dP_j = dO.v_j,  Dsum = dO.o = sum_j p_j dP_j,  dS_j = p_j (dP_j - Dsum)
 *   dq   = scale sum_j dS_j k_j
 *   dk_j += scale dS_j q,  dv_j += p_j dO          (summed over every query row and query head of the group)
 * Inputs as for orc_prefill_rows plus dout [tq, Hq, D] of the same dtype, and o (nullable, same dtype and
 * layout as dout): a stored forward output.  Without o, Dsum is the exact sum_j p_j dP_j; with o it is
 * the row dot dO.o of the stored output, as a backward that reads the saved output computes it (equal to
 * the former when o is the exact output; a rounded o shifts every dS_j of the row by -p_j * the dot of
 * dO with the rounding).  Outputs fp64 dq [tq, Hq, D], dk and dv [tk, Hkv, D] (fully written).  One task
 * per (sequence, KV head), so no two tasks touch the same output.
 */
int orc_prefill_bwd(int dtype, const void *q, const void *k, const void *v, const void *dout, const void *o,
                    const int32_t *cu_q, const int32_t *cu_k, int B, int Hq, int Hkv, int D, double scale, int causal,
                    double *dq, double *dk, double *dv)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || D <= 0)
        return -1;
    const int G = Hq / Hkv;
    const size_t tq = B ? (size_t)cu_q[B] : 0, tk = B ? (size_t)cu_k[B] : 0;
    memset(dq, 0, sizeof(double) * tq * Hq * D);
    memset(dk, 0, sizeof(double) * tk * Hkv * D);
    memset(dv, 0, sizeof(double) * tk * Hkv * D);
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int b = 0; b < B; ++b)
        for (int g = 0; g < Hkv; ++g) {
            const int Lq = cu_q[b + 1] - cu_q[b], Lk = cu_k[b + 1] - cu_k[b];
            double *K = malloc(sizeof(double) * ((size_t)Lk * D + 1));
            double *V = malloc(sizeof(double) * ((size_t)Lk * D + 1));
            double *qd = malloc(sizeof(double) * D), *go = malloc(sizeof(double) * D);
            double *s = malloc(sizeof(double) * ((size_t)Lk + 1)), *dp = malloc(sizeof(double) * ((size_t)Lk + 1));
            for (int j = 0; j < Lk; ++j)
                for (int d = 0; d < D; ++d) {
                    const size_t src = ((size_t)(cu_k[b] + j) * Hkv + g) * D + d;
                    K[(size_t)j * D + d] = widen(k, dtype, src);
                    V[(size_t)j * D + d] = widen(v, dtype, src);
                }
            for (int hh = 0; hh < G; ++hh) {
                const int h = g * G + hh;
                for (int i = 0; i < Lq; ++i) {
                    const size_t row = ((size_t)(cu_q[b] + i) * Hq + h) * D;
                    int n = Lk;
                    if (causal) {
                        n = i + 1 + (Lk - Lq);
                        n = n < 0 ? 0 : (n > Lk ? Lk : n);
                    }
                    if (n == 0)
                        continue; /* a row with no key: o = 0 regardless of q, k, v */
                    for (int d = 0; d < D; ++d) {
                        qd[d] = widen(q, dtype, row + d);
                        go[d] = widen(dout, dtype, row + d);
                    }
                    double m = -INFINITY;
                    for (int j = 0; j < n; ++j) {
                        s[j] = scale * dot(qd, K + (size_t)j * D, D);
                        if (s[j] > m)
                            m = s[j];
                    }
                    double sum = 0.0;
                    for (int j = 0; j < n; ++j)
                        sum += exp(s[j] - m);
                    const double lse = m + log(sum);
                    double dsum = 0.0;
                    for (int j = 0; j < n; ++j) {
                        s[j] = exp(s[j] - lse); /* s now holds p */
                        dp[j] = dot(go, V + (size_t)j * D, D);
                        dsum += s[j] * dp[j];
                    }
                    if (o) {
                        dsum = 0.0;
                        for (int d = 0; d < D; ++d)
                            dsum += go[d] * widen(o, dtype, row + d);
                    }
                    for (int j = 0; j < n; ++j) {
                        const double ds = s[j] * (dp[j] - dsum);
                        const size_t kv = ((size_t)(cu_k[b] + j) * Hkv + g) * D;
                        for (int d = 0; d < D; ++d) {
                            dq[row + d] += scale * ds * K[(size_t)j * D + d];
                            dk[kv + d] += scale * ds * qd[d];
                            dv[kv + d] += s[j] * go[d];
                        }
                    }
                }
            }
            free(K);
            free(V);
            free(qd);
            free(go);
            free(s);
            free(dp);
        }
    return 0;
}

/*
 * Backward of the small-seq cross-attention from its stored attention weights ("ROCm TransformerEngine:
 * Integrate CK varlen cross attention for small-seq (s_q=1, s_kv<=16)", change list: the backward takes
 * grad_V, grad_attn, the softmax backward and grad_Q / grad_K, and reads the weights the forward wrote).
 * Per (sequence b, head h) with s = cu_kv[b+1] - cu_kv[b] keys, stored weights w_j = w[b, h, 0, j]
 * (entries j >= s are padding and not read) and output gradient dO:
 *   grad_V:   dv_j = w_j dO
 *   grad_attn: dw_j = dO . v_j
 *   softmax backward: ds_j = w_j (dw_j - sum_j' w_j' dw_j')
 *   grad_Q:   dq = scale sum_j ds_j k_j          grad_K: dk_j = scale ds_j q
 * q, dout [B, H, D]; k, v [total_kv, H, D]; w [B, H, 1, max_s]; all of dtype; outputs fp64 dq [B, H, D],
 * dk, dv [total_kv, H, D], fully written.  Each key belongs to one sequence, so tasks never overlap.
 */
int orc_smallseq_bwd(int dtype, const void *q, const void *k, const void *v, const void *w, const void *dout,
                     const int32_t *cu_kv, int B, int H, int D, int max_s, double scale, double *dq, double *dk,
                     double *dv)
{
    if (B < 0 || H <= 0 || D <= 0 || max_s < 0)
        return -1;
    const size_t tk = B ? (size_t)cu_kv[B] : 0;
    memset(dq, 0, sizeof(double) * (size_t)B * H * D);
    memset(dk, 0, sizeof(double) * tk * H * D);
    memset(dv, 0, sizeof(double) * tk * H * D);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 16) collapse(2) reduction(| : bad)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            const int n = cu_kv[b + 1] - cu_kv[b];
            if (n < 0 || n > max_s) {
                bad = 1;
                continue;
            }
            const size_t row = ((size_t)b * H + h) * D;
            double *dw = malloc(sizeof(double) * ((size_t)n + 1)), *wj = malloc(sizeof(double) * ((size_t)n + 1));
            double sum = 0.0;
            for (int j = 0; j < n; ++j) {
                const size_t kv = ((size_t)(cu_kv[b] + j) * H + h) * D;
                wj[j] = widen(w, dtype, ((size_t)b * H + h) * max_s + j);
                dw[j] = 0.0;
                for (int d = 0; d < D; ++d)
                    dw[j] += widen(dout, dtype, row + d) * widen(v, dtype, kv + d);
                sum += wj[j] * dw[j];
            }
            for (int j = 0; j < n; ++j) {
                const size_t kv = ((size_t)(cu_kv[b] + j) * H + h) * D;
                const double ds = wj[j] * (dw[j] - sum);
                for (int d = 0; d < D; ++d) {
                    dv[kv + d] = wj[j] * widen(dout, dtype, row + d);
                    dk[kv + d] = scale * ds * widen(q, dtype, row + d);
                    dq[row + d] += scale * ds * widen(k, dtype, kv + d);
                }
            }
            free(dw);
            free(wj);
        }
    return bad ? -1 : 0;
}

/*
 * Multi-token paged decode: the paged cache of "Model-Optimizer: Add split-k decode kernel for skip
 * softmax" (its description keeps multi-token decode on the shared attention kernel, whose summary gives
 * causal masking over variable-length batches).  Sequence b has Lq_b = cu_q[b+1] - cu_q[b] new query
 * tokens, the last Lq_b of its seq_lens[b] cached keys; its token i sees the keys
 * j < clamp(seq_lens[b] - Lq_b + i + 1, 0, seq_lens[b]) (bottom-right causal), key j living in page
 * block_table[b * max_pages + j / page], slot j % page.  Dense definition per row.
 * q [total_q, Hq, D] bf16; caches [num_pages, Hkv, page, D] bf16.  rows: (token, head) pairs;
 * o [n_rows, D], lse [n_rows].
 */
int orc_paged_multi_rows(const void *q, const int32_t *cu_q, const void *kc, const void *vc,
                         const int32_t *block_table, const int32_t *seq_lens, int B, int Hq, int Hkv, int D, int page,
                         int max_pages, double scale, const int32_t *rows, int n_rows, double *o, double *lse)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || D <= 0 || page <= 0)
        return -1;
    const int G = Hq / Hkv, tq = B ? cu_q[B] : 0;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int r = 0; r < n_rows; ++r) {
        const int t = rows[2 * r], h = rows[2 * r + 1];
        if (t < 0 || t >= tq || h < 0 || h >= Hq) {
            bad = 1;
            continue;
        }
        int b = 0;
        while (cu_q[b + 1] <= t)
            ++b;
        const int L = seq_lens[b], Lq = cu_q[b + 1] - cu_q[b], i = t - cu_q[b];
        if (L < 0 || L > max_pages * page) {
            bad = 1;
            continue;
        }
        int n = L - Lq + i + 1;
        n = n < 0 ? 0 : (n > L ? L : n);
        const int g = h / G;
        double *qd = malloc(sizeof(double) * D);
        double *K = malloc(sizeof(double) * ((size_t)n * D + 1));
        double *V = malloc(sizeof(double) * ((size_t)n * D + 1));
        for (int d = 0; d < D; ++d)
            qd[d] = widen(q, ORC_BF16, ((size_t)t * Hq + h) * D + d);
        for (int j = 0; j < n; ++j) {
            const int pg = block_table[(size_t)b * max_pages + j / page];
            for (int d = 0; d < D; ++d) {
                const size_t src = (((size_t)pg * Hkv + g) * page + j % page) * D + d;
                K[(size_t)j * D + d] = widen(kc, ORC_BF16, src);
                V[(size_t)j * D + d] = widen(vc, ORC_BF16, src);
            }
        }
        dense_row(qd, K, V, n, D, scale, o + (size_t)r * D, lse + r, NULL);
        free(qd);
        free(K);
        free(V);
    }
    return bad ? -1 : 0;
}
