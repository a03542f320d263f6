/* Drives every entry point of the fp64 oracle (oracle/oracle.c, built with the address and
 * undefined-behaviour sanitizers) on tiny inputs: fp32 and bf16 varlen prefill in every mode, the paged
 * decode in every mode and with NVFP4 P / V, small-seq forward and backward, the prefill backward with and
 * without a stored output, the multi-token paged decode, the fp rounding and NVFP4 helpers, and a few
 * rejected calls.  Checks that every call returns its expected code and every output is finite (rows that
 * see no key excepted for lse).  Exit status 0 on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_prefill_rows(int, const void *, const void *, const void *, const int32_t *, const int32_t *, int, int, int, int,
                     double, int, int, double, int, int, const int32_t *, int, const uint8_t *, int, double *, double *,
                     uint8_t *);
int orc_decode_rows(const void *, const void *, const void *, const int32_t *, const int32_t *, int, int, int, int, int,
                    int, double, int, double, int, int, const int32_t *, int, const uint8_t *, int, double *, double *,
                    uint8_t *);
int orc_decode_qdq_rows(const void *, const void *, const void *, const int32_t *, const int32_t *, int, int, int, int,
                        int, int, double, double, float, float, const int32_t *, int, const uint8_t *, int, double *,
                        double *, uint8_t *);
int orc_smallseq_rows(int, const void *, const void *, const void *, const int32_t *, int, int, int, int, double,
                      const int32_t *, int, double *, double *, double *);
int orc_prefill_bwd(int, const void *, const void *, const void *, const void *, const void *, const int32_t *,
                    const int32_t *, int, int, int, int, double, int, double *, double *, double *);
int orc_smallseq_bwd(int, const void *, const void *, const void *, const void *, const void *, const int32_t *, int,
                     int, int, int, double, double *, double *, double *);
int orc_paged_multi_rows(const void *, const int32_t *, const void *, const void *, const int32_t *, const int32_t *,
                         int, int, int, int, int, int, double, const int32_t *, int, double *, double *);
int orc_fp_round(int, const float *, float *, size_t);
int orc_nvfp4_qdq(const float *, size_t, int, float, float *);

static int bad = 0;
static uint32_t rng = 12345u;
static float urand(void) /* uniform in [-1, 1) */
{
    rng = rng * 1664525u + 1013904223u;
    return (float)(rng >> 8) / 8388608.0f - 1.0f;
}
static uint16_t to_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    return (uint16_t)(u >> 16);
}
static void expect(int rc, int want, const char *what)
{
    if (rc != want) {
        fprintf(stderr, "%s: returned %d, expected %d\n", what, rc, want);
        ++bad;
    }
}
static void finite(const double *x, size_t n, const char *what)
{
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) {
            fprintf(stderr, "%s: element %zu is not finite\n", what, i);
            ++bad;
            return;
        }
}

enum { D = 16, HQ = 4, HKV = 2, B = 2, PAGE = 4, MAXP = 12, POOL = 30 };

int main(void)
{
    const int32_t cu[B + 1] = {0, 5, 42}; /* lengths 5 and 37 */
    const int tq = 42;
    float *qf = malloc(sizeof(float) * tq * HQ * D), *kf = malloc(sizeof(float) * tq * HKV * D);
    float *vf = malloc(sizeof(float) * tq * HKV * D), *gf = malloc(sizeof(float) * tq * HQ * D);
    uint16_t *qb = malloc(2 * tq * HQ * D), *kb = malloc(2 * tq * HKV * D), *vb = malloc(2 * tq * HKV * D);
    for (int i = 0; i < tq * HQ * D; ++i) {
        qf[i] = urand();
        gf[i] = urand();
        qb[i] = to_bf16(qf[i]);
    }
    for (int i = 0; i < tq * HKV * D; ++i) {
        kf[i] = urand();
        vf[i] = urand();
        kb[i] = to_bf16(kf[i]);
        vb[i] = to_bf16(vf[i]);
    }
    int32_t rows[2 * 42 * HQ];
    for (int t = 0; t < tq; ++t)
        for (int h = 0; h < HQ; ++h) {
            rows[2 * (t * HQ + h)] = t;
            rows[2 * (t * HQ + h) + 1] = h;
        }
    const int nr = tq * HQ, stride = 8;
    double *o = malloc(sizeof(double) * nr * D), *lse = malloc(sizeof(double) * nr);
    uint8_t *map = malloc((size_t)nr * stride);
    for (int dt = 0; dt < 2; ++dt)
        for (int causal = 0; causal < 2; ++causal)
            for (int mode = 0; mode < 3; ++mode) {
                const void *q = dt ? (const void *)qb : qf, *k = dt ? (const void *)kb : kf;
                const void *v = dt ? (const void *)vb : vf;
                expect(orc_prefill_rows(dt, q, k, v, cu, cu, B, HQ, HKV, D, 0.25, causal, mode, 0.1, 8, 3, rows, nr,
                                        NULL, stride, o, lse, mode == 1 ? map : NULL), 0, "prefill");
                finite(o, (size_t)nr * D, "prefill o");
                finite(lse, nr, "prefill lse");
                if (mode == 1) { /* replay the map just written */
                    expect(orc_prefill_rows(dt, q, k, v, cu, cu, B, HQ, HKV, D, 0.25, causal, 1, 0.0, 8, 1, rows, nr,
                                            map, stride, o, lse, NULL), 0, "prefill replay");
                    finite(o, (size_t)nr * D, "prefill replay o");
                }
            }
    expect(orc_prefill_rows(0, qf, kf, vf, cu, cu, B, 3, HKV, D, 0.25, 1, 0, 0.0, 8, 1, rows, 1, NULL, 0, o, lse,
                            NULL), -1, "prefill Hq % Hkv");
    /* paged decode: pages of 4 keys, the pool's pages in a scrambled order */
    uint16_t *kc = malloc(2 * POOL * HKV * PAGE * D), *vc = malloc(2 * POOL * HKV * PAGE * D);
    for (int i = 0; i < POOL * HKV * PAGE * D; ++i) {
        kc[i] = to_bf16(urand());
        vc[i] = to_bf16(urand());
    }
    int32_t bt[B * MAXP], sl[B] = {5, 37};
    for (int i = 0; i < B * MAXP; ++i)
        bt[i] = (i * 7) % POOL;
    int32_t drows[2 * B * HQ];
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < HQ; ++h) {
            drows[2 * (b * HQ + h)] = b;
            drows[2 * (b * HQ + h) + 1] = h;
        }
    for (int mode = 0; mode < 3; ++mode) {
        expect(orc_decode_rows(qb, kc, vc, bt, sl, B, HQ, HKV, D, PAGE, MAXP, 0.25, mode, 0.1, 8, 4, drows, B * HQ,
                               NULL, stride, o, lse, mode == 1 ? map : NULL), 0, "decode");
        finite(o, (size_t)B * HQ * D, "decode o");
    }
    expect(orc_decode_qdq_rows(qb, kc, vc, bt, sl, B, HQ, HKV, D, PAGE, MAXP, 0.25, 0.1, 1.0f, 1.0f, drows, B * HQ,
                               NULL, stride, o, lse, map), 0, "decode nvfp4");
    finite(o, (size_t)B * HQ * D, "decode nvfp4 o");
    expect(orc_decode_qdq_rows(qb, kc, vc, bt, sl, B, HQ, HKV, D, PAGE, MAXP, 0.25, 0.1, -1.0f, 1.0f, drows, 1, NULL,
                               0, o, lse, NULL), -1, "decode nvfp4 negative amax");
    sl[1] = MAXP * PAGE + 1;
    expect(orc_decode_rows(qb, kc, vc, bt, sl, B, HQ, HKV, D, PAGE, MAXP, 0.25, 0, 0.0, 8, 1, drows, B * HQ, NULL, 0, o,
                           lse, NULL), -1, "decode seq_len past the table");
    sl[1] = 37;
    /* multi-token decode: 2 and 3 new tokens */
    const int32_t cuq[B + 1] = {0, 2, 5};
    int32_t mrows[2 * 5 * HQ];
    for (int t = 0; t < 5; ++t)
        for (int h = 0; h < HQ; ++h) {
            mrows[2 * (t * HQ + h)] = t;
            mrows[2 * (t * HQ + h) + 1] = h;
        }
    expect(orc_paged_multi_rows(qb, cuq, kc, vc, bt, sl, B, HQ, HKV, D, PAGE, MAXP, 0.25, mrows, 5 * HQ, o, lse), 0,
           "multi");
    finite(o, (size_t)5 * HQ * D, "multi o");
    /* small-seq: 3 sequences of 0, 4 and 16 keys over H = 4 heads */
    const int32_t cus[4] = {0, 0, 4, 20};
    double *w = malloc(sizeof(double) * 3 * HQ * 16), *ls = malloc(sizeof(double) * 3 * HQ);
    int32_t srows[2 * 3 * HQ];
    for (int b = 0; b < 3; ++b)
        for (int h = 0; h < HQ; ++h) {
            srows[2 * (b * HQ + h)] = b;
            srows[2 * (b * HQ + h) + 1] = h;
        }
    expect(orc_smallseq_rows(0, qf, qf, gf, cus, 3, HQ, D, 16, 0.25, srows, 3 * HQ, o, w, ls), 0, "small-seq");
    finite(o, (size_t)3 * HQ * D, "small-seq o");
    finite(w, (size_t)3 * HQ * 16, "small-seq w");
    expect(orc_smallseq_rows(0, qf, qf, gf, cus, 3, HQ, D, 8, 0.25, srows, 3 * HQ, o, w, NULL), -1,
           "small-seq length above max_s");
    float *wf = malloc(sizeof(float) * 3 * HQ * 16);
    for (int i = 0; i < 3 * HQ * 16; ++i)
        wf[i] = (float)w[i];
    double *dq = malloc(sizeof(double) * tq * HQ * D), *dk = malloc(sizeof(double) * tq * HQ * D);
    double *dv = malloc(sizeof(double) * tq * HQ * D);
    expect(orc_smallseq_bwd(0, qf, qf, gf, wf, gf, cus, 3, HQ, D, 16, 0.25, dq, dk, dv), 0, "small-seq backward");
    finite(dq, (size_t)3 * HQ * D, "small-seq dq");
    /* prefill backward, fp32 and bf16, with the exact Dsum and with a stored output */
    for (int dt = 0; dt < 2; ++dt)
        for (int with_o = 0; with_o < 2; ++with_o) {
            const void *q = dt ? (const void *)qb : qf, *k = dt ? (const void *)kb : kf;
            const void *v = dt ? (const void *)vb : vf, *g = dt ? (const void *)qb : gf;
            expect(orc_prefill_bwd(dt, q, k, v, g, with_o ? g : NULL, cu, cu, B, HQ, HKV, D, 0.25, 1, dq, dk, dv), 0,
                   "prefill backward");
            finite(dq, (size_t)tq * HQ * D, "dq");
            finite(dk, (size_t)tq * HKV * D, "dk");
            finite(dv, (size_t)tq * HKV * D, "dv");
        }
    /* rounding helpers */
    float y[64], z[160];
    for (int i = 0; i < 64; ++i)
        y[i] = fabsf(urand()) * 500.0f;
    expect(orc_fp_round(0, y, z, 64), 0, "e2m1");
    expect(orc_fp_round(1, y, z, 64), 0, "e4m3");
    y[3] = -1.0f;
    expect(orc_fp_round(1, y, z, 64), -1, "e4m3 negative");
    expect(orc_nvfp4_qdq(qf, 4, 40, 1.0f, z), 0, "nvfp4 (a partial block of 8)");
    expect(orc_nvfp4_qdq(qf, 1, 16, 0.0f, z), -1, "nvfp4 amax 0");
    free(qf); free(kf); free(vf); free(gf); free(qb); free(kb); free(vb); free(o); free(lse); free(map);
    free(kc); free(vc); free(w); free(ls); free(wf); free(dq); free(dk); free(dv);
    printf("oracle driver: %d failures\n", bad);
    return bad ? 1 : 0;
}
