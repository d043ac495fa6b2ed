/*
 * Drives every entry point of the C oracle (oracle/ep_oracle.c) on small
 * seeded inputs -- node-limited and unlimited routing, LL / HT / per-rank
 * layouts with invalid and repeated routing entries, quantisation, packing,
 * the identity expert, combine (all rows and a subset) and the combine
 * adjoint with and without expert outputs -- so that a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer sees every path.  Test
 * infrastructure: it links the oracle only.  Prints one line, exits 0.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_route(const float *scores, int64_t n_tok, int E, int N, int K, int M, int32_t *topk_idx);
int orc_layout_ll(const int32_t *topk, int S, int T, int K, int E, int slots, int32_t *counts,
                  int32_t *slot_map, int32_t *err);
int orc_layout_ht(const int32_t *topk, int S, int T, int K, int E, int N, int G, int32_t *c1, int32_t *off1,
                  int32_t *node_row, int32_t *c2, int32_t *off2, int32_t *row2, int32_t *err);
int orc_layout_ht_rank(const int32_t *topk, int S, int T, int K, int E, int R, int32_t *c2, int32_t *off2,
                       int32_t *row2, int32_t *err);
void orc_meta_ht_rank(const int32_t *topk, const float *w, int64_t n_tok, int K, int E, int R,
                      const int32_t *row2, int32_t *meta_topk, float *meta_w);
void orc_quantize_row(const uint16_t *x, int H, uint8_t *q, float *scales);
void orc_token_row(const uint16_t *x, int H, int fp8, uint8_t *dst);
void orc_pack_ll(const uint16_t *x, int64_t n_tok, int T, int H, int K, int fp8, const int32_t *slot_map,
                 int64_t msg_bytes, uint8_t *buf);
void orc_pack_ht(const uint16_t *x, const int32_t *topk, const float *w, int64_t i0, int64_t n_tok, int T, int H, int K,
                 int N, int fp8, const int32_t *node_row, const int32_t *row2, uint8_t *stage1,
                 int32_t *meta1_tok, int32_t *meta1_src, int32_t *meta1_topk, float *meta1_w, uint8_t *stage2,
                 int32_t *meta2_src, int32_t *meta2_tok, int32_t *meta2_k);
void orc_dequant_rows(const uint8_t *rows, int64_t row_stride, int64_t n, int H, int fp8, uint16_t *y);
void orc_combine(const uint16_t *Y, int64_t ld_y, const float *w, const int32_t *loc, int K, int H,
                 const int64_t *which, int64_t n_out, uint16_t *out);
void orc_combine_backward(const uint16_t *g, const uint16_t *Y, int64_t ld_y, const float *w,
                          const int32_t *loc, int64_t n, int K, int H, uint16_t *dY, double *dw,
                          double *dw_abs);

enum { S = 3, T = 37, NT = S * T, E = 32, N = 4, G = 2, R = N * G, K = 5, M = 2, H = 256 };

static uint32_t state = 99u;
static uint32_t rnd(void) {
    state = state * 1664525u + 1013904223u;
    return state >> 8;
}

static void *xalloc(size_t n) {
    void *p = calloc(n ? n : 1, 1);
    if (!p) {
        printf("oracle sanitizer run: out of memory\n");
        exit(1);
    }
    return p;
}

static int64_t sum(const int32_t *a, int n) {
    int64_t s = 0;
    for (int i = 0; i < n; ++i) s += a[i];
    return s;
}

int main(void) {
    float *scores = xalloc(sizeof(float) * NT * E);
    uint16_t *x = xalloc(sizeof(uint16_t) * NT * H);
    float *w = xalloc(sizeof(float) * NT * K);
    for (int i = 0; i < NT * E; ++i) scores[i] = (float)(rnd() & 0xFFFF) / 65536.0f;
    for (int i = 0; i < NT * H; ++i) x[i] = (uint16_t)(rnd() & 0xFFFF & ~0x7F80u) | 0x3F00u;  /* finite bf16 */
    for (int i = 0; i < 4; ++i) memset(x + 5 * H + 128 * (i & 1), 0, 128 * sizeof(uint16_t)); /* zero blocks */
    for (int i = 0; i < NT * K; ++i) w[i] = (float)(rnd() % 1000) / 1000.0f;

    int32_t *topk = xalloc(sizeof(int32_t) * NT * K);
    int32_t *topk0 = xalloc(sizeof(int32_t) * NT * K);
    if (orc_route(scores, NT, E, N, K, M, topk) != 0 || orc_route(scores, NT, E, N, K, 0, topk0) != 0) {
        printf("oracle sanitizer run: route failed\n");
        return 1;
    }
    topk[2 * K + 1] = E + 3;          /* out of range */
    topk[7 * K + 3] = topk[7 * K + 0]; /* repeated */
    topk[11 * K + 0] = -1;

    /* LL layout and pack */
    int32_t *counts = xalloc(sizeof(int32_t) * E * S), *slot = xalloc(sizeof(int32_t) * NT * K), err = 0;
    if (orc_layout_ll(topk, S, T, K, E, T, counts, slot, &err) != 0) return 1;
    const int64_t row_fp8 = H + H / 128 * 4, msg = row_fp8 + 16;
    uint8_t *llbuf = xalloc((size_t)E * S * T * msg);
    orc_pack_ll(x, NT, T, H, K, 1, slot, msg, llbuf);
    uint8_t *llbuf16 = xalloc((size_t)E * S * T * (2 * H + 16));
    orc_pack_ll(x, NT, T, H, K, 0, slot, 2 * H + 16, llbuf16);

    /* HT layout and pack */
    int32_t *c1 = xalloc(sizeof(int32_t) * R), *off1 = xalloc(sizeof(int32_t) * R);
    int32_t *node_row = xalloc(sizeof(int32_t) * NT * N);
    int32_t *c2 = xalloc(sizeof(int32_t) * E), *off2 = xalloc(sizeof(int32_t) * E);
    int32_t *row2 = xalloc(sizeof(int32_t) * NT * K);
    if (orc_layout_ht(topk, S, T, K, E, N, G, c1, off1, node_row, c2, off2, row2, &err) != 0) return 1;
    const int64_t rows1 = sum(c1, R), rows2 = sum(c2, E);
    uint8_t *st1 = xalloc((size_t)rows1 * row_fp8), *st2 = xalloc((size_t)rows2 * row_fp8);
    int32_t *m1t = xalloc(sizeof(int32_t) * rows1), *m1s = xalloc(sizeof(int32_t) * rows1);
    int32_t *m1k = xalloc(sizeof(int32_t) * rows1 * K);
    float *m1w = xalloc(sizeof(float) * rows1 * K);
    int32_t *m2s = xalloc(sizeof(int32_t) * rows2), *m2t = xalloc(sizeof(int32_t) * rows2);
    int32_t *m2k = xalloc(sizeof(int32_t) * rows2);
    orc_pack_ht(x, topk, w, 0, NT, T, H, K, N, 1, node_row, row2, st1, m1t, m1s, m1k, m1w, st2, m2s, m2t, m2k);

    /* per-rank stage 2 */
    int32_t *rc2 = xalloc(sizeof(int32_t) * R), *roff2 = xalloc(sizeof(int32_t) * R);
    int32_t *rrow2 = xalloc(sizeof(int32_t) * NT * K);
    if (orc_layout_ht_rank(topk, S, T, K, E, R, rc2, roff2, rrow2, &err) != 0) return 1;
    const int64_t rrows = sum(rc2, R);
    int32_t *mtk = xalloc(sizeof(int32_t) * rrows * K);
    float *mw = xalloc(sizeof(float) * rrows * K);
    orc_meta_ht_rank(topk, w, NT, K, E, R, rrow2, mtk, mw);

    /* quantisation, token rows, identity expert */
    uint8_t *q = xalloc(H);
    float *sc = xalloc(sizeof(float) * H / 128);
    uint8_t *tr = xalloc(2 * H);
    orc_quantize_row(x, H, q, sc);
    orc_token_row(x, H, 1, tr);
    orc_token_row(x, H, 0, tr);
    uint16_t *y = xalloc(sizeof(uint16_t) * rows2 * H);
    orc_dequant_rows(st2, row_fp8, rows2, H, 1, y);
    uint16_t *y16 = xalloc(sizeof(uint16_t) * E * S * T * H);
    orc_dequant_rows(llbuf16, 2 * H + 16, (int64_t)E * S * T, H, 0, y16);

    /* combine: every token, then a subset */
    uint16_t *out = xalloc(sizeof(uint16_t) * NT * H);
    orc_combine(y, H, w, row2, K, H, NULL, NT, out);
    int64_t which[3] = {0, NT / 2, NT - 1};
    orc_combine(y, H, w, row2, K, H, which, 3, out);

    /* combine adjoint, with and without expert outputs */
    uint16_t *dY = xalloc(sizeof(uint16_t) * rows2 * H);
    double *dw = xalloc(sizeof(double) * NT * K), *dwa = xalloc(sizeof(double) * NT * K);
    orc_combine_backward(x, y, H, w, row2, NT, K, H, dY, dw, dwa);
    orc_combine_backward(x, NULL, H, w, row2, NT, K, H, dY, dw, dwa);

    printf("oracle sanitizer run: OK (%lld stage-1 rows, %lld stage-2 rows, %lld per-rank rows, error bits %d)\n",
           (long long)rows1, (long long)rows2, (long long)rrows, err);
    free(scores); free(x); free(w); free(topk); free(topk0); free(counts); free(slot); free(llbuf);
    free(llbuf16); free(c1); free(off1); free(node_row); free(c2); free(off2); free(row2); free(st1);
    free(st2); free(m1t); free(m1s); free(m1k); free(m1w); free(m2s); free(m2t); free(m2k); free(rc2);
    free(roff2); free(rrow2); free(mtk); free(mw); free(q); free(sc); free(tr); free(y); free(y16);
    free(out); free(dY); free(dw); free(dwa);
    return 0;
}
