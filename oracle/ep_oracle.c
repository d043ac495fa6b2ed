/*
 * ep_oracle.c -- plain, slow, single-threaded CPU oracle for MoE
 * expert-parallel dispatch and combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant generator with the HIP library; the two are fed
 * the same seeded inputs and their outputs are compared.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -shared -fPIC ep_oracle.c -lm
 * (no fast-math: every float operation below is one IEEE binary32 operation,
 * round to nearest even, in the order written).
 *
 * Sources (page titles; sections):
 *  [DeepEP] "NVSHMEM and DeepEP: GPU-initiated communication"
 *      - high-throughput mode: node-limited routing (each node scored by the
 *        sum of its two best expert scores, keep the best 4 nodes, pick the
 *        top-8 experts inside them), one copy per destination node sent to
 *        the same-position ("same rail") GPU, then an intra-node forward;
 *        FP8 payload with one fp32 scale per 128 elements (7168 + 56*4 B).
 *      - low-latency mode: fixed slots per (local expert, source rank),
 *        message = FP8 data + scales + a small 16-byte header (7408 B).
 *      - combine returns the weighted sum of expert outputs in BF16.
 *  [NCCL-EP] "NCCL EP paper notes" (lpnh.cn)
 *      - tensor layouts: tokens [num_tokens x hidden], routing
 *        [num_tokens x top_k]; LL output 3-D expert-major, HT output 2-D with
 *        per-expert counts marking boundaries, deterministic order.
 *      - message sizes: dispatch 14352 B (BF16) / 7408 B (FP8), combine
 *        14336 B (BF16) for hidden 7168.
 *
 * Where the pages leave a step open, the reading taken here is stated at the
 * function that implements it.
 *
 * Parity pins: every function here is checked by the CPU test-suite against
 * values the pages print, closed forms, library routines (torch casts, numpy
 * sorts) or brute force; none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Device-error bits reported for invalid routing entries (same meaning as the
 * library's public error word, restated here; no shared header). */
#define ORC_ERR_BAD_INDEX 1
#define ORC_ERR_DUP_INDEX 2

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

/* bfloat16 -> float: the bf16 bits are the high half of the binary32 word. */
float orc_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* float -> bfloat16, round to nearest, ties to even, by definition: the two
 * bf16 neighbours of f are its truncation and the next value away from zero;
 * pick the nearer, and on an exact tie the one whose last mantissa bit is 0.
 * Magnitudes from the largest finite bf16 plus half its spacing upwards
 * round to infinity (IEEE 754 overflow); infinities stay infinite.  NaN is
 * outside the contract and gives the canonical quiet NaN 0x7FC0. */
uint16_t orc_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if (f != f) return 0x7FC0;              /* NaN: the canonical quiet NaN */
    uint32_t lo = u & 0xFFFF0000u;          /* truncation toward zero      */
    uint32_t hi = lo + 0x10000u;            /* next bf16 away from zero    */
    if (lo == u) return (uint16_t)(lo >> 16);
    float flo;
    memcpy(&flo, &lo, 4);
    /* Rounding works as if the exponent range were unbounded: above the
     * largest finite bf16 the next candidate is 2^128, and choosing it is an
     * overflow to infinity (hi is then the bit pattern of +-inf). */
    double hi_mag;
    if ((hi & 0x7F800000u) == 0x7F800000u) {
        hi_mag = ldexp(1.0, 128);
    } else {
        float fhi;
        memcpy(&fhi, &hi, 4);
        hi_mag = fabs((double)fhi);
    }
    double a = fabs((double)f), dlo = a - fabs((double)flo), dhi = hi_mag - a;
    if (dlo < dhi) return (uint16_t)(lo >> 16);
    if (dhi < dlo) return (uint16_t)(hi >> 16);
    return (uint16_t)(((lo >> 16) & 1u) ? (hi >> 16) : (lo >> 16));
}

/* Value of a non-negative OCP FP8 E4M3 ("E4M3FN") code 0..126: 4 exponent
 * bits with bias 7, 3 mantissa bits, subnormals at exponent field 0, no
 * infinities, 0x7F is NaN.  Largest finite value 0x7E = 448. */
double orc_e4m3_value(int code)
{
    int e = (code >> 3) & 15, m = code & 7;
    if (e == 0) return ldexp((double)m, -9);            /* m/8 * 2^(1-7) */
    return ldexp(1.0 + m / 8.0, e - 7);
}

/* float -> E4M3: nearest representable value, ties to the even code, finite
 * magnitudes beyond 448 saturate to +-448, the sign of zero is kept.
 * The bracketing pair is found by bisection over the monotone code table;
 * the decision compares |v| with the exact midpoint (exact in double).
 * A NaN gets the format's NaN code S.1111.111 (its sign bit as it comes). */
uint8_t orc_e4m3_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v)) return sign | 0x7F;
    double a = fabs((double)v);
    if (a >= 448.0) return sign | 0x7E;
    int lo = 0, hi = 126;              /* value(lo) <= a < value(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (orc_e4m3_value(mid) <= a) lo = mid; else hi = mid;
    }
    double half = (orc_e4m3_value(lo) + orc_e4m3_value(hi)) / 2.0;
    int code;
    if (a < half) code = lo;
    else if (a > half) code = hi;
    else code = (lo & 1) ? hi : lo;
    return sign | (uint8_t)code;
}

float orc_e4m3_decode(uint8_t q)
{
    double v = orc_e4m3_value(q & 0x7F);
    return (float)((q & 0x80) ? -v : v);
}

/* ------------------------------------------------------------------------ */
/* A1  Node-limited top-k routing  [DeepEP, high-throughput mode]           */
/* ------------------------------------------------------------------------ */
/*
 * scores: float32 [n_tok, E].  Experts are laid out in contiguous blocks:
 * expert e lives on GPU e / (E/R) and node (e / (E/R)) / G, so node n owns
 * experts [n*E/N, (n+1)*E/N).
 *
 * If 0 < M < N: each node's score is the float32 sum, largest first, of its
 * J = ceil(K/M) largest expert scores (J = 2 at K = 8, M = 4, the page's
 * "top-2 per node"); the M best nodes are kept, ties going to the lower node
 * index.  Otherwise every expert is a candidate.  The K best candidates are
 * written in descending score order, ties going to the lower expert index.
 * Both selections are repeated arg-max, the plainest form of "top".
 */
int orc_route(const float *scores, int64_t n_tok, int E, int N, int K, int M,
              int32_t *topk_idx)
{
    if (E <= 0 || N <= 0 || E % N != 0 || K <= 0 || K > E) return -1;
    const int P = E / N;
    const int limited = (M > 0 && M < N);
    const int J = limited ? (K + M - 1) / M : 0;
    if (limited && J > P) return -1;
    unsigned char *allowed = malloc((size_t)E);
    unsigned char *taken = malloc((size_t)E);
    unsigned char *node_kept = malloc((size_t)N);
    unsigned char *used = malloc((size_t)P);
    float *node_score = malloc(sizeof(float) * (size_t)N);
    if (!allowed || !taken || !node_kept || !used || !node_score) return -2;

    for (int64_t t = 0; t < n_tok; ++t) {
        const float *s = scores + t * (int64_t)E;
        if (limited) {
            for (int n = 0; n < N; ++n) {
                /* J largest of the node's P scores, largest first. */
                memset(used, 0, (size_t)P);
                float acc = 0.0f;
                for (int j = 0; j < J; ++j) {
                    int best = -1;
                    for (int p = 0; p < P; ++p)
                        if (!used[p] && (best < 0 || s[n * P + p] > s[n * P + best])) best = p;
                    used[best] = 1;
                    acc = (j == 0) ? s[n * P + best] : acc + s[n * P + best];
                }
                node_score[n] = acc;
            }
            memset(node_kept, 0, (size_t)N);
            for (int m = 0; m < M; ++m) {
                int best = -1;
                for (int n = 0; n < N; ++n)
                    if (!node_kept[n] && (best < 0 || node_score[n] > node_score[best])) best = n;
                node_kept[best] = 1;
            }
            for (int e = 0; e < E; ++e) allowed[e] = node_kept[e / P];
        } else {
            memset(allowed, 1, (size_t)E);
        }
        memset(taken, 0, (size_t)E);
        for (int k = 0; k < K; ++k) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (allowed[e] && !taken[e] && (best < 0 || s[e] > s[best])) best = e;
            taken[best] = 1;
            topk_idx[t * K + k] = best;
        }
    }
    free(allowed); free(taken); free(node_kept); free(used); free(node_score);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Validity of routing entries (caller-supplied topk_idx)                    */
/* ------------------------------------------------------------------------ */
/* An entry is used only if 0 <= e < E and it does not repeat an earlier entry
 * of the same token; anything else is reported and then ignored (no slot, no
 * row, no contribution to the combine). */
static int entry_valid(const int32_t *row, int k, int E, int32_t *err)
{
    int32_t e = row[k];
    if (e < 0 || e >= E) { *err |= ORC_ERR_BAD_INDEX; return 0; }
    for (int j = 0; j < k; ++j)
        if (row[j] == e) { *err |= ORC_ERR_DUP_INDEX; return 0; }
    return 1;
}

/* ------------------------------------------------------------------------ */
/* A2 (LL)  Fixed slots per (expert, source rank)  [DeepEP, low-latency]     */
/* ------------------------------------------------------------------------ */
/*
 * Tokens are [S sources x T tokens]; token i = s*T + t.  Each expert reserves
 * `slots` slots for every source rank, so the whole receive space is the
 * expert-major array [E][S][slots] (rank r's partition is experts
 * r*E/R .. r*E/R + E/R - 1, i.e. a contiguous [E/R][S][slots] block).
 * Reading taken (the page leaves slot order open): a (token, k) entry gets
 * slot = number of earlier entries of the same source that chose the same
 * expert, scanning tokens ascending then k ascending.
 * Outputs: counts[e*S + s]; slot_map[i*K + k] = (e*S + s)*slots + slot, or -1.
 * Returns 0, or -3 if some (source, expert) needs more than `slots` slots.
 */
int orc_layout_ll(const int32_t *topk, int S, int T, int K, int E, int slots,
                  int32_t *counts, int32_t *slot_map, int32_t *err)
{
    memset(counts, 0, sizeof(int32_t) * (size_t)E * (size_t)S);
    for (int s = 0; s < S; ++s)
        for (int t = 0; t < T; ++t) {
            const int64_t i = (int64_t)s * T + t;
            const int32_t *row = topk + i * K;
            for (int k = 0; k < K; ++k) {
                if (!entry_valid(row, k, E, err)) { slot_map[i * K + k] = -1; continue; }
                const int e = row[k];
                const int slot = counts[e * S + s]++;
                if (slot >= slots) return -3;
                slot_map[i * K + k] = (int32_t)(((int64_t)e * S + s) * slots + slot);
            }
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* A2 (HT)  Node-dedup stage-1 rows and expert-grouped stage-2 rows          */
/* ------------------------------------------------------------------------ */
/*
 * Stage 1 (hop 1): one row per (token, distinct destination node n).  The
 * row goes to the same-position GPU on node n: rank d = n*G + (s mod G).
 * Reading taken: the source's own node is also given a row (in its own
 * same-position rank, i.e. itself); the page's traffic metric counts only
 * the other nodes.  Rows of all ranks sit in one array grouped by d
 * ascending (off1 = exclusive scan of c1), ordered inside a rank by
 * (source, token) ascending -- the deterministic order of the HT layout.
 *   c1[d], off1[d]; node_row[i*N + n] = global stage-1 row, or -1.
 *
 * Stage 2 (hop 2, intra-node forward): one row per valid (token, k), at the
 * GPU owning expert e, grouped by expert; since rank r owns a contiguous
 * block of experts, grouping by (rank, local expert) is grouping by e.
 * off2 = exclusive scan of c2 over e; inside an expert rows follow
 * (source, token) ascending.
 *   c2[e], off2[e]; row2[i*K + k] = global stage-2 row, or -1.
 */
int orc_layout_ht(const int32_t *topk, int S, int T, int K, int E, int N, int G,
                  int32_t *c1, int32_t *off1, int32_t *node_row,
                  int32_t *c2, int32_t *off2, int32_t *row2, int32_t *err)
{
    const int R = N * G;
    if (E % R != 0) return -1;
    const int per_node = E / N;
    const int64_t n_tok = (int64_t)S * T;
    unsigned char *hit = malloc((size_t)N);
    int32_t *run1 = calloc((size_t)R, sizeof(int32_t));
    int32_t *run2 = calloc((size_t)E, sizeof(int32_t));
    if (!hit || !run1 || !run2) return -2;
    memset(c1, 0, sizeof(int32_t) * (size_t)R);
    memset(c2, 0, sizeof(int32_t) * (size_t)E);

    /* Counting pass. */
    for (int64_t i = 0; i < n_tok; ++i) {
        const int s = (int)(i / T);
        const int32_t *row = topk + i * K;
        memset(hit, 0, (size_t)N);
        int32_t dummy = 0;
        for (int k = 0; k < K; ++k) {
            if (!entry_valid(row, k, E, &dummy)) continue;
            hit[row[k] / per_node] = 1;
            c2[row[k]]++;
        }
        for (int n = 0; n < N; ++n)
            if (hit[n]) c1[n * G + s % G]++;
    }
    /* Exclusive scans. */
    int32_t acc = 0;
    for (int d = 0; d < R; ++d) { off1[d] = acc; acc += c1[d]; }
    acc = 0;
    for (int e = 0; e < E; ++e) { off2[e] = acc; acc += c2[e]; }

    /* Assignment pass, in (source, token, k) order. */
    for (int64_t i = 0; i < n_tok; ++i) {
        const int s = (int)(i / T);
        const int32_t *row = topk + i * K;
        memset(hit, 0, (size_t)N);
        for (int k = 0; k < K; ++k) {
            if (!entry_valid(row, k, E, err)) { row2[i * K + k] = -1; continue; }
            const int e = row[k];
            hit[e / per_node] = 1;
            row2[i * K + k] = off2[e] + run2[e]++;
        }
        for (int n = 0; n < N; ++n) {
            if (!hit[n]) { node_row[i * N + n] = -1; continue; }
            const int d = n * G + s % G;
            node_row[i * N + n] = off1[d] + run1[d]++;
        }
    }
    free(hit); free(run1); free(run2);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* A2 (HT), stage 2 per destination rank  [DeepEP, high-throughput mode]     */
/* ------------------------------------------------------------------------ */
/*
 * The alternative the page's traffic study compares: one copy per
 * destination GPU.  Stage 2 gets one row per (token, distinct rank
 * r = e / (E/R) among its valid entries), grouped by rank ascending and
 * ordered (source, token) inside a rank.  Reading taken: the row belongs to
 * the token's first entry (k order) on that rank; the token's other entries
 * on the same rank get -1, so every row appears once in a token's map.
 *   c2[r], off2[r] (R entries); row2[i*K + k] = global stage-2 row, or -1.
 * Stage 1 is unchanged (orc_layout_ht).
 */
int orc_layout_ht_rank(const int32_t *topk, int S, int T, int K, int E, int R,
                       int32_t *c2, int32_t *off2, int32_t *row2, int32_t *err)
{
    if (R <= 0 || E % R != 0) return -1;
    const int L = E / R;
    const int64_t n_tok = (int64_t)S * T;
    unsigned char *hit = malloc((size_t)R);
    int32_t *run = calloc((size_t)R, sizeof(int32_t));
    if (!hit || !run) return -2;
    memset(c2, 0, sizeof(int32_t) * (size_t)R);
    for (int64_t i = 0; i < n_tok; ++i) {
        const int32_t *row = topk + i * K;
        memset(hit, 0, (size_t)R);
        int32_t dummy = 0;
        for (int k = 0; k < K; ++k) {
            if (!entry_valid(row, k, E, &dummy)) continue;
            const int r = row[k] / L;
            if (!hit[r]) { hit[r] = 1; c2[r]++; }
        }
    }
    int32_t acc = 0;
    for (int r = 0; r < R; ++r) { off2[r] = acc; acc += c2[r]; }
    for (int64_t i = 0; i < n_tok; ++i) {
        const int32_t *row = topk + i * K;
        memset(hit, 0, (size_t)R);
        for (int k = 0; k < K; ++k) {
            row2[i * K + k] = -1;
            if (!entry_valid(row, k, E, err)) continue;
            const int r = row[k] / L;
            if (hit[r]) continue;
            hit[r] = 1;
            row2[i * K + k] = off2[r] + run[r]++;
        }
    }
    free(hit); free(run);
    return 0;
}

/* What a rank receives with each per-rank stage-2 row (DeepEP's received
 * top-k form): for the token's entry kk, its local expert index
 * e - r*(E/R) if it is a valid entry on the row's rank r, else -1; and its
 * weight, else 0 (weights omitted when w is NULL).  Rows are those of
 * row2 from orc_layout_ht_rank. */
void orc_meta_ht_rank(const int32_t *topk, const float *w, int64_t n_tok, int K, int E,
                      int R, const int32_t *row2, int32_t *meta_topk, float *meta_w)
{
    const int L = E / R;
    for (int64_t i = 0; i < n_tok; ++i) {
        const int32_t *row = topk + i * K;
        for (int k = 0; k < K; ++k) {
            const int32_t dst = row2[i * K + k];
            if (dst < 0) continue;
            const int r = row[k] / L;
            for (int kk = 0; kk < K; ++kk) {
                int32_t dummy = 0;
                const int here = entry_valid(row, kk, E, &dummy) && row[kk] / L == r;
                meta_topk[(int64_t)dst * K + kk] = here ? row[kk] - r * L : -1;
                if (meta_w) meta_w[(int64_t)dst * K + kk] = here ? w[i * K + kk] : 0.0f;
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* A3  FP8 E4M3 quantisation, one fp32 scale per 128 elements  [DeepEP]      */
/* ------------------------------------------------------------------------ */
/*
 * For each block of 128 consecutive elements of a row:
 *   amax  = max |x|                      (x = the bf16 value, exact in fp32)
 *   scale = amax / 448   (fp32 division) -- the stored scale; dequantised
 *                                            value = decode(q) * scale
 *   q     = E4M3(x / scale)  (fp32 division, then nearest-even E4M3)
 * A block whose amax is 0 stores scale 0 and all codes 0x00.
 * Readings taken: the stored scale is amax/448 (not its inverse); the code
 * is computed by dividing by the stored scale.
 */
void orc_quantize_row(const uint16_t *x, int H, uint8_t *q, float *scales)
{
    for (int b = 0; b < H / 128; ++b) {
        float amax = 0.0f;
        for (int j = 0; j < 128; ++j) {
            float a = fabsf(orc_bf16_to_f32(x[b * 128 + j]));
            if (a > amax) amax = a;
        }
        if (amax == 0.0f) {
            scales[b] = 0.0f;
            memset(q + b * 128, 0, 128);
            continue;
        }
        float scale = amax / 448.0f;
        scales[b] = scale;
        for (int j = 0; j < 128; ++j) {
            float v = orc_bf16_to_f32(x[b * 128 + j]) / scale;
            q[b * 128 + j] = orc_e4m3_encode(v);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* A4-A6  Row / message images                                               */
/* ------------------------------------------------------------------------ */
/*
 * FP8 row  = [q: H bytes][scales: H/128 fp32, little-endian]  (7392 B @7168)
 * BF16 row = [x: H bf16]                                       (14336 B)
 * LL message = row + 16-byte header {src_token, src_rank, k, 0} as int32
 *            (7408 B FP8 / 14352 B BF16 at hidden 7168).
 * Reading taken: header after the payload and its four int32 fields as
 * above (the pages only say "a small header" of 16 bytes).
 */
/* The row image of one token (what both stage-1 and stage-2 rows hold). */
void orc_token_row(const uint16_t *x, int H, int fp8, uint8_t *dst)
{
    /* scales are written through a bounce buffer: dst + H may be unaligned */
    if (fp8) {
        float sc[1024];
        orc_quantize_row(x, H, dst, sc);
        memcpy(dst + H, sc, sizeof(float) * (size_t)(H / 128));
    } else {
        memcpy(dst, x, (size_t)H * 2);
    }
}

/* LL pack: every valid (i, k) writes the message into slot slot_map[i*K+k]
 * of the [E][S][slots] receive space (msg_bytes apart). */
void orc_pack_ll(const uint16_t *x, int64_t n_tok, int T, int H, int K, int fp8,
                 const int32_t *slot_map, int64_t msg_bytes, uint8_t *buf)
{
    const int64_t row_bytes = fp8 ? (int64_t)H + (H / 128) * 4 : (int64_t)H * 2;
    uint8_t *img = malloc((size_t)row_bytes);
    for (int64_t i = 0; i < n_tok; ++i) {
        orc_token_row(x + i * H, H, fp8, img);
        for (int k = 0; k < K; ++k) {
            int32_t slot = slot_map[i * K + k];
            if (slot < 0) continue;
            uint8_t *m = buf + (int64_t)slot * msg_bytes;
            memcpy(m, img, (size_t)row_bytes);
            int32_t hdr[4] = {(int32_t)(i % T), (int32_t)(i / T), k, 0};
            memcpy(m + row_bytes, hdr, 16);
        }
    }
    free(img);
}

/* HT pack: stage-1 rows (one per destination node) and stage-2 rows (one per
 * valid k), with their structure-of-arrays metadata:
 *   stage 1: meta1_tok[row]=t, meta1_src[row]=s, meta1_topk[row*K..]=topk_idx
 *            of the token, meta1_w[row*K..]=topk_weights (if w != NULL)
 *   stage 2: meta2_src[row]=s, meta2_tok[row]=t, meta2_k[row]=k
 * The n_tok tokens given are tokens i0 .. i0+n_tok-1 of the batch (token
 * i = s*T + t); x, topk, w, node_row and row2 start at token i0, the row
 * arrays are the whole batch's.
 * With both stage pointers NULL only the metadata is produced (x unused). */
void orc_pack_ht(const uint16_t *x, const int32_t *topk, const float *w,
                 int64_t i0, int64_t n_tok, int T, int H, int K, int N, int fp8,
                 const int32_t *node_row, const int32_t *row2,
                 uint8_t *stage1, int32_t *meta1_tok, int32_t *meta1_src,
                 int32_t *meta1_topk, float *meta1_w,
                 uint8_t *stage2, int32_t *meta2_src, int32_t *meta2_tok,
                 int32_t *meta2_k)
{
    const int64_t row_bytes = fp8 ? (int64_t)H + (H / 128) * 4 : (int64_t)H * 2;
    uint8_t *img = malloc((size_t)row_bytes);
    for (int64_t i = 0; i < n_tok; ++i) {
        const int32_t t = (int32_t)((i0 + i) % T), s = (int32_t)((i0 + i) / T);
        if (stage1 || stage2) orc_token_row(x + i * H, H, fp8, img);
        for (int n = 0; n < N; ++n) {
            int32_t r = node_row[i * N + n];
            if (r < 0) continue;
            if (stage1) memcpy(stage1 + (int64_t)r * row_bytes, img, (size_t)row_bytes);
            meta1_tok[r] = t;
            meta1_src[r] = s;
            for (int k = 0; k < K; ++k) {
                meta1_topk[(int64_t)r * K + k] = topk[i * K + k];
                if (w) meta1_w[(int64_t)r * K + k] = w[i * K + k];
            }
        }
        for (int k = 0; k < K; ++k) {
            int32_t r = row2[i * K + k];
            if (r < 0) continue;
            if (stage2) memcpy(stage2 + (int64_t)r * row_bytes, img, (size_t)row_bytes);
            meta2_src[r] = s;
            meta2_tok[r] = t;
            meta2_k[r] = k;
        }
    }
    free(img);
}

/* ------------------------------------------------------------------------ */
/* Identity expert (test aid): FP8 row -> BF16 row                           */
/* ------------------------------------------------------------------------ */
/* y = bf16(decode(q) * scale) with one fp32 multiply; a BF16 row is copied. */
void orc_dequant_rows(const uint8_t *rows, int64_t row_stride, int64_t n, int H,
                      int fp8, uint16_t *y)
{
    for (int64_t r = 0; r < n; ++r) {
        const uint8_t *src = rows + r * row_stride;
        if (!fp8) { memcpy(y + r * H, src, (size_t)H * 2); continue; }
        for (int h = 0; h < H; ++h) {
            float sc;
            memcpy(&sc, src + H + 4 * (h / 128), 4);
            y[r * H + h] = orc_f32_to_bf16(orc_e4m3_decode(src[h]) * sc);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* A7  Combine: weighted top-k gather-reduce  [DeepEP; NCCL-EP combine]      */
/* ------------------------------------------------------------------------ */
/*
 * out[i][h] = bf16( sum_k w[i][k] * Y[loc[i][k]][h] ), accumulated in fp32
 * as a chain of fused multiply-adds in k order starting from +0.  Entries
 * with loc < 0 (invalid routing entries) contribute nothing.
 * Reading taken: the accumulation order is k = 0..K-1 and each step is one
 * fused multiply-add (fmaf), so the result is defined to the last bit.
 * Only tokens listed in `which` (or all if which == NULL) are computed;
 * out has one row per listed token.
 */
void orc_combine(const uint16_t *Y, int64_t ld_y, const float *w,
                 const int32_t *loc, int K, int H, const int64_t *which,
                 int64_t n_out, uint16_t *out)
{
    for (int64_t o = 0; o < n_out; ++o) {
        const int64_t i = which ? which[o] : o;
        for (int h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
                const int32_t r = loc[i * K + k];
                if (r < 0) continue;
                acc = fmaf(w[i * K + k], orc_bf16_to_f32(Y[(int64_t)r * ld_y + h]), acc);
            }
            out[o * H + h] = orc_f32_to_bf16(acc);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Backward pass: reuse of the forward handle                                */
/* ------------------------------------------------------------------------ */
/* [NCCL-EP] usage (training in HT mode): the backward pass walks the layers
 * in reverse and reuses each layer's handle -- the loss gradient is
 * dispatched to the experts, the experts run their backward, and the
 * experts' gradients are combined back to the tokens.  The pages give no
 * arithmetic for it; the reading here is the adjoint of the forward maps,
 * with the FP8 quantisation of the forward dispatch taken as the identity
 * (straight-through):
 *
 * combine forward   out[t] = sum_k w[t,k] * Y[loc(t,k)]
 *   backward        dY[loc(t,k)][h] = bf16( w[t,k] * g[t][h] )  (one fp32
 *                                     multiply, then bf16 nearest-even)
 *                   dw[t,k] = sum_h g[t][h] * Y[loc(t,k)][h]
 * dw is returned in fp64 (products of two bf16 values are exact in fp64),
 * with sum_h |g * Y| beside it for the fp32 error bound of a device sum.
 * Entries with loc < 0 write no row and get dw = 0.  dY uses Y's row stride.
 *
 * dispatch forward  rows[loc(t,k)] = x[t]
 *   backward        dx[t] = bf16( sum over valid k, in k order, from +0 )
 *                   of dRows[loc(t,k)] -- orc_combine with unit weights
 *                   (fma(1, y, acc) rounds exactly as y + acc). */
void orc_combine_backward(const uint16_t *g, const uint16_t *Y, int64_t ld_y,
                          const float *w, const int32_t *loc, int64_t n, int K,
                          int H, uint16_t *dY, double *dw, double *dw_abs)
{
    for (int64_t t = 0; t < n; ++t) {
        for (int k = 0; k < K; ++k) {
            const int32_t r = loc[t * K + k];
            double s = 0.0, a = 0.0;
            if (r >= 0) {
                for (int h = 0; h < H; ++h) {
                    const float gv = orc_bf16_to_f32(g[t * H + h]);
                    const float prod = w[t * K + k] * gv;
                    dY[(int64_t)r * ld_y + h] = orc_f32_to_bf16(prod);
                    if (Y) {
                        const double p = (double)gv * (double)orc_bf16_to_f32(Y[(int64_t)r * ld_y + h]);
                        s += p;
                        a += fabs(p);
                    }
                }
            }
            if (dw) dw[t * K + k] = s;
            if (dw_abs) dw_abs[t * K + k] = a;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Array forms of the scalar conversions (for the pins)                      */
/* ------------------------------------------------------------------------ */
void orc_f32_to_bf16_n(const float *x, int64_t n, uint16_t *y)
{
    for (int64_t i = 0; i < n; ++i) y[i] = orc_f32_to_bf16(x[i]);
}

void orc_e4m3_encode_n(const float *x, int64_t n, uint8_t *y)
{
    for (int64_t i = 0; i < n; ++i) y[i] = orc_e4m3_encode(x[i]);
}
