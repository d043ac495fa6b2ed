/*
 * A plain C99 client of libep: the HT hot path driven through include/ep.h
 * alone (no Python, no torch), with HIP used only for device memory and the
 * stream.
 *
 *   route -> handle -> FP8 dispatch (stage-1 and stage-2 rows) -> identity
 *   expert on the stage-2 rows -> combine with weights 1/2, 1/2
 *
 * The tokens are chosen so that every step is exact: each 128-element block
 * holds one +-448 and otherwise integers in [-16, 16], so its scale is
 * 448/448 = 1 and every value is an E4M3 code ("NVSHMEM and DeepEP":
 * one fp32 scale per 128 elements); the identity expert returns the token;
 * and 1/2 x + 1/2 x = x in fp32.  The combined output must therefore equal
 * the input bit for bit.  The program also checks the receive count, the
 * device error word and a few rejected calls, prints one line and exits 0
 * on success, 1 on any failure.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "ep.h"

enum { N = 2, G = 2, E = 16, K = 2, H = 512, S = 2, T = 64, NTOK = S * T };

#define CHECK_HIP(call)                                                        \
    do {                                                                       \
        hipError_t e_ = (call);                                                \
        if (e_ != hipSuccess) {                                                \
            printf("ep_c_client: FAIL %s -> %s\n", #call, hipGetErrorString(e_)); \
            exit(1);                                                           \
        }                                                                      \
    } while (0)

#define CHECK_EP(call)                                                         \
    do {                                                                       \
        ep_status_t s_ = (call);                                               \
        if (s_ != EP_OK) {                                                     \
            printf("ep_c_client: FAIL %s -> %s (hip %d)\n", #call,             \
                   ep_status_string(s_), ep_last_hip_error());                 \
            exit(1);                                                           \
        }                                                                      \
    } while (0)

static uint32_t lcg_state = 12345u;
static uint32_t lcg(void) {
    lcg_state = lcg_state * 1664525u + 1013904223u;
    return lcg_state >> 8;
}

/* bf16 bits of a float that bf16 holds exactly (the upper half). */
static uint16_t bf16_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

static ep_tensor_t tensor2d(void *data, int32_t dtype, int64_t rows, int64_t cols, int32_t tag) {
    ep_tensor_t t;
    memset(&t, 0, sizeof t);
    t.data = data;
    t.dtype = dtype;
    t.ndim = 2;
    t.sizes[0] = rows;
    t.sizes[1] = cols;
    t.strides[0] = cols;
    t.strides[1] = 1;
    t.tag = tag;
    return t;
}

int main(void) {
    /* host inputs */
    static float scores[NTOK * E];
    static uint16_t x[NTOK * H];
    static float weights[NTOK * K];
    static uint16_t out[NTOK * H];
    for (int i = 0; i < NTOK * E; ++i) scores[i] = (float)(lcg() & 0xFFFF) / 65536.0f;
    for (int i = 0; i < NTOK; ++i) {
        for (int b = 0; b < H / 128; ++b) {
            const int big = (int)(lcg() % 128);
            for (int j = 0; j < 128; ++j) {
                float v = (float)((int)(lcg() % 33) - 16);
                if (j == big) v = (lcg() & 1) ? 448.0f : -448.0f;
                x[i * H + b * 128 + j] = bf16_bits(v);
            }
        }
        for (int k = 0; k < K; ++k) weights[i * K + k] = 0.5f;
    }

    hipStream_t stream;
    CHECK_HIP(hipStreamCreate(&stream));
    float *d_scores, *d_w;
    uint16_t *d_x, *d_out, *d_y;
    int32_t *d_topk, *d_counts;
    CHECK_HIP(hipMalloc((void **)&d_scores, sizeof scores));
    CHECK_HIP(hipMalloc((void **)&d_w, sizeof weights));
    CHECK_HIP(hipMalloc((void **)&d_x, sizeof x));
    CHECK_HIP(hipMalloc((void **)&d_out, sizeof out));
    CHECK_HIP(hipMalloc((void **)&d_topk, NTOK * K * sizeof(int32_t)));
    CHECK_HIP(hipMalloc((void **)&d_counts, E * sizeof(int32_t)));
    CHECK_HIP(hipMalloc((void **)&d_y, (size_t)NTOK * K * H * sizeof(uint16_t)));
    CHECK_HIP(hipMemcpy(d_scores, scores, sizeof scores, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_w, weights, sizeof weights, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_x, x, sizeof x, hipMemcpyHostToDevice));

    ep_config_t cfg;
    memset(&cfg, 0, sizeof cfg);
    cfg.mode = EP_MODE_HT;
    cfg.num_nodes = N;
    cfg.ranks_per_node = G;
    cfg.num_experts = E;
    cfg.top_k = K;
    cfg.max_nodes_per_token = 0;
    cfg.hidden = H;
    cfg.max_tokens_per_rank = T;
    cfg.num_src_ranks = S;
    cfg.payload = EP_DTYPE_FP8_E4M3;
    ep_group_t g;
    CHECK_EP(ep_create_group(&cfg, stream, &g));

    ep_tensor_t t_scores = tensor2d(d_scores, EP_DTYPE_F32, NTOK, E, EP_TAG_TOKENS);
    ep_tensor_t t_topk = tensor2d(d_topk, EP_DTYPE_I32, NTOK, K, EP_TAG_TOPK_IDX);
    ep_tensor_t t_x = tensor2d(d_x, EP_DTYPE_BF16, NTOK, H, EP_TAG_TOKENS);
    ep_tensor_t t_w = tensor2d(d_w, EP_DTYPE_F32, NTOK, K, EP_TAG_TOPK_WEIGHTS);
    ep_tensor_t t_out = tensor2d(d_out, EP_DTYPE_BF16, NTOK, H, EP_TAG_TOKENS);
    ep_tensor_t t_counts;
    memset(&t_counts, 0, sizeof t_counts);
    t_counts.data = d_counts;
    t_counts.dtype = EP_DTYPE_I32;
    t_counts.ndim = 1;
    t_counts.sizes[0] = E;
    t_counts.strides[0] = 1;
    t_counts.tag = EP_TAG_TOKENS_PER_EXPERT;

    /* rejected calls enqueue nothing */
    ep_handle_t h;
    if (ep_create_handle(g, NULL, stream, &h) != EP_ERR_INVALID_ARGUMENT) {
        printf("ep_c_client: FAIL a NULL topk_idx was accepted\n");
        return 1;
    }
    ep_tensor_t t_big = tensor2d(d_topk, EP_DTYPE_I32, S * (T + 1), K, EP_TAG_TOPK_IDX);
    if (ep_create_handle(g, &t_big, stream, &h) != EP_ERR_CAPACITY) {
        printf("ep_c_client: FAIL more tokens than max_tokens_per_rank were accepted\n");
        return 1;
    }
    if (strcmp(ep_status_string(EP_ERR_CAPACITY), "EP_ERR_CAPACITY") != 0) {
        printf("ep_c_client: FAIL status string\n");
        return 1;
    }

    CHECK_EP(ep_route(g, &t_scores, &t_topk, stream));
    CHECK_EP(ep_create_handle(g, &t_topk, stream, &h));
    CHECK_EP(ep_dispatch(h, &t_x, NULL, &t_w, &t_counts, 0, stream));
    int64_t rows = 0;
    CHECK_EP(ep_handle_get_num_recv(h, -1, &rows));   /* blocking */
    if (rows != (int64_t)NTOK * K) {
        printf("ep_c_client: FAIL %lld stage-2 rows, expected %d\n", (long long)rows, NTOK * K);
        return 1;
    }
    ep_tensor_t st2;
    CHECK_EP(ep_get_buffer(g, EP_BUF_HT_STAGE2, &st2));
    st2.sizes[0] = rows;
    ep_tensor_t t_y = tensor2d(d_y, EP_DTYPE_BF16, rows, H, EP_TAG_TOKENS);
    CHECK_EP(ep_dequantize_rows(g, &st2, &t_y, stream));
    CHECK_EP(ep_combine(h, &t_y, &t_w, &t_out, 0, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    CHECK_HIP(hipMemcpy(out, d_out, sizeof out, hipMemcpyDeviceToHost));
    int32_t counts[E];
    CHECK_HIP(hipMemcpy(counts, d_counts, sizeof counts, hipMemcpyDeviceToHost));
    int32_t err = -1;
    CHECK_EP(ep_get_device_error(g, &err));

    long long mismatches = 0, count_sum = 0;
    for (int i = 0; i < NTOK * H; ++i) mismatches += out[i] != x[i];
    for (int e = 0; e < E; ++e) count_sum += counts[e];
    CHECK_EP(ep_destroy_handle(h));
    CHECK_EP(ep_destroy_group(g));
    hipFree(d_scores);
    hipFree(d_w);
    hipFree(d_x);
    hipFree(d_out);
    hipFree(d_topk);
    hipFree(d_counts);
    hipFree(d_y);
    hipStreamDestroy(stream);

    if (mismatches != 0 || count_sum != (long long)NTOK * K || err != 0) {
        printf("ep_c_client: FAIL %lld mismatching elements, %lld counted entries, device error %d\n",
               mismatches, count_sum, err);
        return 1;
    }
    printf("ep_c_client: OK (%d tokens, %lld stage-2 rows, output equals input bit for bit)\n", NTOK,
           (long long)rows);
    return 0;
}
