/* c_gpu_relayout.c -- the relayouts driven from plain C through include/h3.h,
 * with device memory from the HIP runtime and no Python in between.  56 heads
 * over P = 6 ragged ranks (10,10,9,9,9,9), 3 planes, a token count that is not
 * a multiple of anything: seq2head of every rank, checked element by element
 * against dst[j*K+p][t][h][d] = src[t][p][hb_j+h][d] computed here from the
 * partition; then head2seq of plane 1 back to [N][H][D], checked against the
 * source plane; then the same seq2head with a chunk cap.  Exits non-zero on
 * failure.  Built and run by tests/test_gpu_c_abi.py. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "h3.h"

#define N_TOKENS 777
#define N_HEADS 56
#define PLANES 3
#define WORLD 6
#define D H3_HEAD_DIM

static int failures = 0;

#define CHECK(cond)                                                     \
    do {                                                                \
        if (!(cond)) {                                                  \
            printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);      \
            ++failures;                                                 \
        }                                                               \
    } while (0)

#define HIP_OK(call)                                                    \
    do {                                                                \
        hipError_t e_ = (call);                                         \
        if (e_ != hipSuccess) {                                         \
            printf("HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
            return 2;                                                   \
        }                                                               \
    } while (0)

/* a distinct 16-bit pattern per element (bits only; nothing is computed) */
static uint16_t pattern(int64_t t, int p, int h, int d) {
    return (uint16_t)((t * 7919 + p * 104729 + h * 131 + d * 3) & 0xffff);
}

int main(void) {
    const size_t plane_row = (size_t)N_HEADS * D;             /* elements per token and plane */
    const size_t src_elems = (size_t)N_TOKENS * PLANES * plane_row;
    uint16_t *src = (uint16_t *)malloc(src_elems * sizeof(uint16_t));
    if (!src) return 2;
    for (int64_t t = 0; t < N_TOKENS; ++t)
        for (int p = 0; p < PLANES; ++p)
            for (int h = 0; h < N_HEADS; ++h)
                for (int d = 0; d < D; ++d) src[((t * PLANES + p) * N_HEADS + h) * D + d] = pattern(t, p, h, d);

    int64_t hb[WORLD], hn[WORLD];
    for (int j = 0; j < WORLD; ++j) CHECK(h3_partition(N_HEADS, WORLD, j, &hb[j], &hn[j]) == H3_OK);
    CHECK(hn[0] == 10 && hn[1] == 10 && hn[2] == 9 && hn[5] == 9);

    void *d_src = NULL, *d_dst[WORLD * PLANES], *d_out = NULL;
    HIP_OK(hipMalloc(&d_src, src_elems * sizeof(uint16_t)));
    HIP_OK(hipMemcpy(d_src, src, src_elems * sizeof(uint16_t), hipMemcpyHostToDevice));
    for (int j = 0; j < WORLD; ++j)
        for (int p = 0; p < PLANES; ++p)
            HIP_OK(hipMalloc(&d_dst[j * PLANES + p], (size_t)N_TOKENS * hn[j] * D * sizeof(uint16_t)));
    HIP_OK(hipMalloc(&d_out, (size_t)N_TOKENS * plane_row * sizeof(uint16_t)));

    for (int pass = 0; pass < 2; ++pass) {
        h3_layout L;
        memset(&L, 0, sizeof L);
        L.n_tokens = N_TOKENS;
        L.n_heads = N_HEADS;
        L.head_dim = D;
        L.n_planes = PLANES;
        L.world = WORLD;
        L.rank = -1;
        /* pass 1: a cap of 100 tokens of a whole plane per launch */
        L.max_chunk_bytes = pass ? (int64_t)100 * N_HEADS * D * 2 : 0;
        h3_plan_info info;
        h3_status st = h3_seq2head(&L, d_src, d_dst, NULL, &info);
        CHECK(st == H3_OK);
        if (st != H3_OK) {
            printf("h3_seq2head: %s\n", h3_last_error());
            break;
        }
        CHECK(info.chunks == (pass ? 8 : 1));
        CHECK(info.launches == PLANES * info.chunks);
        HIP_OK(hipDeviceSynchronize());
        int bad = 0;
        for (int j = 0; j < WORLD && !bad; ++j)
            for (int p = 0; p < PLANES && !bad; ++p) {
                const size_t n = (size_t)N_TOKENS * hn[j] * D;
                uint16_t *got = (uint16_t *)malloc(n * sizeof(uint16_t));
                if (!got) return 2;
                HIP_OK(hipMemcpy(got, d_dst[j * PLANES + p], n * sizeof(uint16_t), hipMemcpyDeviceToHost));
                for (int64_t t = 0; t < N_TOKENS && !bad; ++t)
                    for (int h = 0; h < hn[j] && !bad; ++h)
                        for (int d = 0; d < D; ++d)
                            if (got[((size_t)t * hn[j] + h) * D + d] != pattern(t, p, (int)(hb[j] + h), d)) {
                                printf("seq2head mismatch: pass %d rank %d plane %d token %lld head %d d %d\n",
                                       pass, j, p, (long long)t, h, d);
                                bad = 1;
                                break;
                            }
                free(got);
            }
        CHECK(!bad);
    }

    /* head2seq of plane 1 from every rank back to [N][H][D] */
    {
        h3_layout L;
        memset(&L, 0, sizeof L);
        L.n_tokens = N_TOKENS;
        L.n_heads = N_HEADS;
        L.head_dim = D;
        L.n_planes = 1;
        L.world = WORLD;
        L.rank = -1;
        const void *parts[WORLD];
        for (int j = 0; j < WORLD; ++j) parts[j] = d_dst[j * PLANES + 1];
        CHECK(h3_head2seq(&L, parts, d_out, NULL, NULL) == H3_OK);
        HIP_OK(hipDeviceSynchronize());
        const size_t n = (size_t)N_TOKENS * plane_row;
        uint16_t *got = (uint16_t *)malloc(n * sizeof(uint16_t));
        if (!got) return 2;
        HIP_OK(hipMemcpy(got, d_out, n * sizeof(uint16_t), hipMemcpyDeviceToHost));
        size_t wrong = 0;
        for (int64_t t = 0; t < N_TOKENS; ++t)
            for (int h = 0; h < N_HEADS; ++h)
                for (int d = 0; d < D; ++d)
                    wrong += got[((size_t)t * N_HEADS + h) * D + d] != pattern(t, 1, h, d);
        CHECK(wrong == 0);
        free(got);
    }

    /* a misaligned destination is rejected before anything is enqueued */
    {
        h3_layout L;
        memset(&L, 0, sizeof L);
        L.n_tokens = N_TOKENS;
        L.n_heads = N_HEADS;
        L.head_dim = D;
        L.n_planes = 1;
        L.world = WORLD;
        L.rank = -1;
        const void *parts[WORLD];
        for (int j = 0; j < WORLD; ++j) parts[j] = d_dst[j * PLANES];
        CHECK(h3_head2seq(&L, parts, (char *)d_out + 2, NULL, NULL) == H3_ERR_ARG);
    }

    for (int i = 0; i < WORLD * PLANES; ++i) HIP_OK(hipFree(d_dst[i]));
    HIP_OK(hipFree(d_src));
    HIP_OK(hipFree(d_out));
    free(src);
    if (failures) {
        printf("c gpu relayout: %d failed checks\n", failures);
        return 1;
    }
    printf("c gpu relayout: ok\n");
    return 0;
}
