/* c_abi_check.c -- include/h3.h compiled as plain C99 and linked against
 * libh3.so: the host-only helpers and the argument checks that return before
 * any device work, so the program runs without a GPU.  Built and run by
 * tests/test_c_abi.py; exits non-zero on the first failed check's count. */
#include <stdio.h>
#include <string.h>

#include "h3.h"

static int failures = 0;

#define CHECK(cond)                                                     \
    do {                                                                \
        if (!(cond)) {                                                  \
            printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);      \
            ++failures;                                                 \
        }                                                               \
    } while (0)

int main(void) {
    int64_t begin = -1, count = -1;

    /* quotient / remainder split: 56 heads over 6 ranks is 10,10,9,9,9,9 */
    CHECK(h3_partition(56, 6, 0, &begin, &count) == H3_OK && begin == 0 && count == 10);
    CHECK(h3_partition(56, 6, 1, &begin, &count) == H3_OK && begin == 10 && count == 10);
    CHECK(h3_partition(56, 6, 2, &begin, &count) == H3_OK && begin == 20 && count == 9);
    CHECK(h3_partition(56, 6, 5, &begin, &count) == H3_OK && begin == 47 && count == 9);
    CHECK(h3_partition(5, 6, 0, &begin, &count) == H3_ERR_EMPTY_PARTITION);
    CHECK(strlen(h3_last_error()) > 0);
    CHECK(h3_partition(5, 0, 0, &begin, &count) == H3_ERR_EMPTY_PARTITION);

    /* clip and rebase: segments 96, 160, 256 against two intervals */
    {
        const int64_t cu[4] = {0, 96, 256, 512};
        int32_t seg[3];
        int64_t lo[3], hi[3];
        CHECK(h3_clip_segments(cu, 3, 256, 512, seg, lo, hi) == 1);
        CHECK(seg[0] == 2 && lo[0] == 0 && hi[0] == 256);
        CHECK(h3_clip_segments(cu, 3, 50, 300, seg, lo, hi) == 3);
        CHECK(seg[0] == 0 && lo[0] == 0 && hi[0] == 46);
        CHECK(seg[1] == 1 && lo[1] == 46 && hi[1] == 206);
        CHECK(seg[2] == 2 && lo[2] == 206 && hi[2] == 250);
        CHECK(h3_clip_segments(cu, 3, 0, 512, NULL, NULL, NULL) == 3);
        CHECK(h3_clip_segments(cu, 3, 300, 200, seg, lo, hi) == -1);
    }

    CHECK(strcmp(h3_status_string(H3_OK), "H3_OK") == 0);
    CHECK(strcmp(h3_status_string(H3_ERR_ALIAS), "H3_ERR_ALIAS") == 0);
    CHECK(strlen(h3_version()) >= 5);

    /* rejected before anything reaches the device */
    CHECK(h3_seq2head(NULL, NULL, NULL, NULL, NULL) == H3_ERR_ARG);
    {
        const int64_t cu[2] = {0, 64};
        h3_plan_info info;
        memset(&info, 0xff, sizeof info);
        CHECK(h3_packed_attn(NULL, NULL, NULL, NULL, NULL, 64, 1, H3_HEAD_DIM, cu, 1, 0.0884f, NULL, &info) ==
              H3_ERR_ARG);
        CHECK(info.launches == 0);
    }
    CHECK(h3_packed_attn_backward_workspace(0, 4, 1) == 0);
    CHECK(h3_packed_attn_backward_workspace(64, 2, 1) >= (int64_t)64 * 2 * H3_HEAD_DIM * 2);
    CHECK(h3_packed_attn_backward_workspace(64, 2, 0) < h3_packed_attn_backward_workspace(64, 2, 1));

    if (failures) {
        printf("c abi: %d failed checks\n", failures);
        return 1;
    }
    printf("c abi: ok\n");
    return 0;
}
