/* C99 client of libvarattn.so: the header compiles as C and the host-only
 * entry points link and behave (no device is touched: every call below
 * either needs no HIP call or fails its argument checks first). */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "var_attn.h"

static int failures = 0;
#define CHECK(cond)                                                              \
    do {                                                                         \
        if (!(cond)) {                                                           \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);  \
            ++failures;                                                          \
        }                                                                        \
    } while (0)

int main(void) {
    const int32_t g[13] = {1, 2, 4, 6, 8, 12, 16, 20, 24, 32, 40, 48, 64};
    var_schedule sched = {13, g, g};
    int64_t first = -1, n_q = -1, kv = -1;
    CHECK(var_schedule_extent(&sched, 12, 13, &first, &n_q, &kv) == VAR_OK);
    CHECK(first == 6425 && n_q == 4096 && kv == 10521);
    CHECK(var_schedule_extent(&sched, 13, 13, NULL, NULL, NULL) == VAR_ERR_RANGE);
    CHECK(strlen(var_last_error()) > 0);

    var_mask_params mp = {64, 64, 7, 7, 2, 2};
    int32_t n_qt = 0, n_kt = 0;
    CHECK(var_tile_mask_dims(&sched, 12, 13, &mp, 0, &n_qt, &n_kt) == VAR_OK);
    CHECK(n_qt == 64 && n_kt == 165);

    var_attn_desc d;
    memset(&d, 0, sizeof(d));
    d.batch = 2; d.heads = 16; d.head_dim = 96;   /* unsupported head dim: rejected before any HIP call */
    d.q_scale_begin = 12; d.q_scale_end = 13; d.in_dtype = VAR_BF16; d.out_dtype = VAR_F32;
    var_layout l = {2 * 16 * 4096 * 96, 4096 * 96, 96};
    char fake[16];
    CHECK(var_attn_dense(&sched, &d, fake, l, fake, l, fake, l, fake, l, NULL, NULL, 0, NULL) == VAR_ERR_UNSUPPORTED);
    CHECK(var_attn_dense(NULL, &d, fake, l, fake, l, fake, l, fake, l, NULL, NULL, 0, NULL) == VAR_ERR_NULL);

    int32_t splits = 0;
    int64_t ws = -1;
    d.head_dim = 128;
    CHECK(var_attn_split_plan(&sched, &d, 0, 0, &splits, &ws) == VAR_OK);
    CHECK(splits == 1 && ws == 0);   /* the last step fills the GPU without splits */

    CHECK(var_quantize_e4m3(2, 16, 100, 128, NULL, l, NULL, l, NULL, 2, 100, NULL) == VAR_OK);   /* nothing to do */
    CHECK(var_quantize_e4m3(2, 16, 100, 120, fake, l, NULL, l, NULL, 2, 0, NULL) == VAR_ERR_UNSUPPORTED);

    CHECK(strcmp(var_status_string(VAR_ERR_CAPACITY), "VAR_ERR_CAPACITY") == 0);
    if (failures == 0) printf("c abi: ok\n");
    return failures ? 1 : 0;
}
