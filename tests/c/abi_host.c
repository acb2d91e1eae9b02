/* A plain C11 client of libmoe's host-only entry points: the header must
 * compile as C and every call below runs without a GPU (validation, sizes
 * and status strings only; nothing is enqueued). */
#include <stdio.h>
#include <string.h>

#include "moe.h"

static int fail(const char *what) {
    fprintf(stderr, "FAIL: %s\n", what);
    return 1;
}

int main(void) {
    moe_desc d;
    memset(&d, 0, sizeof d);
    d.T = 4096;
    d.d = 4096;
    d.d_ff = 14336;
    d.E = 8;
    d.k = 2;
    d.gate = MOE_GATE_RENORM;
    d.act = MOE_ACT_SWIGLU;
    d.dtype = MOE_DTYPE_BF16;
    d.capacity_factor = 1.25;

    size_t ws = 0;
    if (moe_workspace_size(&d, &ws) != MOE_OK || ws == 0) return fail("moe_workspace_size");
    int64_t C = 0;
    if (moe_capacity(&d, &C) != MOE_OK || C != 1280) return fail("moe_capacity");

    moe_shared sh;
    memset(&sh, 0, sizeof sh);
    sh.n_shared = 2;
    size_t ws_sh = 0;
    if (moe_workspace_size_shared(&d, &sh, &ws_sh) != MOE_OK || ws_sh <= ws)
        return fail("moe_workspace_size_shared");
    sh.n_shared = MOE_MAX_SHARED + 1;
    if (moe_workspace_size_shared(&d, &sh, &ws_sh) != MOE_ERR_INVALID_ARG)
        return fail("shared count limit");

    /* e4m3 weights need a decode-sized batch: T = 4096 is refused */
    moe_fp8_experts f8;
    memset(&f8, 0, sizeof f8);
    if (moe_expert_ffn_fp8(&d, (const void *)16, (const int32_t *)16, &f8, (float *)16,
                           (void *)16, ws, NULL) != MOE_ERR_UNSUPPORTED)
        return fail("fp8 shape support");
    if (moe_quantize_e4m3(7, NULL, 1, 1, NULL, NULL, NULL) != MOE_ERR_INVALID_ARG)
        return fail("moe_quantize_e4m3 dtype");

    d.k = 9; /* k > E */
    if (moe_workspace_size(&d, &ws) != MOE_ERR_INVALID_ARG) return fail("k > E");
    if (strcmp(moe_status_string(MOE_OK), "MOE_OK") != 0) return fail("moe_status_string");
    printf("ok %zu %zu\n", ws, ws_sh);
    return 0;
}
