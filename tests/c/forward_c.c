/* A plain C11 client of libmoe on the GPU: allocates device memory through
 * the HIP runtime's C API, runs moe_forward on seeded inputs of a small
 * Mixtral-style layer (T = 300, d = 256, d_ff = 512, E = 8, top-2,
 * SwiGLU, bf16), and checks that the output is finite, that a second call
 * gives the same bits, and that the staged entry points (moe_route,
 * moe_dispatch, moe_expert_ffn, moe_combine) give the same bits as well.
 * Prints "ok <checksum>" and exits 0 on success. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe.h"

#define CHECK_HIP(x)                                                     \
    do {                                                                 \
        hipError_t e_ = (x);                                             \
        if (e_ != hipSuccess) {                                          \
            fprintf(stderr, "HIP error %d at line %d\n", (int)e_, __LINE__); \
            return 1;                                                    \
        }                                                                \
    } while (0)
#define CHECK_MOE(x)                                                     \
    do {                                                                 \
        int r_ = (x);                                                    \
        if (r_ != MOE_OK) {                                              \
            fprintf(stderr, "%s at line %d\n", moe_status_string(r_), __LINE__); \
            return 1;                                                    \
        }                                                                \
    } while (0)

static uint64_t lcg = 0x9E3779B97F4A7C15ull;
static double uniform01(void) {
    lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
    return ((lcg >> 11) + 0.5) / 9007199254740992.0;
}
static float normal(void) { /* Box-Muller */
    const double u = uniform01(), v = uniform01();
    return (float)(sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v));
}
static uint16_t to_bf16(float f) { /* round to nearest even */
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static void *dev_copy(const void *h, size_t bytes) {
    void *p = NULL;
    if (hipMalloc(&p, bytes) != hipSuccess) return NULL;
    if (h && hipMemcpy(p, h, bytes, hipMemcpyHostToDevice) != hipSuccess) return NULL;
    return p;
}

int main(void) {
    moe_desc desc;
    memset(&desc, 0, sizeof desc);
    desc.T = 300;
    desc.d = 256;
    desc.d_ff = 512;
    desc.E = 8;
    desc.k = 2;
    desc.gate = MOE_GATE_RENORM;
    desc.act = MOE_ACT_SWIGLU;
    desc.dtype = MOE_DTYPE_BF16;
    desc.capacity_factor = 0.0;
    const size_t T = 300, d = 256, f = 512, E = 8, k = 2;

    uint16_t *x = malloc(T * d * 2), *w1 = malloc(E * f * d * 2), *w3 = malloc(E * f * d * 2),
             *w2 = malloc(E * d * f * 2);
    float *wr = malloc(E * d * 4);
    if (!x || !w1 || !w3 || !w2 || !wr) return 1;
    for (size_t i = 0; i < T * d; ++i) x[i] = to_bf16(normal());
    for (size_t i = 0; i < E * d; ++i) wr[i] = normal() / 16.0f;
    for (size_t i = 0; i < E * f * d; ++i) w1[i] = to_bf16(normal() / 16.0f);
    for (size_t i = 0; i < E * f * d; ++i) w3[i] = to_bf16(normal() / 16.0f);
    for (size_t i = 0; i < E * d * f; ++i) w2[i] = to_bf16(normal() / 22.627417f);

    void *dx = dev_copy(x, T * d * 2), *dw1 = dev_copy(w1, E * f * d * 2),
         *dw3 = dev_copy(w3, E * f * d * 2), *dw2 = dev_copy(w2, E * d * f * 2);
    float *dwr = dev_copy(wr, E * d * 4);
    void *dy = dev_copy(NULL, T * d * 2), *dy2 = dev_copy(NULL, T * d * 2);
    int32_t *idx = dev_copy(NULL, T * k * 4), *routed = dev_copy(NULL, E * 4),
            *kept = dev_copy(NULL, E * 4), *offs = dev_copy(NULL, (E + 1) * 4),
            *ros = dev_copy(NULL, T * k * 4), *tor = dev_copy(NULL, T * k * 4);
    float *gates = dev_copy(NULL, T * k * 4), *stats = dev_copy(NULL, (2 * E + 2) * 4);
    uint8_t *dropped = dev_copy(NULL, T * k);
    void *xperm = dev_copy(NULL, T * k * d * 2);
    float *yperm = dev_copy(NULL, T * k * d * 4);
    if (!dx || !dw1 || !dw3 || !dw2 || !dwr || !dy || !dy2 || !idx || !routed || !kept || !offs ||
        !ros || !tor || !gates || !stats || !dropped || !xperm || !yperm)
        return 1;
    size_t ws_bytes = 0;
    CHECK_MOE(moe_workspace_size(&desc, &ws_bytes));
    void *ws = dev_copy(NULL, ws_bytes);
    if (!ws) return 1;

    uint16_t *y1 = malloc(T * d * 2), *y2 = malloc(T * d * 2), *y3 = malloc(T * d * 2);
    if (!y1 || !y2 || !y3) return 1;
    for (int rep = 0; rep < 2; ++rep) {
        CHECK_MOE(moe_forward(&desc, dx, dwr, NULL, NULL, dw1, dw3, dw2, dy, NULL, NULL, NULL, NULL,
                              NULL, NULL, NULL, NULL, NULL, ws, ws_bytes, NULL));
        CHECK_HIP(hipDeviceSynchronize());
        CHECK_HIP(hipMemcpy(rep == 0 ? y1 : y2, dy, T * d * 2, hipMemcpyDeviceToHost));
    }
    /* the staged entry points */
    CHECK_MOE(moe_route(&desc, dx, dwr, NULL, NULL, idx, gates, stats, ws, ws_bytes, NULL));
    CHECK_MOE(moe_dispatch(&desc, dx, idx, routed, kept, offs, ros, tor, dropped, xperm, ws, ws_bytes,
                           NULL));
    CHECK_MOE(moe_expert_ffn(&desc, xperm, offs, dw1, dw3, dw2, yperm, ws, ws_bytes, NULL));
    CHECK_MOE(moe_combine(&desc, yperm, ros, gates, dy2, NULL));
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(y3, dy2, T * d * 2, hipMemcpyDeviceToHost));

    double checksum = 0.0;
    for (size_t i = 0; i < T * d; ++i) {
        uint32_t u = (uint32_t)y1[i] << 16;
        float v;
        memcpy(&v, &u, 4);
        if (!isfinite(v)) {
            fprintf(stderr, "non-finite output at %zu\n", i);
            return 1;
        }
        checksum += fabs((double)v);
    }
    if (checksum == 0.0) {
        fprintf(stderr, "all-zero output\n");
        return 1;
    }
    if (memcmp(y1, y2, T * d * 2) != 0) {
        fprintf(stderr, "two moe_forward calls differ\n");
        return 1;
    }
    if (memcmp(y1, y3, T * d * 2) != 0) {
        fprintf(stderr, "staged entry points differ from moe_forward\n");
        return 1;
    }
    printf("ok %.6f\n", checksum);
    return 0;
}
