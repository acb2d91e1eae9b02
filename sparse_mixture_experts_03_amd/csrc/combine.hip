// combine.hip -- gate-weighted combine of the expert outputs.
//
// Page "Mixture of experts" (rayaq.ca), Mechanics, "Replacing the
// feed-forward block": y = sum over the selected experts of g_i E_i(x);
// Implementation: the gated expert outputs are added back per token (the
// listing's index_add_), so a token with two experts gets both; "Capacity
// and dropped tokens": a dropped assignment skips the expert, so it adds
// nothing here, and a token dropped from every expert gets 0 (its residual,
// outside the layer, carries it).
//
// When the down projection split K in two, the two partial rows are added
// (first half + second half) before the gate multiplies them.
//
// With shared experts and the block residual (section "Total versus active
// parameters": shared experts every token visits; Implementation: the block
// adds the layer output to its hidden state), the same pass then adds the
// token's row of the shared experts' summed output (its two K halves first,
// when split) and the residual last, before the single rounding to the act
// dtype.
//
// combine_kernel: one wave per (token, group of 256-column chunks),
// grid-stride; each lane owns 4 consecutive columns of a chunk and sums the
// k slots in slot order in fp32, then stores fp32 or bf16 (a scalar
// variant serves widths that are not a multiple of 4).  Every output element is
// written exactly once, so no memset and no atomics are needed.  The rows
// it reads (expert outputs, their second K halves, the shared experts' rows,
// the residual) are read once, so they are loaded non-temporally and do
// not displace the caches' contents (Mixtral prefill combine 65 -> 55 us);
// y, which the next layer reads, is stored normally.
#include "moe_internal.h"

namespace moe {

namespace {

// Shared experts' summed output and the residual (SH kernels only).
struct SharedIn {
    const float *ysh;   // [T][d] fp32, or nullptr
    const float *ysh2;  // second K half of ysh, or nullptr
    const void *res;    // [T][d] in the act dtype, or nullptr
};

typedef float f32x4v __attribute__((ext_vector_type(4)));

// a 16-byte load of data read once
__device__ __forceinline__ float4 ld_once(const float *p) {
    const f32x4v v = __builtin_nontemporal_load((const f32x4v *)p);
    return make_float4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ float4 add4(float4 a, float4 b) {
    a.x += b.x;
    a.y += b.y;
    a.z += b.z;
    a.w += b.w;
    return a;
}

// KC: k when it is a compile-time constant (the slot loop unrolled, so all
// of a chunk group's loads are issued together), 0 for any k.  SH: add the
// shared experts and the residual after the routed slots.
template <bool BF16, bool VEC4, int KC, bool SH>
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ y_perm,
                                                      const float *__restrict__ part2,
                                                      const int32_t *__restrict__ row_of_slot,
                                                      const float *__restrict__ gates, int T,
                                                      int d, int k, int G, SharedIn sh,
                                                      void *__restrict__ y) {
    const int lane = threadIdx.x & 63;
    if (VEC4) {
        // one wave per (token, group of G 256-column chunks): the token's k
        // rows and gates are read once per group, then the group's chunks
        // follow, four at a time with their loads in flight
        const int nch = (d + 255) / 256;
        const int ngrp = (nch + G - 1) / G;
        for (int64_t it = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); it < (int64_t)T * ngrp;
             it += (int64_t)gridDim.x * 4) {
            const int t = (int)(it / ngrp);
            const int grp = (int)(it - (int64_t)t * ngrp);
            const int cend = min(d, (grp + 1) * G * 256);
            const int32_t *rs = row_of_slot + (int64_t)t * k;
            const float *gs = gates + (int64_t)t * k;
#pragma unroll 4
            for (int c = grp * G * 256 + lane * 4; c < cend; c += 256) {
                float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                for (int s = 0; s < (KC ? KC : k); ++s) {
                    const int r = rs[s];
                    if (r < 0) continue;
                    const float g = gs[s];
                    float4 v = ld_once(y_perm + (int64_t)r * d + c);
                    if (part2) {
                        const float4 u = ld_once(part2 + (int64_t)r * d + c);
                        v.x += u.x;
                        v.y += u.y;
                        v.z += u.z;
                        v.w += u.w;
                    }
                    a.x = fmaf(g, v.x, a.x);
                    a.y = fmaf(g, v.y, a.y);
                    a.z = fmaf(g, v.z, a.z);
                    a.w = fmaf(g, v.w, a.w);
                }
                if (SH) {
                    const int64_t o = (int64_t)t * d + c;
                    if (sh.ysh) {
                        float4 v = ld_once(sh.ysh + o);
                        if (sh.ysh2) v = add4(v, ld_once(sh.ysh2 + o));
                        a = add4(a, v);
                    }
                    if (sh.res) {
                        if (BF16) {
                            typedef unsigned u32x2v __attribute__((ext_vector_type(2)));
                            const u32x2v rv = __builtin_nontemporal_load((const u32x2v *)((const uint16_t *)sh.res + o));
                            const uint2 r = make_uint2(rv[0], rv[1]);
                            a.x += bf16_to_f32((uint16_t)(r.x & 0xffffu));
                            a.y += bf16_to_f32((uint16_t)(r.x >> 16));
                            a.z += bf16_to_f32((uint16_t)(r.y & 0xffffu));
                            a.w += bf16_to_f32((uint16_t)(r.y >> 16));
                        } else {
                            a = add4(a, ld_once((const float *)sh.res + o));
                        }
                    }
                }
                if (BF16) {
                    uint2 o;
                    o.x = (uint32_t)f32_to_bf16(a.x) | ((uint32_t)f32_to_bf16(a.y) << 16);
                    o.y = (uint32_t)f32_to_bf16(a.z) | ((uint32_t)f32_to_bf16(a.w) << 16);
                    *(uint2 *)((uint16_t *)y + (int64_t)t * d + c) = o;
                } else {
                    *(float4 *)((float *)y + (int64_t)t * d + c) = a;
                }
            }
        }
        return;
    }
    for (int t = blockIdx.x * 4 + (threadIdx.x >> 6); t < T; t += gridDim.x * 4) {
        const int32_t *rs = row_of_slot + (int64_t)t * k;
        const float *gs = gates + (int64_t)t * k;
        {
            for (int c = lane; c < d; c += 64) {
                float a = 0.f;
                for (int s = 0; s < k; ++s) {
                    const int r = rs[s];
                    if (r < 0) continue;
                    float v = y_perm[(int64_t)r * d + c];
                    if (part2) v += part2[(int64_t)r * d + c];
                    a = fmaf(gs[s], v, a);
                }
                if (SH) {
                    const int64_t o = (int64_t)t * d + c;
                    if (sh.ysh) {
                        float v = sh.ysh[o];
                        if (sh.ysh2) v += sh.ysh2[o];
                        a += v;
                    }
                    if (sh.res)
                        a += BF16 ? bf16_to_f32(((const uint16_t *)sh.res)[o]) : ((const float *)sh.res)[o];
                }
                if (BF16)
                    ((uint16_t *)y)[(int64_t)t * d + c] = f32_to_bf16(a);
                else
                    ((float *)y)[(int64_t)t * d + c] = a;
            }
        }
    }
}

}  // namespace

namespace {

template <bool SH>
hipError_t combine_any(const Shape &s, const float *y_perm, const float *y_perm_part2,
                       const int32_t *row_of_slot, const float *gates, const SharedIn &sh, void *y,
                       hipStream_t st) {
    const bool v4 = (s.d % 4) == 0;
    // chunks per wave: whole rows when there are many tokens, single
    // 256-column chunks when there are few (so that enough waves run)
    const int nch = (s.d + 255) / 256;
    int G = (int)(((int64_t)s.T * nch) / 2048);
    G = G < 1 ? 1 : (G > nch ? nch : G);
    const int64_t items = v4 ? (int64_t)s.T * ((nch + G - 1) / G) : (int64_t)s.T;
    int64_t blocks = (items + 3) / 4;
    if (blocks > 16384) blocks = 16384;
    const bool bf = s.dtype == 1;
    auto kern = bf ? (v4 ? combine_kernel<true, true, 0, SH> : combine_kernel<true, false, 0, SH>)
                   : (v4 ? combine_kernel<false, true, 0, SH> : combine_kernel<false, false, 0, SH>);
    if (v4) {
        // common k: slot loop unrolled
        if (s.k == 1) kern = bf ? combine_kernel<true, true, 1, SH> : combine_kernel<false, true, 1, SH>;
        if (s.k == 2) kern = bf ? combine_kernel<true, true, 2, SH> : combine_kernel<false, true, 2, SH>;
        if (s.k == 4) kern = bf ? combine_kernel<true, true, 4, SH> : combine_kernel<false, true, 4, SH>;
        if (s.k == 8) kern = bf ? combine_kernel<true, true, 8, SH> : combine_kernel<false, true, 8, SH>;
    }
    launch_kernel(kern, dim3((unsigned)blocks), dim3(256), 0, st, y_perm, y_perm_part2, row_of_slot,
                  gates, s.T, s.d, s.k, G, sh, y);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const Shape &s, const float *y_perm, const float *y_perm_part2,
                          const int32_t *row_of_slot, const float *gates, void *y,
                          hipStream_t st) {
    return combine_any<false>(s, y_perm, y_perm_part2, row_of_slot, gates,
                              SharedIn{nullptr, nullptr, nullptr}, y, st);
}

hipError_t launch_combine_shared(const Shape &s, const float *y_perm, const float *y_perm_part2,
                                 const int32_t *row_of_slot, const float *gates, const float *y_sh,
                                 const float *y_sh_part2, const void *residual, void *y,
                                 hipStream_t st) {
    if (y_sh == nullptr && residual == nullptr)
        return launch_combine(s, y_perm, y_perm_part2, row_of_slot, gates, y, st);
    return combine_any<true>(s, y_perm, y_perm_part2, row_of_slot, gates,
                             SharedIn{y_sh, y_sh_part2, residual}, y, st);
}

}  // namespace moe
