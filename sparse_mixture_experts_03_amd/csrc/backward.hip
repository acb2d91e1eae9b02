// backward.hip -- the layer's backward (training gradients).
//
// Page "Mixture of experts" (rayaq.ca), Mechanics: the top-k choice is
// discrete, the gate values are differentiable, and that is how the router
// learns ("Replacing the feed-forward block"); the load-balancing loss
// aux = E sum f_i P_i has d aux / d P_i = E f_i, f being a count ("The
// load-balancing loss"); the z statistic is mean lse^2.  The routing of
// the forward (top-k indices, gates, capacity drops, the permutation) is
// an input and is held fixed.
//
// The expert part runs through the forward's grouped GEMM launchers
// (C = A B^T over the ragged per-expert row blocks), so every operand must
// be K-contiguous: the weights are transposed once per call (W2 to
// [E][d_ff][d]; W1 and W3 side by side to [E][d][n_up d_ff]).  The kernels
// here:
//   transpose_kernel       64 x 64 tiles through LDS, batched, any strides
//   act_fwd_kernel         H = act(a1, a3) from the recomputed pre-activations
//   combine_bwd_kernel     per kept row: dE = g dy_t (bf16), dg = <dy_t, E(x_t)>
//   act_bwd_kernel         dA = [da1 | da3] from dH and the pre-activations
//   logits_kernel          p = softmax(W_r x + b + n), lse (fp32; 32 tokens
//                          per block sharing each W_r read); for d a
//                          multiple of 64 the logits run on matrix cores
//                          instead (split_wr_kernel, the weight-gradient
//                          GEMM, logits_finish_kernel)
//   router_bwd_kernel      dh_t from dg (gate convention), aux and z terms
//   dx_kernel              dx_t = sum over kept slots of dX_perm + W_r^T dh_t
//                          (the product on fp32 matrix cores)
//   dwr_partial_kernel, dwr_reduce_kernel, dbias_kernel
//                          dW_r = sum_t dh_t x_t^T (token splits, then the
//                          splits in order), db = sum_t dh_t; dW_r runs on
//                          matrix cores instead when it fits (split_dh_kernel,
//                          the weight-gradient GEMM, dwr_sum_kernel)
//   pad_offsets_kernel     each expert's start in the padded row layout
//                          (row counts rounded up to 64)
//   transpose_padded_kernel  the activations transposed into that layout
//                          (K-contiguous rows, zero pads)
//   wgrad_kernel           weight gradients: per expert, C = P^T Q over its
//                          k range, 128 x 128 tiles, for operands past
//                          2 GiB; otherwise the forward's 256 x 256 tile
//                          runs them (its weight-gradient form, in
//                          expert_gemm.hip)
// fp32 layers use the same steps with plain kernels where the bf16 path
// uses matrix cores: transpose_f32_kernel for the weights, the fp32
// grouped GEMM of the forward, and wgrad_f32_kernel (one thread per weight,
// the expert's rows in order).
// Every sum has a fixed order (no atomics); results are reproducible.
#include "moe_internal.h"

namespace moe {

namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ float wave_max_f32b(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// activations in the layer's storage type: bf16 bits or fp32
__device__ __forceinline__ float ld_elem(const uint16_t *p, int64_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ float ld_elem(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ void st_elem(uint16_t *p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
__device__ __forceinline__ void st_elem(float *p, int64_t i, float v) { p[i] = v; }

// dst[b][c][r] = src[b][r][c] for r < R, c < C (bf16); strides in elements.
// VEC: 4-element (8-byte) reads along c and writes along r (C, R, the
// strides and the bases multiples of 4); otherwise one element at a time.
// With row offsets, matrix b is skipped when expert b has no rows: nothing
// reads its transposed weights then (skewed routing leaves most experts of
// a fine-grained layer without rows).
template <bool VEC>
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t *__restrict__ src, int64_t R,
                                                        int64_t C, int64_t lds, int64_t sbs,
                                                        uint16_t *__restrict__ dst, int64_t ldd,
                                                        int64_t dbs, const int32_t *__restrict__ offsets) {
    if (offsets && offsets[blockIdx.z + 1] == offsets[blockIdx.z]) return;   // uniform in the block
    __shared__ uint16_t tile[64][66];
    const int64_t c0 = (int64_t)blockIdx.x * 64, r0 = (int64_t)blockIdx.y * 64;
    const uint16_t *s = src + (int64_t)blockIdx.z * sbs;
    uint16_t *d = dst + (int64_t)blockIdx.z * dbs;
    if (VEC) {
        // 64 rows x 16 groups of 4 = 1024 groups, 4 per thread
        const int g = threadIdx.x & 15, rr = threadIdx.x >> 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t r = r0 + rr + 16 * i, c = c0 + 4 * g;
            uint2 v = make_uint2(0, 0);
            if (r < R && c < C) v = *(const uint2 *)(s + r * lds + c);
            tile[rr + 16 * i][4 * g + 0] = (uint16_t)(v.x & 0xffffu);
            tile[rr + 16 * i][4 * g + 1] = (uint16_t)(v.x >> 16);
            tile[rr + 16 * i][4 * g + 2] = (uint16_t)(v.y & 0xffffu);
            tile[rr + 16 * i][4 * g + 3] = (uint16_t)(v.y >> 16);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int cc = rr + 16 * i;
            const int64_t c = c0 + cc, r = r0 + 4 * g;
            if (c < C && r < R) {
                uint2 v;
                v.x = (uint32_t)tile[4 * g + 0][cc] | ((uint32_t)tile[4 * g + 1][cc] << 16);
                v.y = (uint32_t)tile[4 * g + 2][cc] | ((uint32_t)tile[4 * g + 3][cc] << 16);
                *(uint2 *)(d + c * ldd + r) = v;
            }
        }
        return;
    }
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t r = r0 + ty + 4 * i, c = c0 + tx;
        tile[ty + 4 * i][tx] = (r < R && c < C) ? s[r * lds + c] : (uint16_t)0;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t c = c0 + ty + 4 * i, r = r0 + tx;
        if (r < R && c < C) d[c * ldd + r] = tile[tx][ty + 4 * i];
    }
}

// poff[e] = sum over e' < e of (offsets[e'+1] - offsets[e']) rounded up to
// 64, poff[E] the total: one wave, experts e and e + 64 on lane e % 64
// (E <= 128), two inclusive scans by shuffles.
__global__ __launch_bounds__(64) void pad_offsets_kernel(const int32_t *__restrict__ offsets, int E,
                                                         int32_t *__restrict__ poff) {
    const int l = threadIdx.x;
    int c0 = 0, c1 = 0;
    if (l < E) c0 = (offsets[l + 1] - offsets[l] + 63) & ~63;
    if (l + 64 < E) c1 = (offsets[l + 65] - offsets[l + 64] + 63) & ~63;
    int s0 = c0, s1 = c1;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u0 = __shfl_up(s0, o), u1 = __shfl_up(s1, o);
        if (l >= o) {
            s0 += u0;
            s1 += u1;
        }
    }
    const int tot0 = __shfl(s0, 63), tot1 = __shfl(s1, 63);
    if (l < E) poff[l] = s0 - c0;
    if (l + 64 < E) poff[l + 64] = tot0 + s1 - c1;
    if (l == 0) poff[E] = tot0 + tot1;
}

// The padded transpose: block (x, y) takes source columns 64x.. and padded
// positions 64y..; a 64-wide run of positions lies inside one expert's
// range (every range starts on a multiple of 64), found by binary search
// over poff; its source rows are offsets[e] + (64y - poff[e]) + i for the
// expert's count, zeros past it.  VEC as in transpose_kernel.
template <bool VEC>
__global__ __launch_bounds__(256) void transpose_padded_kernel(const uint16_t *__restrict__ src, int64_t C,
                                                               int64_t lds, const int32_t *__restrict__ offsets,
                                                               const int32_t *__restrict__ poff, int E,
                                                               uint16_t *__restrict__ dst, int64_t ldp) {
    __shared__ uint16_t tile[64][66];
    const int64_t c0 = (int64_t)blockIdx.x * 64;
    const int j0 = (int)blockIdx.y * 64;
    if (j0 >= poff[E]) return;
    int lo = 0, hi = E - 1;   // largest e with poff[e] <= j0
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (poff[mid] <= j0) lo = mid;
        else hi = mid - 1;
    }
    const int e = lo;
    const int64_t rb = (int64_t)offsets[e] + (j0 - poff[e]);
    const int nv = min(64, offsets[e + 1] - offsets[e] - (j0 - poff[e]));   // valid rows (may be <= 0)
    if (VEC) {
        const int g = threadIdx.x & 15, rr = threadIdx.x >> 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rr + 16 * i;
            const int64_t c = c0 + 4 * g;
            uint2 v = make_uint2(0, 0);
            if (r < nv && c < C) v = *(const uint2 *)(src + (rb + r) * lds + c);
            tile[r][4 * g + 0] = (uint16_t)(v.x & 0xffffu);
            tile[r][4 * g + 1] = (uint16_t)(v.x >> 16);
            tile[r][4 * g + 2] = (uint16_t)(v.y & 0xffffu);
            tile[r][4 * g + 3] = (uint16_t)(v.y >> 16);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int cc = rr + 16 * i;
            const int64_t c = c0 + cc;
            if (c < C) {
                uint2 v;
                v.x = (uint32_t)tile[4 * g + 0][cc] | ((uint32_t)tile[4 * g + 1][cc] << 16);
                v.y = (uint32_t)tile[4 * g + 2][cc] | ((uint32_t)tile[4 * g + 3][cc] << 16);
                *(uint2 *)(dst + c * ldp + j0 + 4 * g) = v;
            }
        }
        return;
    }
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = ty + 4 * i;
        const int64_t c = c0 + tx;
        tile[r][tx] = (r < nv && c < C) ? src[(rb + r) * lds + c] : (uint16_t)0;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t c = c0 + ty + 4 * i;
        if (c < C) dst[c * ldp + j0 + tx] = tile[tx][ty + 4 * i];
    }
}

// H[r][f] = act(a1, a3) for the kept rows (r < offsets[E])
template <typename HT>
__global__ __launch_bounds__(256) void act_fwd_kernel(const float *__restrict__ a1,
                                                      const float *__restrict__ a3,
                                                      const int32_t *__restrict__ offsets, int E,
                                                      int d_ff, int act, HT *__restrict__ H) {
    const int64_t n = (int64_t)offsets[E] * d_ff;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        st_elem(H, i, apply_act(act, a1[i], act == ACT_SWIGLU ? a3[i] : 0.f));
}

// one wave per kept row: its token and slot, dE = g dy_t, dg = <dy_t, Y_r>
template <typename DT>
__global__ __launch_bounds__(256) void combine_bwd_kernel(
    const DT *__restrict__ dy, const float *__restrict__ Y, const int32_t *__restrict__ token_of_row,
    const int32_t *__restrict__ row_of_slot, const float *__restrict__ gates,
    const int32_t *__restrict__ offsets, int E, int k, int d, DT *__restrict__ dE,
    float *__restrict__ dg) {
    const int lane = threadIdx.x & 63;
    const int rows = offsets[E];
    for (int r = blockIdx.x * 4 + (threadIdx.x >> 6); r < rows; r += gridDim.x * 4) {
        const int t = token_of_row[r];
        int s = 0;
        for (int q = 0; q < k; ++q)
            if (row_of_slot[(int64_t)t * k + q] == r) s = q;
        const float g = gates[(int64_t)t * k + s];
        float dot = 0.f;
        for (int o = lane; o < d; o += 64) {
            const float v = ld_elem(dy, (int64_t)t * d + o);
            dot = fmaf(v, Y[(int64_t)r * d + o], dot);
            st_elem(dE, (int64_t)r * d + o, g * v);
        }
        dot = wave_sum_f32(dot);
        if (lane == 0) dg[(int64_t)t * k + s] = dot;
    }
}

// dA[r] = [da1 | da3] (storage type; width n_up * d_ff) from dH and the
// pre-activations
template <typename DT>
__global__ __launch_bounds__(256) void act_bwd_kernel(const float *__restrict__ a1,
                                                      const float *__restrict__ a3,
                                                      const float *__restrict__ dH,
                                                      const int32_t *__restrict__ offsets, int E,
                                                      int d_ff, int act, DT *__restrict__ dA) {
    const int64_t n = (int64_t)offsets[E] * d_ff;
    const int nup = act == ACT_SWIGLU ? 2 : 1;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int64_t r = i / d_ff, f = i - r * d_ff;
        DT *row = dA + r * nup * d_ff;
        float da1, da3;
        act_bwd_f32(act, a1[i], act == ACT_SWIGLU ? a3[i] : 0.f, dH[i], da1, da3);
        st_elem(row, f, da1);
        if (act == ACT_SWIGLU) st_elem(row, d_ff + f, da3);
    }
}

// logits for few experts (E <= 32): one wave per token (lane i: experts i,
// i + 64), softmax, lse
template <typename XT>
__global__ __launch_bounds__(256) void logits_wave_kernel(const XT *__restrict__ x,
                                                     const float *__restrict__ Wr,
                                                     const float *__restrict__ bias,
                                                     const float *__restrict__ noise, int T, int d,
                                                     int E, float *__restrict__ p,
                                                     float *__restrict__ lse) {
    const int lane = threadIdx.x & 63;
    for (int t = blockIdx.x * 4 + (threadIdx.x >> 6); t < T; t += gridDim.x * 4) {
        float h0 = -INFINITY, h1 = -INFINITY;
        for (int i = 0; i < E; ++i) {
            float acc = 0.f;
            for (int j = lane; j < d; j += 64)
                acc = fmaf(ld_elem(x, (int64_t)t * d + j), Wr[(int64_t)i * d + j], acc);
            acc = wave_sum_f32(acc);
            if (bias) acc += bias[i];
            if (noise) acc += noise[(int64_t)t * E + i];
            if (i == lane) h0 = acc;
            if (i == lane + 64) h1 = acc;
        }
        const float m = wave_max_f32b(fmaxf(h0, h1));
        const float e0 = lane < E ? expf(h0 - m) : 0.f;
        const float e1 = lane + 64 < E ? expf(h1 - m) : 0.f;
        const float sum = wave_sum_f32(e0 + e1);
        if (lane < E) p[(int64_t)t * E + lane] = e0 / sum;
        if (lane + 64 < E) p[(int64_t)t * E + lane + 64] = e1 / sum;
        if (lane == 0) lse[t] = m + logf(sum);
    }
}

// logits in fp32, then p = softmax and lse: a block per 32 tokens (8 per
// wave), their rows of x staged in LDS 1024 columns at a time; lane i
// accumulates experts i and i + 64 for the wave's 8 tokens, reading its own
// W_r rows 4 columns at a time, each x value a broadcast from LDS.
constexpr int LG_TB = 32, LG_TW = 8, LG_DC = 1024;
template <typename XT>
__global__ __launch_bounds__(256) void logits_kernel(const XT *__restrict__ x,
                                                     const float *__restrict__ Wr,
                                                     const float *__restrict__ bias,
                                                     const float *__restrict__ noise, int T, int d,
                                                     int E, float *__restrict__ p,
                                                     float *__restrict__ lse) {
    __shared__ float xs[LG_TB][LG_DC + 4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * LG_TB;
    const bool e0 = lane < E, e1 = lane + 64 < E;
    float acc0[LG_TW], acc1[LG_TW];
#pragma unroll
    for (int u = 0; u < LG_TW; ++u) acc0[u] = acc1[u] = 0.f;
    for (int c0 = 0; c0 < d; c0 += LG_DC) {
        const int cw = min(LG_DC, d - c0);
        __syncthreads();
        for (int q = threadIdx.x; q < LG_TB * cw; q += 256) {
            const int tt = q / cw, j = q - tt * cw;
            xs[tt][j] = t0 + tt < T ? ld_elem(x, (int64_t)(t0 + tt) * d + c0 + j) : 0.f;
        }
        __syncthreads();
        const float *w0 = Wr + (int64_t)lane * d + c0, *w1 = Wr + (int64_t)(lane + 64) * d + c0;
#pragma unroll 4
        for (int j = 0; j < cw; j += 4) {
            float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = make_float4(0.f, 0.f, 0.f, 0.f);
            if (e0) a = *(const float4 *)(w0 + j);
            if (e1) b = *(const float4 *)(w1 + j);
#pragma unroll
            for (int u = 0; u < LG_TW; ++u) {
                const float *xr = &xs[wave * LG_TW + u][j];
                acc0[u] = fmaf(xr[0], a.x, fmaf(xr[1], a.y, fmaf(xr[2], a.z, fmaf(xr[3], a.w, acc0[u]))));
                acc1[u] = fmaf(xr[0], b.x, fmaf(xr[1], b.y, fmaf(xr[2], b.z, fmaf(xr[3], b.w, acc1[u]))));
            }
        }
    }
#pragma unroll
    for (int u = 0; u < LG_TW; ++u) {
        const int t = t0 + wave * LG_TW + u;
        if (t >= T) break;
        float h0 = -INFINITY, h1 = -INFINITY;
        if (e0) h0 = acc0[u] + (bias ? bias[lane] : 0.f) + (noise ? noise[(int64_t)t * E + lane] : 0.f);
        if (e1) h1 = acc1[u] + (bias ? bias[lane + 64] : 0.f) + (noise ? noise[(int64_t)t * E + lane + 64] : 0.f);
        const float m = wave_max_f32b(fmaxf(h0, h1));
        const float x0 = e0 ? expf(h0 - m) : 0.f;
        const float x1 = e1 ? expf(h1 - m) : 0.f;
        const float sum = wave_sum_f32(x0 + x1);
        if (e0) p[(int64_t)t * E + lane] = x0 / sum;
        if (e1) p[(int64_t)t * E + lane + 64] = x1 / sum;
        if (lane == 0) lse[t] = m + logf(sum);
    }
}

// one wave per token: dh from the gate convention, then the aux and z terms
__global__ __launch_bounds__(256) void router_bwd_kernel(
    const float *__restrict__ p, const float *__restrict__ lse, const int32_t *__restrict__ topk_idx,
    const float *__restrict__ gates, const float *__restrict__ dg, const int32_t *__restrict__ row_of_slot,
    const float *__restrict__ f, int T, int E, int k, int gate, float alpha_aux, float alpha_z,
    float *__restrict__ dh) {
    const int lane = threadIdx.x & 63;
    for (int t = blockIdx.x * 4 + (threadIdx.x >> 6); t < T; t += gridDim.x * 4) {
        const float *pt = p + (int64_t)t * E;
        const float p0 = lane < E ? pt[lane] : 0.f, p1 = lane + 64 < E ? pt[lane + 64] : 0.f;
        float d0 = 0.f, d1 = 0.f;
        // <g, dg> (renormalised) or <p_sel, dg> (Switch), in slot order
        float dot = 0.f;
        for (int s = 0; s < k; ++s) {
            const int64_t q = (int64_t)t * k + s;
            const float dgs = row_of_slot[q] >= 0 ? dg[q] : 0.f;
            const int e = topk_idx[q];
            dot += (gate == 0 ? gates[q] : pt[e]) * dgs;
        }
        for (int s = 0; s < k; ++s) {
            const int64_t q = (int64_t)t * k + s;
            const float dgs = row_of_slot[q] >= 0 ? dg[q] : 0.f;
            const int e = topk_idx[q];
            if (gate == 0) {
                const float v = gates[q] * (dgs - dot);
                if (e == lane) d0 += v;
                if (e == lane + 64) d1 += v;
            } else {
                if (e == lane) d0 += p0 * dgs;
                if (e == lane + 64) d1 += p1 * dgs;
            }
        }
        if (gate != 0) {
            d0 -= p0 * dot;
            d1 -= p1 * dot;
        }
        if (alpha_aux != 0.f) {
            const float a0 = lane < E ? (float)E * f[lane] / (float)T : 0.f;
            const float a1 = lane + 64 < E ? (float)E * f[lane + 64] / (float)T : 0.f;
            const float pa = wave_sum_f32(p0 * a0 + p1 * a1);
            d0 += alpha_aux * p0 * (a0 - pa);
            d1 += alpha_aux * p1 * (a1 - pa);
        }
        if (alpha_z != 0.f) {
            const float c = alpha_z * 2.f / (float)T * lse[t];
            d0 += c * p0;
            d1 += c * p1;
        }
        if (lane < E) dh[(int64_t)t * E + lane] = d0;
        if (lane + 64 < E) dh[(int64_t)t * E + lane + 64] = d1;
    }
}

// dx[t] = sum over kept slots (slot order) of dXp[row] + W_r^T dh_t.  The
// product is a GEMM with K = E on v_mfma_f32_16x16x4_f32 (fp32 operands,
// products exact as in fp32 FMAs, fp32 accumulation in k order; twice the
// rate of unpacked fp32 FMAs): a block per 64 tokens x 64 columns.  Chunks
// of 32 experts of dh (64 x 32) and W_r (32 x 64) are staged in LDS by rows;
// wave w takes tokens 16w .. 16w + 15 and four 16-column fragments, lane l
// reading dh[16w + l % 16][k + l / 16] and W_r[k + l / 16][16n + l % 16]
// (accumulator r of lane l: token 4 (l / 16) + r, column l % 16).  The
// product goes back through LDS, and four threads per token row add the
// kept slots' rows of dXp (slot order) and store 64 contiguous columns.
constexpr int DX_TT = 64, DX_JJ = 64, DX_KC = 32;
__global__ __launch_bounds__(256) void dx_kernel(const float *__restrict__ dXp,
                                                 const int32_t *__restrict__ row_of_slot,
                                                 const float *__restrict__ dh,
                                                 const float *__restrict__ Wr, int T, int d, int E,
                                                 int k, float *__restrict__ dx) {
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    constexpr int SOPS = DX_TT * (DX_KC + 1) + DX_KC * (DX_JJ + 1), SOUT = DX_TT * (DX_JJ + 1);
    __shared__ float sm[SOPS > SOUT ? SOPS : SOUT];       // both operands, then the output tile
    float(*sA)[DX_KC + 1] = (float(*)[DX_KC + 1])sm;      // [64][33]
    float(*sB)[DX_JJ + 1] = (float(*)[DX_JJ + 1])(sm + DX_TT * (DX_KC + 1));   // [32][65]
    float(*sC)[DX_JJ + 1] = (float(*)[DX_JJ + 1])sm;      // [64][65]
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lk = lane >> 4;
    const int t0 = blockIdx.x * DX_TT, j0 = blockIdx.y * DX_JJ;
    f32x4_t acc[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // staging: thread tid loads 8 consecutive dh values of token tid / 4 and
    // 8 consecutive W_r values of expert row tid / 8
    const int ar = tid >> 2, ac = (tid & 3) * 8;
    const int br = tid >> 3, bc = (tid & 7) * 8;
    for (int kc = 0; kc < E; kc += DX_KC) {
        float av[8], bv[8];
        {
            const int t = t0 + ar, kk = kc + ac;
            if (t < T && (E & 3) == 0 && kk + 8 <= E) {
                const float4 u0 = *(const float4 *)(dh + (int64_t)t * E + kk);
                const float4 u1 = *(const float4 *)(dh + (int64_t)t * E + kk + 4);
                av[0] = u0.x, av[1] = u0.y, av[2] = u0.z, av[3] = u0.w;
                av[4] = u1.x, av[5] = u1.y, av[6] = u1.z, av[7] = u1.w;
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) av[q] = (t < T && kk + q < E) ? dh[(int64_t)t * E + kk + q] : 0.f;
            }
            const int kb = kc + br, j = j0 + bc;
            if (kb < E && (d & 3) == 0 && j + 8 <= d) {
                const float4 u0 = *(const float4 *)(Wr + (int64_t)kb * d + j);
                const float4 u1 = *(const float4 *)(Wr + (int64_t)kb * d + j + 4);
                bv[0] = u0.x, bv[1] = u0.y, bv[2] = u0.z, bv[3] = u0.w;
                bv[4] = u1.x, bv[5] = u1.y, bv[6] = u1.z, bv[7] = u1.w;
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) bv[q] = (kb < E && j + q < d) ? Wr[(int64_t)kb * d + j + q] : 0.f;
            }
        }
        __syncthreads();   // the previous chunk's fragments have been read
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            sA[ar][ac + q] = av[q];
            sB[br][bc + q] = bv[q];
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < DX_KC / 4; ++q) {
            const float a = sA[16 * w + lr][4 * q + lk];
#pragma unroll
            for (int n = 0; n < 4; ++n)
                acc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, sB[4 * q + lk][16 * n + lr], acc[n], 0, 0, 0);
        }
    }
    __syncthreads();
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) sC[16 * w + 4 * lk + r][16 * n + lr] = acc[n][r];
    __syncthreads();
    // four threads per token row, 16 columns each
    const int t = t0 + (tid >> 2), c0 = (tid & 3) * 16;
    if (t >= T) return;
    float v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) v[q] = 0.f;
    const bool vec = (d & 3) == 0 && j0 + c0 + 16 <= d;   // 16-byte rows
    for (int sl = 0; sl < k; ++sl) {
        const int row = row_of_slot[(int64_t)t * k + sl];
        if (row < 0) continue;
        const float *src = dXp + (int64_t)row * d + j0 + c0;
        if (vec) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 u = *(const float4 *)(src + 4 * q);
                v[4 * q] += u.x, v[4 * q + 1] += u.y, v[4 * q + 2] += u.z, v[4 * q + 3] += u.w;
            }
        } else {
#pragma unroll
            for (int q = 0; q < 16; ++q)
                if (j0 + c0 + q < d) v[q] += src[q];
        }
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) v[q] += sC[tid >> 2][c0 + q];
    float *dst = dx + (int64_t)t * d + j0 + c0;
    if (vec) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *(float4 *)(dst + 4 * q) = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    } else {
#pragma unroll
        for (int q = 0; q < 16; ++q)
            if (j0 + c0 + q < d) dst[q] = v[q];
    }
}

// dW_r[i][j] = sum_t dh[t][i] x[t][j] in two passes with a fixed order: a
// thread per (column j, split of the tokens) sums its tokens in order for
// 16 experts at a time into partials [split][i][j]; then the splits are
// added in split order.
constexpr int DWR_EG = 16, DWR_SPLITS = 64;
template <typename XT>
__global__ __launch_bounds__(256) void dwr_partial_kernel(const float *__restrict__ dh,
                                                          const XT *__restrict__ x, int T, int d,
                                                          int E, float *__restrict__ part) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    const int i0 = blockIdx.y * DWR_EG;
    const int sp = blockIdx.z;
    if (j >= d) return;
    const int t0 = (int)((int64_t)sp * T / DWR_SPLITS), t1 = (int)((int64_t)(sp + 1) * T / DWR_SPLITS);
    float acc[DWR_EG];
#pragma unroll
    for (int u = 0; u < DWR_EG; ++u) acc[u] = 0.f;
#pragma unroll 8
    for (int t = t0; t < t1; ++t) {
        const float xv = ld_elem(x, (int64_t)t * d + j);
#pragma unroll
        for (int u = 0; u < DWR_EG; ++u)
            if (i0 + u < E) acc[u] = fmaf(dh[(int64_t)t * E + i0 + u], xv, acc[u]);
    }
#pragma unroll
    for (int u = 0; u < DWR_EG; ++u)
        if (i0 + u < E) part[((int64_t)sp * E + i0 + u) * d + j] = acc[u];
}

__global__ __launch_bounds__(256) void dwr_reduce_kernel(const float *__restrict__ part, int64_t n,
                                                         float *__restrict__ dWr) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        float s = 0.f;
        for (int sp = 0; sp < DWR_SPLITS; ++sp) s += part[sp * n + i];
        dWr[i] = s;
    }
}

// dbias[i] = sum_t dh[t][i]: one block per expert, 256 strided partials
// added in thread order
__global__ __launch_bounds__(256) void dbias_kernel(const float *__restrict__ dh, int T, int E,
                                                    float *__restrict__ dbias) {
    __shared__ float part[256];
    const int i = blockIdx.x;
    float acc = 0.f;
    for (int t = threadIdx.x; t < T; t += 256) acc += dh[(int64_t)t * E + i];
    part[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        float s = 0.f;
        for (int u = 0; u < 256; ++u) s += part[u];
        dbias[i] = s;
    }
}

// dh [T][E] -> the three bf16 terms, transposed: P[q Ep + e][t] for t < Tp
// (zeros for t >= T or e >= E); 64 x 64 tiles through LDS.
__global__ __launch_bounds__(256) void split_dh_kernel(const float *__restrict__ dh, int T, int E, int Ep,
                                                       int64_t Tp, uint16_t *__restrict__ P) {
    __shared__ float tile[64][65];
    const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int t = t0 + ty + 4 * i, e = e0 + tx;
        tile[ty + 4 * i][tx] = (t < T && e < E) ? dh[(int64_t)t * E + e] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int e = e0 + ty + 4 * i;
        const int64_t t = t0 + tx;
        if (e < Ep && t < Tp) {
            const float v = tile[tx][ty + 4 * i];
            const uint16_t hi = f32_to_bf16(v);
            const float r1 = v - bf16_to_f32(hi);   // exact
            const uint16_t mid = f32_to_bf16(r1);
            const uint16_t lo = f32_to_bf16(r1 - bf16_to_f32(mid));
            P[(int64_t)e * Tp + t] = hi;
            P[(int64_t)(Ep + e) * Tp + t] = mid;
            P[(int64_t)(2 * Ep + e) * Tp + t] = lo;
        }
    }
}

// W_r [E][d] -> its three bf16 terms as rows e, Ep + e, 2 Ep + e of Ws
// [3 Ep][d] (zero rows for e >= E)
__global__ __launch_bounds__(256) void split_wr_kernel(const float *__restrict__ Wr, int E, int Ep, int d,
                                                       uint16_t *__restrict__ Ws) {
    const int64_t n = (int64_t)Ep * d;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int e = (int)(i / d);
        const float v = e < E ? Wr[i] : 0.f;
        const uint16_t hi = f32_to_bf16(v);
        const float r1 = v - bf16_to_f32(hi);   // exact
        const uint16_t mid = f32_to_bf16(r1);
        Ws[i] = hi;
        Ws[n + i] = mid;
        Ws[2 * n + i] = f32_to_bf16(r1 - bf16_to_f32(mid));
    }
}

// p and lse from the partial logits C [ns][T][3 Ep]: one wave per token,
// lane i holds experts i and i + 64 (E <= 128)
__global__ __launch_bounds__(256) void logits_finish_kernel(const float *__restrict__ C, int ns, int T, int E,
                                                            int Ep, const float *__restrict__ bias,
                                                            const float *__restrict__ noise,
                                                            float *__restrict__ p, float *__restrict__ lse) {
    const int lane = threadIdx.x & 63;
    const int64_t stride = (int64_t)T * 3 * Ep;
    for (int t = blockIdx.x * 4 + (threadIdx.x >> 6); t < T; t += gridDim.x * 4) {
        float h[2] = {-INFINITY, -INFINITY};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int e = lane + 64 * u;
            if (e < E) {
                float a = 0.f;
                for (int q = 2; q >= 0; --q)
                    for (int sp = 0; sp < ns; ++sp) a += C[sp * stride + (int64_t)t * 3 * Ep + q * Ep + e];
                if (bias) a += bias[e];
                if (noise) a += noise[(int64_t)t * E + e];
                h[u] = a;
            }
        }
        const float m = wave_max_f32b(fmaxf(h[0], h[1]));
        const float e0 = lane < E ? expf(h[0] - m) : 0.f;
        const float e1 = lane + 64 < E ? expf(h[1] - m) : 0.f;
        const float sum = wave_sum_f32(e0 + e1);
        if (lane < E) p[(int64_t)t * E + lane] = e0 / sum;
        if (lane + 64 < E) p[(int64_t)t * E + lane + 64] = e1 / sum;
        if (lane == 0) lse[t] = m + logf(sum);
    }
}

// idx = {0, T, 0, Tp, then the ns + 1 token-range starts (multiples of 64)}
__global__ void dwr_index_kernel(int T, int64_t Tp, int ns, int32_t *__restrict__ idx) {
    const int i = threadIdx.x;
    if (i == 0) {
        idx[0] = 0;
        idx[1] = T;
        idx[2] = 0;
        idx[3] = (int)Tp;
    }
    const int64_t chunks = Tp / 64;
    for (int j = i; j <= ns; j += blockDim.x) idx[4 + j] = (int)(j * chunks / ns * 64);
}

// dW_r[e][c] = sum over the terms lo, mid, hi, and within each over the
// token ranges in order, of the partial products C[sp][q Ep + e][c]
__global__ __launch_bounds__(256) void dwr_sum_kernel(const float *__restrict__ C, int ns, int E, int Ep,
                                                      int d, float *__restrict__ dWr) {
    const int64_t n = (int64_t)E * d;
    const int64_t stride = (int64_t)3 * Ep * d;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int e = (int)(i / d), c = (int)(i - (int64_t)e * d);
        float a = 0.f;
        for (int q = 2; q >= 0; --q)
            for (int sp = 0; sp < ns; ++sp) a += C[sp * stride + (int64_t)(q * Ep + e) * d + c];
        dWr[i] = a;
    }
}

// Weight gradients: for expert e, C_e[m][n] = sum over k in [offsets[e],
// offsets[e+1]) of P[m][k] Q[n][k], P [M][ldk] and Q [N][ldk] bf16
// (k-contiguous; the transposed activations), C [E][M][N] fp32.  128 x 128
// tiles, four waves of 64 x 64 on v_mfma_f32_32x32x16_bf16, 32-wide k
// chunks staged in LDS; the chunk start is aligned down to 8 elements and
// elements outside the expert's range are zeroed.  An expert without rows
// gets zeros.
constexpr int WG_BK = 32, WG_LD = WG_BK + 8;
__global__ __launch_bounds__(256) void wgrad_kernel(const uint16_t *__restrict__ P,
                                                    const uint16_t *__restrict__ Q, int64_t ldk,
                                                    const int32_t *__restrict__ offsets, int M, int N,
                                                    float *__restrict__ C) {
    __shared__ __attribute__((aligned(16))) uint16_t As[128][WG_LD];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[128][WG_LD];
    const int tm = (M + 127) / 128, tn = (N + 127) / 128;
    const int e = blockIdx.x / (tm * tn);
    const int rem = blockIdx.x - e * tm * tn;
    const int m0 = (rem / tn) * 128, n0 = (rem % tn) * 128;
    const int k0 = offsets[e], k1 = offsets[e + 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1, lr = lane & 31, lh = lane >> 5;
    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    for (int kb = k0 & ~7; kb < k1; kb += WG_BK) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int c = threadIdx.x + h * 256;  // 512 chunks of 8 per operand
            const int row = c >> 2, kc = (c & 3) * 8;
            const int kg = kb + kc;
            uint4 va = make_uint4(0, 0, 0, 0), vb = make_uint4(0, 0, 0, 0);
            if (kg < k1) {
                if (m0 + row < M) va = *(const uint4 *)(P + (int64_t)(m0 + row) * ldk + kg);
                if (n0 + row < N) vb = *(const uint4 *)(Q + (int64_t)(n0 + row) * ldk + kg);
                if (kg < k0 || kg + 8 > k1) {
                    uint16_t *ea = (uint16_t *)&va, *eb = (uint16_t *)&vb;
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        if (kg + u < k0 || kg + u >= k1) {
                            ea[u] = 0;
                            eb[u] = 0;
                        }
                }
            }
            *(uint4 *)&As[row][kc] = va;
            *(uint4 *)&Bs[row][kc] = vb;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < WG_BK / 16; ++kk) {
            bf16x8_t a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) a[i] = *(const bf16x8_t *)&As[wm * 64 + i * 32 + lr][kk * 16 + lh * 8];
#pragma unroll
            for (int j = 0; j < 2; ++j) b[j] = *(const bf16x8_t *)&Bs[wn * 64 + j * 32 + lr][kk * 16 + lh * 8];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }
    float *Ce = C + (int64_t)e * M * N;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + wn * 64 + j * 32 + lr;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + lh * 4 + (r & 3);
                if (row < M && col < N) Ce[(int64_t)row * N + col] = acc[i][j][r];
            }
        }
}

inline unsigned grid_for(int64_t items, int64_t per_block, int64_t cap) {
    int64_t b = (items + per_block - 1) / per_block;
    if (b > cap) b = cap;
    return (unsigned)(b < 1 ? 1 : b);
}

// fp32 layers (small; plain kernels, one thread per output, sums in a
// fixed order):
// dst[b][c][r] = src[b][r][c] for r < R, c < C; strides in elements
__global__ __launch_bounds__(256) void transpose_f32_kernel(const float *__restrict__ src, int64_t R, int64_t C,
                                                            int64_t lds, int64_t sbs, float *__restrict__ dst,
                                                            int64_t ldd, int64_t dbs, int batch,
                                                            const int32_t *__restrict__ offsets) {
    const int64_t n = (int64_t)batch * R * C;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int64_t b = i / (R * C), rc = i - b * R * C, r = rc / C, c = rc - r * C;
        if (offsets && offsets[b + 1] == offsets[b]) continue;   // an expert without rows
        dst[b * dbs + c * ldd + r] = src[b * sbs + r * lds + c];
    }
}

// C[e][m][n] = sum over the rows r of expert e (in row order) of
// P[r][m] Q[r][n]: the weight gradients of an fp32 layer
__global__ __launch_bounds__(256) void wgrad_f32_kernel(int E, int M, int N, const int32_t *__restrict__ offsets,
                                                        const float *__restrict__ P, int64_t ldp,
                                                        const float *__restrict__ Q, int64_t ldq,
                                                        float *__restrict__ C) {
    const int64_t n_out = (int64_t)E * M * N;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n_out; i += (int64_t)gridDim.x * 256) {
        const int64_t e = i / ((int64_t)M * N), mn = i - e * M * N, m = mn / N, n = mn - m * N;
        float acc = 0.f;
        for (int r = offsets[e]; r < offsets[e + 1]; ++r) acc = fmaf(P[(int64_t)r * ldp + m], Q[(int64_t)r * ldq + n], acc);
        C[i] = acc;
    }
}

}  // namespace

hipError_t launch_transpose_bf16(const void *src, int64_t R, int64_t C, int64_t lds, int64_t sbs,
                                 void *dst, int64_t ldd, int64_t dbs, int batch, hipStream_t st,
                                 const int32_t *offsets) {
    if (R <= 0 || C <= 0 || batch <= 0) return hipSuccess;
    dim3 grid((unsigned)((C + 63) / 64), (unsigned)((R + 63) / 64), (unsigned)batch);
    const bool vec = R % 4 == 0 && C % 4 == 0 && lds % 4 == 0 && ldd % 4 == 0 && sbs % 4 == 0 &&
                     dbs % 4 == 0 && (uintptr_t)src % 8 == 0 && (uintptr_t)dst % 8 == 0;
    if (vec)
        hipLaunchKernelGGL(transpose_kernel<true>, grid, dim3(256), 0, st, (const uint16_t *)src, R, C, lds,
                           sbs, (uint16_t *)dst, ldd, dbs, offsets);
    else
        hipLaunchKernelGGL(transpose_kernel<false>, grid, dim3(256), 0, st, (const uint16_t *)src, R, C, lds,
                           sbs, (uint16_t *)dst, ldd, dbs, offsets);
    return hipGetLastError();
}

int64_t padded_rows_bound(int64_t R, int E) { return (R + 63 * (int64_t)E + 63) / 64 * 64; }

hipError_t launch_pad_offsets(const int32_t *offsets, int E, int32_t *poff, hipStream_t st) {
    if (E < 1 || E > 128) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pad_offsets_kernel, dim3(1), dim3(64), 0, st, offsets, E, poff);
    return hipGetLastError();
}

hipError_t launch_transpose_padded(const void *src, int64_t C, int64_t lds, const int32_t *offsets,
                                   const int32_t *poff, int E, int64_t ldp, void *dst, hipStream_t st) {
    if (C <= 0 || ldp <= 0) return hipSuccess;
    if (ldp % 64 != 0 || ldp / 64 > 65535) return hipErrorInvalidValue;
    dim3 grid((unsigned)((C + 63) / 64), (unsigned)(ldp / 64));
    const bool vec = C % 4 == 0 && lds % 4 == 0 && (uintptr_t)src % 8 == 0 && (uintptr_t)dst % 8 == 0;
    if (vec)
        hipLaunchKernelGGL(transpose_padded_kernel<true>, grid, dim3(256), 0, st, (const uint16_t *)src, C, lds,
                           offsets, poff, E, (uint16_t *)dst, ldp);
    else
        hipLaunchKernelGGL(transpose_padded_kernel<false>, grid, dim3(256), 0, st, (const uint16_t *)src, C, lds,
                           offsets, poff, E, (uint16_t *)dst, ldp);
    return hipGetLastError();
}

hipError_t launch_act_fwd(const Shape &s, const float *a1, const float *a3, const int32_t *offsets,
                          void *H, hipStream_t st) {
    const dim3 g(grid_for((int64_t)s.Tk() * s.d_ff, 256, 16384));
    if (s.dtype == 0)
        hipLaunchKernelGGL(act_fwd_kernel<float>, g, dim3(256), 0, st, a1, a3, offsets, s.E, s.d_ff, s.act,
                           (float *)H);
    else
        hipLaunchKernelGGL(act_fwd_kernel<uint16_t>, g, dim3(256), 0, st, a1, a3, offsets, s.E, s.d_ff, s.act,
                           (uint16_t *)H);
    return hipGetLastError();
}

hipError_t launch_combine_bwd(const Shape &s, const void *dy, const float *Y, const int32_t *token_of_row,
                              const int32_t *row_of_slot, const float *gates, const int32_t *offsets,
                              void *dE, float *dg, hipStream_t st) {
    const dim3 g(grid_for(s.Tk(), 4, 16384));
    if (s.dtype == 0)
        hipLaunchKernelGGL(combine_bwd_kernel<float>, g, dim3(256), 0, st, (const float *)dy, Y, token_of_row,
                           row_of_slot, gates, offsets, s.E, s.k, s.d, (float *)dE, dg);
    else
        hipLaunchKernelGGL(combine_bwd_kernel<uint16_t>, g, dim3(256), 0, st, (const uint16_t *)dy, Y,
                           token_of_row, row_of_slot, gates, offsets, s.E, s.k, s.d, (uint16_t *)dE, dg);
    return hipGetLastError();
}

hipError_t launch_act_bwd(const Shape &s, const float *a1, const float *a3, const float *dH,
                          const int32_t *offsets, void *dA, hipStream_t st) {
    const dim3 g(grid_for((int64_t)s.Tk() * s.d_ff, 256, 16384));
    if (s.dtype == 0)
        hipLaunchKernelGGL(act_bwd_kernel<float>, g, dim3(256), 0, st, a1, a3, dH, offsets, s.E, s.d_ff, s.act,
                           (float *)dA);
    else
        hipLaunchKernelGGL(act_bwd_kernel<uint16_t>, g, dim3(256), 0, st, a1, a3, dH, offsets, s.E, s.d_ff,
                           s.act, (uint16_t *)dA);
    return hipGetLastError();
}

hipError_t launch_transpose_f32(const float *src, int64_t R, int64_t C, int64_t lds, int64_t sbs, float *dst,
                                int64_t ldd, int64_t dbs, int batch, hipStream_t st, const int32_t *offsets) {
    if (R <= 0 || C <= 0 || batch <= 0) return hipSuccess;
    hipLaunchKernelGGL(transpose_f32_kernel, dim3(grid_for((int64_t)batch * R * C, 256, 16384)), dim3(256), 0,
                       st, src, R, C, lds, sbs, dst, ldd, dbs, batch, offsets);
    return hipGetLastError();
}

hipError_t launch_wgrad_f32(int E, int M, int N, const int32_t *offsets, const float *P, int64_t ldp,
                            const float *Q, int64_t ldq, float *C, hipStream_t st) {
    hipLaunchKernelGGL(wgrad_f32_kernel, dim3(grid_for((int64_t)E * M * N, 256, 16384)), dim3(256), 0, st, E, M,
                       N, offsets, P, ldp, Q, ldq, C);
    return hipGetLastError();
}

hipError_t launch_router_bwd(const Shape &s, const void *x, const float *Wr, const float *bias,
                             const float *noise, const int32_t *topk_idx, const float *gates,
                             const float *dg, const int32_t *row_of_slot, const float *f,
                             float alpha_aux, float alpha_z, float *p, float *lse, float *dh,
                             hipStream_t st, bool logits) {
    const unsigned g = grid_for(s.T, 4, 16384);
    if (logits) {
        const dim3 gl((unsigned)((s.T + LG_TB - 1) / LG_TB));
        if (s.dtype == 0) {
            if (s.E <= 32)
                hipLaunchKernelGGL(logits_wave_kernel<float>, dim3(g), dim3(256), 0, st, (const float *)x, Wr,
                                   bias, noise, s.T, s.d, s.E, p, lse);
            else
                hipLaunchKernelGGL(logits_kernel<float>, gl, dim3(256), 0, st, (const float *)x, Wr, bias, noise,
                                   s.T, s.d, s.E, p, lse);
        } else {
            if (s.E <= 32)
                hipLaunchKernelGGL(logits_wave_kernel<uint16_t>, dim3(g), dim3(256), 0, st, (const uint16_t *)x,
                                   Wr, bias, noise, s.T, s.d, s.E, p, lse);
            else
                hipLaunchKernelGGL(logits_kernel<uint16_t>, gl, dim3(256), 0, st, (const uint16_t *)x, Wr, bias,
                                   noise, s.T, s.d, s.E, p, lse);
        }
    }
    hipLaunchKernelGGL(router_bwd_kernel, dim3(g), dim3(256), 0, st, (const float *)p, (const float *)lse,
                       topk_idx, gates, dg, row_of_slot, f, s.T, s.E, s.k, s.gate, alpha_aux, alpha_z, dh);
    return hipGetLastError();
}

hipError_t launch_dx(const Shape &s, const float *dXp, const int32_t *row_of_slot, const float *dh,
                     const float *Wr, float *dx, hipStream_t st) {
    dim3 grid((unsigned)((s.T + DX_TT - 1) / DX_TT), (unsigned)((s.d + DX_JJ - 1) / DX_JJ));
    hipLaunchKernelGGL(dx_kernel, grid, dim3(256), 0, st, dXp, row_of_slot, dh, Wr, s.T, s.d, s.E, s.k, dx);
    return hipGetLastError();
}

size_t dwr_part_floats(const Shape &s) { return (size_t)DWR_SPLITS * s.E * s.d; }

hipError_t launch_dwr(const Shape &s, const float *dh, const void *x, float *part, float *dWr,
                      float *dbias, hipStream_t st) {
    dim3 grid((unsigned)((s.d + 255) / 256), (unsigned)((s.E + DWR_EG - 1) / DWR_EG), DWR_SPLITS);
    if (s.dtype == 0)
        hipLaunchKernelGGL(dwr_partial_kernel<float>, grid, dim3(256), 0, st, dh, (const float *)x, s.T, s.d,
                           s.E, part);
    else
        hipLaunchKernelGGL(dwr_partial_kernel<uint16_t>, grid, dim3(256), 0, st, dh, (const uint16_t *)x, s.T,
                           s.d, s.E, part);
    const int64_t n = (int64_t)s.E * s.d;
    hipLaunchKernelGGL(dwr_reduce_kernel, dim3(grid_for(n, 256, 4096)), dim3(256), 0, st, (const float *)part,
                       n, dWr);
    if (dbias) hipLaunchKernelGGL(dbias_kernel, dim3((unsigned)s.E), dim3(256), 0, st, dh, s.T, s.E, dbias);
    return hipGetLastError();
}

DwrPlan dwr_plan(const Shape &s) {
    DwrPlan pl{};
    pl.Ep = (s.E + 7) / 8 * 8;
    pl.Tp = ((int64_t)s.T + 63) / 64 * 64;
    // E < 16: the token-split kernel is as fast (Mixtral layer, E = 8: 56
    // against 55 us; the three terms fill only 3 Ep of a tile's 256 rows)
    if (s.E < 16 || !wgrad_big_fits(3 * pl.Ep, s.d, pl.Tp) || pl.Tp / 64 > 65535) return pl;   // ns = 0
    // about 512 blocks of 256 x 256 output tiles, each range >= 4 k stages
    const int64_t tiles = (int64_t)((3 * pl.Ep + 255) / 256) * ((s.d + 255) / 256);
    int64_t ns = (512 + tiles - 1) / tiles;
    const int64_t most = pl.Tp / 256 > 0 ? pl.Tp / 256 : 1;
    if (ns > most) ns = most;
    if (ns > 64) ns = 64;
    pl.ns = (int)(ns < 1 ? 1 : ns);
    pl.xt_bytes = (size_t)s.d * pl.Tp * 2;
    pl.p_bytes = (size_t)3 * pl.Ep * pl.Tp * 2;
    pl.c_bytes = (size_t)pl.ns * 3 * pl.Ep * s.d * 4;
    pl.idx_bytes = (size_t)(4 + pl.ns + 1) * 4;
    return pl;
}

LogitsPlan logits_plan(const Shape &s) {
    LogitsPlan pl{};
    pl.Ep = (s.E + 7) / 8 * 8;
    if (s.d % 64 != 0 || s.T % 8 != 0 || !wgrad_big_fits(s.T, 3 * pl.Ep, s.d)) return pl;   // ns = 0
    const int64_t tiles = (int64_t)((s.T + 255) / 256) * ((3 * pl.Ep + 255) / 256);
    int64_t ns = (512 + tiles - 1) / tiles;
    const int64_t most = s.d / 256 > 0 ? s.d / 256 : 1;
    if (ns > most) ns = most;
    if (ns > 64) ns = 64;
    pl.ns = (int)(ns < 1 ? 1 : ns);
    pl.ws_bytes = (size_t)3 * pl.Ep * s.d * 2;
    pl.c_bytes = (size_t)pl.ns * s.T * 3 * pl.Ep * 4;
    pl.idx_bytes = (size_t)(4 + pl.ns + 1) * 4;
    return pl;
}

hipError_t launch_logits_mfma(const Shape &s, const LogitsPlan &pl, const void *x, const float *Wr,
                              const float *bias, const float *noise, void *wsplit, float *cpart,
                              int32_t *idx, float *p, float *lse, hipStream_t st) {
    if (pl.ns < 1) return hipErrorInvalidValue;
    // ranges of d: idx[4 ..] (the first four entries are not used here)
    hipLaunchKernelGGL(dwr_index_kernel, dim3(1), dim3(64), 0, st, s.d, (int64_t)s.d, pl.ns, idx);
    hipLaunchKernelGGL(split_wr_kernel, dim3(grid_for((int64_t)pl.Ep * s.d, 256, 4096)), dim3(256), 0, st, Wr,
                       s.E, pl.Ep, s.d, (uint16_t *)wsplit);
    hipError_t err = launch_wgrad_big(pl.ns, s.T, 3 * pl.Ep, idx + 4, x, wsplit, s.d, cpart, st);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(logits_finish_kernel, dim3(grid_for(s.T, 4, 16384)), dim3(256), 0, st,
                       (const float *)cpart, pl.ns, s.T, s.E, pl.Ep, bias, noise, p, lse);
    return hipGetLastError();
}

hipError_t launch_dwr_mfma(const Shape &s, const DwrPlan &pl, const float *dh, const void *x, void *xt,
                           void *pterms, float *cpart, int32_t *idx, float *dWr, float *dbias,
                           hipStream_t st) {
    if (pl.ns < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(dwr_index_kernel, dim3(1), dim3(64), 0, st, s.T, pl.Tp, pl.ns, idx);
    hipLaunchKernelGGL(split_dh_kernel, dim3((unsigned)(pl.Tp / 64), (unsigned)((pl.Ep + 63) / 64)), dim3(256),
                       0, st, dh, s.T, s.E, pl.Ep, pl.Tp, (uint16_t *)pterms);
    hipError_t err = launch_transpose_padded(x, s.d, s.d, idx, idx + 2, 1, pl.Tp, xt, st);
    if (err != hipSuccess) return err;
    err = launch_wgrad_big(pl.ns, 3 * pl.Ep, s.d, idx + 4, pterms, xt, pl.Tp, cpart, st);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(dwr_sum_kernel, dim3(grid_for((int64_t)s.E * s.d, 256, 4096)), dim3(256), 0, st,
                       (const float *)cpart, pl.ns, s.E, pl.Ep, s.d, dWr);
    if (dbias) hipLaunchKernelGGL(dbias_kernel, dim3((unsigned)s.E), dim3(256), 0, st, dh, s.T, s.E, dbias);
    return hipGetLastError();
}

hipError_t launch_wgrad(int E, int M, int N, const int32_t *offsets, const void *P, const void *Q,
                        int64_t ldk, float *C, hipStream_t st) {
    const unsigned blocks = (unsigned)E * (unsigned)((M + 127) / 128) * (unsigned)((N + 127) / 128);
    hipLaunchKernelGGL(wgrad_kernel, dim3(blocks), dim3(256), 0, st, (const uint16_t *)P, (const uint16_t *)Q,
                       ldk, offsets, M, N, C);
    return hipGetLastError();
}

}  // namespace moe
