// route.hip -- router logits, softmax, top-k, gates and load-balancing
// statistics.
//
// Page "Mixture of experts" (rayaq.ca), Mechanics:
//   "Replacing the feed-forward block": h = W_r x, p = softmax(h);
//   "Top-k gating": keep the k largest logits; Switch gate = full-softmax p,
//     renormalised gate = softmax over the k selected logits; noise, when
//     given, is added to the logits before the top-k;
//   "The load-balancing loss": f_i (share of tokens whose top choice is i),
//     P_i (mean router probability), and the z statistic mean (log sum exp h)^2;
//   Implementation: the router runs in float32.
//
// Kernel route_kernel: one block of 256 threads per ROUTE_TOKENS tokens.
//   1. Logits: a [ROUTE_TOKENS x E] fp32 tile accumulated over d in chunks
//      staged through LDS; each thread owns 4 tokens x 4 experts and sums
//      its dot products sequentially in j (fp32 FMA).
//   2. Per token, one wave holds the E <= 128 logits in registers (lane l:
//      experts l and l+64), reduces max and sum of exponentials with
//      shuffles, and picks the top k by k arg-max reductions over 64-bit
//      keys (orderable logit bits, then the complement of the index so that
//      a tie goes to the lower index).
//   3. Per-block partial sums of p (per expert) and of lse^2 go to the
//      workspace in a fixed order; route_finalize_kernel reduces them in
//      double, in block order, and counts top choices.
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int RT_THREADS = 256;
constexpr int RT_DC = 32;                 // d chunk staged per iteration
constexpr int RT_EMAX = 128;              // logits tile width (MOE_MAX_EXPERTS)

// Monotone map of fp32 bits to uint32: a < b  <=>  ord(a) < ord(b) (no NaN);
// -0 and +0 map to the same key, as they compare equal.
__device__ __forceinline__ uint32_t ord_f32(float f) {
    uint32_t u = (f == 0.f) ? 0u : __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float wave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
    for (int o = 32; o > 0; o >>= 1) {
        unsigned long long w = __shfl_xor(v, o);
        v = w > v ? w : v;
    }
    return v;
}

template <bool BF16>
__device__ __forceinline__ float load_x(const void *x, int64_t i) {
    if (BF16) return bf16_to_f32(((const uint16_t *)x)[i]);
    return ((const float *)x)[i];
}

template <bool BF16>
__global__ __launch_bounds__(RT_THREADS) void route_kernel(
    const void *__restrict__ x, const float *__restrict__ Wr, const float *__restrict__ bias,
    const float *__restrict__ noise, int T, int d, int E, int k, int gate_switch,
    int32_t *__restrict__ topk_idx, float *__restrict__ gates, float *__restrict__ part_P,
    float *__restrict__ part_lse2) {
    __shared__ float xs[ROUTE_TOKENS][RT_DC + 1];
    __shared__ float wsh[RT_EMAX][RT_DC + 1];
    __shared__ float hl[ROUTE_TOKENS][RT_EMAX + 1];
    __shared__ float pw[4][RT_EMAX];
    __shared__ float lw[4];

    const int tid = threadIdx.x;
    const int t0 = blockIdx.x * ROUTE_TOKENS;
    const int tg = tid >> 5;  // 8 token groups of 4 tokens
    const int eg = tid & 31;  // 32 expert groups; experts eg + 32*j

    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

    for (int c0 = 0; c0 < d; c0 += RT_DC) {
        // stage x[t0 .. t0+32)[c0 .. c0+32) and W_r[0..E)[c0 .. c0+32)
        for (int i = tid; i < ROUTE_TOKENS * RT_DC; i += RT_THREADS) {
            int r = i / RT_DC, c = i % RT_DC;
            int t = t0 + r;
            xs[r][c] = (t < T && c0 + c < d) ? load_x<BF16>(x, (int64_t)t * d + c0 + c) : 0.f;
        }
        for (int i = tid; i < RT_EMAX * RT_DC; i += RT_THREADS) {
            int r = i / RT_DC, c = i % RT_DC;
            wsh[r][c] = (r < E && c0 + c < d) ? Wr[(int64_t)r * d + c0 + c] : 0.f;
        }
        __syncthreads();
#pragma unroll 4
        for (int c = 0; c < RT_DC; ++c) {
            float xv[4], wv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) xv[i] = xs[tg * 4 + i][c];
#pragma unroll
            for (int j = 0; j < 4; ++j) wv[j] = wsh[eg + 32 * j][c];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(xv[i], wv[j], acc[i][j]);
        }
        __syncthreads();
    }

    // logits + bias + noise into LDS
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int r = tg * 4 + i, t = t0 + r;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int e = eg + 32 * j;
            float h = acc[i][j];
            if (e < E && t < T) {
                if (bias) h += bias[e];
                if (noise) h += noise[(int64_t)t * E + e];
            }
            hl[r][e] = h;
        }
    }
    __syncthreads();

    // per-token softmax / top-k / gates: wave w takes tokens w, w+4, ...
    const int lane = tid & 63, w = tid >> 6;
    const int e0 = lane, e1 = lane + 64;
    const bool v0 = e0 < E, v1 = e1 < E;
    float psum0 = 0.f, psum1 = 0.f, lsum = 0.f;
    for (int r = w; r < ROUTE_TOKENS; r += 4) {
        const int t = t0 + r;
        if (t >= T) break;
        const float h0 = v0 ? hl[r][e0] : -INFINITY;
        const float h1 = v1 ? hl[r][e1] : -INFINITY;
        const float m = wave_max(fmaxf(h0, h1));
        const float x0 = v0 ? expf(h0 - m) : 0.f;
        const float x1 = v1 ? expf(h1 - m) : 0.f;
        const float s = wave_sum(x0 + x1);
        const float inv = 1.f / s;
        psum0 += x0 * inv;
        psum1 += x1 * inv;
        const float lse = m + logf(s);
        lsum += lse * lse;

        unsigned long long k0 = v0 ? ((unsigned long long)ord_f32(h0) << 32) | (0xffffffffu - (uint32_t)e0) : 0ull;
        unsigned long long k1 = v1 ? ((unsigned long long)ord_f32(h1) << 32) | (0xffffffffu - (uint32_t)e1) : 0ull;
        // lane (s & 63) keeps slot s: register 0 for s < 64, register 1 above
        float h_top = 0.f, den = 0.f, sh0 = 0.f, sh1 = 0.f;
        int si0 = 0, si1 = 0;
        for (int sl = 0; sl < k; ++sl) {
            unsigned long long best = wave_max_u64(k0 > k1 ? k0 : k1);
            int bi = (int)(0xffffffffu - (uint32_t)(best & 0xffffffffull));
            bi = bi < 0 ? 0 : bi;  // unreachable while k <= E (validated on the host)
            if (bi == e0) k0 = 0ull;
            if (bi == e1) k1 = 0ull;
            float hb = hl[r][bi];  // the selected logit (same address on every lane)
            if (sl == 0) h_top = hb;
            den += expf(hb - h_top);  // slot order, identical on every lane
            if (lane == (sl & 63)) {
                if (sl < 64) { sh0 = hb; si0 = bi; }
                else         { sh1 = hb; si1 = bi; }
            }
        }
        for (int sl = lane, j = 0; sl < k; sl += 64, ++j) {
            float hb = j ? sh1 : sh0;
            float g = gate_switch ? expf(hb - m) * inv : expf(hb - h_top) / den;
            topk_idx[(int64_t)t * k + sl] = j ? si1 : si0;
            gates[(int64_t)t * k + sl] = g;
        }
    }
    // block partials in a fixed order: waves 0..3.  lsum is the same on
    // every lane of a wave (it sums wave-uniform values).
    pw[w][e0] = psum0;
    pw[w][e1] = psum1;
    if (lane == 0) lw[w] = lsum;
    __syncthreads();
    if (tid < E) {
        float a = pw[0][tid] + pw[1][tid];
        a += pw[2][tid];
        a += pw[3][tid];
        part_P[(int64_t)blockIdx.x * E + tid] = a;
    }
    if (tid == 0) part_lse2[blockIdx.x] = ((lw[0] + lw[1]) + lw[2]) + lw[3];
}

__global__ __launch_bounds__(256) void route_finalize_kernel(
    const int32_t *__restrict__ topk_idx, const float *__restrict__ part_P,
    const float *__restrict__ part_lse2, int T, int E, int k, int nblk,
    float *__restrict__ stats) {
    __shared__ int cnt[RT_EMAX];
    __shared__ double fP[RT_EMAX];
    __shared__ double zsh;
    const int tid = threadIdx.x;
    if (tid < RT_EMAX) cnt[tid] = 0;
    __syncthreads();
    for (int t = tid; t < T; t += blockDim.x) atomicAdd(&cnt[topk_idx[(int64_t)t * k]], 1);
    if (tid == 64) {
        double z = 0.0;
        for (int b = 0; b < nblk; ++b) z += (double)part_lse2[b];
        zsh = z / (double)T;
    }
    __syncthreads();
    if (tid < E) {
        double P = 0.0;
        for (int b = 0; b < nblk; ++b) P += (double)part_P[(int64_t)b * E + tid];
        P /= (double)T;
        double f = (double)cnt[tid] / (double)T;
        stats[tid] = (float)f;
        stats[E + tid] = (float)P;
        fP[tid] = f * P;
    }
    __syncthreads();
    if (tid == 0) {
        double a = 0.0;
        for (int i = 0; i < E; ++i) a += fP[i];
        stats[2 * E] = (float)((double)E * a);
        stats[2 * E + 1] = (float)zsh;
    }
}

}  // namespace

hipError_t launch_route(const Shape &s, const void *x, const float *Wr, const float *bias,
                        const float *noise, int32_t *topk_idx, float *gates, float *part_P,
                        float *part_lse2, hipStream_t st) {
    dim3 grid(route_blocks(s)), block(RT_THREADS);
    if (s.dtype == 1)
        hipLaunchKernelGGL(route_kernel<true>, grid, block, 0, st, x, Wr, bias, noise, s.T, s.d,
                           s.E, s.k, s.gate, topk_idx, gates, part_P, part_lse2);
    else
        hipLaunchKernelGGL(route_kernel<false>, grid, block, 0, st, x, Wr, bias, noise, s.T, s.d,
                           s.E, s.k, s.gate, topk_idx, gates, part_P, part_lse2);
    return hipGetLastError();
}

hipError_t launch_route_finalize(const Shape &s, const int32_t *topk_idx, const float *part_P,
                                 const float *part_lse2, float *stats, hipStream_t st) {
    hipLaunchKernelGGL(route_finalize_kernel, dim3(1), dim3(256), 0, st, topk_idx, part_P,
                       part_lse2, s.T, s.E, s.k, route_blocks(s), stats);
    return hipGetLastError();
}

}  // namespace moe
