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
// bf16 activations (the MFMA path), two kernels:
//   router_logits_kernel  v_mfma_f32_16x16x32_bf16 over a 64-token x E tile,
//     split over d into slices (so that a 32-token decode batch still
//     spreads over many CUs); each slice writes fp32 partial logits.  The
//     fp32 router matrix is split exactly into three bf16 terms as it is
//     staged, W = hi + mid + lo: hi = bf16(W), mid = bf16(W - hi),
//     lo = bf16(W - hi - mid); each difference is exact in fp32 and the last
//     one has at most 8 significant bits, so the three terms sum to W.  A
//     bf16 token times a bf16 term is exact in fp32, hence
//     x.W = x.hi + x.mid + x.lo with fp32 accumulation: an fp32 router whose
//     only rounding is in the accumulation, computed on bf16 MFMA.
//   route_epilogue_kernel  per token: partial logits summed in slice order,
//     plus bias and noise, then the shared per-token epilogue below.
// fp32 activations: route_f32_kernel, a plain fp32 FMA tile over d staged
//   through LDS, then the same per-token epilogue.
//
// Per-token epilogue (one wave per token, E <= 128 logits in registers:
// lane l holds experts l and l+64): max and sum of exponentials by shuffle
// reductions, top-k by k arg-max reductions over 64-bit keys (orderable
// logit bits, then the complement of the index, so a tie goes to the lower
// index), gates, and per-block partials: sums of p and counts of top
// choices (per expert) and the sum of lse^2, in a fixed order.
// route_stats_kernel reduces the partials in double in a fixed order.
#include "moe_internal.h"

namespace moe {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int RT_THREADS = 256;
constexpr int RT_DC = 32;      // d chunk of the fp32 path
constexpr int RT_EMAX = 128;   // MOE_MAX_EXPERTS
constexpr int RL_BM = 64;      // tokens per logits block
constexpr int RL_KC = 64;      // d chunk per iteration
constexpr int RL_LDK = RL_KC + 8;

// Monotone map of fp32 bits to uint32: a < b  <=>  ord(a) < ord(b) (no NaN);
// -0 and +0 map to the same key, as they compare equal.
__device__ __forceinline__ uint32_t ord_f32(float f) {
    uint32_t u = (f == 0.f) ? 0u : __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave reductions on the VALU's cross-lane moves (DPP) instead of LDS
// permutes: within each row of 16 lanes, swap neighbours (quad_perm 1,0,3,2),
// pairs (2,3,0,1), then mirror the half-rows and the row, so that every lane
// of a row holds the row's result; the four rows are then read with
// readlane and combined in row order (a fixed order, so sums are
// reproducible).  DPP control codes: quad_perm 0xB1 and 0x4E, row_half_mirror
// 0x141, row_mirror 0x140.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long v) {
    const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
    return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ float rows_f32(float v, int r) { return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), r)); }

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_f32<0xB1>(v));
    v = fmaxf(v, dpp_f32<0x4E>(v));
    v = fmaxf(v, dpp_f32<0x141>(v));
    v = fmaxf(v, dpp_f32<0x140>(v));
    return fmaxf(fmaxf(rows_f32(v, 0), rows_f32(v, 16)), fmaxf(rows_f32(v, 32), rows_f32(v, 48)));
}

__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f32<0xB1>(v);
    v += dpp_f32<0x4E>(v);
    v += dpp_f32<0x141>(v);
    v += dpp_f32<0x140>(v);
    return ((rows_f32(v, 0) + rows_f32(v, 16)) + rows_f32(v, 32)) + rows_f32(v, 48);
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
    unsigned long long w;
    w = dpp_u64<0xB1>(v);
    v = w > v ? w : v;
    w = dpp_u64<0x4E>(v);
    v = w > v ? w : v;
    w = dpp_u64<0x141>(v);
    v = w > v ? w : v;
    w = dpp_u64<0x140>(v);
    v = w > v ? w : v;
    unsigned long long best = 0ull;
#pragma unroll
    for (int r = 0; r < 64; r += 16) {
        const unsigned long long x = ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), r) << 32) |
                                     (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, r);
        best = x > best ? x : best;
    }
    return best;
}

// Reductions within groups of G = 8 or 16 lanes (a token per group): the
// same DPP steps as wave_max, stopped at the group.
template <int G>
__device__ __forceinline__ float group_max(float v) {
    v = fmaxf(v, dpp_f32<0xB1>(v));
    v = fmaxf(v, dpp_f32<0x4E>(v));
    v = fmaxf(v, dpp_f32<0x141>(v));
    if (G == 16) v = fmaxf(v, dpp_f32<0x140>(v));
    return v;
}
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    v += dpp_f32<0xB1>(v);
    v += dpp_f32<0x4E>(v);
    v += dpp_f32<0x141>(v);
    if (G == 16) v += dpp_f32<0x140>(v);
    return v;
}
template <int G>
__device__ __forceinline__ unsigned long long group_max_u64(unsigned long long v) {
    unsigned long long w;
    w = dpp_u64<0xB1>(v);
    v = w > v ? w : v;
    w = dpp_u64<0x4E>(v);
    v = w > v ? w : v;
    w = dpp_u64<0x141>(v);
    v = w > v ? w : v;
    if (G == 16) {
        w = dpp_u64<0x140>(v);
        v = w > v ? w : v;
    }
    return v;
}

// softmax_topk_block for E <= G: lane l serves expert l % G of token
// l / G of the wave's current group of 64 / G tokens, so a wave takes 8
// (E <= 8) or 4 (E <= 16) tokens at a time.  Same results as the one-token-
// per-wave form (every reduction is within the token's lanes); the block
// partials are added in (wave, token group) order.
template <int G, int TILE, int NW>
__device__ void softmax_topk_grouped(const float (*hl)[RT_EMAX + 1], int t0, int T, int E, int k,
                                     int gate_switch, int32_t *__restrict__ topk_idx,
                                     float *__restrict__ gates, float *__restrict__ part_P,
                                     float *__restrict__ part_lse2, int *topk_sh, float *P_sh,
                                     float *lse2_sh) {
    constexpr int TPW = 64 / G;   // tokens per wave at a time
    __shared__ float pwg[NW][64];
    __shared__ float lsg[NW][TPW];
    __shared__ int topchg[TILE];
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int g = lane / G, e = lane % G;
    const bool ve = e < E;
    float psum = 0.f, lsum = 0.f;
    for (int r0 = w * TPW; r0 < TILE; r0 += NW * TPW) {
        if (t0 + r0 >= T) break;   // uniform in the wave
        const int r = r0 + g, t = t0 + r;
        const bool vt = r < TILE && t < T;
        const bool v = ve && vt;
        const float h = v ? hl[r][e] : -INFINITY;
        const float m = group_max<G>(h);
        const float x = v ? expf(h - m) : 0.f;
        const float s = group_sum<G>(x);
        const float inv = 1.f / s;
        if (v) psum += x * inv;
        const float lse = m + logf(s);
        if (vt && e == 0) lsum += lse * lse;
        unsigned long long key = v ? ((unsigned long long)ord_f32(h) << 32) | (0xffffffffu - (uint32_t)e) : 0ull;
        float h_top = 0.f, den = 0.f, my_hb = 0.f;
        int my_bi = 0;
        for (int sl = 0; sl < k; ++sl) {
            const unsigned long long best = group_max_u64<G>(key);
            int bi = (int)(0xffffffffu - (uint32_t)(best & 0xffffffffull));
            bi = bi < 0 ? 0 : bi;  // only for a token past T (its key is 0)
            if (bi == e) key = 0ull;
            const float hb = vt ? hl[r][bi] : 0.f;
            if (sl == 0) {
                h_top = hb;
                if (vt && e == 0) topchg[r] = bi;
            }
            den += expf(hb - h_top);  // slot order, identical on the token's lanes
            if (e == sl) {
                my_hb = hb;
                my_bi = bi;
            }
        }
        if (vt && e < k) {
            const float gt = gate_switch ? expf(my_hb - m) * inv : expf(my_hb - h_top) / den;
            topk_idx[(int64_t)t * k + e] = my_bi;
            if (topk_sh) topk_sh[t * k + e] = my_bi;  // LDS copy (small batches)
            gates[(int64_t)t * k + e] = gt;
        }
    }
    pwg[w][lane] = psum;
    if (e == 0) lsg[w][g] = lsum;
    __syncthreads();
    if (tid < E) {
        float a = 0.f;
        for (int v = 0; v < NW; ++v)
#pragma unroll
            for (int q = 0; q < TPW; ++q) a += pwg[v][q * G + tid];
        const int64_t nblk = gridDim.x;
        int c = 0;
        for (int r = 0, nr = min(TILE, T - t0); r < nr; ++r) c += topchg[r] == tid;
        part_P[(int64_t)tid * nblk + blockIdx.x] = a;
        part_P[(int64_t)(E + tid) * nblk + blockIdx.x] = (float)c;
        if (P_sh) P_sh[tid] = a;
    }
    if (tid == 0) {
        float a = 0.f;
        for (int v = 0; v < NW; ++v)
#pragma unroll
            for (int q = 0; q < TPW; ++q) a += lsg[v][q];
        part_lse2[blockIdx.x] = a;
        if (lse2_sh) *lse2_sh = a;
    }
}

// The per-token epilogue over a block's logits tile hl[TILE][.]
// (already synchronised), NW waves, wave w taking tokens w, w + NW, ...
// Every thread of the block must call it.  Block partials, for a grid of
// nblk blocks: part_P[e * nblk + b] = sum of p_e over the block's tokens
// (waves in order), part_P[(E + e) * nblk + b] = how many of them have e as
// their top choice (an exact small integer in a float), part_lse2[b].
template <int TILE, int NW = 4>
__device__ void softmax_topk_block(const float (*hl)[RT_EMAX + 1], int t0, int T, int E, int k,
                                   int gate_switch, int32_t *__restrict__ topk_idx,
                                   float *__restrict__ gates, float *__restrict__ part_P,
                                   float *__restrict__ part_lse2, int *topk_sh = nullptr,
                                   float *P_sh = nullptr, float *lse2_sh = nullptr) {
    if (E <= 8) {
        softmax_topk_grouped<8, TILE, NW>(hl, t0, T, E, k, gate_switch, topk_idx, gates, part_P, part_lse2,
                                          topk_sh, P_sh, lse2_sh);
        return;
    }
    if (E <= 16) {
        softmax_topk_grouped<16, TILE, NW>(hl, t0, T, E, k, gate_switch, topk_idx, gates, part_P, part_lse2,
                                           topk_sh, P_sh, lse2_sh);
        return;
    }
    __shared__ float pw[NW][RT_EMAX];
    __shared__ float lw[NW];
    __shared__ int topch[TILE];   // each token's top choice
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int e0 = lane, e1 = lane + 64;
    const bool v0 = e0 < E, v1 = e1 < E;
    float psum0 = 0.f, psum1 = 0.f, lsum = 0.f;
    for (int r = w; r < TILE; r += NW) {
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
            if (sl == 0) {
                h_top = hb;
                if (lane == 0) topch[r] = bi;
            }
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
            if (topk_sh) topk_sh[t * k + sl] = j ? si1 : si0;  // LDS copy (small batches)
            gates[(int64_t)t * k + sl] = g;
        }
    }
    // block partials in a fixed order: waves 0..NW-1.  lsum is the same on
    // every lane of a wave (it sums wave-uniform values).
    pw[w][e0] = psum0;
    pw[w][e1] = psum1;
    if (lane == 0) lw[w] = lsum;
    __syncthreads();
    if (tid < E) {
        float a = pw[0][tid];
#pragma unroll
        for (int v = 1; v < NW; ++v) a += pw[v][tid];
        const int64_t nblk = gridDim.x;
        int c = 0;
        for (int r = 0, nr = min(TILE, T - t0); r < nr; ++r) c += topch[r] == tid;
        part_P[(int64_t)tid * nblk + blockIdx.x] = a;
        part_P[(int64_t)(E + tid) * nblk + blockIdx.x] = (float)c;
        if (P_sh) P_sh[tid] = a;
    }
    if (tid == 0) {
        float a = lw[0];
#pragma unroll
        for (int v = 1; v < NW; ++v) a += lw[v];
        part_lse2[blockIdx.x] = a;
        if (lse2_sh) *lse2_sh = a;
    }
}

// ---- fp32 activations ----------------------------------------------------

__global__ __launch_bounds__(RT_THREADS) void route_f32_kernel(
    const float *__restrict__ x, const float *__restrict__ Wr, const float *__restrict__ bias,
    const float *__restrict__ noise, int T, int d, int E, int k, int gate_switch,
    int32_t *__restrict__ topk_idx, float *__restrict__ gates, float *__restrict__ part_P,
    float *__restrict__ part_lse2, unsigned *__restrict__ arrivals) {
    constexpr int TILE = ROUTE_TOKENS_F32;
    __shared__ float xs[TILE][RT_DC + 1];
    __shared__ float wsh[RT_EMAX][RT_DC + 1];
    __shared__ float hl[TILE][RT_EMAX + 1];

    const int tid = threadIdx.x;
    const int t0 = blockIdx.x * TILE;
    const int tg = tid >> 5;  // 8 token groups of 4 tokens
    const int eg = tid & 31;  // 32 expert groups; experts eg + 32*j

    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

    for (int c0 = 0; c0 < d; c0 += RT_DC) {
        for (int i = tid; i < TILE * RT_DC; i += RT_THREADS) {
            int r = i / RT_DC, c = i % RT_DC;
            int t = t0 + r;
            xs[r][c] = (t < T && c0 + c < d) ? x[(int64_t)t * d + c0 + c] : 0.f;
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
    if (blockIdx.x == 0 && tid == 0) *arrivals = 0u;
    softmax_topk_block<TILE>(hl, t0, T, E, k, gate_switch, topk_idx, gates, part_P, part_lse2);
}

// ---- bf16 activations: exact three-term split + MFMA ---------------------

// Logit partials of tokens [64*bx, +64) over the d slice of blockIdx.y.
// MFMA 16x16x32 layout (lane l): A row l % 16, k 8*(l/16)..+8; B column
// l % 16, same k; accumulator r holds row 4*(l/16) + r, column l % 16.
// The block reads its slice of the fp32 router matrix and splits it into
// the three bf16 terms as it stages it in LDS (rows q * E_PAD + e hold
// term q of expert e; rows of experts >= E are zero).
template <int E_PAD, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t *__restrict__ x,
                                                            const float *__restrict__ Wr,
                                                            int T, int d, int E, int slice,
                                                            float *__restrict__ part) {
    constexpr int TMW = RL_BM / 16 / WAVES_M;   // 16-token tiles per wave
    constexpr int TNW = E_PAD / 16 / WAVES_N;   // 16-expert tiles per wave
    constexpr int WROWS = 3 * E_PAD;
    constexpr int CPR = RL_KC / 8;                       // 16-byte bf16 chunks per x row
    constexpr int WCPR = RL_KC / 4;                      // 16-byte fp32 chunks per W row
    constexpr int XCH = (RL_BM * CPR + 255) / 256;       // x chunks per thread
    constexpr int WCH = (E_PAD * WCPR + 255) / 256;      // W chunks per thread
    static_assert(WAVES_M * WAVES_N == 4 && TMW >= 1 && TNW >= 1, "wave split");
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][RL_BM][RL_LDK];
    __shared__ __attribute__((aligned(16))) uint16_t wsh[2][WROWS][RL_LDK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int t0 = blockIdx.x * RL_BM;
    const int kbeg = blockIdx.y * slice;
    const int kend = min(d, kbeg + slice);

    uint4 rx[XCH];
    float4 rw[WCH];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < XCH; ++i) {
            const int c = tid + i * 256;
            const int r = c / CPR, kc = (c % CPR) * 8;
            const bool ok = c < RL_BM * CPR && t0 + r < T && k0 + kc < kend;
            rx[i] = ok ? *(const uint4 *)(x + (int64_t)(t0 + r) * d + k0 + kc) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < WCH; ++i) {
            const int c = tid + i * 256;
            const int e = c / WCPR, kc = (c % WCPR) * 4;
            const bool ok = c < E_PAD * WCPR && e < E && k0 + kc < kend;
            rw[i] = ok ? *(const float4 *)(Wr + (int64_t)e * d + k0 + kc)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < XCH; ++i) {
            const int c = tid + i * 256;
            if (c < RL_BM * CPR) *(uint4 *)&xs[buf][c / CPR][(c % CPR) * 8] = rx[i];
        }
#pragma unroll
        for (int i = 0; i < WCH; ++i) {
            const int c = tid + i * 256;
            if (c < E_PAD * WCPR) {
                // W = hi + mid + lo exactly: hi = bf16(W), mid = bf16(W - hi),
                // lo = bf16(W - hi - mid); each difference is exact in fp32
                // and the last has at most 8 significant bits
                const int e = c / WCPR, kc = (c % WCPR) * 4;
                const float w[4] = {rw[i].x, rw[i].y, rw[i].z, rw[i].w};
                uint16_t t[3][4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint16_t hi = f32_to_bf16(w[j]);
                    const float r1 = w[j] - bf16_to_f32(hi);
                    const uint16_t mid = f32_to_bf16(r1);
                    const float r2 = r1 - bf16_to_f32(mid);
                    t[0][j] = hi;
                    t[1][j] = mid;
                    t[2][j] = f32_to_bf16(r2);
                }
#pragma unroll
                for (int q = 0; q < 3; ++q)
                    *(uint2 *)&wsh[buf][q * E_PAD + e][kc] =
                        make_uint2((uint32_t)t[q][0] | ((uint32_t)t[q][1] << 16),
                                   (uint32_t)t[q][2] | ((uint32_t)t[q][3] << 16));
            }
        }
    };

    f32x4_t acc[TMW][TNW];
#pragma unroll
    for (int i = 0; i < TMW; ++i)
#pragma unroll
        for (int j = 0; j < TNW; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int nchunks = (kend - kbeg + RL_KC - 1) / RL_KC;
    const int lr = lane & 15, lk = (lane >> 4) * 8;
    if (nchunks > 0) {
        gload(kbeg);
        lstore(0);
    }
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {
        const int cur = c & 1;
        if (c + 1 < nchunks) gload(kbeg + (c + 1) * RL_KC);
#pragma unroll
        for (int kk = 0; kk < RL_KC; kk += 32) {
            bf16x8_t a[TMW];
#pragma unroll
            for (int i = 0; i < TMW; ++i)
                a[i] = *(const bf16x8_t *)&xs[cur][(wm * TMW + i) * 16 + lr][kk + lk];
#pragma unroll
            for (int q = 0; q < 3; ++q)
#pragma unroll
                for (int j = 0; j < TNW; ++j) {
                    const bf16x8_t b =
                        *(const bf16x8_t *)&wsh[cur][q * E_PAD + (wn * TNW + j) * 16 + lr][kk + lk];
#pragma unroll
                    for (int i = 0; i < TMW; ++i)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b, acc[i][j], 0, 0, 0);
                }
        }
        if (c + 1 < nchunks) lstore(cur ^ 1);
        __syncthreads();
    }
    float *pp = part + (int64_t)blockIdx.y * T * E;
#pragma unroll
    for (int i = 0; i < TMW; ++i)
#pragma unroll
        for (int j = 0; j < TNW; ++j) {
            const int e = (wn * TNW + j) * 16 + lr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = t0 + (wm * TMW + i) * 16 + (lane >> 4) * 4 + r;
                if (t < T && e < E) pp[(int64_t)t * E + e] = acc[i][j][r];
            }
        }
}

// The three bf16 terms of W_r (the same split as the logits kernel makes
// in LDS), stacked: row q * epad + e of ws holds term q of expert e, rows
// of experts >= E are zero.  Thread: 4 consecutive k of one expert.  Block
// 0 also writes the row offsets {0, T} of the router GEMM's one row group.
__global__ __launch_bounds__(256) void router_wsplit_kernel(const float *__restrict__ Wr, int E, int epad,
                                                            int d, int T, uint16_t *__restrict__ ws,
                                                            int32_t *__restrict__ roffs) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // 4-wide group
    if (blockIdx.x == 0 && threadIdx.x < 2) roffs[threadIdx.x] = threadIdx.x ? T : 0;
    const int dq = d / 4;
    if (i >= (int64_t)epad * dq) return;
    const int e = (int)(i / dq), kc = (int)(i - (int64_t)e * dq) * 4;
    float w[4] = {0.f, 0.f, 0.f, 0.f};
    if (e < E) {
        const float4 v = *(const float4 *)(Wr + (int64_t)e * d + kc);
        w[0] = v.x, w[1] = v.y, w[2] = v.z, w[3] = v.w;
    }
    uint16_t t[3][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint16_t hi = f32_to_bf16(w[j]);
        const float r1 = w[j] - bf16_to_f32(hi);
        const uint16_t mid = f32_to_bf16(r1);
        const float r2 = r1 - bf16_to_f32(mid);
        t[0][j] = hi;
        t[1][j] = mid;
        t[2][j] = f32_to_bf16(r2);
    }
#pragma unroll
    for (int q = 0; q < 3; ++q)
        *(uint2 *)(ws + ((int64_t)q * epad + e) * d + kc) =
            make_uint2((uint32_t)t[q][0] | ((uint32_t)t[q][1] << 16), (uint32_t)t[q][2] | ((uint32_t)t[q][3] << 16));
}

// Logit (t, e) is the sum over partials o < nouter (outer stride souter)
// and i < ninner (inner stride sinner) of part[o, i][t * stride_t + e],
// added in (o, i) order: the d slices of the logits kernel (nouter slices,
// one inner), or the K halves and the three W_r terms of the router GEMM.
// Each thread handles up to 4 (token, expert) entries of the block's tile
// with all its loads of one partial in flight together.
__global__ __launch_bounds__(RT_THREADS) void route_epilogue_kernel(
    const float *__restrict__ part, int nouter, int64_t souter, int ninner, int sinner, int stride_t,
    const float *__restrict__ bias, const float *__restrict__ noise, int T, int E, int k,
    int gate_switch, int32_t *__restrict__ topk_idx, float *__restrict__ gates,
    float *__restrict__ part_P, float *__restrict__ part_lse2, unsigned *__restrict__ arrivals) {
    constexpr int TILE = ROUTE_TOKENS_BF16;
    __shared__ float hl[TILE][RT_EMAX + 1];
    constexpr int MAXQ = TILE * RT_EMAX / RT_THREADS;
    const int t0 = blockIdx.x * TILE;
    const int tid = threadIdx.x;
    const int64_t base = (int64_t)t0 * E;
    const int npairs = min(TILE, T - t0) * E;
    float h[MAXQ];
    int64_t off[MAXQ];
#pragma unroll
    for (int q = 0; q < MAXQ; ++q) {
        const int i = tid + q * RT_THREADS;
        const int r = i / E, e = i - r * E;
        h[q] = 0.f;
        off[q] = (int64_t)(t0 + r) * stride_t + e;
    }
    for (int o = 0; o < nouter; ++o)
        for (int in = 0; in < ninner; ++in) {
            const float *ps = part + o * souter + (int64_t)in * sinner;
#pragma unroll
            for (int q = 0; q < MAXQ; ++q) {
                const int i = tid + q * RT_THREADS;
                if (i < npairs) h[q] += ps[off[q]];
            }
        }
#pragma unroll
    for (int q = 0; q < MAXQ; ++q) {
        const int i = tid + q * RT_THREADS;
        if (i < npairs) {
            const int r = i / E, e = i - r * E;
            float v = h[q];
            if (bias) v += bias[e];
            if (noise) v += noise[base + i];
            hl[r][e] = v;
        }
    }
    if (blockIdx.x == 0 && tid == 0) *arrivals = 0u;
    __syncthreads();
    softmax_topk_block<TILE>(hl, t0, T, E, k, gate_switch, topk_idx, gates, part_P, part_lse2);
}

// Statistics in double, every sum in a fixed order.  route_stats_kernel:
// block e < E reduces expert e's block partials of p (thread t takes blocks
// t, t+256, ...; then the 256 thread sums are added in thread order) and
// adds up its block counts of top choices; block E reduces the lse^2
// partials the same way.  The last block to finish (an integer arrival
// counter, zeroed by the route kernel that runs before) adds the f_e P_e in
// expert order for aux and writes aux and z, then re-zeroes the counter.
__device__ __forceinline__ double block_sum_fixed(double v, double *red) {
    const int tid = threadIdx.x;
    red[tid] = v;
    __syncthreads();
    // threads 0..15 each add 16 consecutive values in order, then thread 0
    // adds the 16 group sums in order
    if (tid < 16) {
        double g = 0.0;
#pragma unroll
        for (int i = 0; i < 16; ++i) g += red[tid * 16 + i];
        red[256 + tid] = g;
    }
    __syncthreads();
    double total = 0.0;
    if (tid == 0)
#pragma unroll
        for (int i = 0; i < 16; ++i) total += red[256 + i];
    return total;  // valid in thread 0
}

__global__ __launch_bounds__(256) void route_stats_kernel(
    const int32_t *__restrict__ topk_idx, const float *__restrict__ part_P,
    const float *__restrict__ part_lse2, int T, int E, int k, int nblk,
    float *__restrict__ stats, double *__restrict__ fP, unsigned *__restrict__ arrivals) {
    __shared__ double red[256 + 16];
    __shared__ int cnt[4];
    __shared__ int last;
    const int tid = threadIdx.x;
    const int e = blockIdx.x;
    if (e == E) {
        double z = 0.0;
        for (int b = tid; b < nblk; b += 256) z += (double)part_lse2[b];
        z = block_sum_fixed(z, red);
        if (tid == 0) fP[E] = z / (double)T;
    } else {
        // expert e's block partials are contiguous: p sums, then top-choice
        // counts
        const float *pp = part_P + (int64_t)e * nblk;
        const float *pc = part_P + (int64_t)(E + e) * nblk;
        double acc = 0.0;
        int c = 0;
#pragma unroll 8
        for (int b = tid; b < nblk; b += 256) {
            acc += (double)pp[b];
            c += (int)pc[b];
        }
        // integer count: the order of the additions does not matter
        for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
        if ((tid & 63) == 0) cnt[tid >> 6] = c;
        const double P = block_sum_fixed(acc, red) / (double)T;
        if (tid == 0) {
            const double f = (double)(cnt[0] + cnt[1] + cnt[2] + cnt[3]) / (double)T;
            stats[e] = (float)f;
            stats[E + e] = (float)P;
            fP[e] = f * P;
        }
    }
    if (tid == 0) {
        __threadfence();
        last = atomicAdd(arrivals, 1u) == (unsigned)E;
    }
    __syncthreads();
    if (last) {
        // every block's f_e P_e (and z) is visible: all threads load them
        // at once, thread 0 adds them in expert order
        __threadfence();
        for (int i = tid; i <= E; i += 256)
            red[i] = __hip_atomic_load(fP + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (tid == 0) {
            double a = 0.0;
            for (int i = 0; i < E; ++i) a += red[i];
            stats[2 * E] = (float)((double)E * a);
            stats[2 * E + 1] = (float)red[E];
            *arrivals = 0u;
        }
    }
}

// Small batches: one block of 16 waves finishes the routing.  The logits of
// the T <= 64 tokens (slices added in slice order, then bias and noise) go
// to LDS, the shared per-token epilogue runs over all of them (its block
// partials are then the whole sums), and the statistics follow as in
// route_stats_kernel: P and z from the partials in double, f from the top
// choices, aux over experts in order.  The dispatch, when asked for, counts
// the assignments per expert (integer LDS atomics), forms kept counts and
// offsets, then wave 0 ranks the T*k assignments in order, 64 at a time:
// lanes with the same expert are grouped by ballot and ranked by popcount
// of the lower lanes, on top of a per-expert running count.
constexpr int RS_THREADS = 1024;

__global__ __launch_bounds__(RS_THREADS) void route_small_kernel(
    const float *__restrict__ part, int nsplit, const float *__restrict__ bias,
    const float *__restrict__ noise, int T, int E, int k, int gate_switch, int64_t C,
    int32_t *__restrict__ topk_idx, float *__restrict__ gates, float *__restrict__ part_P,
    float *__restrict__ part_lse2, float *__restrict__ stats, int32_t *__restrict__ routed,
    int32_t *__restrict__ kept, int32_t *__restrict__ offsets, int32_t *__restrict__ row_of_slot,
    int32_t *__restrict__ token_of_row, uint8_t *__restrict__ dropped) {
    constexpr int TILE = ROUTE_SMALL_T;
    __shared__ float hl[TILE][RT_EMAX + 1];
    __shared__ int cnt[RT_EMAX], off[RT_EMAX], run[RT_EMAX], topc[RT_EMAX];
    __shared__ int tk[ROUTE_SMALL_TK];
    __shared__ float Psh[RT_EMAX], lse2sh;
    __shared__ int sh_total;
    const int tid = threadIdx.x;
    const int TE = T * E;
    for (int i = tid; i < TE; i += RS_THREADS) {
        // the slices are added in slice order; each group's loads are all
        // issued before the first add, so the group costs one memory round
        // trip rather than one per slice
        constexpr int G = 32;
        float v = 0.f;
        for (int s0 = 0; s0 < nsplit; s0 += G) {
            float buf[G];
#pragma unroll
            for (int u = 0; u < G; ++u)
                if (s0 + u < nsplit) buf[u] = part[(int64_t)(s0 + u) * TE + i];
#pragma unroll
            for (int u = 0; u < G; ++u)
                if (s0 + u < nsplit) v += buf[u];
        }
        const int t = i / E, e = i - t * E;
        if (bias) v += bias[e];
        if (noise) v += noise[i];
        hl[t][e] = v;
    }
    if (tid < RT_EMAX) {
        cnt[tid] = 0;
        topc[tid] = 0;
    }
    __syncthreads();
    softmax_topk_block<TILE, RS_THREADS / 64>(hl, 0, T, E, k, gate_switch, topk_idx, gates, part_P,
                                              part_lse2, tk, Psh, &lse2sh);
    __syncthreads();

    // statistics
    const int Tk = T * k;
    for (int j = tid; j < Tk; j += RS_THREADS) {
        const int e = tk[j];
        atomicAdd(&cnt[e], 1);                         // integer: order-free
        if (j % k == 0) atomicAdd(&topc[e], 1);
    }
    __syncthreads();
    if (tid == 0) {
        double a = 0.0;
        for (int e = 0; e < E; ++e) {
            const double f = (double)topc[e] / (double)T;
            const double P = (double)Psh[e] / (double)T;
            stats[e] = (float)f;
            stats[E + e] = (float)P;
            a += f * P;
        }
        stats[2 * E] = (float)((double)E * a);
        stats[2 * E + 1] = (float)((double)lse2sh / (double)T);
    }
    if (routed == nullptr) return;

    // dispatch
    if (tid == 0) {
        int o = 0;
        for (int e = 0; e < E; ++e) {
            const int kc = (C >= 0 && cnt[e] > C) ? (int)C : cnt[e];
            off[e] = o;
            run[e] = 0;
            routed[e] = cnt[e];
            kept[e] = kc;
            offsets[e] = o;
            o += kc;
        }
        offsets[E] = o;
        sh_total = o;
    }
    __syncthreads();
    if (tid < 64) {
        const int lane = tid;
        const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        for (int j0 = 0; j0 < Tk; j0 += 64) {
            const int j = j0 + lane;
            const bool valid = j < Tk;
            const int ej = valid ? tk[j] : -1;
            bool act = valid;
            int rank = 0;
            while (true) {
                const unsigned long long am = __ballot(act);
                if (am == 0ull) break;
                const int leader = __ffsll((long long)am) - 1;
                const int e0 = __builtin_amdgcn_readlane(ej, leader);  // leader is wave-uniform
                const bool m = act && ej == e0;
                const unsigned long long mm = __ballot(m);
                if (m) {
                    rank = run[e0] + __popcll(mm & lt_mask);
                    act = false;
                }
                // every lane has read run[e0] above before the leader adds
                if (lane == leader) run[e0] += __popcll(mm);
            }
            if (valid) {
                if (C < 0 || rank < C) {
                    const int row = off[ej] + rank;
                    row_of_slot[j] = row;
                    token_of_row[row] = j / k;
                    dropped[j] = 0;
                } else {
                    row_of_slot[j] = -1;
                    dropped[j] = 1;
                }
            }
        }
    }
    // rows past the last kept one hold no token
    for (int r = sh_total + tid; r < Tk; r += RS_THREADS) token_of_row[r] = -1;
}

template <int E_PAD, int WM, int WN>
void launch_logits(const Shape &s, const void *x, const float *Wr, float *part, hipStream_t st) {
    dim3 grid((unsigned)((s.T + RL_BM - 1) / RL_BM), (unsigned)route_nsplit(s));
    hipLaunchKernelGGL((router_logits_kernel<E_PAD, WM, WN>), grid, dim3(256), 0, st,
                       (const uint16_t *)x, Wr, s.T, s.d, s.E, route_slice(s), part);
}

}  // namespace

int route_epad(const Shape &s) {
    if (s.E <= 16) return 16;
    if (s.E <= 32) return 32;
    if (s.E <= 64) return 64;
    return 128;
}

// d slice per split: whole 64-wide chunks, enough slices to give the GPU
// about 512 blocks, each slice at least two chunks, at most 8 slices (32
// for a small batch, whose block count is tiny and whose single finishing
// block adds the slices back at little cost).
int route_slice(const Shape &s) {
    const int tiles = (s.T + RL_BM - 1) / RL_BM;
    const int chunks = (s.d + RL_KC - 1) / RL_KC;
    const int want = (512 + tiles - 1) / tiles;
    int maxsplit = chunks / 2 > 1 ? chunks / 2 : 1;
    const int cap = route_small(s) ? 32 : 8;  // the epilogue adds the slices back
    if (maxsplit > cap) maxsplit = cap;
    int nsplit = want < maxsplit ? want : maxsplit;
    if (nsplit < 1) nsplit = 1;
    return (chunks + nsplit - 1) / nsplit * RL_KC;
}

int route_nsplit(const Shape &s) {
    const int slice = route_slice(s);
    return (s.d + slice - 1) / slice;
}

// The GEMM pays off where the logits kernel re-splits a large W_r for every
// 64-token tile: many experts and a batch past the small-batch kernel.  The
// 256-row kernel needs d % 64 == 0 and its operand offsets within 32 bits.
bool route_gemm(const Shape &s) {
    if (s.dtype != 1 || route_small(s) || route_epad(s) < 64 || s.d % 64 != 0) return false;
    return (int64_t)s.T * s.d * 2 < (int64_t(1) << 31) && (int64_t)3 * route_epad(s) * s.d * 2 < (int64_t(1) << 31);
}

// K halves: when the 256 x 256 output tiles would fill less than one round
// of the CUs and the 64-wide K stages split evenly.
int route_gemm_nsplit(const Shape &s) {
    const int64_t tiles = (int64_t)((s.T + 255) / 256) * ((3 * route_epad(s) + 255) / 256);
    return tiles < 256 && (s.d / 64) % 2 == 0 ? 2 : 1;
}

static size_t route_wsplit_matrix_bytes(const Shape &s) {
    return ((size_t)3 * route_epad(s) * s.d * 2 + 255) / 256 * 256;
}

size_t route_part_floats(const Shape &s) {
    if (route_gemm(s)) return (size_t)route_gemm_nsplit(s) * s.T * 3 * route_epad(s);
    return (size_t)route_nsplit(s) * s.T * s.E;
}

size_t route_wsplit_bytes(const Shape &s) {
    return route_gemm(s) ? route_wsplit_matrix_bytes(s) + 256 : 0;
}

hipError_t launch_route(const Shape &s, const void *x, const float *Wr, const float *bias,
                        const float *noise, int32_t *topk_idx, float *gates, float *part_P,
                        float *part_lse2, float *part_logits, void *wsplit, unsigned *arrivals,
                        hipStream_t st) {
    const dim3 grid(route_blocks(s)), block(RT_THREADS);
    if (s.dtype == 0) {
        hipLaunchKernelGGL(route_f32_kernel, grid, block, 0, st, (const float *)x, Wr, bias, noise,
                           s.T, s.d, s.E, s.k, s.gate, topk_idx, gates, part_P, part_lse2,
                           arrivals);
        return hipGetLastError();
    }
    if (route_gemm(s)) {
        if (wsplit == nullptr) return hipErrorInvalidValue;
        const int epad = route_epad(s), N = 3 * epad;
        uint16_t *wm = (uint16_t *)wsplit;
        int32_t *roffs = (int32_t *)((char *)wsplit + route_wsplit_matrix_bytes(s));
        const int64_t groups = (int64_t)epad * (s.d / 4);
        hipLaunchKernelGGL(router_wsplit_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, st, Wr,
                           s.E, epad, s.d, s.T, wm, roffs);
        const hipError_t err = launch_router_gemm(s, x, wm, roffs, part_logits, st);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(route_epilogue_kernel, grid, block, 0, st, (const float *)part_logits,
                           route_gemm_nsplit(s), (int64_t)s.T * N, 3, epad, N, bias, noise, s.T, s.E, s.k,
                           s.gate, topk_idx, gates, part_P, part_lse2, arrivals);
        return hipGetLastError();
    }
    switch (route_epad(s)) {
    case 16: launch_logits<16, 4, 1>(s, x, Wr, part_logits, st); break;
    case 32: launch_logits<32, 4, 1>(s, x, Wr, part_logits, st); break;
    case 64: launch_logits<64, 2, 2>(s, x, Wr, part_logits, st); break;
    default: launch_logits<128, 1, 4>(s, x, Wr, part_logits, st); break;
    }
    hipLaunchKernelGGL(route_epilogue_kernel, grid, block, 0, st, (const float *)part_logits,
                       route_nsplit(s), (int64_t)s.T * s.E, 1, 0, s.E, bias, noise, s.T, s.E, s.k, s.gate,
                       topk_idx, gates, part_P, part_lse2, arrivals);
    return hipGetLastError();
}

hipError_t launch_route_finalize(const Shape &s, const int32_t *topk_idx, const float *part_P,
                                 const float *part_lse2, float *stats, double *fP,
                                 unsigned *arrivals, hipStream_t st) {
    hipLaunchKernelGGL(route_stats_kernel, dim3(s.E + 1), dim3(256), 0, st, topk_idx, part_P,
                       part_lse2, s.T, s.E, s.k, route_blocks(s), stats, fP, arrivals);
    return hipGetLastError();
}

hipError_t launch_route_small(const Shape &s, const void *x, const float *Wr, const float *bias,
                              const float *noise, int32_t *topk_idx, float *gates, float *stats,
                              const DispatchOut *disp, float *part_P, float *part_lse2,
                              float *part_logits, hipStream_t st) {
    if (!route_small(s)) return hipErrorInvalidValue;
    switch (route_epad(s)) {
    case 16: launch_logits<16, 4, 1>(s, x, Wr, part_logits, st); break;
    case 32: launch_logits<32, 4, 1>(s, x, Wr, part_logits, st); break;
    case 64: launch_logits<64, 2, 2>(s, x, Wr, part_logits, st); break;
    default: launch_logits<128, 1, 4>(s, x, Wr, part_logits, st); break;
    }
    hipLaunchKernelGGL(route_small_kernel, dim3(1), dim3(RS_THREADS), 0, st, (const float *)part_logits,
                       route_nsplit(s), bias, noise, s.T, s.E, s.k, s.gate, s.C, topk_idx, gates,
                       part_P, part_lse2, stats, disp ? disp->routed : nullptr,
                       disp ? disp->kept : nullptr, disp ? disp->offsets : nullptr,
                       disp ? disp->row_of_slot : nullptr, disp ? disp->token_of_row : nullptr,
                       disp ? disp->dropped : nullptr);
    return hipGetLastError();
}

}  // namespace moe
