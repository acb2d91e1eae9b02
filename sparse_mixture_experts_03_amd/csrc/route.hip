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
// bf16 activations (the MFMA path):
//   route_fused_kernel (batches past the small-batch kernel, d % 64 == 0):
//     after router_wsplit_kernel has split W_r once into its three bf16
//     terms (below), one kernel per token tile computes the logits on MFMA
//     and finishes the routing in its epilogue -- see its comment.
//   Otherwise two kernels:
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
// Per-token epilogue (one token per group of 8 or 16 lanes, E <= 128
// logits in registers: for E > 16 lane c of a 16-lane row holds experts c,
// c + 16, ...): max and sum of exponentials by DPP reductions within the
// group, top-k by k rounds of two reductions on orderable logit bits (the
// largest key, then the lowest index holding it, so a tie goes to the lower
// index), gates, and per-block partials: sums of p and counts of top
// choices (per expert) and the sum of lse^2, in a fixed order.
// route_stats_kernel reduces the partials in double in a fixed order.
#include <type_traits>

#include "moe_internal.h"
#include "route_stats.h"

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
// Its inverse (a zero comes back as +0, which no use below tells from -0).
__device__ __forceinline__ float unord_f32(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// Exponential, logarithm and reciprocal on the hardware's transcendental
// unit (v_exp_f32 = 2^x, v_log_f32 = log2 x, v_rcp_f32): about 1e-6
// relative error on the epilogue's arguments (the rounding of x * log2 e
// dominates), which no routing decision depends on -- the choices compare
// the logits themselves.
__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }
__device__ __forceinline__ float log_hw(float x) { return __builtin_amdgcn_logf(x) * 0.693147180559945309f; }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }

// Reductions within groups of G = 8 or 16 lanes (one token per group) on
// the VALU's cross-lane moves (DPP) instead of LDS permutes: swap
// neighbours (quad_perm 1,0,3,2), pairs (2,3,0,1), then mirror the
// half-rows and (G = 16) the row, so that every lane of the group holds the
// group's result, bit for bit the same on every lane (each step combines two
// equal-shaped partial results commutatively).  DPP control codes: quad_perm
// 0xB1 and 0x4E, row_half_mirror 0x141, row_mirror 0x140.  Maxima and
// minima run on unsigned integers (ordered logit keys, expert indices),
// where the move folds into the max/min instruction.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
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
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
    v = max(v, dpp_u32<0xB1>(v));
    v = max(v, dpp_u32<0x4E>(v));
    v = max(v, dpp_u32<0x141>(v));
    if (G == 16) v = max(v, dpp_u32<0x140>(v));
    return v;
}
template <int G>
__device__ __forceinline__ uint32_t group_min_u32(uint32_t v) {
    v = min(v, dpp_u32<0xB1>(v));
    v = min(v, dpp_u32<0x4E>(v));
    v = min(v, dpp_u32<0x141>(v));
    if (G == 16) v = min(v, dpp_u32<0x140>(v));
    return v;
}

// Top-k over ordered keys: each round takes the group's largest key, then
// the lowest expert index holding it (so a tie goes to the lower index, and
// -0 ties with +0, which share a key), and clears that key.  A padding
// expert or a taken one has key 0, below every logit's, so with k <= E a
// real expert always wins.

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
                                     float *lse2_sh, int pslot, int pslots) {
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
        const float h = v ? hl[r][e] : 0.f;
        uint32_t key = v ? ord_f32(h) : 0u;
        const float m = unord_f32(group_max_u32<G>(key));
        const float x = v ? exp_hw(h - m) : 0.f;
        const float s = group_sum<G>(x);
        const float inv = rcp_hw(s);
        if (v) psum += x * inv;
        const float lse = m + log_hw(s);
        if (vt && e == 0) lsum += lse * lse;
        float h_top = 0.f, den = 0.f, my_hb = 0.f;
        int my_bi = 0;
        for (int sl = 0; sl < k; ++sl) {
            const uint32_t b = group_max_u32<G>(key);
            const uint32_t bi = group_min_u32<G>(key == b ? (uint32_t)e : 0xffffffffu);
            if ((uint32_t)e == bi) key = 0u;
            const float hb = unord_f32(b);   // the key holds the logit
            if (sl == 0) {
                h_top = hb;
                if (vt && e == 0) topchg[r] = (int)bi;
            }
            den += exp_hw(hb - h_top);  // slot order, identical on the token's lanes
            if (e == sl) {
                my_hb = hb;
                my_bi = (int)bi;
            }
        }
        if (vt && e < k) {
            const float gt = gate_switch ? exp_hw(my_hb - m) * inv : exp_hw(my_hb - h_top) * rcp_hw(den);
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
        const int64_t nblk = pslots;
        int c = 0;
        for (int r = 0, nr = min(TILE, T - t0); r < nr; ++r) c += topchg[r] == tid;
        part_P[(int64_t)tid * nblk + pslot] = a;
        part_P[(int64_t)(E + tid) * nblk + pslot] = (float)c;
        if (P_sh) P_sh[tid] = a;
    }
    if (tid == 0) {
        float a = 0.f;
        for (int v = 0; v < NW; ++v)
#pragma unroll
            for (int q = 0; q < TPW; ++q) a += lsg[v][q];
        part_lse2[pslot] = a;
        if (lse2_sh) *lse2_sh = a;
    }
}

// softmax_topk_block for 16 < E <= 16 V: one token per row of 16 lanes
// (waves past the first NW of the block only join its barriers),
// lane c of a row holding experts c, c + 16, ..., c + 16 (V - 1), so a wave
// serves 4 tokens at once and every reduction stays within a row (DPP
// moves only: no readlane, no LDS).  Each lane first reduces its V values
// (max, sum in v order, largest key, lowest index), then the row.
// Selected slot s is kept by lane s % 16 of the row, in its register
// s / 16 (one register when k <= 16).  Partials: per expert, the waves'
// row sums added in (wave, row) order.
template <int V, int TILE, int NW>
__device__ __forceinline__ void softmax_topk_rows(const float (*hl)[RT_EMAX + 1], int t0, int T, int E, int k,
                                                  int gate_switch, int32_t *__restrict__ topk_idx,
                                                  float *__restrict__ gates, float *__restrict__ part_P,
                                                  float *__restrict__ part_lse2, int *topk_sh, float *P_sh,
                                                  float *lse2_sh, int pslot, int pslots) {
    __shared__ float pwr[NW][V][64];
    __shared__ float lsr[NW][4];
    __shared__ int topcr[TILE];
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    float psum[V], lsum = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) psum[v] = 0.f;
    for (int r0 = w * 4; w < NW && r0 < TILE; r0 += NW * 4) {
        if (t0 + r0 >= T) break;   // uniform in the wave
        const int r = r0 + g, t = t0 + r;
        const bool vt = r < TILE && t < T;
        float h[V];
        uint32_t key[V];
        bool ve[V];
#pragma unroll
        for (int v = 0; v < V; ++v) {
            ve[v] = c + 16 * v < E;
            // a row past the batch holds no token: finite stand-ins, nothing stored
            h[v] = ve[v] && vt ? hl[r][c + 16 * v] : 0.f;
            key[v] = ve[v] ? ord_f32(h[v]) : 0u;
        }
        uint32_t km = key[0];
#pragma unroll
        for (int v = 1; v < V; ++v) km = max(km, key[v]);
        const float mx = unord_f32(group_max_u32<16>(km));
        float xv[V], sl = 0.f;
#pragma unroll
        for (int v = 0; v < V; ++v) {
            xv[v] = ve[v] ? exp_hw(h[v] - mx) : 0.f;
            sl += xv[v];
        }
        const float sm = group_sum<16>(sl);
        const float inv = rcp_hw(sm);
        if (vt) {
#pragma unroll
            for (int v = 0; v < V; ++v) psum[v] += xv[v] * inv;
            const float lse = mx + log_hw(sm);
            lsum += lse * lse;
        }
        // NS slot registers per lane: 1 when k <= 16, else V
        auto select = [&](auto ns_c) {
            constexpr int NS = decltype(ns_c)::value;
            float sh[NS];
            int si[NS];
#pragma unroll
            for (int q = 0; q < NS; ++q) {
                sh[q] = 0.f;
                si[q] = 0;
            }
            float h_top = 0.f, den = 0.f;
            for (int s = 0; s < k; ++s) {
                uint32_t b = key[0];
#pragma unroll
                for (int v = 1; v < V; ++v) b = max(b, key[v]);
                b = group_max_u32<16>(b);
                uint32_t cand = 0xffffffffu;
#pragma unroll
                for (int v = V - 1; v >= 0; --v) cand = key[v] == b ? (uint32_t)(c + 16 * v) : cand;
                const uint32_t bi = group_min_u32<16>(cand);
#pragma unroll
                for (int v = 0; v < V; ++v) key[v] = (uint32_t)(c + 16 * v) == bi ? 0u : key[v];
                const float hb = unord_f32(b);   // the key holds the logit
                if (s == 0) {
                    h_top = hb;
                    if (c == 0 && vt) topcr[r] = (int)bi;
                }
                den += exp_hw(hb - h_top);   // slot order, identical on the row's lanes
                if (NS == 1) {
                    if (c == s) {
                        sh[0] = hb;
                        si[0] = (int)bi;
                    }
                } else if (c == (s & 15)) {
#pragma unroll
                    for (int q = 0; q < NS; ++q)
                        if (q == (s >> 4)) {
                            sh[q] = hb;
                            si[q] = (int)bi;
                        }
                }
            }
            if (vt) {
                const float rden = rcp_hw(den);
#pragma unroll
                for (int q = 0; q < NS; ++q) {
                    const int s = c + 16 * q;
                    if (s < k) {
                        const float gt = gate_switch ? exp_hw(sh[q] - mx) * inv : exp_hw(sh[q] - h_top) * rden;
                        topk_idx[(int64_t)t * k + s] = si[q];
                        if (topk_sh) topk_sh[t * k + s] = si[q];   // LDS copy (small batches)
                        gates[(int64_t)t * k + s] = gt;
                    }
                }
            }
        };
        if (k <= 16)
            select(std::integral_constant<int, 1>{});
        else
            select(std::integral_constant<int, V>{});
    }
    if (w < NW) {
#pragma unroll
        for (int v = 0; v < V; ++v) pwr[w][v][lane] = psum[v];
        if (c == 0) lsr[w][g] = lsum;
    }
    __syncthreads();
    if (tid < E) {
        const int v = tid >> 4, cc = tid & 15;
        float a = 0.f;
        for (int wv = 0; wv < NW; ++wv)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) a += pwr[wv][v][16 * gg + cc];
        int cnt = 0;
        for (int r = 0, nr = min(TILE, T - t0); r < nr; ++r) cnt += topcr[r] == tid;
        part_P[(int64_t)tid * pslots + pslot] = a;
        part_P[(int64_t)(E + tid) * pslots + pslot] = (float)cnt;
        if (P_sh) P_sh[tid] = a;
    }
    if (tid == 0) {
        float a = 0.f;
        for (int wv = 0; wv < NW; ++wv)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) a += lsr[wv][gg];
        part_lse2[pslot] = a;
        if (lse2_sh) *lse2_sh = a;
    }
}

// The per-token epilogue over a block's logits tile hl[TILE][.]
// (already synchronised), NW waves, wave w taking tokens w, w + NW, ...
// Every thread of the block must call it.  Inlined into its kernel: as a
// call it would run with a stack and without the caller's constants.  Partials of tile pslot out of
// pslots (by default the block's index in the grid): part_P[e * pslots + b]
// = sum of p_e over the tile's tokens (waves in order), part_P[(E + e) *
// pslots + b] = how many of them have e as their top choice (an exact small
// integer in a float), part_lse2[b].
template <int TILE, int NW = 4>
__device__ __forceinline__ void softmax_topk_block(const float (*hl)[RT_EMAX + 1], int t0, int T, int E, int k,
                                   int gate_switch, int32_t *__restrict__ topk_idx,
                                   float *__restrict__ gates, float *__restrict__ part_P,
                                   float *__restrict__ part_lse2, int *topk_sh = nullptr,
                                   float *P_sh = nullptr, float *lse2_sh = nullptr,
                                   int pslot = -1, int pslots = 0) {
    if (pslot < 0) {
        pslot = blockIdx.x;
        pslots = gridDim.x;
    }
    if (E <= 8) {
        softmax_topk_grouped<8, TILE, NW>(hl, t0, T, E, k, gate_switch, topk_idx, gates, part_P, part_lse2,
                                          topk_sh, P_sh, lse2_sh, pslot, pslots);
        return;
    }
    if (E <= 16) {
        softmax_topk_grouped<16, TILE, NW>(hl, t0, T, E, k, gate_switch, topk_idx, gates, part_P, part_lse2,
                                           topk_sh, P_sh, lse2_sh, pslot, pslots);
        return;
    }
    if (E <= 32) {
        softmax_topk_rows<2, TILE, NW>(hl, t0, T, E, k, gate_switch, topk_idx, gates, part_P, part_lse2,
                                       topk_sh, P_sh, lse2_sh, pslot, pslots);
        return;
    }
    if (E <= 64) {
        softmax_topk_rows<4, TILE, NW>(hl, t0, T, E, k, gate_switch, topk_idx, gates, part_P, part_lse2,
                                       topk_sh, P_sh, lse2_sh, pslot, pslots);
        return;
    }
    softmax_topk_rows<8, TILE, NW>(hl, t0, T, E, k, gate_switch, topk_idx, gates, part_P, part_lse2, topk_sh,
                                   P_sh, lse2_sh, pslot, pslots);
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
    // every bias and noise load is issued before the first add (clamped
    // indices): one memory round trip
    float bv[4], nz[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int ec = min(eg + 32 * j, E - 1);
        bv[j] = bias ? bias[ec] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) nz[i][j] = noise ? noise[(int64_t)min(t0 + tg * 4 + i, T - 1) * E + ec] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int r = tg * 4 + i, t = t0 + r;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int e = eg + 32 * j;
            float h = acc[i][j];
            if (e < E && t < T) {
                if (bias) h += bv[j];
                if (noise) h += nz[i][j];
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
// in LDS), stacked: row q * epad + e holds term q of expert e, rows of
// experts >= E are zero.  Stored for the fused router's fragment loads:
// [d / 32][3 epad][32] -- the 32 columns k = 32 c .. 32 c + 31 of every row
// together, so 16 consecutive rows of one such block (one MFMA B fragment)
// are one contiguous kilobyte.  Thread: 4 consecutive k of one expert.
__global__ __launch_bounds__(256) void router_wsplit_kernel(const float *__restrict__ Wr, int E, int epad,
                                                            int d, uint16_t *__restrict__ ws) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // 4-wide group
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
        *(uint2 *)(ws + (((int64_t)(kc >> 5) * 3 + q) * epad + e) * 32 + (kc & 31)) =
            make_uint2((uint32_t)t[q][0] | ((uint32_t)t[q][1] << 16), (uint32_t)t[q][2] | ((uint32_t)t[q][3] << 16));
}

// The fused router for bf16 batches past the small-batch kernel with more
// than 32 experts: one block per tile of BT tokens, all E_PAD experts, the
// whole of d.  The logits go from the MFMAs to LDS and through the per-token
// epilogue in the same kernel; they never reach memory.
//
// Products: x (bf16) against the three stacked bf16 terms of W_r, stored
// [d / 32][3][E_PAD][32] (router_wsplit_kernel), all three added into the
// same fp32 accumulator
// on v_mfma_f32_16x16x32_bf16, so a logit is an fp32 sum of exact products
// of x with W_r's 24 significant bits.
//
// NCW + 1 waves.  Wave NCW only loads x: 64-wide k stages of the tile go from
// global memory straight into an LDS ring of NBUF stages (buffer loads to
// LDS, no registers), NBUF - 1 stages ahead; before each block barrier it
// waits until the next stage has landed.  Its loads are the only ones in
// its own in-order return queue, so the compute waves' loads never wait
// behind them.  Compute waves 0 .. NCW - 1 (8 for 128 experts and tiles
// of 32 or 64 tokens, two per SIMD, so that one computes while the other
// waits; else 4) each own NG =
// E_PAD / (16 NCW) groups of 16 experts (all three terms): they load their weight fragments from L2 straight into registers
// PW - 1 stages ahead (a ring of PW register slots, the stage loop unrolled
// by PW) and multiply them with the tile's x fragments read from the ring.
// MFMA step j in {0, 1} of a stage covers k 32j .. 32j + 31, lane group
// g = lane / 16 supplying k 32j + 8g .. +8 of both operands; a weight
// fragment of a step is one contiguous kilobyte.  A stage's rows are
// 128 bytes; chunk s of row r sits in slot s ^ f(r), f(r) = (r % 8) ^
// ((r / 8) % 2), so the 16 rows a fragment read serves fall on distinct
// banks (the loader fetches chunk (lane % 8) ^ f(row) into slot lane % 8).
//
// After the last stage the ring becomes the logit tile: bias and noise
// are added, and the compute waves run the shared per-token epilogue; the
// statistic partials are indexed by tile.
template <int E_PAD, int BT, int PW, int NCW>
__global__ __launch_bounds__(64 * (NCW + 1)) void route_fused_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wsplit, const float *__restrict__ bias,
    const float *__restrict__ noise, int T, int d, int E, int k, int gate_switch,
    int32_t *__restrict__ topk_idx, float *__restrict__ gates, float *__restrict__ part_P,
    float *__restrict__ part_lse2, unsigned *__restrict__ arrivals) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int NG = E_PAD / (16 * NCW);      // 16-expert groups per compute wave
    constexpr int TM = BT / 16;                 // 16-token fragments
    constexpr int NBUF = BT == 64 ? 8 : 16;     // x stages in the ring
    constexpr int LPS = BT / 8;                 // loader instructions per stage (8 rows each)
    constexpr int SB = BT * 128;                // bytes per stage
    constexpr int RING = NBUF * SB;
    constexpr int HLB = BT * (RT_EMAX + 1) * 4;
    static_assert(NG >= 1 && NG * 16 * NCW == E_PAD && TM >= 1 && (NBUF - 2) * LPS <= 63, "tile shape");
    __shared__ __attribute__((aligned(1024))) char lds[RING > HLB ? RING : HLB];
    float(*hl)[RT_EMAX + 1] = (float(*)[RT_EMAX + 1])lds;

    const int tile = blockIdx.x, t0 = tile * BT;
    const int nst = d / 64;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, lr = lane & 15;
    if (tile == 0 && tid == 0) *arrivals = 0u;
    f32x4_t acc[TM][NG];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) acc[i][gi] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    if (wave == NCW) {
        // the loader: rows past the batch read its last token (their logits
        // are never used); offsets from the tile's first row
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc((void *)(x + (int64_t)t0 * d), 0, 0x7fffffff, 0x00020000);
        const int last = T - 1 - t0;
        uint32_t voff[LPS];
#pragma unroll
        for (int q = 0; q < LPS; ++q) {
            const int r = q * 8 + (lane >> 3);
            const int f = (r & 7) ^ ((r >> 3) & 1);
            voff[q] = ((uint32_t)min(r, last) * (uint32_t)d + (uint32_t)(((lane & 7) ^ f) * 8)) * 2u;
        }
        auto issue = [&](int st) {
            const int sc = min(st, nst - 1);   // past the end: the last stage again, into a ring slot nobody reads
            char *dst = lds + (st % NBUF) * SB;
#pragma unroll
            for (int q = 0; q < LPS; ++q)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rsrc, (__attribute__((address_space(3))) void *)(dst + q * 1024), 16, voff[q], sc * 128, 0, 0);
        };
        for (int s = 0; s < NBUF - 1; ++s) issue(s);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NBUF - 2) * LPS) : "memory");   // stage 0 has landed
        __syncthreads();
        for (int st = 0; st < nst; ++st) {
            issue(st + NBUF - 1);   // into the slot stage st - 1 left, which every wave has finished
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NBUF - 2) * LPS) : "memory");   // stage st + 1 has landed
            __syncthreads();
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no ring write in flight when it becomes the logit tile
    } else {
        // compute wave `wave`: experts (wave * NG + gi) * 16 + lr, all three terms
        const uint16_t *wrow[NG][3];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
#pragma unroll
            for (int q = 0; q < 3; ++q)
                wrow[gi][q] = wsplit + (int64_t)(q * E_PAD + (wave * NG + gi) * 16 + lr) * 32 + 8 * g;
        uint4 wr[PW][NG][3][2];
        auto load_w = [&](auto slot_c, int st) {
            constexpr int slot = decltype(slot_c)::value;
            const int sc = min(st, nst - 1);
#pragma unroll
            for (int gi = 0; gi < NG; ++gi)
#pragma unroll
                for (int q = 0; q < 3; ++q)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        wr[slot][gi][q][h] =
                            *(const uint4 *)(wrow[gi][q] + (int64_t)(2 * sc + h) * (3 * E_PAD * 32));
        };
        const int fsw = (lr & 7) ^ ((lr >> 3) & 1);
        int st = 0;
        // one stage from ring slot st % NBUF and weight slot `cur`; the
        // weights of stage st + PW - 1 are fetched into the slot stage st - 1
        // left
        auto stage = [&](auto cur_c) {
            constexpr int cur = decltype(cur_c)::value;
            constexpr std::integral_constant<int, (cur + PW - 1) % PW> nxt_c{};
            load_w(nxt_c, st + PW - 1);
            const char *xb = lds + (st % NBUF) * SB;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                bf16x8_t a[TM];
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    a[i] = *(const bf16x8_t *)(xb + (i * 16 + lr) * 128 + (((4 * j + g) ^ fsw) * 16));
#pragma unroll
                for (int q = 0; q < 3; ++q)
#pragma unroll
                    for (int gi = 0; gi < NG; ++gi) {
                        const bf16x8_t b = __builtin_bit_cast(bf16x8_t, wr[cur][gi][q][j]);
#pragma unroll
                        for (int i = 0; i < TM; ++i)
                            acc[i][gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b, acc[i][gi], 0, 0, 0);
                    }
            }
            __syncthreads();
            ++st;
        };
        load_w(std::integral_constant<int, 0>{}, 0);
        if constexpr (PW > 2) load_w(std::integral_constant<int, 1>{}, 1);
        if constexpr (PW > 3) load_w(std::integral_constant<int, 2>{}, 2);
        __syncthreads();
        if constexpr (PW == 2) {
            while (st + 1 < nst) {
                stage(std::integral_constant<int, 0>{});
                stage(std::integral_constant<int, 1>{});
            }
            if (st < nst) stage(std::integral_constant<int, 0>{});
        } else {
            static_assert(PW == 4, "weight ring of 2 or 4 slots");
            while (st + 3 < nst) {
                stage(std::integral_constant<int, 0>{});
                stage(std::integral_constant<int, 1>{});
                stage(std::integral_constant<int, 2>{});
                stage(std::integral_constant<int, 3>{});
            }
            if (st < nst) stage(std::integral_constant<int, 0>{});
            if (st < nst) stage(std::integral_constant<int, 1>{});
            if (st < nst) stage(std::integral_constant<int, 2>{});
        }
    }
    __syncthreads();   // the ring is free: it becomes the logit tile

    // accumulator r of lane l (compute waves): token i * 16 + 4 g + r, expert
    // (wave * NG + gi) * 16 + lr
    if (wave < NCW) {
        // every bias and noise load of the lane is issued before the first
        // add (clamped indices, so none is conditional): one memory round
        // trip instead of one per logit
        float bv[NG], nz[TM][NG][4];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            const int ec = min((wave * NG + gi) * 16 + lr, E - 1);
            bv[gi] = bias ? bias[ec] : 0.f;
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    nz[i][gi][r] = noise ? noise[(int64_t)min(t0 + i * 16 + 4 * g + r, T - 1) * E + ec] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int gi = 0; gi < NG; ++gi)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = i * 16 + 4 * g + r, t = t0 + row;
                    const int e = (wave * NG + gi) * 16 + lr;
                    float v = acc[i][gi][r];
                    if (e < E && t < T) {
                        if (bias) v += bv[gi];
                        if (noise) v += nz[i][gi][r];
                    }
                    hl[row][e] = v;
                }
    }
    __syncthreads();
    // E_PAD / 16 logits per lane cover every E of this padding (E > E_PAD / 2).
    // The compute waves take the tokens.
    softmax_topk_rows<E_PAD / 16, BT, NCW>(hl, t0, T, E, k, gate_switch, topk_idx, gates, part_P, part_lse2,
                                         nullptr, nullptr, nullptr, tile, gridDim.x);
#endif
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
    // every bias and noise load is issued before the first add (clamped
    // indices): one memory round trip
    float bv[MAXQ], nz[MAXQ];
#pragma unroll
    for (int q = 0; q < MAXQ; ++q) {
        const int i = min(tid + q * RT_THREADS, npairs - 1);
        bv[q] = bias ? bias[i % E] : 0.f;
        nz[q] = noise ? noise[base + i] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < MAXQ; ++q) {
        const int i = tid + q * RT_THREADS;
        if (i < npairs) {
            const int r = i / E, e = i - r * E;
            float v = h[q];
            if (bias) v += bv[q];
            if (noise) v += nz[q];
            hl[r][e] = v;
        }
    }
    if (blockIdx.x == 0 && tid == 0) *arrivals = 0u;
    __syncthreads();
    softmax_topk_block<TILE>(hl, t0, T, E, k, gate_switch, topk_idx, gates, part_P, part_lse2);
}

// Statistics in double, every sum in a fixed order (route_stats_block, in
// route_stats.h): E + 1 blocks, the last to finish writing aux and z.
__global__ __launch_bounds__(256) void route_stats_kernel(
    const float *__restrict__ part_P, const float *__restrict__ part_lse2, int T, int E, int nblk,
    float *__restrict__ stats, double *__restrict__ fP, unsigned *__restrict__ arrivals) {
    route_stats_block(blockIdx.x, part_P, part_lse2, T, E, nblk, stats, fP, arrivals);
}

// Small batches: one block of 16 waves finishes the routing.  The logits of
// the T <= 64 tokens (slices added in slice order, then bias and noise) go
// to LDS, the shared per-token epilogue runs over all of them (its block
// partials are then the whole sums), and the statistics follow as in
// route_stats_kernel: P and z from the partials in double, f from the top
// choices, aux over experts in order.  The dispatch, when asked for, counts
// the assignments per expert (integer LDS atomics), forms kept counts and
// offsets, then wave 0 ranks the T*k assignments in order, 64 at a time:
// lanes with the same expert are found bit by bit of the expert index (one
// ballot per bit) and ranked by popcount
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
        const int t = i / E, e = i - t * E;
        // bias and noise are loaded with the first group of slices
        const float bv = bias ? bias[e] : 0.f, nz = noise ? noise[i] : 0.f;
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
        if (bias) v += bv;
        if (noise) v += nz;
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
            const unsigned long long mm = lanes_with_same_expert(ej, valid, expert_bits(E));
            const int below = __popcll(mm & lt_mask);
            const int rank = valid ? run[ej] + below : 0;
            // every lane has read run[] above before the group's lowest lane adds
            if (valid && below == 0) run[ej] += __popcll(mm);
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

// The fused router serves bf16 batches past the small-batch kernel with
// more than 32 experts and d a multiple of its 64-wide k stages.  Token
// tiles as large as still give about 256 blocks (each block reads all of
// the weight terms from L2, so fewer, larger tiles read fewer bytes):
// 64 tokens for at least 16384, 32 for at least 8192, else 16.
bool route_fused(const Shape &s) {
    return s.dtype == 1 && !route_small(s) && s.d % 64 == 0 && route_epad(s) >= 64;
}

int route_fused_bt(const Shape &s) { return s.T >= 16384 ? 64 : (s.T >= 8192 ? 32 : 16); }

int route_fused_ntiles(const Shape &s) { return (s.T + route_fused_bt(s) - 1) / route_fused_bt(s); }

static size_t route_wsplit_matrix_bytes(const Shape &s) {
    return ((size_t)3 * route_epad(s) * s.d * 2 + 255) / 256 * 256;
}

size_t route_part_floats(const Shape &s) {
    if (route_fused(s)) return 0;
    return (size_t)route_nsplit(s) * s.T * s.E;
}

size_t route_wsplit_bytes(const Shape &s) { return route_fused(s) ? route_wsplit_matrix_bytes(s) : 0; }

int route_stat_blocks(const Shape &s) { return route_fused(s) ? route_fused_ntiles(s) : route_blocks(s); }

namespace {

template <int E_PAD, int BT>
void launch_fused(const Shape &s, const void *x, const uint16_t *wm, const float *bias, const float *noise,
                  int32_t *topk_idx, float *gates, float *part_P, float *part_lse2, unsigned *arrivals,
                  hipStream_t st) {
    constexpr int NCW = E_PAD == 128 && BT >= 32 ? 8 : 4;
    hipLaunchKernelGGL((route_fused_kernel<E_PAD, BT, 2, NCW>), dim3((unsigned)route_fused_ntiles(s)),
                       dim3(64 * (NCW + 1)), 0,
                       st, (const uint16_t *)x, wm, bias, noise, s.T, s.d, s.E, s.k, s.gate, topk_idx, gates,
                       part_P, part_lse2, arrivals);
}

template <int E_PAD>
void launch_fused_e(const Shape &s, const void *x, const uint16_t *wm, const float *bias, const float *noise,
                    int32_t *topk_idx, float *gates, float *part_P, float *part_lse2, unsigned *arrivals,
                    hipStream_t st) {
    switch (route_fused_bt(s)) {
    case 64: launch_fused<E_PAD, 64>(s, x, wm, bias, noise, topk_idx, gates, part_P, part_lse2, arrivals, st); break;
    case 32: launch_fused<E_PAD, 32>(s, x, wm, bias, noise, topk_idx, gates, part_P, part_lse2, arrivals, st); break;
    default: launch_fused<E_PAD, 16>(s, x, wm, bias, noise, topk_idx, gates, part_P, part_lse2, arrivals, st); break;
    }
}

}  // namespace

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
    if (route_fused(s)) {
        if (wsplit == nullptr) return hipErrorInvalidValue;
        const int epad = route_epad(s);
        uint16_t *wm = (uint16_t *)wsplit;
        const int64_t groups = (int64_t)epad * (s.d / 4);
        hipLaunchKernelGGL(router_wsplit_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, st, Wr,
                           s.E, epad, s.d, wm);
        if (epad == 64)
            launch_fused_e<64>(s, x, wm, bias, noise, topk_idx, gates, part_P, part_lse2, arrivals, st);
        else
            launch_fused_e<128>(s, x, wm, bias, noise, topk_idx, gates, part_P, part_lse2, arrivals, st);
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
    (void)topk_idx;
    hipLaunchKernelGGL(route_stats_kernel, dim3(s.E + 1), dim3(256), 0, st, part_P, part_lse2, s.T, s.E,
                       route_stat_blocks(s), stats, fP, arrivals);
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
