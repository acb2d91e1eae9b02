// moe_internal.h -- internal declarations of libmoe (not part of the ABI).
//
// Each kernel family lives in its own .hip file and exports a host-side
// launcher declared here; moe_api.cpp validates arguments, carves the
// workspace and calls the launchers in order on the caller's stream.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Start/stop events for the next kernel launched through launch_kernel():
// moe_forward's stage-event hook for a stage that is one kernel (expert
// up).  The launch itself timestamps them, so timing the stage puts no
// commands between the kernels.  Per host thread; one launch consumes them.
struct LaunchEvents {
    hipEvent_t start, stop;
};
LaunchEvents &next_launch_events();
template <typename F, typename... Args>
inline void launch_kernel(F kernel, dim3 grid, dim3 block, unsigned shm, hipStream_t st,
                          Args... args) {
    LaunchEvents &le = next_launch_events();
    const LaunchEvents ev = le;
    le = LaunchEvents{nullptr, nullptr};
    hipExtLaunchKernelGGL(kernel, grid, block, shm, st, ev.start, ev.stop, 0u, args...);
}

// Problem sizes plus the derived capacity (C < 0: no limit).
struct Shape {
    int T, d, d_ff, E, k;
    int gate, act, dtype;
    int64_t C;
    int64_t Tk() const { return (int64_t)T * k; }
};

// ---- router: the per-token epilogue runs one block per route_tile() tokens
// (32 for fp32 activations, whose block also computes the logits; 8 for
// bf16, so that many waves work on the tokens at once)
constexpr int ROUTE_TOKENS_F32 = 32;
constexpr int ROUTE_TOKENS_BF16 = 8;
inline int route_tile(const Shape &s) { return s.dtype == 1 ? ROUTE_TOKENS_BF16 : ROUTE_TOKENS_F32; }
inline int route_blocks(const Shape &s) { return (s.T + route_tile(s) - 1) / route_tile(s); }

// bf16 path: logits computed in route_nsplit() slices of d, each
// route_slice() wide, against E padded to route_epad() experts.
int route_epad(const Shape &s);
int route_slice(const Shape &s);
int route_nsplit(const Shape &s);

// bf16 batches past the small-batch kernel with more than 32 experts and
// d % 64 == 0 (route_fused): W_r is split once into its three bf16 terms,
// stacked as a [3 * route_epad()][d] matrix, and one kernel computes each
// tile of route_fused_bt() tokens' logits on MFMA and finishes its routing
// (softmax, top-k, gates, statistic partials) without writing the logits.
bool route_fused(const Shape &s);
int route_fused_bt(const Shape &s);
int route_fused_ntiles(const Shape &s);
// statistic partials per expert: one per route block, or per fused tile
int route_stat_blocks(const Shape &s);
// floats of the logit partials in the workspace, and bytes of the split
// matrix (fused router)
size_t route_part_floats(const Shape &s);
size_t route_wsplit_bytes(const Shape &s);

// arrivals: a 4-byte counter in the workspace (zeroed by launch_route's
// kernels, used and re-zeroed by the statistics kernel); fP: E + 1 doubles.
// wsplit: route_wsplit_bytes() of workspace (used when route_fused()).
hipError_t launch_route(const Shape &s, const void *x, const float *Wr, const float *bias,
                        const float *noise, int32_t *topk_idx, float *gates, float *part_P,
                        float *part_lse2, float *part_logits, void *wsplit, unsigned *arrivals,
                        hipStream_t st);
// Small bf16 batches (T <= ROUTE_SMALL_T tokens, T*k <= ROUTE_SMALL_TK):
// after the logits, one block finishes the routing -- slices summed,
// softmax, top-k, gates, statistics and (when the dispatch outputs are
// given) the dispatch -- in place of the epilogue, statistics and dispatch
// kernels.  The results equal theirs: every integer output bit for bit, and
// the statistics up to the grouping of the partial sums (one block here).
constexpr int ROUTE_SMALL_T = 64;
constexpr int ROUTE_SMALL_TK = 2048;
inline bool route_small(const Shape &s) {
    return s.dtype == 1 && s.T <= ROUTE_SMALL_T && s.Tk() <= ROUTE_SMALL_TK;
}
struct DispatchOut {
    int32_t *routed, *kept, *offsets, *row_of_slot, *token_of_row;
    uint8_t *dropped;
};
hipError_t launch_route_small(const Shape &s, const void *x, const float *Wr, const float *bias,
                              const float *noise, int32_t *topk_idx, float *gates, float *stats,
                              const DispatchOut *disp, float *part_P, float *part_lse2,
                              float *part_logits, hipStream_t st);
hipError_t launch_route_finalize(const Shape &s, const int32_t *topk_idx, const float *part_P,
                                 const float *part_lse2, float *stats, double *fP,
                                 unsigned *arrivals, hipStream_t st);

// ---- dispatch: capacity, stable permutation, gather ----------------------
// Assignments per dispatch block (256 per round; more rounds when T*k is
// large); per-chunk expert histograms [chunks][E] int32 live in the
// workspace.
int dispatch_chunk(const Shape &s);
int dispatch_chunks(const Shape &s);
// The statistics' inputs and outputs (those of launch_route_finalize), for a
// dispatch launch that also finishes the statistics in extra blocks.
struct RouteStatsIn {
    const float *part_P, *part_lse2;
    int nblk;
    float *stats;
    double *fP;
    unsigned *arrivals;
};
// zero_ctr (n_zero words), when given, is cleared by the ranking launch:
// the tile counters of the expert GEMMs that follow (launch_expert_up/down).
hipError_t launch_dispatch(const Shape &s, const int32_t *topk_idx, int32_t *routed,
                           int32_t *kept, int32_t *offsets, int32_t *row_of_slot,
                           int32_t *token_of_row, uint8_t *dropped, int32_t *chunk_counts,
                           hipStream_t st, const RouteStatsIn *stats = nullptr,
                           unsigned *zero_ctr = nullptr, int n_zero = 0);
// Clears n words (a one-block kernel; no memset node in a captured graph).
hipError_t launch_zero_u32(unsigned *p, int n, hipStream_t st);
hipError_t launch_gather(const Shape &s, const void *x, const int32_t *token_of_row,
                         const int32_t *offsets, void *x_perm, hipStream_t st);

// Shared experts (every token, no gate), all S of them as one dense layer:
// the up projection is one row group of T rows against the S experts' W1
// (and W3) stacked as [S*d_ff][d] (their native layout), so H_sh is
// [T][S*d_ff] with expert j at columns j*d_ff; the down projection is one
// GEMM with K = S*d_ff against W2 repacked as [d][S*d_ff] (expert j's
// columns at j*d_ff), which sums the S experts' outputs in its fp32
// accumulation, in expert order.  shared_shape() is that layer's shape.
inline Shape shared_shape(const Shape &s, int S) {
    Shape q = s;
    q.E = 1;
    q.k = 1;
    q.C = -1;
    q.d_ff = S * s.d_ff;
    return q;
}
// Row offsets {0, T} of the single row group; for S > 1 also the W2
// repack W2cat[o][j*d_ff + f] = W2s[j][o][f] (act dtype).
size_t shared_w2cat_bytes(const Shape &s, int S);
hipError_t launch_shared_prep(const Shape &s, int S, const void *W2s, void *W2cat,
                              int32_t *offsets, hipStream_t st);

// ---- expert FFN: grouped GEMMs over ragged per-expert row blocks --------
// a_rows: row r of A is A[a_rows[r]] (the gather done by the loads);
// nullptr: row r is A[r].
// tctr: TILE_CTR_WORDS words, zero when the launch starts (or nullptr):
// the 256-row tile kernel's per-XCD tile counters, which let its blocks
// stay resident and take tiles in turn.  Each launch needs its own (or the
// same ones cleared again); the other kernels ignore them.
constexpr int TILE_CTR_WORDS = 8;
hipError_t launch_expert_up(const Shape &s, const void *x_perm, const int32_t *a_rows,
                            const int32_t *offsets, const void *W1, const void *W3, void *H,
                            hipStream_t st, unsigned *tctr);
// The down projection may split K in two (down_ksplit(s) == 2, when its
// tiles would not fill three rounds of the CUs): the second half's partial
// sums go to y_perm_part2 (same layout as y_perm) and must be added, either
// by launch_add_partial or by the combine (which adds them before gating).
int down_ksplit(const Shape &s);
hipError_t launch_expert_down(const Shape &s, const void *H, const int32_t *offsets,
                              const void *W2, float *y_perm, float *y_perm_part2,
                              hipStream_t st, unsigned *tctr);
hipError_t launch_add_partial(const Shape &s, float *y_perm, const float *part2,
                              const int32_t *offsets, hipStream_t st);

// ---- expert weights in e4m3 (decode batches) ------------------------------
// Row-wise post-training quantisation (dtype 1: bf16 input, 0: fp32).
hipError_t launch_quantize_e4m3(int dtype, const void *W, int64_t rows, int64_t cols, uint8_t *q,
                                float *scales, hipStream_t st);
// The e4m3-weight expert GEMMs exist for the weight-streaming shapes only:
// bf16 activations, at most 48 rows per expert, d and d_ff multiples of 128.
bool fp8_supported(const Shape &s);
// packed: the codes are in the streaming tile layout (launch_pack_stream)
// instead of row-major.
hipError_t launch_expert_up_fp8(const Shape &s, const void *A, const int32_t *a_rows,
                                const int32_t *offsets, const uint8_t *W1, const uint8_t *W3,
                                const float *S1, const float *S3, void *H, hipStream_t st,
                                bool packed = false);
hipError_t launch_expert_down_fp8(const Shape &s, const void *H, const int32_t *offsets,
                                  const uint8_t *W2, const float *S2, float *y_perm, hipStream_t st,
                                  bool packed = false);

// ---- weights in the streaming tile layout ------------------------------
// [rows][cols] of esz-byte elements (2: bf16, 1: e4m3 codes) -> the
// layout the weight-streaming kernels read with one contiguous KB per load
// instruction (rows % 16 == 0, cols % 128 == 0; see pack_stream_kernel).
hipError_t launch_pack_stream(int esz, const void *W, int64_t rows, int64_t cols, void *out, hipStream_t st);
// bf16 expert GEMMs on packed weights, for the shapes fp8_supported() accepts
hipError_t launch_expert_up_packed(const Shape &s, const void *x, const int32_t *a_rows, const int32_t *offsets,
                                   const void *W1, const void *W3, void *H, hipStream_t st);
hipError_t launch_expert_down_packed(const Shape &s, const void *H, const int32_t *offsets, const void *W2,
                                     float *y_perm, hipStream_t st);

// ---- backward (training gradients) --------------------------------------
// batched transposes of the expert weights; with row offsets (may be
// nullptr) the matrices of experts without rows are skipped
hipError_t launch_transpose_bf16(const void *src, int64_t R, int64_t C, int64_t lds, int64_t sbs,
                                 void *dst, int64_t ldd, int64_t dbs, int batch, hipStream_t st,
                                 const int32_t *offsets);
// fp32 layers' backward: batched transpose (dst[b][c][r] = src[b][r][c]) and
// the per-expert weight gradients C[e][m][n] = sum over e's rows of P[r][m] Q[r][n]
hipError_t launch_transpose_f32(const float *src, int64_t R, int64_t C, int64_t lds, int64_t sbs, float *dst,
                                int64_t ldd, int64_t dbs, int batch, hipStream_t st, const int32_t *offsets);
hipError_t launch_wgrad_f32(int E, int M, int N, const int32_t *offsets, const float *P, int64_t ldp,
                            const float *Q, int64_t ldq, float *C, hipStream_t st);
hipError_t launch_act_fwd(const Shape &s, const float *a1, const float *a3, const int32_t *offsets,
                          void *H, hipStream_t st);
hipError_t launch_combine_bwd(const Shape &s, const void *dy, const float *Y, const int32_t *token_of_row,
                              const int32_t *row_of_slot, const float *gates, const int32_t *offsets,
                              void *dE, float *dg, hipStream_t st);
hipError_t launch_act_bwd(const Shape &s, const float *a1, const float *a3, const float *dH,
                          const int32_t *offsets, void *dA, hipStream_t st);
// logits: false when p and lse are already there (launch_logits_mfma)
hipError_t launch_router_bwd(const Shape &s, const void *x, const float *Wr, const float *bias,
                             const float *noise, const int32_t *topk_idx, const float *gates,
                             const float *dg, const int32_t *row_of_slot, const float *f,
                             float alpha_aux, float alpha_z, float *p, float *lse, float *dh,
                             hipStream_t st, bool logits = true);
hipError_t launch_dx(const Shape &s, const float *dXp, const int32_t *row_of_slot, const float *dh,
                     const float *Wr, float *dx, hipStream_t st);
size_t dwr_part_floats(const Shape &s);
hipError_t launch_dwr(const Shape &s, const float *dh, const void *x, float *part, float *dWr,
                      float *dbias, hipStream_t st);
// Weight gradients read the activations transposed into a padded layout:
// expert e's kept rows become positions poff[e] .. poff[e] + count_e - 1 of
// each row, poff[e] = the sum over e' < e of count_e' rounded up to 64, and
// the pad positions up to poff[e + 1] hold zeros.  padded_rows_bound bounds
// poff[E] (a multiple of 64) for R kept rows at most.
int64_t padded_rows_bound(int64_t R, int E);
hipError_t launch_pad_offsets(const int32_t *offsets, int E, int32_t *poff, hipStream_t st);
// dst[c][poff[e] + i] = src[offsets[e] + i][c] (bf16, c < C, row stride lds
// of src, ldp of dst), zeros on the pad positions; positions past poff[E]
// are not written.
hipError_t launch_transpose_padded(const void *src, int64_t C, int64_t lds, const int32_t *offsets,
                                   const int32_t *poff, int E, int64_t ldp, void *dst, hipStream_t st);
// C[e][m][n] = sum over k in [koff[e], koff[e+1]) of P[m][k] Q[n][k]
// (P [M][ldk], Q [N][ldk] bf16, C fp32).  launch_wgrad: 128 x 128 tiles, any
// k range; launch_wgrad_big: the 256 x 256 direct-to-LDS tiles of the
// forward's grouped GEMM, for k ranges that start and end on multiples of
// 64 (the padded layout), M and N multiples of 8 and both operands under
// 2 GiB (wgrad_big_fits).
// dW_r = sum over tokens of dh_t x_t^T on matrix cores: dh [T][E] fp32 split
// into three bf16 terms (hi, mid = the rest's bf16, lo = what remains; their
// sum carries dh's 24 significant bits), stacked as the rows of P [3 Ep][Tp]
// (Ep = E rounded up to 8, Tp = T rounded up to 64, zero pads), x transposed
// to [d][Tp]; the weight-gradient GEMM over ns token ranges (its "experts")
// writes ns partial [3 Ep][d] products, which dwr_sum adds term by term
// (lo, mid, hi), range by range in order.  ns == 0: not used (E < 16, or K
// too large for 32-bit buffer offsets); the token-split kernel runs instead.
struct DwrPlan {
    int Ep, ns;
    int64_t Tp;
    size_t xt_bytes, p_bytes, c_bytes, idx_bytes;
};
DwrPlan dwr_plan(const Shape &s);
hipError_t launch_dwr_mfma(const Shape &s, const DwrPlan &pl, const float *dh, const void *x, void *xt,
                           void *pterms, float *cpart, int32_t *idx, float *dWr, float *dbias,
                           hipStream_t st);
// The router logits of the backward on matrix cores: W_r split into the
// same three bf16 terms (rows q Ep + e of Ws [3 Ep][d]), h = x Ws^T through
// the weight-gradient GEMM over ns ranges of d (its "experts"; x is already
// [T][d], K-contiguous), the partial products added term by term (lo, mid,
// hi) and range by range in order, then bias, noise, softmax and lse.
// ns == 0: not used (d not a multiple of 64, T not a multiple of 8, or
// operands past 32-bit offsets); the fp32 kernels run instead.
struct LogitsPlan {
    int Ep, ns;
    size_t ws_bytes, c_bytes, idx_bytes;
};
LogitsPlan logits_plan(const Shape &s);
hipError_t launch_logits_mfma(const Shape &s, const LogitsPlan &pl, const void *x, const float *Wr,
                              const float *bias, const float *noise, void *wsplit, float *cpart,
                              int32_t *idx, float *p, float *lse, hipStream_t st);
hipError_t launch_wgrad(int E, int M, int N, const int32_t *koff, const void *P, const void *Q,
                        int64_t ldk, float *C, hipStream_t st);
bool wgrad_big_fits(int M, int N, int64_t ldk);
hipError_t launch_wgrad_big(int E, int M, int N, const int32_t *koff, const void *P, const void *Q,
                            int64_t ldk, float *C, hipStream_t st);

// ---- static scratch of moe_forward_noalloc --------------------------------
// The device address of the current device's copy of the library's static
// scratch array (MOE_NOALLOC_SCRATCH_BYTES), looked up on first use per
// device and kept.
hipError_t noalloc_scratch(void **ptr);

// ---- combine -------------------------------------------------------------
// y_perm_part2: nullptr, or the second K half of a split down projection.
hipError_t launch_combine(const Shape &s, const float *y_perm, const float *y_perm_part2,
                          const int32_t *row_of_slot, const float *gates, void *y,
                          hipStream_t st);

// Combine plus the shared experts' summed row (y_sh [T][d] fp32, or
// nullptr; y_sh_part2 its second K half, or nullptr) and the residual (act
// dtype, or nullptr), added in that order after the routed slots.
hipError_t launch_combine_shared(const Shape &s, const float *y_perm, const float *y_perm_part2,
                                 const int32_t *row_of_slot, const float *gates, const float *y_sh,
                                 const float *y_sh_part2, const void *residual, void *y,
                                 hipStream_t st);

}  // namespace moe

// ---- device helpers shared by the kernels --------------------------------
#if defined(__HIPCC__)
namespace moe {

// fp32 -> bf16 bits, round to nearest even (NaN becomes a quiet NaN).
// The lanes of the wave whose expert equals this lane's (valid lanes only;
// 0 for an invalid lane), found bit by bit: for each of the nbits low bits
// of e (nbits uniform, 2^nbits >= E), keep the lanes whose bit agrees.  One
// ballot per bit, whatever the number of distinct experts in the wave.  A
// lane's rank among its expert's lanes in lane order is then the popcount
// of the mask below it, and the group's lowest lane can publish its size.
__device__ __forceinline__ unsigned long long lanes_with_same_expert(int e, bool valid, int nbits) {
    unsigned long long m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const unsigned long long bm = __ballot(bit);
        m &= bit ? bm : ~bm;
    }
    return valid ? m : 0ull;
}
// Bits that tell apart the expert indices 0 .. E - 1.
__host__ __device__ inline int expert_bits(int E) {
    int b = 0;
    while ((1 << b) < E) ++b;
    return b;
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));


// Expert activations of the GEMM epilogues (ACT_NONE: the down projection).
constexpr int ACT_RELU = 0, ACT_GELU = 1, ACT_SWIGLU = 2, ACT_NONE = 3;

// SwiGLU uses the hardware exp2 and reciprocal (about 1 ulp each; the
// result is rounded to bf16, 8 bits, right after).  GELU keeps erff.
__device__ __forceinline__ float apply_act(int act, float a1, float a3) {
    if (act == ACT_SWIGLU)
        return a1 * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.44269504088896341f * a1)) * a3;
    if (act == ACT_GELU) return 0.5f * a1 * (1.f + erff(a1 * 0.70710678118654752f));
    if (act == ACT_RELU) return fmaxf(a1, 0.f);
    return a1;
}

// Activation backward of one element: u = a1, v = a3 (SwiGLU), g = dH; da1
// and (SwiGLU) da3 as bf16 bits.  SwiGLU: H = silu(u) v; GELU (erf form);
// ReLU (derivative 0 at u = 0).
__device__ __forceinline__ void act_bwd_f32(int act, float u, float v, float g, float &da1, float &da3) {
    da3 = 0.f;
    if (act == ACT_SWIGLU) {
        const float sg = 1.f / (1.f + expf(-u));
        da1 = g * v * sg * (1.f + u * (1.f - sg));
        da3 = g * u * sg;
    } else if (act == ACT_GELU) {
        const float Phi = 0.5f * (1.f + erff(u * 0.70710678118654752f));
        const float phi = expf(-0.5f * u * u) * 0.39894228040143268f;
        da1 = g * (Phi + u * phi);
    } else {
        da1 = u > 0.f ? g : 0.f;
    }
}
__device__ __forceinline__ void act_bwd_elem(int act, float u, float v, float g, uint16_t &da1,
                                             uint16_t &da3) {
    float a, b;
    act_bwd_f32(act, u, v, g, a, b);
    da1 = f32_to_bf16(a);
    if (act == ACT_SWIGLU) da3 = f32_to_bf16(b);
}

}  // namespace moe
#endif
