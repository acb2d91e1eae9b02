// dispatch.hip -- capacity, stable permutation by expert, and gather.
//
// Page "Mixture of experts" (rayaq.ca), Mechanics, "Capacity and dropped
// tokens": each expert has C slots, filled in position (token) order;
// assignments beyond C are dropped and skip the expert.  Implementation
// section: the per-expert token lists are in token order, and production
// kernels replace the loop over experts by a sort of tokens by expert.
//
// dispatch_kernel: one block per expert e (grid = E), 256 threads.
//   A. Histogram of all T*k assignments over experts with LDS integer
//      atomics (a count is order-independent, so the result is exact and
//      reproducible).  From it every block knows routed_e, kept_e =
//      min(routed_e, C) and its row offset sum_{e' < e} kept_e'.
//   B. Rank of every assignment of expert e in token order: the block
//      sweeps the assignments t-major in chunks of 256; a 64-lane ballot
//      and popcount give each lane its rank inside the wave, four wave
//      totals in LDS give the wave's base, and a running block base carries
//      the count across chunks.  No atomic decides any order.
//      rank < C: row = offset_e + rank, else dropped.
// gather_kernel: x_perm[r] = x[token_of_row[r]] for r < offsets[E]; one
//   wave per row, 16-byte loads and stores, grid-stride over rows.
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int DP_THREADS = 256;
constexpr int DP_EMAX = 128;

__global__ __launch_bounds__(DP_THREADS) void dispatch_kernel(
    const int32_t *__restrict__ topk_idx, int64_t Tk, int k, int E, int64_t C,
    int32_t *__restrict__ routed, int32_t *__restrict__ kept, int32_t *__restrict__ offsets,
    int32_t *__restrict__ row_of_slot, int32_t *__restrict__ token_of_row,
    uint8_t *__restrict__ dropped) {
    __shared__ int hist[DP_EMAX];
    __shared__ int wsum[DP_THREADS / 64];
    __shared__ int sh_off, sh_total;
    const int tid = threadIdx.x;
    const int e = blockIdx.x;
    const int lane = tid & 63, w = tid >> 6;

    if (tid < DP_EMAX) hist[tid] = 0;
    __syncthreads();
    for (int64_t j = tid; j < Tk; j += DP_THREADS) atomicAdd(&hist[topk_idx[j]], 1);
    __syncthreads();
    if (tid == 0) {
        int64_t off = 0, tot = 0;
        for (int i = 0; i < E; ++i) {
            int64_t kp = (C >= 0 && hist[i] > C) ? C : hist[i];
            if (i < e) off += kp;
            tot += kp;
        }
        sh_off = (int)off;
        sh_total = (int)tot;
        int64_t ke = (C >= 0 && hist[e] > C) ? C : hist[e];
        routed[e] = hist[e];
        kept[e] = (int)ke;
        offsets[e] = (int)off;
        if (e == E - 1) offsets[E] = (int)tot;
    }
    __syncthreads();
    const int off = sh_off, total = sh_total;

    int64_t base = 0;
    const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int64_t j0 = 0; j0 < Tk; j0 += DP_THREADS) {
        const int64_t j = j0 + tid;
        const bool pred = (j < Tk) && (topk_idx[j] == e);
        const unsigned long long b = __ballot(pred);
        if (lane == 0) wsum[w] = __popcll(b);
        __syncthreads();
        int wbase = 0, btot = 0;
#pragma unroll
        for (int i = 0; i < DP_THREADS / 64; ++i) {
            int c = wsum[i];
            wbase += (i < w) ? c : 0;
            btot += c;
        }
        if (pred) {
            const int64_t rank = base + wbase + __popcll(b & lt_mask);
            if (C < 0 || rank < C) {
                const int row = off + (int)rank;
                row_of_slot[j] = row;
                token_of_row[row] = (int)(j / k);
                dropped[j] = 0;
            } else {
                row_of_slot[j] = -1;
                dropped[j] = 1;
            }
        }
        base += btot;
        __syncthreads();  // wsum is rewritten by the next chunk
    }
    // rows past the last kept one hold no token
    for (int64_t r = (int64_t)total + (int64_t)e * DP_THREADS + tid; r < Tk;
         r += (int64_t)E * DP_THREADS)
        token_of_row[r] = -1;
}

// One wave per permuted row; row_bytes is a multiple of VEC.
template <typename V>
__global__ __launch_bounds__(256) void gather_kernel(const char *__restrict__ x,
                                                     const int32_t *__restrict__ token_of_row,
                                                     const int32_t *__restrict__ offsets, int E,
                                                     int64_t row_bytes, char *__restrict__ x_perm) {
    const int lane = threadIdx.x & 63;
    const int64_t n = offsets[E];
    const int64_t nv = row_bytes / (int64_t)sizeof(V);
    for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < n;
         r += (int64_t)gridDim.x * 4) {
        const V *src = (const V *)(x + (int64_t)token_of_row[r] * row_bytes);
        V *dst = (V *)(x_perm + r * row_bytes);
        for (int64_t c = lane; c < nv; c += 64) dst[c] = src[c];
    }
}

}  // namespace

hipError_t launch_dispatch(const Shape &s, const int32_t *topk_idx, int32_t *routed,
                           int32_t *kept, int32_t *offsets, int32_t *row_of_slot,
                           int32_t *token_of_row, uint8_t *dropped, hipStream_t st) {
    hipLaunchKernelGGL(dispatch_kernel, dim3(s.E), dim3(DP_THREADS), 0, st, topk_idx, s.Tk(), s.k,
                       s.E, s.C, routed, kept, offsets, row_of_slot, token_of_row, dropped);
    return hipGetLastError();
}

hipError_t launch_gather(const Shape &s, const void *x, const int32_t *token_of_row,
                         const int32_t *offsets, void *x_perm, hipStream_t st) {
    const int64_t row_bytes = (int64_t)s.d * (s.dtype == 1 ? 2 : 4);
    int64_t blocks = (s.Tk() + 3) / 4;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    if (row_bytes % 16 == 0)
        hipLaunchKernelGGL(gather_kernel<uint4>, dim3((unsigned)blocks), dim3(256), 0, st,
                           (const char *)x, token_of_row, offsets, s.E, row_bytes, (char *)x_perm);
    else if (row_bytes % 4 == 0)
        hipLaunchKernelGGL(gather_kernel<uint32_t>, dim3((unsigned)blocks), dim3(256), 0, st,
                           (const char *)x, token_of_row, offsets, s.E, row_bytes, (char *)x_perm);
    else
        hipLaunchKernelGGL(gather_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, st,
                           (const char *)x, token_of_row, offsets, s.E, row_bytes, (char *)x_perm);
    return hipGetLastError();
}

}  // namespace moe
