// dispatch.hip -- capacity, stable permutation by expert, and gather.
//
// Page "Mixture of experts" (rayaq.ca), Mechanics, "Capacity and dropped
// tokens": each expert has C slots, filled in position (token) order;
// assignments beyond C are dropped and skip the expert.  Implementation
// section: the per-expert token lists are in token order, and production
// kernels replace the loop over experts by a sort of tokens by expert.
//
// The T*k assignments are read t-major (token t, slot s at j = t*k + s),
// which is token order within every expert (an expert appears at most once
// per token).  They are cut into chunks of 256 (1024 when T*k is large).
//   dispatch_count_kernel (one block per chunk): per-chunk histogram over
//     experts with LDS integer atomics (a count does not depend on the
//     order of the additions).  Skipped when there is a single chunk: the
//     ranking block then counts its own chunk.
//   dispatch_rank_kernel (one block per chunk): every block derives, from
//     all chunk histograms, routed_e, kept_e = min(routed_e, C), the row
//     offsets (exclusive prefix of kept_e) and, for its own chunk, how many
//     assignments of each expert precede it.  It then ranks its chunk in
//     order, 256 assignments per round: inside a wave, lanes with the same
//     expert are grouped by ballot (leader's expert, then the lanes that
//     match it) and ranked by popcount of the lower lanes; a table of
//     per-wave counts in LDS adds the waves before, and a per-expert
//     running count carries the rounds.  No atomic decides any order.
//     rank < C: row = offset_e + rank; else dropped.
// gather_kernel: x_perm[r] = x[token_of_row[r]] for r < offsets[E]; one
//   wave per row, 16-byte loads and stores, grid-stride over rows.
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int DP_THREADS = 256;
constexpr int DP_EMAX = 128;

__global__ __launch_bounds__(DP_THREADS) void dispatch_count_kernel(
    const int32_t *__restrict__ topk_idx, int64_t Tk, int E, int chunk,
    int32_t *__restrict__ chunk_counts) {
    __shared__ int hist[DP_EMAX];
    const int tid = threadIdx.x;
    if (tid < DP_EMAX) hist[tid] = 0;
    __syncthreads();
    const int64_t j0 = (int64_t)blockIdx.x * chunk;
    for (int q = 0; q < chunk / DP_THREADS; ++q) {
        const int64_t j = j0 + q * DP_THREADS + tid;
        if (j < Tk) atomicAdd(&hist[topk_idx[j]], 1);
    }
    __syncthreads();
    if (tid < E) chunk_counts[(int64_t)blockIdx.x * E + tid] = hist[tid];
}

__global__ __launch_bounds__(DP_THREADS) void dispatch_rank_kernel(
    const int32_t *__restrict__ topk_idx, int64_t Tk, int k, int E, int64_t C, int chunk_len,
    int nchunks, const int32_t *__restrict__ chunk_counts, int32_t *__restrict__ routed,
    int32_t *__restrict__ kept, int32_t *__restrict__ offsets, int32_t *__restrict__ row_of_slot,
    int32_t *__restrict__ token_of_row, uint8_t *__restrict__ dropped) {
    __shared__ int running[DP_EMAX];  // assignments of e before the current round
    __shared__ int off[DP_EMAX];      // first row of expert e
    __shared__ int keptc[DP_EMAX];
    __shared__ int wcnt[DP_THREADS / 64][DP_EMAX];
    __shared__ int sh_total;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int chunk = blockIdx.x;

    if (nchunks == 1) {
        // a single chunk counts its own assignments (no histogram kernel ran)
        if (tid < DP_EMAX) running[tid] = 0;
        __syncthreads();
        for (int64_t j = tid; j < Tk; j += DP_THREADS) atomicAdd(&running[topk_idx[j]], 1);
        __syncthreads();
    }
    if (tid < E) {
        int before = 0, tot = 0;
        if (nchunks == 1) {
            tot = running[tid];
        } else {
#pragma unroll 8
            for (int c = 0; c < nchunks; ++c) {
                const int v = chunk_counts[(int64_t)c * E + tid];
                before += (c < chunk) ? v : 0;
                tot += v;
            }
        }
        running[tid] = before;
        keptc[tid] = (C >= 0 && tot > C) ? (int)C : tot;
        if (chunk == 0) {
            routed[tid] = tot;
            kept[tid] = keptc[tid];
        }
    }
    __syncthreads();
    if (tid == 0) {
        int o = 0;
        for (int e = 0; e < E; ++e) {
            off[e] = o;
            o += keptc[e];
        }
        sh_total = o;
        if (chunk == 0) {
            for (int e = 0; e < E; ++e) offsets[e] = off[e];
            offsets[E] = o;
        }
    }
    __syncthreads();

    const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int64_t j0 = (int64_t)chunk * chunk_len;
    for (int round = 0; round < chunk_len / DP_THREADS; ++round) {
        for (int i = tid; i < (DP_THREADS / 64) * DP_EMAX; i += DP_THREADS) (&wcnt[0][0])[i] = 0;
        __syncthreads();
        const int64_t j = j0 + round * DP_THREADS + tid;
        const bool valid = j < Tk;
        const int ej = valid ? topk_idx[j] : -1;
        // group the wave's lanes by expert, in lane (= assignment) order
        bool act = valid;
        int rank_w = 0;
        while (true) {
            const unsigned long long am = __ballot(act);
            if (am == 0ull) break;
            const int leader = __ffsll((long long)am) - 1;
            const int e0 = __builtin_amdgcn_readlane(ej, leader);  // leader is wave-uniform
            const bool m = act && ej == e0;
            const unsigned long long mm = __ballot(m);
            if (m) {
                rank_w = __popcll(mm & lt_mask);
                act = false;
            }
            if (lane == leader) wcnt[w][e0] = __popcll(mm);
        }
        __syncthreads();
        if (valid) {
            int rank = running[ej] + rank_w;
            for (int v = 0; v < w; ++v) rank += wcnt[v][ej];
            if (C < 0 || rank < C) {
                const int row = off[ej] + rank;
                row_of_slot[j] = row;
                token_of_row[row] = (int)(j / k);
                dropped[j] = 0;
            } else {
                row_of_slot[j] = -1;
                dropped[j] = 1;
            }
        }
        __syncthreads();
        if (tid < E) {
            int add = 0;
            for (int v = 0; v < DP_THREADS / 64; ++v) add += wcnt[v][tid];
            running[tid] += add;
        }
        __syncthreads();
    }
    // rows past the last kept one hold no token
    for (int64_t r = (int64_t)sh_total + (int64_t)chunk * DP_THREADS + tid; r < Tk;
         r += (int64_t)nchunks * DP_THREADS)
        token_of_row[r] = -1;
}

// One wave per permuted row; row_bytes is a multiple of sizeof(V).
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

int dispatch_chunk(const Shape &s) { return s.Tk() >= 32768 ? 4 * DP_THREADS : DP_THREADS; }
int dispatch_chunks(const Shape &s) {
    return (int)((s.Tk() + dispatch_chunk(s) - 1) / dispatch_chunk(s));
}

hipError_t launch_dispatch(const Shape &s, const int32_t *topk_idx, int32_t *routed,
                           int32_t *kept, int32_t *offsets, int32_t *row_of_slot,
                           int32_t *token_of_row, uint8_t *dropped, int32_t *chunk_counts,
                           hipStream_t st) {
    const int nch = dispatch_chunks(s);
    const int chunk = dispatch_chunk(s);
    if (nch > 1)
        hipLaunchKernelGGL(dispatch_count_kernel, dim3(nch), dim3(DP_THREADS), 0, st, topk_idx,
                           s.Tk(), s.E, chunk, chunk_counts);
    hipLaunchKernelGGL(dispatch_rank_kernel, dim3(nch), dim3(DP_THREADS), 0, st, topk_idx, s.Tk(),
                       s.k, s.E, s.C, chunk, nch, (const int32_t *)chunk_counts, routed, kept,
                       offsets, row_of_slot, token_of_row, dropped);
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
