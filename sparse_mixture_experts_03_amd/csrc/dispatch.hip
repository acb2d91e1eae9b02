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
//     ranking block then counts its own chunk.  Both kernels load their
//     chunk's indices in one round trip into LDS and check them there.
//   dispatch_rank_kernel (one block per chunk): every block derives, from
//     all chunk histograms, routed_e, kept_e = min(routed_e, C), the row
//     offsets (exclusive prefix of kept_e) and, for its own chunk, how many
//     assignments of each expert precede it.  It then ranks its chunk in
//     order, 256 assignments per round: inside a wave, the lanes with the
//     same expert are found bit by bit of the expert index (one ballot per
//     bit) and ranked by popcount of the lower lanes; a table of
//     per-wave counts in LDS adds the waves before, and a per-expert
//     running count carries the rounds.  No atomic decides any order.
//     rank < C: row = offset_e + rank; else dropped.
// gather_kernel: x_perm[r] = x[token_of_row[r]] for r < offsets[E]; one
//   wave per row, 16-byte loads and stores, grid-stride over rows.
#include "moe_internal.h"
#include "route_stats.h"

namespace moe {

namespace {

constexpr int DP_THREADS = 256;
constexpr int DP_EMAX = 128;
constexpr int DP_MAXR = 4;   // rounds of DP_THREADS assignments per chunk (chunk <= 1024)

// The expert of assignment j (token j / k, slot j % k), whose index e was
// read, or -1 when the assignment is not a valid choice: an index outside
// [0, E), or an expert the token already chose in an earlier slot.  Routing
// from moe_route never has either; moe_dispatch takes caller indices, and
// an invalid one is treated as dropped (not routed, no row) instead of
// indexing the LDS histograms out of range or giving an expert more rows
// than tokens.  The token's earlier slots come from tkc, the chunk's
// indices in LDS (chunk start j0), or from memory when the token began in
// the previous chunk.
__device__ __forceinline__ int valid_expert(int e, int64_t j, int64_t j0, int k, int E, const int *tkc,
                                            const int32_t *__restrict__ topk_idx) {
    if ((unsigned)e >= (unsigned)E) return -1;
    for (int64_t i = j - j % k; i < j; ++i)
        if ((i >= j0 ? tkc[i - j0] : topk_idx[i]) == e) return -1;
    return e;
}

__global__ __launch_bounds__(DP_THREADS) void dispatch_count_kernel(
    const int32_t *__restrict__ topk_idx, int64_t Tk, int k, int E, int chunk,
    int32_t *__restrict__ chunk_counts) {
    __shared__ int hist[DP_EMAX];
    __shared__ int tkc[DP_MAXR * DP_THREADS];   // the chunk's expert indices
    const int tid = threadIdx.x;
    const int nr = chunk / DP_THREADS;
    const int64_t j0 = (int64_t)blockIdx.x * chunk;
    // all of the chunk's loads in flight together, then validity from LDS
    int raw[DP_MAXR];
#pragma unroll
    for (int q = 0; q < DP_MAXR; ++q) {
        const int64_t j = j0 + q * DP_THREADS + tid;
        raw[q] = (q < nr && j < Tk) ? topk_idx[j] : -1;
    }
#pragma unroll
    for (int q = 0; q < DP_MAXR; ++q)
        if (q < nr) tkc[q * DP_THREADS + tid] = raw[q];
    if (tid < DP_EMAX) hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < DP_MAXR; ++q) {
        const int64_t j = j0 + q * DP_THREADS + tid;
        if (q < nr && j < Tk) {
            const int e = valid_expert(raw[q], j, j0, k, E, tkc, topk_idx);
            if (e >= 0) atomicAdd(&hist[e], 1);
        }
    }
    __syncthreads();
    if (tid < E) chunk_counts[(int64_t)blockIdx.x * E + tid] = hist[tid];
}

// Blocks past the last chunk (when moe_forward passes the statistics'
// arguments) finish the load-balancing statistics instead (route_stats.h),
// so that reduction runs beside the ranking rather than as its own launch.
struct StatsArgs {
    const float *part_P, *part_lse2;
    int T, nblk;
    float *stats;
    double *fP;
    unsigned *arrivals;
    unsigned *zero_ctr;   // words cleared by block 0 (the GEMMs' tile counters)
    int n_zero;
};

__global__ __launch_bounds__(DP_THREADS) void dispatch_rank_kernel(
    const int32_t *__restrict__ topk_idx, int64_t Tk, int k, int E, int64_t C, int chunk_len,
    int nchunks, const int32_t *__restrict__ chunk_counts, int32_t *__restrict__ routed,
    int32_t *__restrict__ kept, int32_t *__restrict__ offsets, int32_t *__restrict__ row_of_slot,
    int32_t *__restrict__ token_of_row, uint8_t *__restrict__ dropped, StatsArgs sa) {
    if ((int)blockIdx.x >= nchunks) {
        route_stats_block((int)blockIdx.x - nchunks, sa.part_P, sa.part_lse2, sa.T, E, sa.nblk, sa.stats, sa.fP,
                          sa.arrivals);
        return;
    }
    __shared__ int running[DP_EMAX];  // assignments of e before the current round
    __shared__ int off[DP_EMAX];      // first row of expert e
    __shared__ int keptc[DP_EMAX];
    __shared__ int wcnt[DP_THREADS / 64][DP_EMAX];
    __shared__ int tkc[DP_MAXR * DP_THREADS];   // the chunk's expert indices
    __shared__ int sh_total;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int chunk = blockIdx.x;
    const int nr = chunk_len / DP_THREADS;      // rounds of 256 assignments
    if (chunk == 0 && tid < sa.n_zero) sa.zero_ctr[tid] = 0u;
    const int64_t j0 = (int64_t)chunk * chunk_len;

    // One memory round trip for everything the ranking reads: the chunk
    // histograms (expert tid's count in every chunk) and this chunk's
    // indices are all loaded before the first use.
    int before = 0, tot = 0;
    if (nchunks > 1 && tid < E) {
#pragma unroll 32
        for (int c = 0; c < nchunks; ++c) {
            const int v = chunk_counts[(int64_t)c * E + tid];
            before += (c < chunk) ? v : 0;
            tot += v;
        }
    }
    int raw[DP_MAXR];
#pragma unroll
    for (int q = 0; q < DP_MAXR; ++q) {
        const int64_t j = j0 + q * DP_THREADS + tid;
        raw[q] = (q < nr && j < Tk) ? topk_idx[j] : -1;
    }
#pragma unroll
    for (int q = 0; q < DP_MAXR; ++q)
        if (q < nr) tkc[q * DP_THREADS + tid] = raw[q];
    if (tid < DP_EMAX) running[tid] = 0;
    __syncthreads();
    // assignment j's expert, or -1 when it is not a valid choice
    int ej[DP_MAXR];
#pragma unroll
    for (int q = 0; q < DP_MAXR; ++q) {
        const int64_t j = j0 + q * DP_THREADS + tid;
        ej[q] = (q < nr && j < Tk) ? valid_expert(raw[q], j, j0, k, E, tkc, topk_idx) : -1;
    }
    if (nchunks == 1) {
        // a single chunk counts its own assignments (no histogram kernel ran)
#pragma unroll
        for (int q = 0; q < DP_MAXR; ++q)
            if (ej[q] >= 0) atomicAdd(&running[ej[q]], 1);
        __syncthreads();
        if (tid < E) tot = running[tid];
    }
    if (tid < E) {
        running[tid] = before;
        keptc[tid] = (C >= 0 && tot > C) ? (int)C : tot;
        if (chunk == 0) {
            routed[tid] = tot;
            kept[tid] = keptc[tid];
        }
    }
    __syncthreads();
    if (tid < 64) {
        // exclusive prefix of the kept counts over the experts: wave 0, two
        // experts per lane (lane l: experts l and l + 64), shuffle scans
        const int k0 = tid < E ? keptc[tid] : 0, k1 = tid + 64 < E ? keptc[tid + 64] : 0;
        int i0 = k0, i1 = k1;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int u0 = __shfl_up(i0, o), u1 = __shfl_up(i1, o);
            if (tid >= o) {
                i0 += u0;
                i1 += u1;
            }
        }
        const int tot0 = __shfl(i0, 63);
        i1 += tot0;
        if (tid < E) off[tid] = i0 - k0;
        if (tid + 64 < E) off[tid + 64] = i1 - k1;
        const int total = __shfl(i1, 63);
        if (tid == 0) sh_total = total;
        if (chunk == 0) {
            if (tid < E) offsets[tid] = i0 - k0;
            if (tid + 64 < E) offsets[tid + 64] = i1 - k1;
            if (tid == 0) offsets[E] = total;
        }
    }
    __syncthreads();

    const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int nbits = expert_bits(E);
#pragma unroll
    for (int round = 0; round < DP_MAXR; ++round) {
        if (round >= nr) break;
        for (int i = tid; i < (DP_THREADS / 64) * DP_EMAX; i += DP_THREADS) (&wcnt[0][0])[i] = 0;
        __syncthreads();
        const int64_t j = j0 + round * DP_THREADS + tid;
        const bool inrange = j < Tk;
        const int e_j = ej[round];
        const bool valid = e_j >= 0;
        // the wave's lanes with this lane's expert, in lane (= assignment) order
        const unsigned long long mm = lanes_with_same_expert(e_j, valid, nbits);
        const int rank_w = __popcll(mm & lt_mask);
        if (valid && rank_w == 0) wcnt[w][e_j] = __popcll(mm);   // the group's lowest lane
        __syncthreads();
        if (valid) {
            int rank = running[e_j] + rank_w;
            for (int v = 0; v < w; ++v) rank += wcnt[v][e_j];
            if (C < 0 || rank < C) {
                const int row = off[e_j] + rank;
                row_of_slot[j] = row;
                token_of_row[row] = (int)(j / k);
                dropped[j] = 0;
            } else {
                row_of_slot[j] = -1;
                dropped[j] = 1;
            }
        } else if (inrange) {   // not a valid choice: dropped
            row_of_slot[j] = -1;
            dropped[j] = 1;
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
                           hipStream_t st, const RouteStatsIn *stats, unsigned *zero_ctr, int n_zero) {
    const int nch = dispatch_chunks(s);
    const int chunk = dispatch_chunk(s);
    if (nch > 1)
        hipLaunchKernelGGL(dispatch_count_kernel, dim3(nch), dim3(DP_THREADS), 0, st, topk_idx,
                           s.Tk(), s.k, s.E, chunk, chunk_counts);
    if (n_zero > DP_THREADS) return hipErrorInvalidValue;
    StatsArgs sa{};
    unsigned blocks = (unsigned)nch;
    if (stats) {
        sa = StatsArgs{stats->part_P, stats->part_lse2, s.T, stats->nblk, stats->stats, stats->fP, stats->arrivals,
                       nullptr, 0};
        blocks += (unsigned)s.E + 1;
    }
    sa.zero_ctr = zero_ctr;
    sa.n_zero = zero_ctr ? n_zero : 0;
    hipLaunchKernelGGL(dispatch_rank_kernel, dim3(blocks), dim3(DP_THREADS), 0, st, topk_idx, s.Tk(),
                       s.k, s.E, s.C, chunk, nch, (const int32_t *)chunk_counts, routed, kept,
                       offsets, row_of_slot, token_of_row, dropped, sa);
    return hipGetLastError();
}

namespace {
__global__ __launch_bounds__(256) void zero_u32_kernel(unsigned *__restrict__ p, int n) {
    for (int i = threadIdx.x; i < n; i += 256) p[i] = 0u;
}
}  // namespace

hipError_t launch_zero_u32(unsigned *p, int n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

hipError_t launch_gather(const Shape &s, const void *x, const int32_t *token_of_row,
                         const int32_t *offsets, void *x_perm, hipStream_t st) {
    const int64_t row_bytes = (int64_t)s.d * (s.dtype == 1 ? 2 : 4);
    int64_t blocks = (s.Tk() + 3) / 4;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    if (row_bytes % 16 == 0)
        launch_kernel(gather_kernel<uint4>, dim3((unsigned)blocks), dim3(256), 0, st, (const char *)x,
                      token_of_row, offsets, s.E, row_bytes, (char *)x_perm);
    else if (row_bytes % 4 == 0)
        launch_kernel(gather_kernel<uint32_t>, dim3((unsigned)blocks), dim3(256), 0, st, (const char *)x,
                      token_of_row, offsets, s.E, row_bytes, (char *)x_perm);
    else
        launch_kernel(gather_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, st, (const char *)x,
                      token_of_row, offsets, s.E, row_bytes, (char *)x_perm);
    return hipGetLastError();
}

}  // namespace moe
