// route_stats.h -- the load-balancing statistics' final reduction, shared
// by the statistics kernel (moe_route) and the dispatch launch of
// moe_forward, which runs it in extra blocks beside the ranking.
//
// Page "Mixture of experts" (rayaq.ca), Mechanics, "The load-balancing
// loss": f_i = share of tokens whose top choice is i, P_i = mean router
// probability of i, aux = E sum_i f_i P_i, and the z statistic mean_t
// (log sum exp h_t)^2.
//
// Inputs are the route kernels' per-block partials: part_P[e * nblk + b]
// (sum of p_e over block b's tokens), part_P[(E + e) * nblk + b] (how many
// of them chose e first, an exact integer in a float), part_lse2[b].
// route_stats_block(e) for e < E reduces expert e's partials in double
// (thread t takes blocks t, t + 256, ...; the 256 thread sums are then
// added in a fixed tree order) and writes f_e and P_e; e == E reduces the
// lse^2 partials.  The last of the E + 1 blocks to finish (an integer
// arrival counter, zeroed by the route kernel before) adds the f_e P_e in
// expert order for aux, writes aux and z, and re-zeroes the counter.
// The f_e P_e values (and z) pass between blocks through agent-scope
// atomic stores and loads, which are coherent across the XCDs' L2 caches
// without writing them back or invalidating them (a fence per block did
// both, and held up the loads of every kernel block beside them); each
// block waits for its store to complete before it counts its arrival.
// Every thread of the block must call it.
#pragma once

#include "moe_internal.h"

namespace moe {

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

__device__ __forceinline__ void route_stats_block(int e, const float *__restrict__ part_P,
                                                  const float *__restrict__ part_lse2, int T, int E, int nblk,
                                                  float *__restrict__ stats, double *__restrict__ fP,
                                                  unsigned *__restrict__ arrivals) {
    __shared__ double red[256 + 16];
    __shared__ int cnt[4];
    __shared__ int last;
    const int tid = threadIdx.x;
    if (e == E) {
        double z = 0.0;
        for (int b = tid; b < nblk; b += 256) z += (double)part_lse2[b];
        z = block_sum_fixed(z, red);
        if (tid == 0) __hip_atomic_store(fP + E, z / (double)T, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
            __hip_atomic_store(fP + e, f * P, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (tid == 0) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the store above has completed
        last = __hip_atomic_fetch_add(arrivals, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)E;
    }
    __syncthreads();
    if (last) {
        // every block's f_e P_e (and z) has been stored: all threads load
        // them at once, thread 0 adds them in expert order
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

}  // namespace moe
