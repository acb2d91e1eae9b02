// shared.hip -- operands of the shared experts.
//
// Page "Mixture of experts" (rayaq.ca), Mechanics, "Total versus active
// parameters": DeepSeek-V3's layer has, beside many small routed experts,
// shared experts that every token visits.  No routing decision touches
// them, so all S of them form one dense layer on all T tokens:
//   up:   H_sh[t][j*d_ff + f] = act(x_t . W1s[j][f]) [* (x_t . W3s[j][f])]
//         -- one row group against W1s/W3s read as [S*d_ff][d], their own
//         layout;
//   down: y_sh[t][o] = sum over j, f of H_sh[t][j*d_ff + f] * W2s[j][o][f]
//         -- one GEMM with K = S*d_ff against W2 laid out [d][S*d_ff].
// shared_prep_kernel writes the row offsets {0, T} of the single row group
// and, for S > 1, that W2 layout (W2cat[o][j*d_ff + f] = W2s[j][o][f]): one
// wave per (j, o) row, 16-byte copies when a row allows them.
#include "moe_internal.h"

namespace moe {

namespace {

template <typename V>
__global__ __launch_bounds__(256) void shared_prep_kernel(const char *__restrict__ W2s,
                                                          char *__restrict__ W2cat, int S, int d,
                                                          int64_t row_bytes, int T,
                                                          int32_t *__restrict__ offsets) {
    if (blockIdx.x == 0 && threadIdx.x < 2) offsets[threadIdx.x] = threadIdx.x == 0 ? 0 : T;
    if (W2cat == nullptr) return;
    const int lane = threadIdx.x & 63;
    const int64_t nrows = (int64_t)S * d;
    const int64_t nv = row_bytes / (int64_t)sizeof(V);
    for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < nrows;
         r += (int64_t)gridDim.x * 4) {
        const int64_t j = r / d, o = r - j * d;
        const V *src = (const V *)(W2s + r * row_bytes);                       // W2s[j][o][:]
        V *dst = (V *)(W2cat + (o * S + j) * row_bytes);                       // W2cat[o][j*d_ff:]
        for (int64_t i = lane; i < nv; i += 64) dst[i] = src[i];
    }
}

}  // namespace

size_t shared_w2cat_bytes(const Shape &s, int S) {
    if (S <= 1) return 0;
    return (size_t)S * (size_t)s.d * (size_t)s.d_ff * (s.dtype == 1 ? 2 : 4);
}

hipError_t launch_shared_prep(const Shape &s, int S, const void *W2s, void *W2cat,
                              int32_t *offsets, hipStream_t st) {
    const int64_t row_bytes = (int64_t)s.d_ff * (s.dtype == 1 ? 2 : 4);
    const bool repack = S > 1;
    int64_t blocks = repack ? ((int64_t)S * s.d + 3) / 4 : 1;
    if (blocks > 8192) blocks = 8192;
    char *dst = repack ? (char *)W2cat : nullptr;
    if (row_bytes % 16 == 0)
        hipLaunchKernelGGL(shared_prep_kernel<uint4>, dim3((unsigned)blocks), dim3(256), 0, st,
                           (const char *)W2s, dst, S, s.d, row_bytes, s.T, offsets);
    else
        hipLaunchKernelGGL(shared_prep_kernel<uint32_t>, dim3((unsigned)blocks), dim3(256), 0, st,
                           (const char *)W2s, dst, S, s.d, row_bytes, s.T, offsets);
    return hipGetLastError();
}

}  // namespace moe
