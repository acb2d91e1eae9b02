// expert_fp8.hip -- expert weights in 8-bit floating point (OCP E4M3) for
// decode batches.
//
// Page "Mixture of experts" (rayaq.ca), Mechanics, "Total versus active
// parameters": decoding at small batch sizes is limited by reading expert
// weights; "Tradeoffs": quantisation helps serving.  The glossary page
// "Mixture of Experts (MoE)" (inferensys.com, inference optimization), in
// its entry on model quantization, describes post-training quantisation of
// a trained model's weights.  Here each weight row i is stored as e4m3
// codes q[i][:] with one fp32 scale s[i]: row i = s[i] * value(q[i][:]).
//
// quantize_e4m3_kernel (post-training quantisation; one wave per row,
//   grid-stride over rows): amax = max |w| over the row (exact), s =
//   amax / 448 in fp32 (1 when that is 0), then each w / s (one fp32
//   division, correctly rounded) clamped to [-448, 448] and converted by
//   v_cvt_pk_fp8_f32, which on gfx950 rounds to the nearest OCP e4m3 value,
//   ties to even.
//
// gemm_fp8w_skinny_kernel (the expert GEMMs of a decode batch, at most 16*MT
//   rows per expert, K a multiple of 128): the weight-streaming kernel of
//   the bf16 path with 1-byte weights.  One block per (expert, 16*NT weight
//   rows; for SwiGLU the same rows of W1 and of W3) of KS waves, each taking
//   a contiguous range of K (partials added in wave order through LDS).  A
//   wave streams its rows in 128-wide chunks, PF chunks in a register ring
//   of 16-byte loads (32 bytes of a row per lane per chunk, half the bytes
//   of bf16, so a wave takes more rows than the bf16 kernel).  Lane
//   l = 16g + n holds k = 32g .. 32g+31 of its row; each 8-code group
//   becomes 8 bf16 (v_cvt_pk_f32_fp8, then the
//   upper halves: every finite e4m3 value is exact in bf16) and meets the
//   matching 8 bf16 of A on v_mfma_f32_16x16x32_bf16.  The accumulator of
//   weight row i is the sum over k of A * value(q), so the epilogue
//   multiplies it by s[i] once (for SwiGLU both a1 and a3 by their rows'
//   scales) before the activation.  Experts with no rows exit at once.
#include "moe_internal.h"

namespace moe {

namespace {

// ---- post-training quantisation ----------------------------------------

template <typename T>
__device__ __forceinline__ float load_w(const T *p, int64_t i);
template <>
__device__ __forceinline__ float load_w<float>(const float *p, int64_t i) {
    return p[i];
}
template <>
__device__ __forceinline__ float load_w<uint16_t>(const uint16_t *p, int64_t i) {
    return bf16_to_f32(p[i]);
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ uint32_t e4m3_pair(float a, float b) {
    a = fminf(fmaxf(a, -448.f), 448.f);
    b = fminf(fmaxf(b, -448.f), 448.f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

template <typename T>
__global__ __launch_bounds__(256) void quantize_e4m3_kernel(const T *__restrict__ W, int64_t rows,
                                                            int64_t cols, uint8_t *__restrict__ q,
                                                            float *__restrict__ scales) {
    const int lane = threadIdx.x & 63;
    for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < rows;
         r += (int64_t)gridDim.x * 4) {
        const T *w = W + r * cols;
        float amax = 0.f;
        for (int64_t j = lane; j < cols; j += 64) amax = fmaxf(amax, fabsf(load_w(w, j)));
        amax = wave_max_f32(amax);
        float s = amax / 448.f;
        if (s == 0.f) s = 1.f;
        if (lane == 0) scales[r] = s;
        uint8_t *qr = q + r * cols;
        if (cols % 4 == 0) {
            // four codes per lane and store
            for (int64_t j = (int64_t)lane * 4; j < cols; j += 256) {
                const uint32_t lo = e4m3_pair(load_w(w, j) / s, load_w(w, j + 1) / s);
                const uint32_t hi = e4m3_pair(load_w(w, j + 2) / s, load_w(w, j + 3) / s);
                *(uint32_t *)(qr + j) = lo | (hi << 16);
            }
        } else {
            for (int64_t j = lane; j < cols; j += 64) qr[j] = (uint8_t)(e4m3_pair(load_w(w, j) / s, 0.f) & 0xffu);
        }
    }
}

// ---- weight streaming with e4m3 weights ---------------------------------

constexpr int F8_KC = 128;

// eight e4m3 codes (two dwords) -> eight bf16, exactly
__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, false);
    const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, true);
    const f32x2_t c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, false);
    const f32x2_t d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, true);
    uint4 o;
    o.x = __builtin_amdgcn_perm(__float_as_uint(a[1]), __float_as_uint(a[0]), 0x07060302u);
    o.y = __builtin_amdgcn_perm(__float_as_uint(b[1]), __float_as_uint(b[0]), 0x07060302u);
    o.z = __builtin_amdgcn_perm(__float_as_uint(c[1]), __float_as_uint(c[0]), 0x07060302u);
    o.w = __builtin_amdgcn_perm(__float_as_uint(d[1]), __float_as_uint(d[0]), 0x07060302u);
    return __builtin_bit_cast(bf16x8_t, o);
}

template <int MT, int NT, int PF, int KS, bool DUAL, int ACT, bool OUT_BF16, bool PACKED>
__global__ __launch_bounds__(64 * KS) void gemm_fp8w_skinny_kernel(
    const uint16_t *__restrict__ A, const int32_t *__restrict__ a_rows,
    const int32_t *__restrict__ offsets, int E, const uint8_t *__restrict__ B1,
    const uint8_t *__restrict__ B3, const float *__restrict__ S1, const float *__restrict__ S3,
    void *__restrict__ C, int N, int K) {
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    static_assert(PF % 2 == 0, "the A double buffer needs an even ring length");
    constexpr int NB = DUAL ? 2 : 1;
    constexpr int NACC = MT * NB * NT * 4;
    __shared__ float red[KS > 1 ? KS - 1 : 1][NACC][64];
    const int ntile = (N + 16 * NT - 1) / (16 * NT);
    const int e = blockIdx.x / ntile;
    const int n0 = (blockIdx.x % ntile) * 16 * NT;
    if (e >= E) return;
    const int lo = offsets[e], M = offsets[e + 1] - lo;
    if (M <= 0) return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int nm = min(MT, (M + 15) / 16);
    const int nch_all = K / F8_KC;
    const int cb = (int)((int64_t)wave * nch_all / KS), ce = (int)((int64_t)(wave + 1) * nch_all / KS);

    const uint16_t *a_row[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int ar = lo + min(m * 16 + n, M - 1);
        a_row[m] = A + (int64_t)(a_rows ? a_rows[ar] : ar) * K + (int64_t)cb * F8_KC + g * 32;
    }
    const uint8_t *b_row[NB][NT];
#pragma unroll
    for (int q = 0; q < NB; ++q)
#pragma unroll
        for (int t = 0; t < NT; ++t)
            b_row[q][t] = PACKED ? ((DUAL && q) ? B3 : B1) + (int64_t)e * N * K +
                                       ((int64_t)min(n0 / 16 + t, N / 16 - 1) * (K / F8_KC) + cb) * 2048 +
                                       lane * 16
                                 : ((DUAL && q) ? B3 : B1) + ((int64_t)e * N + min(n0 + t * 16 + n, N - 1)) * K +
                                       (int64_t)cb * F8_KC + g * 32;

    f32x4_t acc[MT][NB][NT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int q = 0; q < NB; ++q)
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[m][q][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    uint4 rb[PF][NB][NT][2];
    // A1: one buffer for the rows of A, refilled after the chunk's MFMAs, on
    // packed weights with a 2-chunk ring and no K split.  The one-matrix
    // 64-row waves then fit in 256 registers and two share a SIMD, each
    // covering the other's start and epilogue (the Switch layer's up
    // projection 147 -> 133 us with bf16 weights, 145 -> 110 us with e4m3
    // codes); the e4m3 decode up projection, still one wave per SIMD, gains
    // 170 -> 165 us; the rest are unchanged.  Row-major codes take the same
    // 64-row short-K shape (Switch up projection 155 -> 119 us).
    constexpr bool A1 = PF == 2 && KS == 1 && (PACKED || (!DUAL && NT == 4));
    uint4 ra[A1 ? 1 : 2][MT][4];
    const int nch = ce - cb;
    auto load_b = [&](int slot, int ch) {
#pragma unroll
        for (int q = 0; q < NB; ++q)
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    rb[slot][q][t][h] = *(const uint4 *)(b_row[q][t] + (PACKED ? (int64_t)ch * 2048 + h * 1024
                                                                              : (int64_t)ch * F8_KC + h * 16));
    };
    auto load_a = [&](int slot, int ch) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
            if (m < nm)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    ra[slot][m][j] = *(const uint4 *)(a_row[m] + (int64_t)ch * F8_KC + j * 8);
    };
#pragma unroll
    for (int p = 0; p < PF - 1; ++p)
        if (p < nch) load_b(p, p);
    if (nch > 0) load_a(0, 0);
    for (int c0 = 0; c0 < nch; c0 += PF) {
#pragma unroll
        for (int sl = 0; sl < PF; ++sl) {
            const int ch = c0 + sl;
            if (ch < nch) {
                if (ch + PF - 1 < nch) load_b((sl + PF - 1) % PF, ch + PF - 1);
                if (!A1 && ch + 1 < nch) load_a((sl + 1) & 1, ch + 1);
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int q = 0; q < NB; ++q)
#pragma unroll
                        for (int t = 0; t < NT; ++t) {
                            // codes k = 32g + 8j .. +8: dwords 2(j%2), 2(j%2)+1 of load j/2
                            const uint4 &w = rb[sl][q][t][j >> 1];
                            const bf16x8_t b = (j & 1) ? e4m3x8_to_bf16(w.z, w.w) : e4m3x8_to_bf16(w.x, w.y);
#pragma unroll
                            for (int m = 0; m < MT; ++m)
                                if (m < nm)
                                    acc[m][q][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                        __builtin_bit_cast(bf16x8_t, ra[A1 ? 0 : (sl & 1)][m][j]), b,
                                        acc[m][q][t], 0, 0, 0);
                        }
                if (A1 && ch + 1 < nch) load_a(0, ch + 1);
            }
        }
    }
    if (KS > 1) {
        if (wave > 0) {
            int i = 0;
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int q = 0; q < NB; ++q)
#pragma unroll
                    for (int t = 0; t < NT; ++t)
#pragma unroll
                        for (int r = 0; r < 4; ++r) red[wave - 1][i++][lane] = acc[m][q][t][r];
        }
        __syncthreads();
        if (wave > 0) return;
#pragma unroll
        for (int w = 1; w < KS; ++w) {
            int i = 0;
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int q = 0; q < NB; ++q)
#pragma unroll
                    for (int t = 0; t < NT; ++t)
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[m][q][t][r] += red[w - 1][i++][lane];
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int col = n0 + t * 16 + n;
        const int cc = min(col, N - 1);
        const float s1 = S1[(int64_t)e * N + cc];
        const float s3 = DUAL ? S3[(int64_t)e * N + cc] : 1.f;
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m * 16 + 4 * g + r;
                if (row < M && col < N) {
                    const float v = apply_act(ACT, acc[m][0][t][r] * s1, DUAL ? acc[m][NB - 1][t][r] * s3 : 0.f);
                    const int64_t o = (int64_t)(lo + row) * N + col;
                    if (OUT_BF16)
                        ((__bf16 *)C)[o] = (__bf16)v;
                    else
                        ((float *)C)[o] = v;
                }
            }
    }
}

// Shapes per wave: 4 (SwiGLU, W1 and W3) or 8 (one matrix) 16-row tiles of
// weights with a 2-chunk ring: 16 KB of weights in flight per wave at 32
// bytes per lane and chunk, and A (re-read from L2 for every chunk) at half
// the weight bytes.  Measured on the Mixtral decode layer against 1 or 2
// tiles with an 8-chunk ring: up projection 180 against 196 us, down 91
// against 100 us.
template <int MT, int NT, bool DUAL, int ACT, bool OUT_BF16, bool PACKED>
hipError_t launch_fp8(const Shape &s, const void *A, const int32_t *a_rows, const int32_t *offsets,
                      const uint8_t *B1, const uint8_t *B3, const float *S1, const float *S3, void *C,
                      int N, int K, hipStream_t st) {
    constexpr int PF = 2;
    const unsigned blocks = (unsigned)s.E * (unsigned)((N + 16 * NT - 1) / (16 * NT));
    // split K over the waves of a block when there are too few column tiles
    // to keep enough weight bytes in flight and K is long
    if (blocks < 4096 && K / F8_KC >= 64)
        launch_kernel((gemm_fp8w_skinny_kernel<MT, NT, PF, 4, DUAL, ACT, OUT_BF16, PACKED>), dim3(blocks), dim3(256), 0,
                      st, (const uint16_t *)A, a_rows, offsets, s.E, B1, B3, S1, S3, C, N, K);
    else
        launch_kernel((gemm_fp8w_skinny_kernel<MT, NT, PF, 1, DUAL, ACT, OUT_BF16, PACKED>), dim3(blocks), dim3(64), 0,
                      st, (const uint16_t *)A, a_rows, offsets, s.E, B1, B3, S1, S3, C, N, K);
    return hipGetLastError();
}

// 16-row tiles of A per expert (2 or 3), 0 when the shape does not fit
inline int fp8_tiles(const Shape &s) {
    int64_t m = s.T;
    if (s.C >= 0 && s.C < m) m = s.C;
    if (m <= 32) return 2;
    if (m <= 48) return 3;
    return 0;
}

}  // namespace

bool fp8_supported(const Shape &s) {
    return s.dtype == 1 && fp8_tiles(s) != 0 && s.d % F8_KC == 0 && s.d_ff % F8_KC == 0;
}

hipError_t launch_quantize_e4m3(int dtype, const void *W, int64_t rows, int64_t cols, uint8_t *q,
                                float *scales, hipStream_t st) {
    int64_t blocks = (rows + 3) / 4;
    if (blocks > 16384) blocks = 16384;
    if (blocks < 1) blocks = 1;
    if (dtype == 1)
        hipLaunchKernelGGL(quantize_e4m3_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, st,
                           (const uint16_t *)W, rows, cols, q, scales);
    else
        hipLaunchKernelGGL(quantize_e4m3_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, st,
                           (const float *)W, rows, cols, q, scales);
    return hipGetLastError();
}

namespace {

template <bool PACKED>
hipError_t up_fp8(const Shape &s, const void *A, const int32_t *a_rows, const int32_t *offsets, const uint8_t *W1,
                  const uint8_t *W3, const float *S1, const float *S3, void *H, hipStream_t st) {
    const int mt = fp8_tiles(s);
    const int N = s.d_ff, K = s.d;
    if (s.act == ACT_SWIGLU)
        return mt == 2 ? launch_fp8<2, 4, true, ACT_SWIGLU, true, PACKED>(s, A, a_rows, offsets, W1, W3, S1, S3, H, N, K, st)
                       : launch_fp8<3, 4, true, ACT_SWIGLU, true, PACKED>(s, A, a_rows, offsets, W1, W3, S1, S3, H, N, K, st);
    // one matrix with a short K (fewer than 16 chunks: the Switch layer's up
    // projection): 64 rows per wave and one A buffer, two waves per SIMD
    // (packed codes 145 -> 110 us, row-major 155 -> 119 us)
    if (s.act != ACT_SWIGLU && K / F8_KC < 16) {
        if (s.act == ACT_GELU)
            return mt == 2 ? launch_fp8<2, 4, false, ACT_GELU, true, PACKED>(s, A, a_rows, offsets, W1, nullptr, S1, nullptr, H, N, K, st)
                           : launch_fp8<3, 4, false, ACT_GELU, true, PACKED>(s, A, a_rows, offsets, W1, nullptr, S1, nullptr, H, N, K, st);
        return mt == 2 ? launch_fp8<2, 4, false, ACT_RELU, true, PACKED>(s, A, a_rows, offsets, W1, nullptr, S1, nullptr, H, N, K, st)
                       : launch_fp8<3, 4, false, ACT_RELU, true, PACKED>(s, A, a_rows, offsets, W1, nullptr, S1, nullptr, H, N, K, st);
    }
    if (s.act == ACT_GELU)
        return mt == 2 ? launch_fp8<2, 8, false, ACT_GELU, true, PACKED>(s, A, a_rows, offsets, W1, nullptr, S1, nullptr, H, N, K, st)
                       : launch_fp8<3, 8, false, ACT_GELU, true, PACKED>(s, A, a_rows, offsets, W1, nullptr, S1, nullptr, H, N, K, st);
    return mt == 2 ? launch_fp8<2, 8, false, ACT_RELU, true, PACKED>(s, A, a_rows, offsets, W1, nullptr, S1, nullptr, H, N, K, st)
                   : launch_fp8<3, 8, false, ACT_RELU, true, PACKED>(s, A, a_rows, offsets, W1, nullptr, S1, nullptr, H, N, K, st);
}

// The down projection takes 8 16-row weight tiles per wave on row-major
// codes and 4 on packed ones (twice the waves; Mixtral decode layer 94.5
// against 89.9 us: with contiguous loads more waves in flight pay).
template <bool PACKED>
hipError_t down_fp8(const Shape &s, const void *H, const int32_t *offsets, const uint8_t *W2, const float *S2,
                    float *y_perm, hipStream_t st) {
    const int mt = fp8_tiles(s);
    const int N = s.d, K = s.d_ff;
    constexpr int NT = PACKED ? 4 : 8;
    return mt == 2 ? launch_fp8<2, NT, false, ACT_NONE, false, PACKED>(s, H, nullptr, offsets, W2, nullptr, S2, nullptr, y_perm, N, K, st)
                   : launch_fp8<3, NT, false, ACT_NONE, false, PACKED>(s, H, nullptr, offsets, W2, nullptr, S2, nullptr, y_perm, N, K, st);
}

}  // namespace

hipError_t launch_expert_up_fp8(const Shape &s, const void *A, const int32_t *a_rows,
                                const int32_t *offsets, const uint8_t *W1, const uint8_t *W3,
                                const float *S1, const float *S3, void *H, hipStream_t st, bool packed) {
    return packed ? up_fp8<true>(s, A, a_rows, offsets, W1, W3, S1, S3, H, st)
                  : up_fp8<false>(s, A, a_rows, offsets, W1, W3, S1, S3, H, st);
}

hipError_t launch_expert_down_fp8(const Shape &s, const void *H, const int32_t *offsets,
                                  const uint8_t *W2, const float *S2, float *y_perm, hipStream_t st, bool packed) {
    return packed ? down_fp8<true>(s, H, offsets, W2, S2, y_perm, st) : down_fp8<false>(s, H, offsets, W2, S2, y_perm, st);
}

}  // namespace moe
