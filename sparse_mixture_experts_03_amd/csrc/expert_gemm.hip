// expert_gemm.hip -- the expert FFNs as grouped matrix multiplies over the
// ragged per-expert row blocks of the permuted tokens.
//
// Page "Mixture of experts" (rayaq.ca), Implementation: the SwiGLU expert
// w2(silu(w1 x) * w3 x) with bias-free Linears, and the remark that
// production kernels replace the loop over experts by a sort of tokens by
// expert plus a grouped matrix multiply with the same arithmetic.
//
// Layouts (all K-contiguous, so both MFMA operands are read K-major with no
// repacking):  A = x_perm [rows][K=d] or H [rows][K=d_ff];
//              W1, W3 [E][N=d_ff][K=d];  W2 [E][N=d][K=d_ff].
// Expert e owns rows [offsets[e], offsets[e+1]), read on the device.
//
// gemm_bf16_kernel: one 256-thread block per (expert, BM-row tile, BN-col
// tile), scheduled XCD-aware (see find_tile); the block finds its expert
// from offsets (surplus blocks exit at once, and an expert with no rows has
// no tiles, so its weights are never read).
// The K loop stages BM x 64 of A and BN x 64 of each weight matrix through
// LDS (double buffered, rows padded by 16 bytes against bank conflicts,
// the next tile prefetched into registers while the current one feeds the
// MFMAs).  Four waves split the tile 2 x 2 (or 1 x 4); each wave issues
// v_mfma_f32_32x32x16_bf16 with fp32 accumulators.  For SwiGLU the block
// loads the same BN rows of W1 and W3 and keeps both accumulators, so the
// epilogue forms silu(a1) * a3 in registers and writes H once in bf16.
// The down projection writes y_perm in fp32.
//
// MFMA 32x32x16 operand layout (lane l of 64): A supplies row l % 32 and
// the 8 consecutive k at 8 * (l / 32); B supplies column l % 32 and the
// same k; accumulator register r of lane l holds row
// 8 * (r / 4) + 4 * (l / 32) + r % 4, column l % 32.
//
// gemm_f32 kernels: a plain fp32 path (one block per row, one thread per
// output column, sequential fp32 FMA over K) for fp32 layers.
#include <atomic>
#include <type_traits>

#include "moe_internal.h"

namespace moe {

namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Tile schedule.  The work is the set of (expert e, column tile n, row tile
// m) with m < ceil(rows_e / BM), ordered e-major, then n, then m.  The 1-D
// grid is an upper bound; block b is mapped XCD-aware: blocks are
// dispatched round-robin over the 8 XCDs (b % 8), so XCD x is given the
// contiguous run [x * per, (x + 1) * per) of the ordered tiles (per = the
// real tile count / 8, rounded up).  The blocks resident on one XCD at a
// time then cover all row tiles of a few column tiles of one expert: each
// weight panel is fetched into that XCD's L2 once and shared, and every XCD
// gets the same amount of real work.  Surplus blocks return at once.
constexpr int NUM_XCD = 8;

template <int BM>
__device__ __forceinline__ bool find_tile(const int32_t *__restrict__ offsets, int E, int ntiles_n,
                                          int &e, int &row0, int &nrows, int &ntile,
                                          int nsplit = 1, int *split = nullptr) {
    int total = 0;
    for (int i = 0; i < E; ++i) total += (offsets[i + 1] - offsets[i] + BM - 1) / BM;
    total *= ntiles_n;
    const int work = total * nsplit;  // K-split index slowest
    const int per = (work + NUM_XCD - 1) / NUM_XCD;
    const int b = blockIdx.x;
    const int slot = b / NUM_XCD;
    if (slot >= per) return false;
    int L = (b % NUM_XCD) * per + slot;
    if (L >= work) return false;
    if (split) *split = L / total;
    L %= total;
    for (int i = 0; i < E; ++i) {
        const int lo = offsets[i], hi = offsets[i + 1];
        const int mt = (hi - lo + BM - 1) / BM;
        const int cnt = mt * ntiles_n;
        if (L < cnt) {
            e = i;
            ntile = L / mt;
            const int m0 = (L % mt) * BM;
            row0 = lo + m0;
            nrows = min(BM, hi - lo - m0);
            return true;
        }
        L -= cnt;
    }
    return false;
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool DUAL, int ACT, bool OUT_BF16>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(
    const uint16_t *__restrict__ A, const int32_t *__restrict__ a_rows,
    const int32_t *__restrict__ offsets, int E, const uint16_t *__restrict__ B1,
    const uint16_t *__restrict__ B3, void *__restrict__ C, int N, int K) {
    constexpr int BK = 64;
    constexpr int LDK = BK + 8;
    constexpr int NB = DUAL ? 2 : 1;
    constexpr int BROWS = NB * BN;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int CPR = BK / 8;                      // 16-byte chunks per row
    constexpr int A_CH = BM * CPR / 256;             // chunks per thread
    constexpr int B_CH = BROWS * CPR / 256;
    static_assert(WAVES_M * WAVES_N == 4, "four waves");
    static_assert(TM >= 1 && TN >= 1 && WM % 32 == 0 && WN % 32 == 0, "wave tile");
    static_assert(A_CH >= 1 && (BM * CPR) % 256 == 0 && (BROWS * CPR) % 256 == 0, "loads");

    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM][LDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BROWS][LDK];

    int e, row0, nrows, ntile;
    if (!find_tile<BM>(offsets, E, (N + BN - 1) / BN, e, row0, nrows, ntile)) return;
    const int n0 = ntile * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    // global source of each 16-byte chunk this thread stages
    const uint16_t *a_src[A_CH];
    int a_row[A_CH], a_kc[A_CH];
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
        const int c = tid + i * 256;
        a_row[i] = c / CPR;
        a_kc[i] = (c % CPR) * 8;
        const int r = min(a_row[i], nrows - 1);  // rows past the expert's last repeat it
        const int ar = row0 + r;
        a_src[i] = A + (int64_t)(a_rows ? a_rows[ar] : ar) * K + a_kc[i];
    }
    const uint16_t *b_src[B_CH];
    int b_row[B_CH], b_kc[B_CH];
    bool b_ok[B_CH];
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
        const int c = tid + i * 256;
        b_row[i] = c / CPR;
        b_kc[i] = (c % CPR) * 8;
        const int which = b_row[i] / BN;
        const int n = n0 + b_row[i] % BN;
        b_ok[i] = n < N;
        const uint16_t *base = (DUAL && which) ? B3 : B1;
        b_src[i] = base + ((int64_t)e * N + (b_ok[i] ? n : 0)) * K + b_kc[i];
    }

    uint4 ra[A_CH], rb[B_CH];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_CH; ++i)
            ra[i] = (k0 + a_kc[i] < K) ? *(const uint4 *)(a_src[i] + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < B_CH; ++i)
            rb[i] = (b_ok[i] && k0 + b_kc[i] < K) ? *(const uint4 *)(b_src[i] + k0)
                                                  : make_uint4(0, 0, 0, 0);
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_CH; ++i) *(uint4 *)&As[buf][a_row[i]][a_kc[i]] = ra[i];
#pragma unroll
        for (int i = 0; i < B_CH; ++i) *(uint4 *)&Bs[buf][b_row[i]][b_kc[i]] = rb[i];
    };

    f32x16_t acc[NB][TM][TN];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[b][i][j][r] = 0.f;

    const int KT = (K + BK - 1) / BK;
    gload(0);
    lstore(0);
    __syncthreads();
    const int lrow = lane & 31, lk = (lane >> 5) * 8;
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) gload((kt + 1) * BK);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            bf16x8_t af[TM], bfr[NB][TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                af[i] = *(const bf16x8_t *)&As[cur][wm * WM + i * 32 + lrow][kk + lk];
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    bfr[b][j] = *(const bf16x8_t *)&Bs[cur][b * BN + wn * WN + j * 32 + lrow][kk + lk];
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[b][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[b][j],
                                                                              acc[b][i][j], 0, 0, 0);
        }
        if (kt + 1 < KT) lstore(cur ^ 1);
        __syncthreads();
    }

    // epilogue: activation (up) or plain store (down)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = n0 + wn * WN + j * 32 + lrow;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * WM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                if (row < nrows && col < N) {
                    const float a1 = acc[0][i][j][r];
                    const float a3 = DUAL ? acc[NB - 1][i][j][r] : 0.f;
                    const float v = apply_act(ACT, a1, a3);
                    const int64_t o = (int64_t)(row0 + row) * N + col;
                    if (OUT_BF16)
                        ((__bf16 *)C)[o] = (__bf16)v;  // v_cvt_pk_bf16_f32, round to nearest even
                    else
                        ((float *)C)[o] = v;
                }
            }
        }
}

// ---- large row tiles: direct-to-LDS loads, 256 x 256 tiles ----------------
//
// gemm_bf16_big_kernel, for experts with many rows and K a multiple of 64.
// A block computes up to 256 rows x 256 weight rows (SwiGLU: 128 rows of W1
// and the same 128 rows of W3, i.e. 128 columns of H) with four waves in a
// 2 x 2 grid.  An expert's row tiles are 256 rows, except its last, which
// takes only as many 64-row slabs as it needs (MI = 1..4 slabs; each wave
// then holds MI 32-row fragments), so a ragged expert pads at most 63 rows
// instead of up to 255.  Tiles are spread over the XCDs by cost
// (find_tile_balanced).  The plain kernel also has half-width tiles (NJ = 2
// column groups per wave instead of 4) for the last round of a run; the
// SwiGLU kernel is built without them (their code alone slowed its whole
// tiles by ~1%).
// Operands go from global memory straight into LDS with
// buffer_load_dwordx4 ... lds (no register staging): instruction j of a
// wave fills 8 LDS rows, lane l writing the 16 bytes at (row + l/8, slot
// l%8).  Slot s of row r holds k-chunk s ^ f(r), f(r) = (r % 8) ^
// ((r / 8) % 2): an XOR swizzle under which any 8 consecutive rows use 8
// different slots and any 16 consecutive rows use 16 different (row parity,
// slot) pairs, so the rows a fragment read serves together fall on distinct
// banks whether the LDS serves 8 or 16 lanes of a 16-byte read per cycle.
// LDS stages of 32 KB per operand: two for A and three for the weights
// (160 KB, all of a gfx950 CU's LDS).  During stage k the A rows of stage
// k+1 and then the weight rows of stage k+2 are issued (first half of the
// stage, under its MFMAs), so weight loads, the ones that miss L2 first,
// have two stages to land and A loads one; at the start of a stage only the
// newest 8 weight loads may still be in flight (loads return in order).
// Fragments for the next 16-wide k step are read from LDS while the current
// step's MFMAs run.
//
// The stage loop carries no vector address arithmetic: a load's address is
// a per-lane offset fixed for the whole tile plus the stage's k offset in
// a scalar register (buffer addressing), and a fragment read is one of
// eight per-lane LDS offsets (operand x k step) plus an immediate (stage,
// fragment row).  The loop is unrolled by two stages so that the A stage
// is a compile-time constant; the weight stage (k mod 3) is a scalar added
// to the weight operand's per-lane offset.
constexpr int BIG_BM = 256;

// Cost-balanced tile schedule for the 256-row kernel.  The work is the
// ordered list of (K split, expert e, column tile n, row tile m) tiles, m
// fastest.  A tile's cost is counted by its 64-row slabs: 18, 20, 22, 25
// for 1..4 slabs (the loads of a whole weight panel are paid for however
// few rows a tile has; measured: a one-slab tile takes about 0.7-0.8 of a
// full one).  XCD x = b % 8 is given the contiguous run of tiles whose
// starting cost lies in [x C / 8, (x+1) C / 8) of the total cost C, and
// its blocks (slot b / 8) take the run's tiles in order; so every XCD gets
// the same amount of work and the row tiles sharing a weight panel run on
// one XCD at the same time.  When all tiles fit in one round of the CUs
// (at most 8 x CUs-per-XCD of them), the runs split the list by count
// instead, so that no XCD has more tiles than CUs.  In the plain (non-SwiGLU) kernel, the last
// partial round of a run, when it would leave at least half of the XCD's
// CUs idle, is done as half-width pieces (two per tile, 128 columns each).
// Each wave computes the schedule by itself,
// one expert per lane (two for E > 64) with shuffle prefix sums: one read
// of offsets and no loop over the experts.
constexpr int BIG_W_FULL = 25;
__device__ __forceinline__ int big_slab_cost(int rows) {
    const int mi = (rows + 63) >> 6;
    return mi >= 4 ? 25 : 16 + 2 * mi;
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o);
        if (lane >= o) v += u;
    }
    return v;
}

__device__ __forceinline__ bool find_tile_balanced(const int32_t *__restrict__ offsets, int E, int ntn,
                                                   int nsplit, int cpx, bool halves_ok, int slot, int &ntot_out,
                                                   int &e, int &row0, int &nrows, int &ntile, int &split,
                                                   int &half) {
    const int lane = threadIdx.x & 63;
    // experts lane and lane + 64; every value taken out of a lane is read
    // with readlane at a uniform lane, so it lands in a scalar register
    int lo[2], rows[2], mt[2], cpc[2], cumT[2], cumC[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int i = lane + 64 * h;
        lo[h] = 0, rows[h] = 0;
        if (i < E) {
            lo[h] = offsets[i];
            rows[h] = offsets[i + 1] - lo[h];
        }
        const int full = rows[h] >> 8, part = rows[h] & 255;
        mt[h] = full + (part ? 1 : 0);
        cpc[h] = BIG_W_FULL * full + (part ? big_slab_cost(part) : 0);   // cost per column tile
        cumT[h] = wave_incl_scan(mt[h] * ntn, lane);
        cumC[h] = wave_incl_scan(cpc[h] * ntn, lane);
    }
    const int T0 = __builtin_amdgcn_readlane(cumT[0], 63), C0 = __builtin_amdgcn_readlane(cumC[0], 63);
    cumT[1] += T0;
    cumC[1] += C0;
    const int Ts = __builtin_amdgcn_readlane(cumT[1], 63);               // tiles per K split
    const int64_t Cs = (int64_t)__builtin_amdgcn_readlane(cumC[1], 63);  // cost per K split
    const int64_t C = Cs * nsplit;
    // first tile whose starting cost is >= X (X <= C)
    auto first_at = [&](int64_t X) -> int {
        if (Cs == 0) return 0;
        const int sp = (int)(X / Cs);
        if (sp >= nsplit) return Ts * nsplit;
        const int Xr = (int)(X - (int64_t)sp * Cs);
        const unsigned long long m0 = __ballot(cumC[0] > Xr), m1 = __ballot(cumC[1] > Xr);
        if (m0 == 0ull && m1 == 0ull) return (sp + 1) * Ts;
        const int h = m0 ? 0 : 1;
        const int ln = __ffsll((long long)(m0 ? m0 : m1)) - 1;
        const int ce = __builtin_amdgcn_readlane(cumC[h], ln), te = __builtin_amdgcn_readlane(cumT[h], ln);
        const int c_e = __builtin_amdgcn_readlane(cpc[h], ln), mt_e = __builtin_amdgcn_readlane(mt[h], ln);
        const int Xe = Xr - (ce - c_e * ntn);          // cost into expert
        const int te0 = te - mt_e * ntn;               // its first tile
        const int n = Xe / c_e, r = Xe - n * c_e;
        const int m = (r + BIG_W_FULL - 1) / BIG_W_FULL;
        const int idx = m <= mt_e - 1 ? n * mt_e + m : (n + 1) * mt_e;
        return sp * Ts + te0 + idx;
    };
    const int x = blockIdx.x % NUM_XCD;
    const int ntot = Ts * nsplit;
    ntot_out = ntot;
    int start, end;
    if (cpx > 0 && ntot <= NUM_XCD * cpx) {
        // one round: every CU takes at most one tile, so the XCDs split the
        // list by count and the slowest tile sets the time (a split by cost
        // would give the XCDs of cheap tiles more tiles than CUs: a second
        // round there)
        start = ntot * x / NUM_XCD;
        end = ntot * (x + 1) / NUM_XCD;
    } else {
        start = first_at(C * x / NUM_XCD);
        end = x == NUM_XCD - 1 ? ntot : first_at(C * (x + 1) / NUM_XCD);
    }
    // The run's last partial round (r tiles on the XCD's cpx CUs): when it
    // would leave at least half of them idle, its tiles are done as two
    // half-width pieces each (half = 1, 2), so the round ends sooner.
    const int n = end - start, r = cpx > 0 ? n % cpx : 0;
    const bool halves = halves_ok && cpx > 0 && r > 0 && 2 * r <= cpx;
    int L;
    half = 0;
    if (!halves || slot < n - r) {
        L = start + slot;
        if (L >= end) return false;
    } else {
        const int p = slot - (n - r);
        if (p >= 2 * r) return false;
        L = start + (n - r) + (p >> 1);
        half = 1 + (p & 1);
    }
    split = L / Ts;
    const int Lr = L - split * Ts;
    const unsigned long long m0 = __ballot(cumT[0] > Lr), m1 = __ballot(cumT[1] > Lr);
    const int h = m0 ? 0 : 1;
    const int ln = __ffsll((long long)(m0 ? m0 : m1)) - 1;
    e = ln + 64 * h;
    const int te = __builtin_amdgcn_readlane(cumT[h], ln), mt_e = __builtin_amdgcn_readlane(mt[h], ln);
    const int Le = Lr - (te - mt_e * ntn);
    ntile = Le / mt_e;
    const int m = Le - ntile * mt_e;
    row0 = __builtin_amdgcn_readlane(lo[h], ln) + m * BIG_BM;
    nrows = min(BIG_BM, __builtin_amdgcn_readlane(rows[h], ln) - m * BIG_BM);
    return true;
}

template <int MI, int NJ, bool DUAL, int ACT, bool OUT_BF16>
__device__ __forceinline__ void big_tile(char *lds, const uint16_t *__restrict__ A,
                                         const int32_t *__restrict__ a_rows,
                                         const uint16_t *__restrict__ B1,
                                         const uint16_t *__restrict__ B3, void *__restrict__ C, int N,
                                         int K, int e, int row0, int nrows, int n0, int KT, int kbeg) {
    // Device pass only: the host pass needs just the kernels' stubs (and
    // its clang rejects these instantiations from the weight-gradient form).
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int BK = 64;
    static_assert(NJ == 4 || NJ == 2, "whole or half-width tiles");
    constexpr int BN = DUAL ? 32 * NJ : 64 * NJ;   // output columns per block
    constexpr int WCOL = DUAL ? 16 * NJ : 32 * NJ;  // output columns per wave column (wn)
    constexpr int ROWB = BK * 2;           // bytes per LDS row (8 slots of 16 bytes)
    constexpr int OPB = 256 * ROWB;        // bytes per operand per stage
    constexpr int WROWS = MI * 32;         // A rows per wave row (wm)
    constexpr int NQA = 2 * MI;            // A loads per wave per stage (8 rows each)
    constexpr int NQB = 2 * NJ;            // weight loads per wave per stage
    constexpr int NQ = NQA + NQB;
    constexpr int NMF = MI * NJ;           // MFMAs per wave per 16-wide k step
    constexpr int NRD = MI + NJ;           // fragment reads per k step
    // the thread index passed through an empty asm: what is derived from it
    // is computed per tile, not hoisted out of a caller's loop over tiles
    // (where it would stay live across the stage loop and spill)
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    // the wave index as a scalar, so LDS destinations (M0) and operand bases
    // are computed on the scalar unit
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    // LDS A rows MI*16*w + 8j + l/8 and weight rows 64w + 8j + l/8 both have
    // f = (l/8) ^ (j % 2), so lane l of load j fetches k-chunk
    // (l % 8) ^ (l / 8) ^ (j % 2).  Per-lane byte offsets into the operand;
    // they do not change from stage to stage.
    const int sub = lane >> 3;
    uint32_t a_off[NQA], b_off[NQB];
    // buffer resources (dword 3 = 0x00020000: raw 32-bit data, no swizzle,
    // bounds not relied on: every offset is in range by construction).
    // Byte offsets stay below 2^31: A is addressed from the tile's first row
    // (or, for rows read through a_rows, from the first row of A, which
    // then has at most T rows), a weight operand from its expert's first
    // row; the host picks this kernel only where those spans fit.
    const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a_rows ? A : A + (int64_t)row0 * K), 0, 0x7fffffff, 0x00020000);
    __amdgpu_buffer_rsrc_t b_rsrc;
    {
#pragma unroll
        for (int j = 0; j < NQA; ++j) {
            const int kchunk = ((lane & 7) ^ sub ^ (j & 1)) * 8;
            const int r = min(wave * (MI * 16) + j * 8 + sub, nrows - 1);
            a_off[j] = ((uint32_t)(a_rows ? a_rows[row0 + r] : r) * (uint32_t)K + kchunk) * 2u;
        }
        // wave w fills LDS weight rows 16 NJ w .. +16 NJ; SwiGLU: waves 0,1
        // the W1 rows of the tile (BN of them), waves 2,3 the same W3 rows
        const uint16_t *bb = ((DUAL && wave >= 2) ? B3 : B1) + (int64_t)e * N * K;
        b_rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)bb, 0, 0x7fffffff, 0x00020000);
        const int brow0 = DUAL ? ((wave * 16 * NJ) & (BN - 1)) : wave * 16 * NJ;
#pragma unroll
        for (int j = 0; j < NQB; ++j) {
            const int kchunk = ((lane & 7) ^ sub ^ (j & 1)) * 8;
            const int r = brow0 + j * 8 + sub;
            b_off[j] = ((uint32_t)min(n0 + r, N - 1) * (uint32_t)K + kchunk) * 2u;
        }
    }
    // global -> LDS load q (0..NQ-1) of a stage: q < NQA from A, else from
    // the weights
    auto issue_one = [&](int stage, int bst, int ka, int kb, int q) {
        if (q < NQA)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                a_rsrc,
                (__attribute__((address_space(3))) void *)(lds + stage * OPB + (wave * (MI * 16) + q * 8) * ROWB),
                16, a_off[q], ka * 2, 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                b_rsrc,
                (__attribute__((address_space(3))) void *)(lds + (2 + bst) * OPB + (wave * 16 * NJ + (q - NQA) * 8) * ROWB),
                16, b_off[q - NQA], kb * 2, 0, 0);
    };

    f32x16_t acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Fragment rows: A rows wm*WROWS + i*32 + lane%32; weight rows of
    // column group j: wn*WCOL + j*32 (DUAL: j < NJ/2 -> W1 rows wn*WCOL +
    // j*32, j >= NJ/2 -> the same W3 rows, 32*NJ further on).  The swizzle only depends on lane % 32 and the k step,
    // so each (operand, k step) has one per-lane offset and every fragment
    // row, stage and operand is an immediate on top of it.  (The weight
    // operand's 64 KB base is part of the per-lane offset, which is made
    // opaque to the compiler so that it does not move the base into the
    // immediate, where it would not fit in the 16-bit offset field.)
    const int lr = lane & 31;
    uint32_t rd_a[4], rd_b[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const uint32_t slot = (uint32_t)(((kk * 2 + (lane >> 5)) ^ (lr & 7) ^ ((lr >> 3) & 1)) * 16);
        rd_a[kk] = (uint32_t)(wm * WROWS + lr) * ROWB + slot;
        rd_b[kk] = 2u * OPB + (uint32_t)(wn * WCOL + lr) * ROWB + slot;
        asm volatile("" : "+v"(rd_a[kk]), "+v"(rd_b[kk]));
    }
    char *const lds0 = lds;
    // fragment read f (0..NRD-1) of k step kk, in the order the MFMAs
    // consume them: A0, B0, ..., B(NJ-1), A1, ..., A(MI-1)
    auto read_one = [&](auto stage_c, int kk, int f, bf16x8_t (&a)[MI], bf16x8_t (&b)[NJ], uint32_t bso) {
        constexpr int stage = decltype(stage_c)::value;
        if (f == 0 || f > NJ) {
            const int i = f == 0 ? 0 : f - NJ;
            a[i] = *(const bf16x8_t *)(lds0 + rd_a[kk] + (stage * OPB + i * 32 * ROWB));
        } else {
            const int j = f - 1;
            const int jo = DUAL ? ((j / (NJ / 2)) * 32 * NJ + (j % (NJ / 2)) * 32) : j * 32;
            b[j] = *(const bf16x8_t *)(lds0 + (rd_b[kk] + bso) + jo * ROWB);
        }
    };

    // A stage is written as explicit bundles in issue order, each closed by
    // a scheduling barrier: 4 k steps of NMF MFMAs (i-major, so consecutive
    // MFMAs never share an accumulator); during each of steps 0..2 the NRD
    // fragment reads of the next step; during steps 0 and 1 the NQ
    // global->LDS loads (A rows of stage k+1, then weight rows of stage
    // k+2), spread evenly (every second MFMA for a full tile: early enough to
    // land in time, spread out so that their issue does not starve the MFMA
    // pipe).  Near the end the loads re-load the last stage into an idle
    // buffer (nobody reads it), which keeps the loop free of branches and
    // the count of loads in flight fixed.
    bf16x8_t fa[2][MI], fb[2][NJ];
    auto stage_body = [&](auto cur_c, int kt, int bcur) {
        constexpr int cur = decltype(cur_c)::value;
        constexpr std::integral_constant<int, cur ^ 1> nxt_c{};
        const int ka = kbeg + min(kt + 1, KT - 1) * BK;
        const int kb = kbeg + min(kt + 2, KT - 1) * BK;
        const int bnext = bcur == 0 ? 2 : bcur - 1;   // (bcur + 2) % 3
        const uint32_t bso = (uint32_t)bcur * OPB;
        // this wave's loads of the stage have landed (only the NQB weight
        // loads of the stage after next, issued last, may still be in
        // flight); after the barrier, everyone's have
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(NQB) : "memory");
        // step 0's fragments in consumption order (kept by the scheduling
        // barriers), so the first MFMA waits for two reads, not all of them
#pragma unroll
        for (int f = 0; f < NRD; ++f) {
            read_one(cur_c, 0, f, fa[0], fb[0], bso);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
            for (int t = 0; t < NMF; ++t) {
                const int i = t / NJ, j = t % NJ;
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk & 1][i], fb[kk & 1][j],
                                                                    acc[i][j], 0, 0, 0);
                if (kk < 2) {
                    // load q with the MFMA u = min(q * 2 NMF / NQ + 1, 2 NMF - 1)
                    // of steps 0..1 (a full tile: every odd MFMA)
                    const int u = kk * NMF + t;
#pragma unroll
                    for (int q = 0; q < NQ; ++q)
                        if (min((q * 2 * NMF) / NQ + 1, 2 * NMF - 1) == u) issue_one(nxt_c, bnext, ka, kb, q);
                }
                if (kk < 3) {
                    // read f with MFMA min(f, NMF - 1) of the step
#pragma unroll
                    for (int f = 0; f < NRD; ++f)
                        if (min(f, NMF - 1) == t)
                            read_one(cur_c, kk + 1, f, fa[(kk + 1) & 1], fb[(kk + 1) & 1], bso);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    // stage 0 of both operands, then the weights' stage 1
#pragma unroll
    for (int q = 0; q < NQ; ++q) issue_one(0, 0, kbeg, kbeg, q);
#pragma unroll
    for (int q = NQA; q < NQ; ++q) issue_one(0, 1, kbeg, kbeg + min(1, KT - 1) * BK, q);
    int kt = 0, bc = 0;
    for (; kt + 1 < KT; kt += 2) {
        stage_body(std::integral_constant<int, 0>{}, kt, bc);
        bc = bc == 2 ? 0 : bc + 1;
        stage_body(std::integral_constant<int, 1>{}, kt + 1, bc);
        bc = bc == 2 ? 0 : bc + 1;
    }
    if (kt < KT) stage_body(std::integral_constant<int, 0>{}, kt, bc);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    if (nrows == MI * 64 && n0 + BN <= N) {
        // whole tile in range: no per-element bounds checks; buffer stores
        // whose row offset is a scalar (row * N * element size) and whose
        // lane offset (row 4 * (lane / 32) of each 8-row group, column
        // lane % 32) is fixed, with the 32-column group as an immediate
        constexpr int ES = OUT_BF16 ? 2 : 4;
        const __amdgpu_buffer_rsrc_t c_rsrc = __builtin_amdgcn_make_buffer_rsrc(
            (char *)C + (int64_t)row0 * N * ES, 0, 0x7fffffff, 0x00020000);
        const uint32_t vo =
            ((uint32_t)(4 * (lane >> 5)) * (uint32_t)N + (uint32_t)(n0 + wn * WCOL + lr)) * ES;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int jj = 0; jj < (DUAL ? NJ / 2 : NJ); ++jj) {
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const uint32_t so =
                        (uint32_t)(wm * WROWS + i * 32 + (r >> 2) * 8 + (r & 3)) * (uint32_t)(N * ES);
                    const float v = DUAL ? apply_act(ACT, acc[i][jj][r], acc[i][jj + NJ / 2][r])
                                         : apply_act(ACT, acc[i][jj][r], 0.f);
                    if (OUT_BF16)
                        __builtin_amdgcn_raw_buffer_store_b16(
                            __builtin_bit_cast(unsigned short, (__bf16)v), c_rsrc, vo + jj * 32 * ES, so, 0);
                    else
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, v), c_rsrc,
                                                              vo + jj * 32 * ES, so, 0);
                }
            }
        return;
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int jj = 0; jj < (DUAL ? NJ / 2 : NJ); ++jj) {
            // one 32 x 32 tile at a time: keeps the activation's temporaries
            // from piling up across tiles
            __builtin_amdgcn_sched_barrier(0);
            const int col = n0 + wn * WCOL + jj * 32 + lr;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * WROWS + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                if (row < nrows && col < N) {
                    const float v = DUAL ? apply_act(ACT, acc[i][jj][r], acc[i][jj + NJ / 2][r])
                                         : apply_act(ACT, acc[i][jj][r], 0.f);
                    const int64_t o = (int64_t)(row0 + row) * N + col;
                    if (OUT_BF16)
                        ((__bf16 *)C)[o] = (__bf16)v;  // v_cvt_pk_bf16_f32, round to nearest even
                    else
                        ((float *)C)[o] = v;
                }
            }
        }
#endif
}

// One tile (or half-width piece, half = 1, 2) of the 256-row kernel, by its
// number of 64-row slabs.
template <bool DUAL, int ACT, bool OUT_BF16>
__device__ __forceinline__ void big_tile_any(char *lds, const uint16_t *__restrict__ A,
                                             const int32_t *__restrict__ a_rows, const uint16_t *__restrict__ B1,
                                             const uint16_t *__restrict__ B3, void *__restrict__ C, int N, int K,
                                             int e, int row0, int nrows, int ntile, int half, int KT, int kbeg) {
    constexpr int BN = DUAL ? 128 : 256;
    const int mi = (nrows + 63) >> 6;   // 64-row slabs this tile needs
    if constexpr (!DUAL) if (half) {
        // half-width piece: columns [ntile * BN + (half - 1) * BN / 2, + BN / 2)
        const int n0 = ntile * BN + (half - 1) * (BN / 2);
        if (mi == 4)
            big_tile<4, 2, DUAL, ACT, OUT_BF16>(lds, A, a_rows, B1, B3, C, N, K, e, row0, nrows, n0, KT, kbeg);
        else if (mi == 3)
            big_tile<3, 2, DUAL, ACT, OUT_BF16>(lds, A, a_rows, B1, B3, C, N, K, e, row0, nrows, n0, KT, kbeg);
        else if (mi == 2)
            big_tile<2, 2, DUAL, ACT, OUT_BF16>(lds, A, a_rows, B1, B3, C, N, K, e, row0, nrows, n0, KT, kbeg);
        else
            big_tile<1, 2, DUAL, ACT, OUT_BF16>(lds, A, a_rows, B1, B3, C, N, K, e, row0, nrows, n0, KT, kbeg);
        return;
    }
    if (mi == 4)
        big_tile<4, 4, DUAL, ACT, OUT_BF16>(lds, A, a_rows, B1, B3, C, N, K, e, row0, nrows, ntile * BN, KT, kbeg);
    else if (mi == 3)
        big_tile<3, 4, DUAL, ACT, OUT_BF16>(lds, A, a_rows, B1, B3, C, N, K, e, row0, nrows, ntile * BN, KT, kbeg);
    else if (mi == 2)
        big_tile<2, 4, DUAL, ACT, OUT_BF16>(lds, A, a_rows, B1, B3, C, N, K, e, row0, nrows, ntile * BN, KT, kbeg);
    else
        big_tile<1, 4, DUAL, ACT, OUT_BF16>(lds, A, a_rows, B1, B3, C, N, K, e, row0, nrows, ntile * BN, KT, kbeg);
}

// WG: the weight-gradient form (launch_wgrad_big).  C_e = P Q^T for each
// expert e over its k range [offsets[e], offsets[e+1]) (multiples of 64:
// the zero-padded transposed activations), with A = P [E][K], B1 = Q [N][K]
// (K the row stride), E = the rows of each C_e, C_ = C [experts][E][N] fp32.
// Block b is tile (e, m, n), rows m*256.., columns n*256.., in (e, m, n)
// order with n fastest: the hardware's round-robin over the XCDs gives
// each XCD every eighth column tile of the same row tiles.  An expert
// without rows writes zeros.
template <bool DUAL, int ACT, bool OUT_BF16, bool WG = false>
__global__ __launch_bounds__(256) void gemm_bf16_big_kernel(
    const uint16_t *__restrict__ A, const int32_t *__restrict__ a_rows,
    const int32_t *__restrict__ offsets, int E, const uint16_t *__restrict__ B1,
    const uint16_t *__restrict__ B3, void *__restrict__ C_, int N, int K, int nsplit,
    void *__restrict__ C_split, int cpx, unsigned *__restrict__ tctr) {
    constexpr int BN = DUAL ? 128 : 256;
    // A stages 0, 1 at 0 and 32 KB; weight stages 0..2 at 64, 96, 128 KB
    __shared__ __attribute__((aligned(1024))) char lds[5 * 256 * 128];

    int e, row0, nrows, ntile, split = 0, half = 0;
    void *C;
    int KT, kbeg;
    if constexpr (WG) {
        const int M = E;
        const int tm = (M + 255) / 256, tn = (N + 255) / 256;
        const int x = (int)blockIdx.x / (tm * tn);
        const int rem = (int)blockIdx.x - x * tm * tn;
        row0 = (rem / tn) * 256;
        ntile = rem % tn;
        nrows = min(256, M - row0);
        kbeg = offsets[x];
        KT = (offsets[x + 1] - kbeg) / 64;
        C = (float *)C_ + (int64_t)x * M * N;
        e = 0;   // the operands carry no per-expert base
        if (KT == 0) {
            const int n0 = ntile * 256, ncols = min(256, N - n0);
            for (int i = threadIdx.x; i < nrows * 256; i += 256)
                if ((i & 255) < ncols) ((float *)C)[(int64_t)(row0 + (i >> 8)) * N + n0 + (i & 255)] = 0.f;
            return;
        }
    } else {
        // Slot s of XCD x = b % 8 is block b's first tile, s = b / 8.  With
        // tile counters (tctr: one per XCD, zero at launch), the grid holds
        // at most one block per CU and the blocks stay resident: after its
        // first slot a block takes slot P + t, P blocks per XCD, t the
        // ticket it draws from its XCD's counter, asking for it when it
        // starts a tile so that the answer arrives during the tile.  Tiles
        // are thus handed out in list order to the block that frees up, as
        // the hardware hands out blocks, without a block launch per tile or
        // blocks left to launch after the work.  Which block computes a tile
        // does not change its result.  Without counters every block takes
        // its one slot.
        const int x = (int)(blockIdx.x % NUM_XCD), P = (int)(gridDim.x / NUM_XCD);
        int slot = (int)(blockIdx.x / NUM_XCD), ntot = 0;
        while (find_tile_balanced(offsets, E, (N + BN - 1) / BN, nsplit, cpx, !DUAL, slot, ntot, e, row0, nrows,
                                  ntile, split, half)) {
            unsigned next = 0;
            if (tctr && threadIdx.x == 0) next = (unsigned)P + atomicAdd(tctr + x, 1u);
            C = split ? C_split : C_;
            KT = K / 64 / nsplit;   // K split: stages [split * KT, (split + 1) * KT), the second
            kbeg = split * KT * 64;  // half writing its partial sums to C_split
            big_tile_any<DUAL, ACT, OUT_BF16>(lds, A, a_rows, B1, B3, C, N, K, e, row0, nrows, ntile, half, KT,
                                              kbeg);
            if (!tctr) return;
            // the LDS stages are free once every wave is past its last
            // stage: word 0 carries the ticket to the block
            __syncthreads();
            if (threadIdx.x == 0) *(volatile unsigned *)lds = next;
            __syncthreads();
            slot = __builtin_amdgcn_readfirstlane((int)*(volatile unsigned *)lds);   // uniform: a scalar
            __syncthreads();   // read before the next tile's loads overwrite it
        }
        return;
    }
    big_tile_any<DUAL, ACT, OUT_BF16>(lds, A, a_rows, B1, B3, C, N, K, e, row0, nrows, ntile, 0, KT, kbeg);
}

// ---- skinny row groups (decode batches): weight streaming ----------------
//
// gemm_bf16_skinny_kernel, for experts with at most 16*MT rows and K a
// multiple of 128.  One block per (expert, 16*NT weight rows) -- for SwiGLU
// the same rows of W1 and of W3 -- of KS waves, each taking a contiguous
// range of K (their partial sums are added in wave order through LDS at the
// end, so the result does not depend on timing).  A wave streams its rows
// in 128-wide chunks, PF chunks in flight in a register ring (16-byte
// loads), and multiplies them with the expert's rows of A (read from L2
// one chunk ahead; only the 16-row tiles the expert fills) on
// v_mfma_f32_16x16x32_bf16.  Within a chunk, lane l = 16g + n holds the 64
// contiguous bytes k = 32g .. 32g+31 of its row, and MFMA j of the chunk
// takes k = 32g + 8j .. +8 from both operands: the same permutation of k on
// both sides, so every product meets its partner as in the plain order.
// MFMA 16x16x32 accumulator: lane l holds rows 4*(l/16) + r, column l % 16.
// Experts with no rows exit at once.
constexpr int SK_KC = 128;

template <int MT, int NT, int PF, int KS, bool DUAL, int ACT, bool OUT_BF16, bool PACKED>
__global__ __launch_bounds__(64 * KS) void gemm_bf16_skinny_kernel(
    const uint16_t *__restrict__ A, const int32_t *__restrict__ a_rows,
    const int32_t *__restrict__ offsets, int E, const uint16_t *__restrict__ B1,
    const uint16_t *__restrict__ B3, void *__restrict__ C, int N, int K) {
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    // chunk ch sits in B slot ch % PF and A slot ch % 2; the unrolled loop
    // below indexes both by its static position sl, which matches only when
    // PF is even
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
    const int nm = min(MT, (M + 15) / 16);  // 16-row tiles of A in use (wave-uniform)
    // wave `wave` takes the contiguous chunk range [cb, ce) of K
    const int nch_all = K / SK_KC;
    const int cb = (int)((int64_t)wave * nch_all / KS), ce = (int)((int64_t)(wave + 1) * nch_all / KS);

    const uint16_t *a_row[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
    {
        const int ar = lo + min(m * 16 + n, M - 1);
        a_row[m] = A + (int64_t)(a_rows ? a_rows[ar] : ar) * K + (int64_t)cb * SK_KC + g * 32;
    }
    const uint16_t *b_row[NB][NT];
#pragma unroll
    for (int q = 0; q < NB; ++q)
#pragma unroll
        for (int t = 0; t < NT; ++t)
            b_row[q][t] = PACKED ? ((DUAL && q) ? B3 : B1) + (int64_t)e * N * K +
                                       ((int64_t)min(n0 / 16 + t, N / 16 - 1) * (K / SK_KC) + cb) * 2048 +
                                       lane * 8
                                 : ((DUAL && q) ? B3 : B1) +
                                       ((int64_t)e * N + min(n0 + t * 16 + n, N - 1)) * K +
                                       (int64_t)cb * SK_KC + g * 32;

    f32x4_t acc[MT][NB][NT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int q = 0; q < NB; ++q)
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[m][q][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    uint4 rb[PF][NB][NT][4];
    // A1: one buffer for the rows of A, refilled after the chunk's MFMAs, on
    // packed weights with a 2-chunk ring and no K split.  The one-matrix
    // 64-row waves then fit in 256 registers and two share a SIMD, each
    // covering the other's start and epilogue (the Switch layer's up
    // projection 147 -> 133 us with bf16 weights, 145 -> 110 us with e4m3
    // codes); the e4m3 decode up projection, still one wave per SIMD, gains
    // 170 -> 165 us; the rest are unchanged.
    constexpr bool A1 = PACKED && PF == 2 && KS == 1;
    uint4 ra[A1 ? 1 : 2][MT][4];
    const int nch = ce - cb;
    auto load_b = [&](int slot, int ch) {
#pragma unroll
        for (int q = 0; q < NB; ++q)
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    rb[slot][q][t][j] = *(const uint4 *)(b_row[q][t] + (PACKED ? (int64_t)ch * 2048 + j * 512
                                                                              : (int64_t)ch * SK_KC + j * 8));
    };
    auto load_a = [&](int slot, int ch) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
            if (m < nm)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    ra[slot][m][j] = *(const uint4 *)(a_row[m] + (int64_t)ch * SK_KC + j * 8);
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
                            const bf16x8_t b = __builtin_bit_cast(bf16x8_t, rb[sl][q][t][j]);
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
        // waves 1..KS-1 hand their partial sums to wave 0, which adds them
        // in wave order
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
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m * 16 + 4 * g + r;
                if (row < M && col < N) {
                    const float v = apply_act(ACT, acc[m][0][t][r], DUAL ? acc[m][NB - 1][t][r] : 0.f);
                    const int64_t o = (int64_t)(lo + row) * N + col;
                    if (OUT_BF16)
                        ((__bf16 *)C)[o] = (__bf16)v;
                    else
                        ((float *)C)[o] = v;
                }
            }
    }
}

// ---- fp32 path -----------------------------------------------------------

__device__ __forceinline__ int expert_of_row(const int32_t *__restrict__ offsets, int E, int r) {
    int e = 0;
    while (e < E - 1 && r >= offsets[e + 1]) ++e;
    return e;
}

__global__ __launch_bounds__(256) void up_f32_kernel(const float *__restrict__ A,
                                                     const int32_t *__restrict__ a_rows,
                                                     const int32_t *__restrict__ offsets, int E,
                                                     const float *__restrict__ W1,
                                                     const float *__restrict__ W3, int act,
                                                     float *__restrict__ H, int d, int d_ff) {
    const int n = offsets[E];
    for (int r = blockIdx.x; r < n; r += gridDim.x) {
        const int e = expert_of_row(offsets, E, r);
        const float *a = A + (int64_t)(a_rows ? a_rows[r] : r) * d;
        for (int f = threadIdx.x; f < d_ff; f += blockDim.x) {
            const float *w1 = W1 + ((int64_t)e * d_ff + f) * d;
            float a1 = 0.f, a3 = 0.f;
            for (int j = 0; j < d; ++j) a1 = fmaf(a[j], w1[j], a1);
            if (act == ACT_SWIGLU) {
                const float *w3 = W3 + ((int64_t)e * d_ff + f) * d;
                for (int j = 0; j < d; ++j) a3 = fmaf(a[j], w3[j], a3);
            }
            H[(int64_t)r * d_ff + f] = apply_act(act, a1, a3);
        }
    }
}

__global__ __launch_bounds__(256) void down_f32_kernel(const float *__restrict__ H,
                                                       const int32_t *__restrict__ offsets, int E,
                                                       const float *__restrict__ W2,
                                                       float *__restrict__ Y, int d, int d_ff) {
    const int n = offsets[E];
    for (int r = blockIdx.x; r < n; r += gridDim.x) {
        const int e = expert_of_row(offsets, E, r);
        const float *h = H + (int64_t)r * d_ff;
        for (int o = threadIdx.x; o < d; o += blockDim.x) {
            const float *w2 = W2 + ((int64_t)e * d + o) * d_ff;
            float a = 0.f;
            for (int f = 0; f < d_ff; ++f) a = fmaf(h[f], w2[f], a);
            Y[(int64_t)r * d + o] = a;
        }
    }
}

// ---- launch configuration ------------------------------------------------

// Upper bound on row tiles: sum_e ceil(kept_e / BM) <= rows / BM + E.
inline unsigned row_tile_bound(const Shape &s, int BM) {
    int64_t rows = s.Tk();
    if (s.C >= 0 && (int64_t)s.E * s.C < rows) rows = (int64_t)s.E * s.C;
    return (unsigned)((rows + BM - 1) / BM + s.E);
}

// Most rows any one expert can receive: each token picks an expert at most
// once, and a capacity caps it further.
inline int64_t max_rows_per_expert(const Shape &s) {
    int64_t m = s.T;
    if (s.C >= 0 && s.C < m) m = s.C;
    return m;
}

// Whether the 256-row kernel's 32-bit buffer offsets (below 2^31, the
// range its buffer resources cover) reach every operand byte: A from the
// tile's first row (256 rows) or, for rows read through a row map, from
// the first of the T rows of x; a weight matrix [N][K] of one expert from
// its first row (N * K = d * d_ff for every projection); C from the tile's
// first row.  Each A or weight span allows one more row for the stage's k
// offset in the scalar offset.
inline bool big_offsets_fit(const Shape &s, int K, bool gathered) {
    const int64_t lim = int64_t(1) << 31;
    const int64_t arows = gathered ? (int64_t)s.T : (int64_t)BIG_BM;
    const int64_t wide = s.d > s.d_ff ? s.d : s.d_ff;
    return (arows + 1) * K * 2 < lim && ((int64_t)s.d * s.d_ff + wide) * 2 < lim &&
           (int64_t)BIG_BM * wide * 4 < lim;
}

// Row-tile height from the mean rows per expert (the counts themselves
// stay on the device).  gathered: A's rows are read through a row map.
inline int pick_bm(const Shape &s, int K, bool gathered = false) {
    int64_t rows = s.Tk();
    if (s.C >= 0 && (int64_t)s.E * s.C < rows) rows = (int64_t)s.E * s.C;
    const int64_t mean = rows / s.E;
    if (mean >= 192 && K % 64 == 0 && big_offsets_fit(s, K, gathered)) return BIG_BM;
    if (mean >= 96) return 128;
    if (mean >= 24) return 64;
    return 32;
}

template <int BM, int BN, int WM_, int WN_, bool DUAL, int ACT, bool OUT_BF16>
hipError_t launch_gemm(const Shape &s, const void *A, const int32_t *a_rows, const int32_t *offsets, const void *B1,
                       const void *B3, void *C, int N, int K, hipStream_t st) {
    const unsigned nt = (unsigned)((N + BN - 1) / BN);
    unsigned blocks = nt * row_tile_bound(s, BM);
    blocks = (blocks + NUM_XCD - 1) / NUM_XCD * NUM_XCD;
    dim3 grid(blocks);
    launch_kernel((gemm_bf16_kernel<BM, BN, WM_, WN_, DUAL, ACT, OUT_BF16>), grid, dim3(256),
                       0, st, (const uint16_t *)A, a_rows, offsets, s.E, (const uint16_t *)B1,
                       (const uint16_t *)B3, C, N, K);
    return hipGetLastError();
}

// CUs per XCD of the current device (looked up once per device; 32 on
// MI355X if the query fails).
int device_cus_per_xcd() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 32;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        int cus = 0;
        n = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus >= NUM_XCD
                ? cus / NUM_XCD
                : 32;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

template <bool DUAL, int ACT, bool OUT_BF16>
hipError_t launch_big(const Shape &s, const void *A, const int32_t *a_rows, const int32_t *offsets, const void *B1,
                      const void *B3, void *C, int N, int K, hipStream_t st, unsigned *tctr, int nsplit = 1,
                      void *C_split = nullptr) {
    constexpr int BN = DUAL ? 128 : 256;
    const unsigned nt = (unsigned)((N + BN - 1) / BN);
    // tiles <= `bound`; an XCD's run costs at most C / 8 plus one full tile,
    // C <= 25 bound, and a tile costs at least 18: runs of at most
    // (25 bound / 8 + 25) / 18 tiles
    const unsigned bound = nt * row_tile_bound(s, BIG_BM) * (unsigned)nsplit;
    // (plus at most cpx / 2 extra slots for the half-width pieces)
    const int cpx = device_cus_per_xcd();
    const unsigned run = (unsigned)(((uint64_t)25 * bound + 8 * 25) / (8 * 18)) + 1 + (unsigned)(cpx / 2);
    // with tile counters: at most one block per CU, the blocks taking tiles
    // until the list is done
    const unsigned blocks = (tctr && run > (unsigned)cpx ? (unsigned)cpx : run) * NUM_XCD;
    launch_kernel((gemm_bf16_big_kernel<DUAL, ACT, OUT_BF16>), dim3(blocks), dim3(256), 0, st,
                       (const uint16_t *)A, a_rows, offsets, s.E, (const uint16_t *)B1,
                       (const uint16_t *)B3, C, N, K, nsplit, C_split, cpx, tctr);
    return hipGetLastError();
}

template <int MT, int NT, int PF, bool DUAL, int ACT, bool OUT_BF16, bool PACKED>
hipError_t launch_skinny(const Shape &s, const void *A, const int32_t *a_rows, const int32_t *offsets, const void *B1,
                         const void *B3, void *C, int N, int K, hipStream_t st) {
    const unsigned blocks = (unsigned)s.E * (unsigned)((N + 16 * NT - 1) / (16 * NT));
    // split K over the waves of a block when there are too few column tiles
    // to keep enough weight bytes in flight and K is long (each wave keeps
    // >= 16 chunks)
    const int nch = K / SK_KC;
    if (blocks < 4096 && nch >= 64) {
        launch_kernel((gemm_bf16_skinny_kernel<MT, NT, PF, 4, DUAL, ACT, OUT_BF16, PACKED>),
                           dim3(blocks), dim3(256), 0, st, (const uint16_t *)A, a_rows, offsets, s.E,
                           (const uint16_t *)B1, (const uint16_t *)B3, C, N, K);
    } else {
        launch_kernel((gemm_bf16_skinny_kernel<MT, NT, PF, 1, DUAL, ACT, OUT_BF16, PACKED>),
                           dim3(blocks), dim3(64), 0, st, (const uint16_t *)A, a_rows, offsets, s.E,
                           (const uint16_t *)B1, (const uint16_t *)B3, C, N, K);
    }
    return hipGetLastError();
}

// 16-row tiles of A the streaming kernel needs (0: it does not apply).
inline int skinny_tiles(const Shape &s, int K) {
    if (K % SK_KC != 0) return 0;
    const int64_t m = max_rows_per_expert(s);
    if (m <= 32) return 2;
    if (m <= 48) return 3;
    return 0;
}

template <bool DUAL, int ACT, bool OUT_BF16, bool PACKED = false>
hipError_t launch_skinny_any(const Shape &s, int mt, const void *A, const int32_t *a_rows, const int32_t *offsets,
                             const void *B1, const void *B3, void *C, int N, int K,
                             hipStream_t st) {
    // SwiGLU: 16 rows of W1 and of W3 per wave, 4-chunk ring; one matrix: 64
    // rows per wave, 2-chunk ring (the rows of A, re-read from L2 for every
    // chunk, then cost 0.5-0.75 of the weight bytes instead of 1-1.5:
    // Switch layer 0.395 -> 0.382 ms per step; more SwiGLU rows per wave
    // were slower), and 128 rows per wave when K is not split over the
    // waves of a block (one wave per SIMD; Switch layer 0.385 -> 0.351 ms
    // per step, its down projection gaining; the split decode down
    // projection is no faster with them)
    if (!DUAL && !((int64_t)s.E * ((N + 63) / 64) < 4096 && K / SK_KC >= 64)) {
        // on packed weights with a short K (fewer than 16 chunks: the Switch
        // layer's up projection) 64 rows per wave with a 2-chunk ring and one
        // A buffer, two waves per SIMD (up projection 150 -> 133 us; its down
        // projection, 24 chunks, keeps 128 rows: 126 against 141 us with 64)
        if (PACKED && K / SK_KC < 16) {
            if (mt == 2) return launch_skinny<2, 4, 2, DUAL, ACT, OUT_BF16, PACKED>(s, A, a_rows, offsets, B1, B3, C, N, K, st);
            return launch_skinny<3, 4, 2, DUAL, ACT, OUT_BF16, PACKED>(s, A, a_rows, offsets, B1, B3, C, N, K, st);
        }
        if (mt == 2) return launch_skinny<2, 8, 2, DUAL, ACT, OUT_BF16, PACKED>(s, A, a_rows, offsets, B1, B3, C, N, K, st);
        return launch_skinny<3, 8, 2, DUAL, ACT, OUT_BF16, PACKED>(s, A, a_rows, offsets, B1, B3, C, N, K, st);
    }
    // (on packed weights a one-matrix product with two A tiles takes 32
    // weight rows per wave instead of 64: Mixtral decode down projection 162
    // against 159 us)
    if (mt == 2)
        return launch_skinny<2, DUAL ? 1 : (PACKED ? 2 : 4), DUAL ? 4 : 2, DUAL, ACT, OUT_BF16, PACKED>(
            s, A, a_rows, offsets, B1, B3, C, N, K, st);
    return launch_skinny<3, DUAL ? 1 : 4, DUAL ? 4 : 2, DUAL, ACT, OUT_BF16, PACKED>(s, A, a_rows, offsets, B1, B3, C,
                                                                                   N, K, st);
}

template <int ACT, bool DUAL>
hipError_t launch_up_bf16(const Shape &s, const void *A, const int32_t *a_rows, const int32_t *offsets, const void *W1,
                          const void *W3, void *H, hipStream_t st, unsigned *tctr) {
    if (const int mt = skinny_tiles(s, s.d))
        return launch_skinny_any<DUAL, ACT, true>(s, mt, A, a_rows, offsets, W1, W3, H, s.d_ff, s.d, st);
    switch (pick_bm(s, s.d, a_rows != nullptr)) {
    case BIG_BM: return launch_big<DUAL, ACT, true>(s, A, a_rows, offsets, W1, W3, H, s.d_ff, s.d, st, tctr);
    case 128: return launch_gemm<128, 128, 2, 2, DUAL, ACT, true>(s, A, a_rows, offsets, W1, W3, H, s.d_ff, s.d, st);
    case 64:  return launch_gemm<64, 128, 2, 2, DUAL, ACT, true>(s, A, a_rows, offsets, W1, W3, H, s.d_ff, s.d, st);
    default:  return launch_gemm<32, 128, 1, 4, DUAL, ACT, true>(s, A, a_rows, offsets, W1, W3, H, s.d_ff, s.d, st);
    }
}

}  // namespace

hipError_t launch_expert_up(const Shape &s, const void *x_perm, const int32_t *a_rows,
                            const int32_t *offsets, const void *W1, const void *W3, void *H,
                            hipStream_t st, unsigned *tctr) {
    if (s.dtype == 0) {
        int64_t blocks = s.Tk() < 16384 ? s.Tk() : 16384;
        launch_kernel(up_f32_kernel, dim3((unsigned)(blocks > 0 ? blocks : 1)), dim3(256), 0,
                           st, (const float *)x_perm, a_rows, offsets, s.E, (const float *)W1,
                           (const float *)W3, s.act, (float *)H, s.d, s.d_ff);
        return hipGetLastError();
    }
    switch (s.act) {
    case ACT_SWIGLU: return launch_up_bf16<ACT_SWIGLU, true>(s, x_perm, a_rows, offsets, W1, W3, H, st, tctr);
    case ACT_GELU:   return launch_up_bf16<ACT_GELU, false>(s, x_perm, a_rows, offsets, W1, nullptr, H, st, tctr);
    default:         return launch_up_bf16<ACT_RELU, false>(s, x_perm, a_rows, offsets, W1, nullptr, H, st, tctr);
    }
}

int down_ksplit(const Shape &s) {
    if (s.dtype == 0 || skinny_tiles(s, s.d_ff) != 0 || pick_bm(s, s.d_ff) != BIG_BM) return 1;
    if (s.d_ff < 4096 || (s.d_ff / 64) % 2 != 0) return 1;
    // expected 256 x 256 output tiles: full row tiles plus about half a
    // partial one per expert; split K in two when they would fill fewer than
    // three rounds of the 256 CUs (one block per CU)
    const int64_t tiles =
        (int64_t)((s.d + 255) / 256) * ((int64_t)row_tile_bound(s, BIG_BM) - s.E + s.E / 2);
    return tiles < 3 * 256 ? 2 : 1;
}

hipError_t launch_expert_down(const Shape &s, const void *H, const int32_t *offsets,
                              const void *W2, float *y_perm, float *y_perm_part2,
                              hipStream_t st, unsigned *tctr) {
    if (s.dtype == 0) {
        int64_t blocks = s.Tk() < 16384 ? s.Tk() : 16384;
        launch_kernel(down_f32_kernel, dim3((unsigned)(blocks > 0 ? blocks : 1)), dim3(256), 0,
                           st, (const float *)H, offsets, s.E, (const float *)W2, y_perm, s.d,
                           s.d_ff);
        return hipGetLastError();
    }
    if (const int mt = skinny_tiles(s, s.d_ff))
        return launch_skinny_any<false, ACT_NONE, false>(s, mt, H, nullptr, offsets, W2, nullptr, y_perm, s.d,
                                                          s.d_ff, st);
    switch (pick_bm(s, s.d_ff)) {
    case BIG_BM:
        if (down_ksplit(s) == 2) {
            if (y_perm_part2 == nullptr) return hipErrorInvalidValue;
            return launch_big<false, ACT_NONE, false>(s, H, nullptr, offsets, W2, nullptr, y_perm, s.d,
                                                       s.d_ff, st, tctr, 2, y_perm_part2);
        }
        return launch_big<false, ACT_NONE, false>(s, H, nullptr, offsets, W2, nullptr, y_perm, s.d, s.d_ff, st,
                                                   tctr);
    case 128: return launch_gemm<128, 128, 2, 2, false, ACT_NONE, false>(s, H, nullptr, offsets, W2, nullptr, y_perm, s.d, s.d_ff, st);
    case 64:  return launch_gemm<64, 128, 2, 2, false, ACT_NONE, false>(s, H, nullptr, offsets, W2, nullptr, y_perm, s.d, s.d_ff, st);
    default:  return launch_gemm<32, 128, 1, 4, false, ACT_NONE, false>(s, H, nullptr, offsets, W2, nullptr, y_perm, s.d, s.d_ff, st);
    }
}

// Expert GEMMs of decode-sized batches on weights in the streaming tile
// layout (pack_stream_kernel): the streaming kernel reads each 16-byte
// unit of a chunk from where its lane needs it, so every load instruction
// of a wave covers 1 KB of contiguous memory.  Same products in the same
// order as on row-major weights, hence the same bits.
hipError_t launch_expert_up_packed(const Shape &s, const void *x, const int32_t *a_rows, const int32_t *offsets,
                                   const void *W1, const void *W3, void *H, hipStream_t st) {
    const int mt = skinny_tiles(s, s.d);
    if (mt == 0 || s.dtype != 1) return hipErrorInvalidValue;
    switch (s.act) {
    case ACT_SWIGLU:
        return launch_skinny_any<true, ACT_SWIGLU, true, true>(s, mt, x, a_rows, offsets, W1, W3, H, s.d_ff, s.d, st);
    case ACT_GELU:
        return launch_skinny_any<false, ACT_GELU, true, true>(s, mt, x, a_rows, offsets, W1, nullptr, H, s.d_ff, s.d,
                                                              st);
    default:
        return launch_skinny_any<false, ACT_RELU, true, true>(s, mt, x, a_rows, offsets, W1, nullptr, H, s.d_ff, s.d,
                                                              st);
    }
}

hipError_t launch_expert_down_packed(const Shape &s, const void *H, const int32_t *offsets, const void *W2,
                                     float *y_perm, hipStream_t st) {
    const int mt = skinny_tiles(s, s.d_ff);
    if (mt == 0 || s.dtype != 1) return hipErrorInvalidValue;
    return launch_skinny_any<false, ACT_NONE, false, true>(s, mt, H, nullptr, offsets, W2, nullptr, y_perm, s.d,
                                                           s.d_ff, st);
}

namespace {

// The streaming tile layout of a [rows][cols] matrix of esz-byte elements
// (esz = 2: bf16, 1: e4m3 codes; rows % 16 == 0, cols % 128 == 0), in
// units of 16 bytes (8 / esz ... 16 / esz elements): blocks of 16 rows x
// 128 columns, block (rb, cb) at index rb * (cols / 128) + cb, each of
// 128 * esz units.  In row n of a block, unit u covers columns
// u * 16 / esz .. +16 / esz; with V = 2 * esz units per 32 columns, unit
// u = V g + r (g = 0..3) is stored at unit position r * 64 + 16 g + n.
// That is the streaming kernels' lane order: lane l = 16 g + n holds row n
// and the columns 32 g .. 32 g + 31 of a 128-column chunk, loading unit
// r of them in its r-th load, so load r of a wave reads positions
// r * 64 .. r * 64 + 63 of the block.  One thread per output unit.
__global__ __launch_bounds__(256) void pack_stream_kernel(const uint4 *__restrict__ W, int64_t rows,
                                                          int64_t cols, int esz, uint4 *__restrict__ out) {
    const int64_t upr = cols * esz / 16;     // units per row
    const int64_t nbc = cols / 128;          // blocks across a row
    const int ub = 128 * esz;                // units per block
    const int V = 2 * esz;
    const int64_t total = rows * upr;
    for (int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x; o < total; o += (int64_t)gridDim.x * 256) {
        const int64_t b = o / ub;
        const int p = (int)(o - b * ub);
        const int r = p >> 6, g = (p >> 4) & 3, n = p & 15;
        const int64_t rb = b / nbc, cb = b - rb * nbc;
        const int64_t i = rb * 16 + n;
        out[o] = W[i * upr + cb * (8 * esz) + V * g + r];
    }
}

}  // namespace

hipError_t launch_pack_stream(int esz, const void *W, int64_t rows, int64_t cols, void *out, hipStream_t st) {
    const int64_t units = rows * cols * esz / 16;
    int64_t blocks = (units + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) return hipSuccess;
    launch_kernel(pack_stream_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const uint4 *)W, rows, cols, esz,
                  (uint4 *)out);
    return hipGetLastError();
}

namespace {

// y_perm[r] += part2[r] for the kept rows (the second K half of a split down
// projection): the same fp32 addition, in the same order, as the combine's
// when it reads both halves.
__global__ __launch_bounds__(256) void add_partial_kernel(float *__restrict__ y,
                                                          const float *__restrict__ p2,
                                                          const int32_t *__restrict__ offsets,
                                                          int E, int d) {
    const int64_t n = (int64_t)offsets[E] * d / 4;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        float4 a = ((float4 *)y)[i];
        const float4 b = ((const float4 *)p2)[i];
        a.x += b.x;
        a.y += b.y;
        a.z += b.z;
        a.w += b.w;
        ((float4 *)y)[i] = a;
    }
}

}  // namespace

hipError_t launch_add_partial(const Shape &s, float *y_perm, const float *part2,
                              const int32_t *offsets, hipStream_t st) {
    int64_t blocks = ((int64_t)(row_tile_bound(s, 1) - s.E) * s.d / 4 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(add_partial_kernel, dim3((unsigned)blocks), dim3(256), 0, st, y_perm, part2,
                       offsets, s.E, s.d);
    return hipGetLastError();
}

bool wgrad_big_fits(int M, int N, int64_t ldk) {
    // 32-bit buffer offsets (row * ldk + k) * 2 for both operands
    const int64_t mx = (int64_t)(M > N ? M : N) * ldk * 2;
    return M % 8 == 0 && N % 8 == 0 && ldk % 64 == 0 && mx < ((int64_t)1 << 31);
}

hipError_t launch_wgrad_big(int E, int M, int N, const int32_t *koff, const void *P, const void *Q,
                            int64_t ldk, float *C, hipStream_t st) {
    if (!wgrad_big_fits(M, N, ldk)) return hipErrorInvalidValue;
    const int64_t blocks = (int64_t)E * ((M + 255) / 256) * ((N + 255) / 256);
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    launch_kernel((gemm_bf16_big_kernel<false, ACT_NONE, false, true>), dim3((unsigned)blocks), dim3(256), 0, st,
                  (const uint16_t *)P, nullptr, koff, M, (const uint16_t *)Q, nullptr, (void *)C, N, (int)ldk, 1,
                  nullptr, 0, nullptr);
    return hipGetLastError();
}


}  // namespace moe
