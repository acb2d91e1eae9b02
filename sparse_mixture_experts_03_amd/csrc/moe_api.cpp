// moe_api.cpp -- the C ABI declared in include/moe.h.
//
// Validates every argument before enqueuing anything, carves the caller's
// workspace, and enqueues the kernel stages on the caller's stream.  Holds
// no state between calls, allocates nothing and never synchronises.
#include "moe.h"

#include <cmath>
#include <cstdint>

#include "moe_internal.h"

namespace {

using moe::Shape;

constexpr size_t kAlign = 256;

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Validates a description and fills the derived shape.
int check_desc(const moe_desc *desc, Shape *s) {
    if (!desc) return MOE_ERR_INVALID_ARG;
    const moe_desc &d = *desc;
    if (d.T < 1 || d.d < 1 || d.d_ff < 1 || d.E < 1 || d.k < 1 || d.k > d.E)
        return MOE_ERR_INVALID_ARG;
    if (d.gate != MOE_GATE_RENORM && d.gate != MOE_GATE_SWITCH) return MOE_ERR_INVALID_ARG;
    if (d.act != MOE_ACT_RELU && d.act != MOE_ACT_GELU && d.act != MOE_ACT_SWIGLU)
        return MOE_ERR_INVALID_ARG;
    if (d.dtype != MOE_DTYPE_F32 && d.dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
    if (!std::isfinite(d.capacity_factor) || d.capacity_factor < 0.0) return MOE_ERR_INVALID_ARG;
    if (d.stage_events == nullptr && d.n_stage_events != 0) return MOE_ERR_INVALID_ARG;
    if (d.n_stage_events < 0) return MOE_ERR_INVALID_ARG;
    if (d.E > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
    if (d.dtype == MOE_DTYPE_BF16 && (d.d % 8 != 0 || d.d_ff % 8 != 0)) return MOE_ERR_UNSUPPORTED;
    // permuted row indices are int32
    if ((int64_t)d.T * d.k >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    s->T = d.T;
    s->d = d.d;
    s->d_ff = d.d_ff;
    s->E = d.E;
    s->k = d.k;
    s->gate = d.gate;
    s->act = d.act;
    s->dtype = d.dtype;
    if (d.capacity_factor > 0.0)
        s->C = (int64_t)std::ceil(d.capacity_factor * (double)d.T * (double)d.k / (double)d.E);
    else
        s->C = -1;
    return MOE_OK;
}

// Workspace layout; every region starts on a 256-byte boundary.
struct Layout {
    size_t part_P, part_lse2, fP, arrivals;         // router partials, f_e*P_e and z, counter
    size_t part_logits;                             // bf16 router: logit slices
    size_t wsplit;                                  // bf16 router GEMM: split W_r (0: none)
    size_t chunk_counts;                            // dispatch: per-chunk expert histograms
    size_t topk_idx, gates, routed, kept, offsets;  // moe_forward's optional outputs
    size_t row_of_slot, token_of_row, dropped, stats;
    size_t x_perm, H, y_perm;
    size_t y_perm2;  // second K half of a split down projection (0: no split)
    size_t tile_ctr; // the 256-row GEMMs' tile counters: routed up, down, shared up, down
    // shared experts (all 0 when there are none)
    size_t sh_offsets;  // {0, T}: their single row group
    size_t w2cat;       // W2 of S > 1 experts as [d][S*d_ff] (0: S <= 1)
    size_t H_sh, y_sh;  // H_sh [T][S*d_ff] act dtype; y_sh [T][d] fp32 (summed over experts)
    size_t y_sh2;       // second K half of their down projection (0: no split)
    size_t total;
};

Layout layout(const Shape &s, int S = 0) {
    Layout L{};
    const size_t elem = s.dtype == MOE_DTYPE_BF16 ? 2 : 4;
    const size_t Tk = (size_t)s.Tk();
    size_t rows = Tk;
    if (s.C >= 0 && (size_t)s.E * (size_t)s.C < rows) rows = (size_t)s.E * (size_t)s.C;
    const size_t nblk = (size_t)moe::route_blocks(s);
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align_up(o + bytes);
        return at;
    };
    L.part_P = take(2 * nblk * s.E * sizeof(float));  // p sums, top-choice counts
    L.part_lse2 = take(nblk * sizeof(float));
    L.fP = take(((size_t)s.E + 1) * sizeof(double));
    L.arrivals = take(sizeof(unsigned));
    L.tile_ctr = take(4 * moe::TILE_CTR_WORDS * sizeof(unsigned));
    if (s.dtype == MOE_DTYPE_BF16) {
        L.part_logits = take(moe::route_part_floats(s) * 4);
        L.wsplit = moe::route_fused(s) ? take(moe::route_wsplit_bytes(s)) : 0;
    }
    L.chunk_counts = take((size_t)moe::dispatch_chunks(s) * (size_t)s.E * 4);
    L.topk_idx = take(Tk * 4);
    L.gates = take(Tk * 4);
    L.routed = take((size_t)s.E * 4);
    L.kept = take((size_t)s.E * 4);
    L.offsets = take(((size_t)s.E + 1) * 4);
    L.row_of_slot = take(Tk * 4);
    L.token_of_row = take(Tk * 4);
    L.dropped = take(Tk);
    L.stats = take((2 * (size_t)s.E + 2) * 4);
    L.x_perm = take(rows * (size_t)s.d * elem);
    L.H = take(rows * (size_t)s.d_ff * elem);
    L.y_perm = take(rows * (size_t)s.d * 4);
    L.y_perm2 = moe::down_ksplit(s) == 2 ? take(rows * (size_t)s.d * 4) : 0;
    if (S > 0) {
        const Shape q = moe::shared_shape(s, S);
        const size_t T = (size_t)s.T;
        L.sh_offsets = take(2 * 4);
        L.w2cat = S > 1 ? take(moe::shared_w2cat_bytes(s, S)) : 0;
        L.H_sh = take(T * (size_t)q.d_ff * elem);
        L.y_sh = take(T * (size_t)s.d * 4);
        L.y_sh2 = moe::down_ksplit(q) == 2 ? take(T * (size_t)s.d * 4) : 0;
    }
    L.total = o;
    return L;
}

template <typename T>
T *at(void *ws, size_t off) {
    return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

int check_ws(const Shape &s, const void *ws, size_t ws_bytes, int S = 0) {
    if (!ws) return MOE_ERR_INVALID_ARG;
    if (ws_bytes < layout(s, S).total) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

// Validates the shared-expert description against the layer's: S in range,
// weights present when S > 0 (W3 exactly for SwiGLU), and the stacked
// hidden width S*d_ff within int32.
int check_shared(const Shape &s, const moe_shared *sh) {
    if (!sh) return MOE_ERR_INVALID_ARG;
    const int S = sh->n_shared;
    if (S < 0 || S > MOE_MAX_SHARED) return MOE_ERR_INVALID_ARG;
    if (S > 0) {
        if (!sh->W1 || !sh->W2) return MOE_ERR_INVALID_ARG;
        if ((s.act == MOE_ACT_SWIGLU) != (sh->W3 != nullptr)) return MOE_ERR_INVALID_ARG;
        if ((int64_t)S * s.d_ff >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    }
    return MOE_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY(expr)                            \
    do {                                         \
        int rc_ = hip_status(expr);              \
        if (rc_ != MOE_OK) return rc_;           \
    } while (0)

// The shared experts on every token as one dense layer through the routed
// experts' GEMM kernels (one row group of T rows): up against the S
// experts' stacked W1/W3 into H_sh [T][S*d_ff], then down with K = S*d_ff
// into y_sh, the experts' summed output (and y_sh2, the second K half, when
// the down projection splits K).
int run_shared_ffn(const Shape &s, const moe_shared *sh, const void *x, float *y_sh, float *y_sh2,
                   void *ws, const Layout &L, hipStream_t st, unsigned *tctr) {
    const int S = sh->n_shared;
    const Shape q = moe::shared_shape(s, S);
    int32_t *offs = at<int32_t>(ws, L.sh_offsets);
    void *w2cat = L.w2cat ? at<char>(ws, L.w2cat) : nullptr;
    void *H = at<char>(ws, L.H_sh);
    MOE_TRY(moe::launch_shared_prep(s, S, sh->W2, w2cat, offs, st));
    MOE_TRY(moe::launch_expert_up(q, x, nullptr, offs, sh->W1, sh->W3, H, st, tctr));
    MOE_TRY(moe::launch_expert_down(q, H, offs, w2cat ? w2cat : sh->W2, y_sh, y_sh2, st,
                                    tctr ? tctr + moe::TILE_CTR_WORDS : nullptr));
    return MOE_OK;
}

}  // namespace

namespace moe {
LaunchEvents &next_launch_events() {
    static thread_local LaunchEvents le{nullptr, nullptr};
    return le;
}
}  // namespace moe

namespace {

struct StageEvents {
    void *const *ev;
    int n;
    int next = 0;
    hipError_t record(hipStream_t st) {
        hipError_t e = hipSuccess;
        if (ev && next < n && ev[next]) e = hipEventRecord((hipEvent_t)ev[next], st);
        ++next;
        return e;
    }
    hipEvent_t at(int j) const { return (ev && j < n) ? (hipEvent_t)ev[j] : nullptr; }
    // the next stage is one kernel: hand its two boundary events to that
    // launch (start and stop timestamps) instead of recording them around it
    void around_next_launch() {
        moe::next_launch_events() = moe::LaunchEvents{at(next), at(next + 1)};
        next += 2;
    }
};

}  // namespace

extern "C" {

int moe_workspace_size(const moe_desc *desc, size_t *bytes) {
    Shape s;
    int rc = check_desc(desc, &s);
    if (rc != MOE_OK) return rc;
    if (!bytes) return MOE_ERR_INVALID_ARG;
    *bytes = layout(s).total;
    return MOE_OK;
}

int moe_capacity(const moe_desc *desc, int64_t *capacity) {
    Shape s;
    int rc = check_desc(desc, &s);
    if (rc != MOE_OK) return rc;
    if (!capacity) return MOE_ERR_INVALID_ARG;
    *capacity = s.C;
    return MOE_OK;
}

int moe_route(const moe_desc *desc, const void *x, const float *W_r, const float *bias,
              const float *noise, int32_t *topk_idx, float *gates, float *stats, void *ws,
              size_t ws_bytes, void *stream) {
    Shape s;
    int rc = check_desc(desc, &s);
    if (rc != MOE_OK) return rc;
    if (!x || !W_r || !topk_idx || !gates || !stats) return MOE_ERR_INVALID_ARG;
    if ((rc = check_ws(s, ws, ws_bytes)) != MOE_OK) return rc;
    const Layout L = layout(s);
    hipStream_t st = (hipStream_t)stream;
    if (moe::route_small(s)) {
        MOE_TRY(moe::launch_route_small(s, x, W_r, bias, noise, topk_idx, gates, stats, nullptr,
                                        at<float>(ws, L.part_P), at<float>(ws, L.part_lse2),
                                        at<float>(ws, L.part_logits),
                                        st));
        return MOE_OK;
    }
    MOE_TRY(moe::launch_route(s, x, W_r, bias, noise, topk_idx, gates, at<float>(ws, L.part_P),
                              at<float>(ws, L.part_lse2), at<float>(ws, L.part_logits),
                              L.wsplit ? at<char>(ws, L.wsplit) : nullptr,
                              at<unsigned>(ws, L.arrivals), st));
    MOE_TRY(moe::launch_route_finalize(s, topk_idx, at<float>(ws, L.part_P),
                                       at<float>(ws, L.part_lse2), stats,
                                       at<double>(ws, L.fP),
                                       at<unsigned>(ws, L.arrivals), st));
    return MOE_OK;
}

int moe_dispatch(const moe_desc *desc, const void *x, const int32_t *topk_idx,
                 int32_t *routed_counts, int32_t *kept_counts, int32_t *offsets,
                 int32_t *row_of_slot, int32_t *token_of_row, uint8_t *dropped, void *x_perm,
                 void *ws, size_t ws_bytes, void *stream) {
    Shape s;
    int rc = check_desc(desc, &s);
    if (rc != MOE_OK) return rc;
    if (!x || !topk_idx || !routed_counts || !kept_counts || !offsets || !row_of_slot ||
        !token_of_row || !dropped || !x_perm)
        return MOE_ERR_INVALID_ARG;
    if ((rc = check_ws(s, ws, ws_bytes)) != MOE_OK) return rc;
    const Layout L = layout(s);
    hipStream_t st = (hipStream_t)stream;
    MOE_TRY(moe::launch_dispatch(s, topk_idx, routed_counts, kept_counts, offsets, row_of_slot,
                                 token_of_row, dropped, at<int32_t>(ws, L.chunk_counts), st));
    // stage events 0 and 1, when given, are the gather launch's start and end
    StageEvents ev{desc->stage_events, desc->n_stage_events};
    ev.around_next_launch();
    MOE_TRY(moe::launch_gather(s, x, token_of_row, offsets, x_perm, st));
    return MOE_OK;
}

int moe_expert_ffn(const moe_desc *desc, const void *x_perm, const int32_t *offsets,
                   const void *W1, const void *W3, const void *W2, float *y_perm, void *ws,
                   size_t ws_bytes, void *stream) {
    Shape s;
    int rc = check_desc(desc, &s);
    if (rc != MOE_OK) return rc;
    if (!x_perm || !offsets || !W1 || !W2 || !y_perm) return MOE_ERR_INVALID_ARG;
    if ((s.act == MOE_ACT_SWIGLU) != (W3 != nullptr)) return MOE_ERR_INVALID_ARG;
    if ((rc = check_ws(s, ws, ws_bytes)) != MOE_OK) return rc;
    const Layout L = layout(s);
    hipStream_t st = (hipStream_t)stream;
    void *H = at<char>(ws, L.H);
    unsigned *tctr = at<unsigned>(ws, L.tile_ctr);
    MOE_TRY(moe::launch_zero_u32(tctr, 2 * moe::TILE_CTR_WORDS, st));
    MOE_TRY(moe::launch_expert_up(s, x_perm, nullptr, offsets, W1, W3, H, st, tctr));
    float *part2 = L.y_perm2 ? at<float>(ws, L.y_perm2) : nullptr;
    MOE_TRY(moe::launch_expert_down(s, H, offsets, W2, y_perm, part2, st, tctr + moe::TILE_CTR_WORDS));
    if (part2) MOE_TRY(moe::launch_add_partial(s, y_perm, part2, offsets, st));
    return MOE_OK;
}

int moe_combine(const moe_desc *desc, const float *y_perm, const int32_t *row_of_slot,
                const float *gates, void *y, void *stream) {
    Shape s;
    int rc = check_desc(desc, &s);
    if (rc != MOE_OK) return rc;
    if (!y_perm || !row_of_slot || !gates || !y) return MOE_ERR_INVALID_ARG;
    MOE_TRY(moe::launch_combine(s, y_perm, nullptr, row_of_slot, gates, y, (hipStream_t)stream));
    return MOE_OK;
}

}  // extern "C"

namespace {

// Workspace of moe_backward (every region 256-byte aligned).  R bounds the
// kept rows; ldk bounds the padded row positions (each expert's rows start
// on a multiple of 64, pads zero) and is the row length of the transposed
// activations; poff holds the E + 1 padded offsets.
struct BwdLayout {
    size_t w2t, wcat;                 // W2 as [E][d_ff][d]; W1 | W3 as [E][d][n_up d_ff]
    size_t x_perm, a1, a3, H, Y, part2;
    size_t dE, dg, dH, dA, dXp;
    size_t dET, HT, dAT, XT;
    size_t p, lse, dh, dwr_part, poff;
    size_t dwr_xt, dwr_p, dwr_c, dwr_idx;   // dW_r on matrix cores (dwr_plan)
    size_t lg_w, lg_c, lg_idx;              // logits on matrix cores (logits_plan)
    size_t tile_ctr;                        // tile counters of the five grouped GEMMs
    size_t total;
    int64_t R, ldk;
};

BwdLayout bwd_layout(const Shape &s) {
    BwdLayout L{};
    const size_t nup = s.act == MOE_ACT_SWIGLU ? 2 : 1;
    int64_t R = s.Tk();
    if (s.C >= 0 && (int64_t)s.E * s.C < R) R = (int64_t)s.E * s.C;
    L.R = R;
    L.ldk = moe::padded_rows_bound(R, s.E);
    const size_t r = (size_t)R, lk = (size_t)L.ldk, d = (size_t)s.d, f = (size_t)s.d_ff, E = (size_t)s.E;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align_up(o + bytes);
        return at;
    };
    L.w2t = take(E * f * d * 2);
    L.wcat = take(E * d * nup * f * 2);
    L.x_perm = take(r * d * 2);
    L.a1 = take(r * f * 4);
    L.a3 = nup == 2 ? take(r * f * 4) : 0;
    L.H = take(r * f * 2);
    L.Y = take(r * d * 4);
    L.part2 = take(r * (nup * f > d ? nup * f : d) * 4);
    L.dE = take(r * d * 2);
    L.dg = take((size_t)s.Tk() * 4);
    L.dH = take(r * f * 4);
    L.dA = take(r * nup * f * 2);
    L.dXp = take(r * d * 4);
    L.dET = take(d * lk * 2);
    L.HT = take(f * lk * 2);
    L.dAT = take(nup * f * lk * 2);
    L.XT = take(d * lk * 2);
    L.p = take((size_t)s.T * E * 4);
    L.lse = take((size_t)s.T * 4);
    L.dh = take((size_t)s.T * E * 4);
    L.poff = take((E + 1) * 4);
    L.tile_ctr = take(5 * moe::TILE_CTR_WORDS * 4);
    const moe::DwrPlan pl = moe::dwr_plan(s);
    if (pl.ns == 0) L.dwr_part = take(moe::dwr_part_floats(s) * 4);
    if (pl.ns > 0) {
        L.dwr_xt = take(pl.xt_bytes);
        L.dwr_p = take(pl.p_bytes);
        L.dwr_c = take(pl.c_bytes);
        L.dwr_idx = take(pl.idx_bytes);
    }
    const moe::LogitsPlan lp = moe::logits_plan(s);
    if (lp.ns > 0) {
        L.lg_w = take(lp.ws_bytes);
        L.lg_c = take(lp.c_bytes);
        L.lg_idx = take(lp.idx_bytes);
    }
    L.total = o;
    return L;
}

// C = A B^T over the per-expert row blocks with N = n, K = kdim (the
// forward's down-projection launcher on a re-labelled shape), adding the
// second K half when it splits K.
int grouped_gemm_f32(const Shape &s, int n, int kdim, const void *A, const int32_t *offsets,
                     const void *B, float *C, float *part2, hipStream_t st, unsigned *tctr) {
    Shape q = s;
    q.d = n;
    q.d_ff = kdim;
    MOE_TRY(moe::launch_expert_down(q, A, offsets, B, C, part2, st, tctr));
    if (moe::down_ksplit(q) == 2) MOE_TRY(moe::launch_add_partial(q, C, part2, offsets, st));
    return MOE_OK;
}

// Validates E4M3 expert weights for this description (shape support first).
int check_fp8(const Shape &s, const moe_fp8_experts *w) {
    if (!w) return MOE_ERR_INVALID_ARG;
    if (!moe::fp8_supported(s)) return MOE_ERR_UNSUPPORTED;
    if (!w->W1 || !w->W2 || !w->s1 || !w->s2) return MOE_ERR_INVALID_ARG;
    const bool swiglu = s.act == MOE_ACT_SWIGLU;
    if (swiglu != (w->W3 != nullptr) || swiglu != (w->s3 != nullptr)) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

// Validates packed expert weights for this description (format, then shape
// support, then the pointers).
int check_packed(const Shape &s, const moe_packed_experts *w) {
    if (!w) return MOE_ERR_INVALID_ARG;
    if (w->format != MOE_WEIGHTS_BF16 && w->format != MOE_WEIGHTS_E4M3) return MOE_ERR_INVALID_ARG;
    if (!moe::fp8_supported(s)) return MOE_ERR_UNSUPPORTED;
    if (!w->W1 || !w->W2) return MOE_ERR_INVALID_ARG;
    const bool swiglu = s.act == MOE_ACT_SWIGLU;
    if (swiglu != (w->W3 != nullptr)) return MOE_ERR_INVALID_ARG;
    if (w->format == MOE_WEIGHTS_E4M3) {
        if (!w->s1 || !w->s2 || swiglu != (w->s3 != nullptr)) return MOE_ERR_INVALID_ARG;
    } else if (w->s1 || w->s2 || w->s3) {
        return MOE_ERR_INVALID_ARG;
    }
    return MOE_OK;
}

// Expert weights of the weight-streaming kernels: e4m3 codes (row-major or
// packed) or packed bf16 values.
struct StreamW {
    bool e4m3, packed;
    const void *W1, *W3, *W2;
    const float *s1, *s3, *s2;
};

StreamW stream_w(const moe_fp8_experts *w) { return StreamW{true, false, w->W1, w->W3, w->W2, w->s1, w->s3, w->s2}; }
StreamW stream_w(const moe_packed_experts *w) {
    return StreamW{w->format == MOE_WEIGHTS_E4M3, true, w->W1, w->W3, w->W2, w->s1, w->s3, w->s2};
}

hipError_t stream_up(const Shape &s, const void *A, const int32_t *a_rows, const int32_t *offsets, const StreamW &w,
                     void *H, hipStream_t st) {
    if (w.e4m3)
        return moe::launch_expert_up_fp8(s, A, a_rows, offsets, (const uint8_t *)w.W1, (const uint8_t *)w.W3, w.s1,
                                         w.s3, H, st, w.packed);
    return moe::launch_expert_up_packed(s, A, a_rows, offsets, w.W1, w.W3, H, st);
}

hipError_t stream_down(const Shape &s, const void *H, const int32_t *offsets, const StreamW &w, float *y_perm,
                       hipStream_t st) {
    if (w.e4m3) return moe::launch_expert_down_fp8(s, H, offsets, (const uint8_t *)w.W2, w.s2, y_perm, st, w.packed);
    return moe::launch_expert_down_packed(s, H, offsets, w.W2, y_perm, st);
}

// moe_forward, moe_forward_shared, moe_forward_fp8 and moe_forward_packed:
// sh == nullptr and f8 == nullptr is moe_forward (seven stages); with sh the
// shared experts run as their own stage between expert-down and the
// combine, which adds them and the residual; with f8 the expert GEMMs are
// the weight-streaming kernels on E4M3 or packed weights (already
// validated by the caller, after the description).
int forward_impl(const moe_desc *desc, const moe_shared *sh, const StreamW *f8,
                 const void *x, const float *W_r, const float *bias, const float *noise,
                 const void *W1, const void *W3, const void *W2, void *y, int32_t *topk_idx,
                 float *gates, int32_t *routed_counts, int32_t *kept_counts, int32_t *offsets,
                 int32_t *row_of_slot, int32_t *token_of_row, uint8_t *dropped, float *stats,
                 void *ws, size_t ws_bytes, void *stream) {
    Shape s;
    int rc = check_desc(desc, &s);
    if (rc != MOE_OK) return rc;
    if (f8) {
        if (!x || !W_r || !y) return MOE_ERR_INVALID_ARG;
    } else {
        if (!x || !W_r || !W1 || !W2 || !y) return MOE_ERR_INVALID_ARG;
        if ((s.act == MOE_ACT_SWIGLU) != (W3 != nullptr)) return MOE_ERR_INVALID_ARG;
    }
    if (sh && (rc = check_shared(s, sh)) != MOE_OK) return rc;
    const int S = sh ? sh->n_shared : 0;
    if ((rc = check_ws(s, ws, ws_bytes, S)) != MOE_OK) return rc;
    const Layout L = layout(s, S);
    if (!topk_idx) topk_idx = at<int32_t>(ws, L.topk_idx);
    if (!gates) gates = at<float>(ws, L.gates);
    if (!routed_counts) routed_counts = at<int32_t>(ws, L.routed);
    if (!kept_counts) kept_counts = at<int32_t>(ws, L.kept);
    if (!offsets) offsets = at<int32_t>(ws, L.offsets);
    if (!row_of_slot) row_of_slot = at<int32_t>(ws, L.row_of_slot);
    if (!token_of_row) token_of_row = at<int32_t>(ws, L.token_of_row);
    if (!dropped) dropped = at<uint8_t>(ws, L.dropped);
    if (!stats) stats = at<float>(ws, L.stats);
    void *H = at<char>(ws, L.H);
    float *y_perm = at<float>(ws, L.y_perm);
    // tile counters, cleared by the dispatch launch (none on the small-batch
    // path, whose kernels need none)
    unsigned *tctr = moe::route_small(s) ? nullptr : at<unsigned>(ws, L.tile_ctr);
    constexpr int CW = moe::TILE_CTR_WORDS;

    hipStream_t st = (hipStream_t)stream;
    StageEvents ev{desc->stage_events, desc->n_stage_events};
    MOE_TRY(ev.record(st));
    if (moe::route_small(s)) {
        // one kernel after the logits does the epilogue, statistics and
        // dispatch; the statistics and dispatch stages are empty
        const moe::DispatchOut disp{routed_counts, kept_counts, offsets,
                                    row_of_slot, token_of_row, dropped};
        MOE_TRY(moe::launch_route_small(s, x, W_r, bias, noise, topk_idx, gates, stats, &disp,
                                        at<float>(ws, L.part_P), at<float>(ws, L.part_lse2),
                                        at<float>(ws, L.part_logits),
                                        st));
        MOE_TRY(ev.record(st));
        MOE_TRY(ev.record(st));
    } else {
        MOE_TRY(moe::launch_route(s, x, W_r, bias, noise, topk_idx, gates, at<float>(ws, L.part_P),
                                  at<float>(ws, L.part_lse2), at<float>(ws, L.part_logits),
                                  L.wsplit ? at<char>(ws, L.wsplit) : nullptr,
                                  at<unsigned>(ws, L.arrivals), st));
        MOE_TRY(ev.record(st));
        // the statistics are finished by extra blocks of the dispatch launch
        // (the same reduction as launch_route_finalize's), so the
        // route-finalize stage is empty
        MOE_TRY(ev.record(st));
        const moe::RouteStatsIn rs{at<float>(ws, L.part_P), at<float>(ws, L.part_lse2),
                                   moe::route_stat_blocks(s), stats, at<double>(ws, L.fP),
                                   at<unsigned>(ws, L.arrivals)};
        MOE_TRY(moe::launch_dispatch(s, topk_idx, routed_counts, kept_counts, offsets, row_of_slot,
                                     token_of_row, dropped, at<int32_t>(ws, L.chunk_counts), st, &rs, tctr,
                                     4 * CW));
    }
    MOE_TRY(ev.record(st));
    // the gather is folded into the up projection's loads: its rows of A are
    // read from x through token_of_row, so x_perm is not materialised here
    ev.around_next_launch();  // events before and after expert-up
    const hipError_t up_err =
        f8 ? stream_up(s, x, token_of_row, offsets, *f8, H, st)
           : moe::launch_expert_up(s, x, token_of_row, offsets, W1, W3, H, st, tctr);
    moe::next_launch_events() = moe::LaunchEvents{nullptr, nullptr};
    MOE_TRY(up_err);
    // the streaming path never splits K across blocks
    float *part2 = (!f8 && L.y_perm2) ? at<float>(ws, L.y_perm2) : nullptr;
    if (f8)
        MOE_TRY(stream_down(s, H, offsets, *f8, y_perm, st));
    else
        MOE_TRY(moe::launch_expert_down(s, H, offsets, W2, y_perm, part2, st, tctr ? tctr + CW : nullptr));
    if (!sh) {
        ev.around_next_launch();  // events before and after the combine (one kernel)
        const hipError_t c_err = moe::launch_combine(s, y_perm, part2, row_of_slot, gates, y, st);
        moe::next_launch_events() = moe::LaunchEvents{nullptr, nullptr};
        MOE_TRY(c_err);
        return MOE_OK;
    }
    MOE_TRY(ev.record(st));
    float *y_sh = nullptr, *y_sh2 = nullptr;
    if (S > 0) {
        y_sh = at<float>(ws, L.y_sh);
        y_sh2 = L.y_sh2 ? at<float>(ws, L.y_sh2) : nullptr;
        if ((rc = run_shared_ffn(s, sh, x, y_sh, y_sh2, ws, L, st, tctr ? tctr + 2 * CW : nullptr)) != MOE_OK)
            return rc;
    }
    MOE_TRY(ev.record(st));
    MOE_TRY(moe::launch_combine_shared(s, y_perm, part2, row_of_slot, gates, y_sh, y_sh2,
                                       sh->residual, y, st));
    MOE_TRY(ev.record(st));
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_forward(const moe_desc *desc, const void *x, const float *W_r, const float *bias,
                const float *noise, const void *W1, const void *W3, const void *W2, void *y,
                int32_t *topk_idx, float *gates, int32_t *routed_counts, int32_t *kept_counts,
                int32_t *offsets, int32_t *row_of_slot, int32_t *token_of_row,
                uint8_t *dropped, float *stats, void *ws, size_t ws_bytes, void *stream) {
    return forward_impl(desc, nullptr, nullptr, x, W_r, bias, noise, W1, W3, W2, y, topk_idx, gates,
                        routed_counts, kept_counts, offsets, row_of_slot, token_of_row, dropped,
                        stats, ws, ws_bytes, stream);
}

int moe_forward_noalloc(const moe_desc *desc, const void *x, const float *W_r, const float *bias,
                        const float *noise, const void *W1, const void *W3, const void *W2,
                        void *y, int32_t *topk_idx, float *gates, int32_t *routed_counts,
                        int32_t *kept_counts, int32_t *offsets, int32_t *row_of_slot,
                        int32_t *token_of_row, uint8_t *dropped, float *stats, void *stream) {
    Shape s;
    int rc = check_desc(desc, &s);
    if (rc != MOE_OK) return rc;
    const size_t need = layout(s).total;
    if (need > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
    void *ws = nullptr;
    if (moe::noalloc_scratch(&ws) != hipSuccess) return MOE_ERR_HIP;
    return forward_impl(desc, nullptr, nullptr, x, W_r, bias, noise, W1, W3, W2, y, topk_idx, gates,
                        routed_counts, kept_counts, offsets, row_of_slot, token_of_row, dropped,
                        stats, ws, need, stream);
}

int moe_workspace_size_shared(const moe_desc *desc, const moe_shared *shared, size_t *bytes) {
    Shape s;
    int rc = check_desc(desc, &s);
    if (rc != MOE_OK) return rc;
    if (!bytes || !shared) return MOE_ERR_INVALID_ARG;
    if (shared->n_shared < 0 || shared->n_shared > MOE_MAX_SHARED) return MOE_ERR_INVALID_ARG;
    if ((int64_t)shared->n_shared * s.d_ff >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    *bytes = layout(s, shared->n_shared).total;
    return MOE_OK;
}

int moe_shared_ffn(const moe_desc *desc, const moe_shared *shared, const void *x,
                   float *y_shared, void *ws, size_t ws_bytes, void *stream) {
    Shape s;
    int rc = check_desc(desc, &s);
    if (rc != MOE_OK) return rc;
    if ((rc = check_shared(s, shared)) != MOE_OK) return rc;
    const int S = shared->n_shared;
    if (S > 0 && (!x || !y_shared)) return MOE_ERR_INVALID_ARG;
    if ((rc = check_ws(s, ws, ws_bytes, S)) != MOE_OK) return rc;
    if (S == 0) return MOE_OK;
    const Layout L = layout(s, S);
    hipStream_t st = (hipStream_t)stream;
    float *y_sh2 = L.y_sh2 ? at<float>(ws, L.y_sh2) : nullptr;
    unsigned *tctr = at<unsigned>(ws, L.tile_ctr) + 2 * moe::TILE_CTR_WORDS;
    MOE_TRY(moe::launch_zero_u32(tctr, 2 * moe::TILE_CTR_WORDS, st));
    if ((rc = run_shared_ffn(s, shared, x, y_shared, y_sh2, ws, L, st, tctr)) != MOE_OK) return rc;
    if (y_sh2)
        MOE_TRY(moe::launch_add_partial(moe::shared_shape(s, S), y_shared, y_sh2,
                                        at<int32_t>(ws, L.sh_offsets), st));
    return MOE_OK;
}

int moe_combine_shared(const moe_desc *desc, const float *y_perm, const int32_t *row_of_slot,
                       const float *gates, const float *y_shared, const void *residual, void *y,
                       void *stream) {
    Shape s;
    int rc = check_desc(desc, &s);
    if (rc != MOE_OK) return rc;
    if (!y_perm || !row_of_slot || !gates || !y) return MOE_ERR_INVALID_ARG;
    MOE_TRY(moe::launch_combine_shared(s, y_perm, nullptr, row_of_slot, gates, y_shared, nullptr,
                                       residual, y, (hipStream_t)stream));
    return MOE_OK;
}

int moe_forward_shared(const moe_desc *desc, const moe_shared *shared, const void *x,
                       const float *W_r, const float *bias, const float *noise, const void *W1,
                       const void *W3, const void *W2, void *y, int32_t *topk_idx, float *gates,
                       int32_t *routed_counts, int32_t *kept_counts, int32_t *offsets,
                       int32_t *row_of_slot, int32_t *token_of_row, uint8_t *dropped,
                       float *stats, void *ws, size_t ws_bytes, void *stream) {
    if (!shared) return MOE_ERR_INVALID_ARG;
    return forward_impl(desc, shared, nullptr, x, W_r, bias, noise, W1, W3, W2, y, topk_idx, gates,
                        routed_counts, kept_counts, offsets, row_of_slot, token_of_row, dropped,
                        stats, ws, ws_bytes, stream);
}

int moe_quantize_e4m3(int32_t dtype, const void *W, int64_t rows, int64_t cols, uint8_t *q,
                      float *scales, void *stream) {
    if (dtype != MOE_DTYPE_F32 && dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
    if (rows < 0 || cols < 1) return MOE_ERR_INVALID_ARG;
    if (rows == 0) return MOE_OK;
    if (!W || !q || !scales) return MOE_ERR_INVALID_ARG;
    MOE_TRY(moe::launch_quantize_e4m3(dtype == MOE_DTYPE_BF16 ? 1 : 0, W, rows, cols, q, scales,
                                      (hipStream_t)stream));
    return MOE_OK;
}

int moe_expert_ffn_fp8(const moe_desc *desc, const void *x_perm, const int32_t *offsets,
                       const moe_fp8_experts *w, float *y_perm, void *ws, size_t ws_bytes,
                       void *stream) {
    Shape s;
    int rc = check_desc(desc, &s);
    if (rc != MOE_OK) return rc;
    if (!x_perm || !offsets || !y_perm) return MOE_ERR_INVALID_ARG;
    if ((rc = check_fp8(s, w)) != MOE_OK) return rc;
    if ((rc = check_ws(s, ws, ws_bytes)) != MOE_OK) return rc;
    const Layout L = layout(s);
    hipStream_t st = (hipStream_t)stream;
    void *H = at<char>(ws, L.H);
    MOE_TRY(moe::launch_expert_up_fp8(s, x_perm, nullptr, offsets, w->W1, w->W3, w->s1, w->s3, H, st));
    MOE_TRY(moe::launch_expert_down_fp8(s, H, offsets, w->W2, w->s2, y_perm, st));
    return MOE_OK;
}

int moe_forward_fp8(const moe_desc *desc, const void *x, const float *W_r, const float *bias,
                    const float *noise, const moe_fp8_experts *w, void *y, int32_t *topk_idx,
                    float *gates, int32_t *routed_counts, int32_t *kept_counts, int32_t *offsets,
                    int32_t *row_of_slot, int32_t *token_of_row, uint8_t *dropped, float *stats,
                    void *ws, size_t ws_bytes, void *stream) {
    if (!w) return MOE_ERR_INVALID_ARG;
    Shape s;
    int rc = check_desc(desc, &s);
    if (rc != MOE_OK) return rc;
    if (!x || !W_r || !y) return MOE_ERR_INVALID_ARG;
    if ((rc = check_fp8(s, w)) != MOE_OK) return rc;
    const StreamW sw = stream_w(w);
    return forward_impl(desc, nullptr, &sw, x, W_r, bias, noise, nullptr, nullptr, nullptr, y,
                        topk_idx, gates, routed_counts, kept_counts, offsets, row_of_slot,
                        token_of_row, dropped, stats, ws, ws_bytes, stream);
}

int moe_pack_stream(int32_t elem_bytes, const void *W, int64_t rows, int64_t cols, void *W_packed,
                    void *stream) {
    if (elem_bytes != 1 && elem_bytes != 2) return MOE_ERR_INVALID_ARG;
    if (rows < 0 || rows % 16 != 0 || cols < 128 || cols % 128 != 0) return MOE_ERR_INVALID_ARG;
    if (rows == 0) return MOE_OK;
    if (!W || !W_packed) return MOE_ERR_INVALID_ARG;
    MOE_TRY(moe::launch_pack_stream(elem_bytes, W, rows, cols, W_packed, (hipStream_t)stream));
    return MOE_OK;
}

int moe_expert_ffn_packed(const moe_desc *desc, const void *x_perm, const int32_t *offsets,
                          const moe_packed_experts *w, float *y_perm, void *ws, size_t ws_bytes,
                          void *stream) {
    Shape s;
    int rc = check_desc(desc, &s);
    if (rc != MOE_OK) return rc;
    if (!x_perm || !offsets || !y_perm) return MOE_ERR_INVALID_ARG;
    if ((rc = check_packed(s, w)) != MOE_OK) return rc;
    if ((rc = check_ws(s, ws, ws_bytes)) != MOE_OK) return rc;
    const Layout L = layout(s);
    hipStream_t st = (hipStream_t)stream;
    void *H = at<char>(ws, L.H);
    const StreamW sw = stream_w(w);
    MOE_TRY(stream_up(s, x_perm, nullptr, offsets, sw, H, st));
    MOE_TRY(stream_down(s, H, offsets, sw, y_perm, st));
    return MOE_OK;
}

int moe_forward_packed(const moe_desc *desc, const void *x, const float *W_r, const float *bias,
                       const float *noise, const moe_packed_experts *w, void *y, int32_t *topk_idx,
                       float *gates, int32_t *routed_counts, int32_t *kept_counts, int32_t *offsets,
                       int32_t *row_of_slot, int32_t *token_of_row, uint8_t *dropped, float *stats,
                       void *ws, size_t ws_bytes, void *stream) {
    if (!w) return MOE_ERR_INVALID_ARG;
    Shape s;
    int rc = check_desc(desc, &s);
    if (rc != MOE_OK) return rc;
    if (!x || !W_r || !y) return MOE_ERR_INVALID_ARG;
    if ((rc = check_packed(s, w)) != MOE_OK) return rc;
    const StreamW sw = stream_w(w);
    return forward_impl(desc, nullptr, &sw, x, W_r, bias, noise, nullptr, nullptr, nullptr, y,
                        topk_idx, gates, routed_counts, kept_counts, offsets, row_of_slot,
                        token_of_row, dropped, stats, ws, ws_bytes, stream);
}

// fp32 layers: the same steps as the bf16 backward with plain fp32 kernels
// (weights transposed by launch_transpose_f32, expert GEMMs through the
// forward's fp32 grouped GEMM, weight gradients by launch_wgrad_f32, the
// router part by the same kernels on fp32 x).
struct BwdLayoutF32 {
    size_t w2t, wcat, x_perm, a1, a3, H, Y, dE, dg, dH, dA, dXp, p, lse, dh, dwr_part, total;
};

static BwdLayoutF32 bwd_layout_f32(const Shape &s) {
    BwdLayoutF32 L{};
    const size_t nup = s.act == MOE_ACT_SWIGLU ? 2 : 1;
    const size_t E = (size_t)s.E, d = (size_t)s.d, f = (size_t)s.d_ff;
    size_t r = (size_t)s.Tk();
    if (s.C >= 0 && E * (size_t)s.C < r) r = E * (size_t)s.C;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align_up(o + bytes);
        return at;
    };
    L.w2t = take(E * f * d * 4);
    L.wcat = take(E * d * nup * f * 4);
    L.x_perm = take(r * d * 4);
    L.a1 = take(r * f * 4);
    L.a3 = nup == 2 ? take(r * f * 4) : 0;
    L.H = take(r * f * 4);
    L.Y = take(r * d * 4);
    L.dE = take(r * d * 4);
    L.dg = take((size_t)s.Tk() * 4);
    L.dH = take(r * f * 4);
    L.dA = take(r * nup * f * 4);
    L.dXp = take(r * d * 4);
    L.p = take((size_t)s.T * E * 4);
    L.lse = take((size_t)s.T * 4);
    L.dh = take((size_t)s.T * E * 4);
    L.dwr_part = take(moe::dwr_part_floats(s) * 4);
    L.total = o;
    return L;
}

static int backward_f32(const Shape &s, const float *x, const float *W_r, const float *bias, const float *noise,
                        const float *W1, const float *W3, const float *W2, const int32_t *topk_idx,
                        const float *gates, const int32_t *offsets, const int32_t *row_of_slot,
                        const int32_t *token_of_row, const float *stats, const float *dy, float alpha_aux,
                        float alpha_z, float *dx, float *dW_r, float *dbias, float *dW1, float *dW3, float *dW2,
                        void *ws, hipStream_t st) {
    const BwdLayoutF32 L = bwd_layout_f32(s);
    const bool swiglu = s.act == MOE_ACT_SWIGLU;
    const int d = s.d, f = s.d_ff, E = s.E, nup = swiglu ? 2 : 1;
    char *w = (char *)ws;
    float *w2t = (float *)(w + L.w2t), *wcat = (float *)(w + L.wcat), *xp = (float *)(w + L.x_perm);
    float *a1 = (float *)(w + L.a1), *a3 = swiglu ? (float *)(w + L.a3) : nullptr, *H = (float *)(w + L.H);
    float *Y = (float *)(w + L.Y), *dE = (float *)(w + L.dE), *dg = (float *)(w + L.dg);
    float *dH = (float *)(w + L.dH), *dA = (float *)(w + L.dA), *dXp = (float *)(w + L.dXp);
    float *p = (float *)(w + L.p), *lse = (float *)(w + L.lse), *dh = (float *)(w + L.dh);
    const int64_t df = (int64_t)d * f;
    int rc;
    // weights as [K][N] operands of the gradient GEMMs: W2 to [E][d_ff][d],
    // W1 | W3 side by side to [E][d][n_up d_ff]
    MOE_TRY(moe::launch_transpose_f32(W2, d, f, f, df, w2t, d, df, E, st, offsets));
    MOE_TRY(moe::launch_transpose_f32(W1, f, d, d, df, wcat, (int64_t)nup * f, (int64_t)nup * df, E, st, offsets));
    if (swiglu)
        MOE_TRY(moe::launch_transpose_f32(W3, f, d, d, df, wcat + f, (int64_t)nup * f, (int64_t)nup * df, E, st,
                                          offsets));
    // recompute the forward's expert part
    MOE_TRY(moe::launch_gather(s, x, token_of_row, offsets, xp, st));
    if ((rc = grouped_gemm_f32(s, f, d, xp, offsets, W1, a1, nullptr, st, nullptr)) != MOE_OK) return rc;
    if (swiglu && (rc = grouped_gemm_f32(s, f, d, xp, offsets, W3, a3, nullptr, st, nullptr)) != MOE_OK) return rc;
    MOE_TRY(moe::launch_act_fwd(s, a1, a3, offsets, H, st));
    if ((rc = grouped_gemm_f32(s, d, f, H, offsets, W2, Y, nullptr, st, nullptr)) != MOE_OK) return rc;
    // combine, down projection and activation backward; dX_perm
    MOE_TRY(moe::launch_combine_bwd(s, dy, Y, token_of_row, row_of_slot, gates, offsets, dE, dg, st));
    if ((rc = grouped_gemm_f32(s, f, d, dE, offsets, w2t, dH, nullptr, st, nullptr)) != MOE_OK) return rc;
    MOE_TRY(moe::launch_act_bwd(s, a1, a3, dH, offsets, dA, st));
    if ((rc = grouped_gemm_f32(s, d, nup * f, dA, offsets, wcat, dXp, nullptr, st, nullptr)) != MOE_OK) return rc;
    // router: gates, load-balancing and z terms; dx, dW_r, dbias
    MOE_TRY(moe::launch_router_bwd(s, x, W_r, bias, noise, topk_idx, gates, dg, row_of_slot, stats, alpha_aux,
                                   alpha_z, p, lse, dh, st, true));
    MOE_TRY(moe::launch_dx(s, dXp, row_of_slot, dh, W_r, dx, st));
    MOE_TRY(moe::launch_dwr(s, dh, x, (float *)(w + L.dwr_part), dW_r, dbias, st));
    // weight gradients over each expert's rows
    MOE_TRY(moe::launch_wgrad_f32(E, d, f, offsets, dE, d, H, f, dW2, st));
    MOE_TRY(moe::launch_wgrad_f32(E, f, d, offsets, dA, (int64_t)nup * f, xp, d, dW1, st));
    if (swiglu) MOE_TRY(moe::launch_wgrad_f32(E, f, d, offsets, dA + f, (int64_t)nup * f, xp, d, dW3, st));
    return MOE_OK;
}

int moe_backward_workspace_size(const moe_desc *desc, size_t *bytes) {
    Shape s;
    int rc = check_desc(desc, &s);
    if (rc != MOE_OK) return rc;
    if (!bytes) return MOE_ERR_INVALID_ARG;
    if (s.dtype != MOE_DTYPE_BF16) {
        *bytes = bwd_layout_f32(s).total;
        return MOE_OK;
    }
    const BwdLayout L = bwd_layout(s);
    if (L.ldk / 64 > 65535) return MOE_ERR_UNSUPPORTED;   // padded transposes' grid
    *bytes = L.total;
    return MOE_OK;
}

int moe_backward(const moe_desc *desc, const void *x, const float *W_r, const float *bias,
                 const float *noise, const void *W1, const void *W3, const void *W2,
                 const int32_t *topk_idx, const float *gates, const int32_t *offsets,
                 const int32_t *row_of_slot, const int32_t *token_of_row, const float *stats,
                 const void *dy, float alpha_aux, float alpha_z, float *dx, float *dW_r,
                 float *dbias, float *dW1, float *dW3, float *dW2, void *ws, size_t ws_bytes,
                 void *stream) {
    Shape s;
    int rc = check_desc(desc, &s);
    if (rc != MOE_OK) return rc;
    if (!x || !W_r || !W1 || !W2 || !topk_idx || !gates || !offsets || !row_of_slot ||
        !token_of_row || !stats || !dy || !dx || !dW_r || !dW1 || !dW2 || !ws)
        return MOE_ERR_INVALID_ARG;
    const bool swiglu = s.act == MOE_ACT_SWIGLU;
    if (swiglu != (W3 != nullptr) || swiglu != (dW3 != nullptr)) return MOE_ERR_INVALID_ARG;
    if (dbias && !bias) return MOE_ERR_INVALID_ARG;
    if (!std::isfinite(alpha_aux) || !std::isfinite(alpha_z)) return MOE_ERR_INVALID_ARG;
    if (s.dtype != MOE_DTYPE_BF16) {
        if (ws_bytes < bwd_layout_f32(s).total) return MOE_ERR_WORKSPACE;
        return backward_f32(s, (const float *)x, W_r, bias, noise, (const float *)W1, (const float *)W3,
                            (const float *)W2, topk_idx, gates, offsets, row_of_slot, token_of_row, stats,
                            (const float *)dy, alpha_aux, alpha_z, dx, dW_r, dbias, dW1, dW3, dW2, ws,
                            (hipStream_t)stream);
    }
    const BwdLayout L = bwd_layout(s);
    // kept rows (rounded per expert to 64) past 65535 * 64: the padded
    // transposes' grid would not fit; rejected before any launch
    if (L.ldk / 64 > 65535) return MOE_ERR_UNSUPPORTED;
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    const int d = s.d, f = s.d_ff, E = s.E, nup = swiglu ? 2 : 1;
    char *w = (char *)ws;
    void *w2t = w + L.w2t, *wcat = w + L.wcat, *xp = w + L.x_perm, *H = w + L.H;
    float *a1 = (float *)(w + L.a1), *a3 = swiglu ? (float *)(w + L.a3) : nullptr;
    float *Y = (float *)(w + L.Y), *part2 = (float *)(w + L.part2), *dg = (float *)(w + L.dg);
    float *dH = (float *)(w + L.dH), *dXp = (float *)(w + L.dXp);
    void *dE = w + L.dE, *dA = w + L.dA;
    void *dET = w + L.dET, *HT = w + L.HT, *dAT = w + L.dAT, *XT = w + L.XT;
    float *p = (float *)(w + L.p), *lse = (float *)(w + L.lse), *dh = (float *)(w + L.dh);
    const int64_t df = (int64_t)d * f;

    // weights as K-contiguous operands of the gradient GEMMs (experts
    // without rows skipped: no GEMM reads their transposed weights)
    MOE_TRY(moe::launch_transpose_bf16(W2, d, f, f, df, w2t, d, df, E, st, offsets));
    MOE_TRY(moe::launch_transpose_bf16(W1, f, d, d, df, wcat, (int64_t)nup * f, (int64_t)nup * df, E, st, offsets));
    if (swiglu)
        MOE_TRY(moe::launch_transpose_bf16(W3, f, d, d, df, (char *)wcat + (size_t)f * 2, (int64_t)nup * f,
                                           (int64_t)nup * df, E, st, offsets));
    // tile counters of the five grouped GEMMs below, cleared once
    unsigned *tc = (unsigned *)(w + L.tile_ctr);
    constexpr int CW = moe::TILE_CTR_WORDS;
    MOE_TRY(moe::launch_zero_u32(tc, 5 * CW, st));
    // recompute the forward's expert part: x rows, pre-activations, H, E(x)
    MOE_TRY(moe::launch_gather(s, x, token_of_row, offsets, xp, st));
    if ((rc = grouped_gemm_f32(s, f, d, xp, offsets, W1, a1, part2, st, tc)) != MOE_OK) return rc;
    if (swiglu && (rc = grouped_gemm_f32(s, f, d, xp, offsets, W3, a3, part2, st, tc + CW)) != MOE_OK) return rc;
    MOE_TRY(moe::launch_act_fwd(s, a1, a3, offsets, H, st));
    if ((rc = grouped_gemm_f32(s, d, f, H, offsets, W2, Y, part2, st, tc + 2 * CW)) != MOE_OK) return rc;
    // combine, down projection and activation backward; dX_perm
    MOE_TRY(moe::launch_combine_bwd(s, dy, Y, token_of_row, row_of_slot, gates, offsets, dE, dg, st));
    if ((rc = grouped_gemm_f32(s, f, d, dE, offsets, w2t, dH, part2, st, tc + 3 * CW)) != MOE_OK) return rc;
    MOE_TRY(moe::launch_act_bwd(s, a1, a3, dH, offsets, dA, st));
    if ((rc = grouped_gemm_f32(s, d, nup * f, dA, offsets, wcat, dXp, part2, st, tc + 4 * CW)) != MOE_OK)
        return rc;
    // router: gates, load-balancing and z terms; dx, dW_r, dbias
    const moe::LogitsPlan lpl = moe::logits_plan(s);
    if (lpl.ns > 0)
        MOE_TRY(moe::launch_logits_mfma(s, lpl, x, W_r, bias, noise, w + L.lg_w, (float *)(w + L.lg_c),
                                        (int32_t *)(w + L.lg_idx), p, lse, st));
    MOE_TRY(moe::launch_router_bwd(s, x, W_r, bias, noise, topk_idx, gates, dg, row_of_slot, stats,
                                   alpha_aux, alpha_z, p, lse, dh, st, lpl.ns == 0));
    MOE_TRY(moe::launch_dx(s, dXp, row_of_slot, dh, W_r, dx, st));
    const moe::DwrPlan dpl = moe::dwr_plan(s);
    if (dpl.ns > 0)
        MOE_TRY(moe::launch_dwr_mfma(s, dpl, dh, x, w + L.dwr_xt, w + L.dwr_p, (float *)(w + L.dwr_c),
                                     (int32_t *)(w + L.dwr_idx), dW_r, dbias, st));
    else
        MOE_TRY(moe::launch_dwr(s, dh, x, (float *)(w + L.dwr_part), dW_r, dbias, st));
    // weight gradients over each expert's rows, from the activations
    // transposed into the padded layout
    int32_t *poff = (int32_t *)(w + L.poff);
    MOE_TRY(moe::launch_pad_offsets(offsets, E, poff, st));
    MOE_TRY(moe::launch_transpose_padded(dE, d, d, offsets, poff, E, L.ldk, dET, st));
    MOE_TRY(moe::launch_transpose_padded(H, f, f, offsets, poff, E, L.ldk, HT, st));
    MOE_TRY(moe::launch_transpose_padded(dA, (int64_t)nup * f, (int64_t)nup * f, offsets, poff, E, L.ldk, dAT, st));
    MOE_TRY(moe::launch_transpose_padded(xp, d, d, offsets, poff, E, L.ldk, XT, st));
    const bool big = moe::wgrad_big_fits(d, f, L.ldk);
    auto wgrad = big ? moe::launch_wgrad_big : moe::launch_wgrad;
    MOE_TRY(wgrad(E, d, f, poff, dET, HT, L.ldk, dW2, st));
    MOE_TRY(wgrad(E, f, d, poff, dAT, XT, L.ldk, dW1, st));
    if (swiglu) MOE_TRY(wgrad(E, f, d, poff, (char *)dAT + (size_t)f * L.ldk * 2, XT, L.ldk, dW3, st));
    return MOE_OK;
}

const char *moe_status_string(int status) {
    switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: valid but not supported by the kernels";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: the HIP runtime reported an error";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace smaller than moe_workspace_size()";
    case MOE_ERR_SCRATCH:
        return "MOE_ERR_SCRATCH: moe_forward_noalloc needs more than its static scratch "
               "(MOE_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown moe status";
    }
}

}  // extern "C"
