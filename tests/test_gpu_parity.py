"""GPU parity against the CPU oracle, element by element, through the C ABI.

Sizes are ones the oracle finishes in seconds but that still span several
row and column tiles, ragged tails in M, N and K, and every row-tile
height the library picks.  Edge cases: T = 1, E = 1, k = E, every token on
one expert, empty experts, capacity 1, exact ties, minimal widths,
determinism, and the staged entry points against moe_forward.
"""
import numpy as np
import pytest
import torch

from sparse_mixture_experts_03_amd import binding as B
from sparse_mixture_experts_03_amd import synth

import harness as H

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
SMALL = {
    # the tiny fp32 layer, full size
    "tiny": W["tiny"],
    # Switch-style: 16 experts, C = ceil(1.25*600/16) = 47, GELU; N and K ragged
    "switch_small": W["switch"].with_(name="switch_small", T=600, d=264, d_ff=392, E=16,
                                      noise_std=1.0 / 16),
    # Mixtral-style SwiGLU, ~175 rows per expert (128-row tiles), N=1000, K=520 ragged
    "mixtral_small": W["mixtral_prefill"].with_(name="mixtral_small", T=700, d=520, d_ff=1000),
    # decode shape: ~8 rows per expert (32-row tiles)
    "decode_small": W["mixtral_decode"].with_(name="decode_small", d=512, d_ff=768),
    # Zipf-skewed, top-4 of 32, cf=1.0: drops, empty experts, 128-row tiles
    "zipf_small": W["finegrained_zipf"].with_(name="zipf_small", T=1500, d=264, d_ff=200, E=32),
    # bf16 ReLU, top-3 of 6, cf=0.8: 64-row tiles, drops
    "relu_bf16": W["tiny"].with_(name="relu_bf16", T=200, d=64, d_ff=136, E=6, k=3, cf=0.8,
                                 dtype="bf16"),
    # 256-row tiles with direct-to-LDS loads: ~600 rows per expert, K % 64 == 0,
    # a partial last column tile (448 = 3*128 + 64), ragged last row tile
    "big_swiglu": W["mixtral_prefill"].with_(name="big_swiglu", T=1200, d=512, d_ff=448, E=4),
    # the same kernel without the dual accumulator: GELU, k = 1, capacity 1.05,
    # partial column tile in the down projection (320 = 256 + 64)
    "big_gelu": W["switch"].with_(name="big_gelu", T=1000, d=320, d_ff=384, E=4, cf=1.05,
                                  noise_std=0.25),
    # the down projection splits K = d_ff in two when its tiles would not
    # fill the CUs: two fp32 partials added before the gate (ragged experts,
    # a partial column tile: 320 = 256 + 64)
    "big_splitk": W["mixtral_prefill"].with_(name="big_splitk", T=1024, d=320, d_ff=4096),
    # Zipf-skewed expert sizes (1842 .. 50 rows): the last row tile of each
    # expert takes 1, 2, 3 or 4 64-row slabs
    "big_slabs": W["mixtral_prefill"].with_(name="big_slabs", T=2048, d=256, d_ff=512, zipf_s=0.8),
    # the same with an odd number of 64-wide k stages (d = 192) and a
    # partial column tile (d_ff = 320 = 2 * 128 + 64)
    "big_slabs_odd": W["mixtral_prefill"].with_(name="big_slabs_odd", T=2500, d=192, d_ff=320,
                                                zipf_s=0.7),
    # a small batch (T <= 64) routed by the single-block routing kernel,
    # with capacity drops (C = ceil(0.5 * 48 * 2 / 8) = 6)
    "small_drops": W["mixtral_decode"].with_(name="small_drops", T=48, d=256, d_ff=384, cf=0.5),
    # weight-streaming kernel (at most 32 rows per expert, K % 128 == 0):
    # every token on both experts -> two full 16-row tiles of A per expert
    "skinny_full": W["mixtral_decode"].with_(name="skinny_full", T=32, d=256, d_ff=384, E=2),
    # ragged counts across one and two 16-row tiles, top-2 of 3
    "skinny_ragged": W["mixtral_decode"].with_(name="skinny_ragged", T=28, d=384, d_ff=256, E=3),
    # non-dual (GELU), k = 1, 40 column tiles
    "skinny_gelu": W["switch"].with_(name="skinny_gelu", T=24, d=128, d_ff=640, E=4, cf=0.0,
                                     noise_std=0.0),
    # up projection with a partial last column tile (136 = 8*16 + 8)
    "skinny_partial_n": W["mixtral_decode"].with_(name="skinny_partial_n", T=16, d=128, d_ff=136, E=4),
    # streaming kernel with three 16-row tiles (capacity 47 rows): GELU with
    # two column tiles per wave, and SwiGLU
    "skinny_mt3_gelu": W["switch"].with_(name="skinny_mt3_gelu", T=600, d=256, d_ff=384, E=16,
                                         noise_std=1.0 / 16),
    "skinny_mt3_swiglu": W["mixtral_decode"].with_(name="skinny_mt3_swiglu", T=300, d=128, d_ff=256,
                                                   E=8, k=1, cf=1.25),
    # streaming kernel with K split over four waves per block (few column
    # tiles, K >= 8192), two and three 16-row tiles
    "skinny_splitk": W["mixtral_decode"].with_(name="skinny_splitk", T=24, d=8192, d_ff=512, E=4),
    "skinny_splitk_mt3": W["mixtral_decode"].with_(name="skinny_splitk_mt3", T=300, d=8192, d_ff=128,
                                                   E=8, k=1, cf=1.25),
    # Switch gate with k = 2, 64-row SwiGLU tiles
    "switch_k2": W["mixtral_prefill"].with_(name="switch_k2", T=500, d=128, d_ff=256, E=16, k=2,
                                            gate="switch", x_rmsnorm=False),
    # router logits as a GEMM against the stacked W_r terms (more than 32
    # experts past the small-batch kernel): E = 100 (padded to 128, 384
    # stacked rows: a partial column tile), ragged T = 700 (256 + 256 + 188
    # rows), an odd number of 64-wide k stages (d = 320: no K split), top-4
    # of 100 with the Zipf router bias
    "router_gemm": W["finegrained_zipf"].with_(name="router_gemm", T=700, d=320, d_ff=256, E=100),
    # the same with E = 64 (192 stacked rows) and the K split in two
    # (d = 256), Switch gate with noise and capacity drops
    "router_gemm_split": W["switch"].with_(name="router_gemm_split", T=300, d=256, d_ff=384, E=64,
                                           noise_std=1.0 / 64),
    # router epilogue with one token per 16-lane group and 4 idle lanes in
    # each (E = 12), top-3, no capacity limit
    "grouped_e12": W["mixtral_prefill"].with_(name="grouped_e12", T=300, d=128, d_ff=192, E=12, k=3,
                                              cf=0.0),
    # k = E: every expert of every token (8-lane groups, 2 idle lanes)
    "k_equals_e": W["mixtral_prefill"].with_(name="k_equals_e", T=200, d=64, d_ff=128, E=6, k=6,
                                             cf=0.0),
    # the fused router (logits and routing in one kernel per token tile):
    # 128-token tiles (T >= 8192) with a ragged last tile (8200 = 64 * 128 +
    # 8), 128 experts padded from 100, K split in 4 (d = 512: 8 stages, 65
    # tiles), top-4 with the Zipf bias and capacity drops
    "fused_bt128": W["finegrained_zipf"].with_(name="fused_bt128", T=8200, d=512, d_ff=32, E=100),
    # 64-token tiles, 48 experts (padded to 64), K split in 8 (d = 1024, 16
    # tiles), Switch gate with noise and drops
    "fused_e48_split8": W["switch"].with_(name="fused_e48_split8", T=1000, d=1024, d_ff=64, E=48,
                                          noise_std=1.0 / 48),
    # 20 experts (padded to 32: two expert groups and two token halves per
    # block), d = 192 (3 stages, split 3 ways, one stage each), top-3
    "fused_e20": W["mixtral_prefill"].with_(name="fused_e20", T=777, d=192, d_ff=64, E=20, k=3,
                                            cf=1.1),
    # many experts on the 256-row tiles: Zipf-skewed top-4 of 64 with drops
    # (SwiGLU up with K = 320, down with K = 512 and a partial column tile,
    # 320 = 256 + 64), and GELU top-1 of 40 without capacity
    "adapt_zipf": W["finegrained_zipf"].with_(name="adapt_zipf", T=4096, d=320, d_ff=512, E=64),
    "adapt_gelu": W["switch"].with_(name="adapt_gelu", T=12000, d=192, d_ff=256, E=40, cf=0.0,
                                    noise_std=1.0 / 40),
    # 9 experts (padded to 16: the grouped epilogue, 16 lanes per token), one
    # 64-token tile plus one token
    "fused_e9": W["mixtral_prefill"].with_(name="fused_e9", T=65, d=128, d_ff=64, E=9, k=2),
}


# cases whose capacity is known to drop assignments (the drop path is exercised)
EXPECT_DROPS = {"switch_small", "zipf_small", "relu_bf16", "big_gelu", "skinny_mt3_gelu",
                "small_drops", "fused_bt128", "fused_e48_split8", "adapt_zipf"}


def _check_all(w, wt, tk, got=None):
    ref = H.reference(w, wt, tk)
    if got is None:
        got = H.run_forward(w, H.device_weights(w, wt), H.device_tokens(w, tk))
    H.assert_routing_exact(w, got, ref)
    H.assert_gates_close(got, ref)
    H.assert_stats_close(w, got, ref)
    H.assert_y_close(w, H.y_float(got["y"]), ref["y"])
    full = (ref["row_of_slot"] < 0).all(axis=1)
    assert (H.y_float(got["y"])[full] == 0).all()
    return ref, got


@pytest.mark.parametrize("name", sorted(SMALL))
def test_forward_matches_oracle(name):
    w = SMALL[name]
    print(f"[parity] {name} T={w.T} d={w.d} d_ff={w.d_ff} E={w.E} k={w.k}", flush=True)
    wt, tk = H.prepare(w)
    ref, got = _check_all(w, wt, tk)
    if name in EXPECT_DROPS:
        assert ref["dropped"].sum() > 0


@pytest.mark.parametrize("name", ["mixtral_small", "zipf_small", "tiny", "switch_small",
                                  "big_splitk", "decode_small", "small_drops", "router_gemm"])
def test_staged_entry_points(name):
    """route, dispatch, expert_ffn and combine called one by one: x_perm is
    the exact gather, y_perm matches the oracle's per-row expert outputs,
    and the final outputs equal moe_forward's bit for bit."""
    w = SMALL[name]
    wt, tk = H.prepare(w)
    dw, dt = H.device_weights(w, wt), H.device_tokens(w, tk)
    st = H.run_staged(w, dw, dt)
    fw = H.run_forward(w, dw, dt)
    for key in fw:
        assert torch.equal(st[key], fw[key]), key
    ref = H.reference(w, wt, tk)
    n = int(ref["offsets"][-1])
    xs = tk["x"][ref["token_of_row"][:n]]
    xp = st["x_perm"][:n]
    xp = xp.view(torch.int16).numpy().view(np.uint16) if w.dtype == "bf16" else xp.numpy()
    assert np.array_equal(xp, xs)
    import oracle
    e_of_row = np.repeat(np.arange(w.E), ref["kept"])
    yp_ref = oracle.expert_ffn(ref["token_of_row"][:n], e_of_row, synth.widen(tk["x"]),
                               synth.widen(wt["W1"]),
                               None if wt["W3"] is None else synth.widen(wt["W3"]),
                               synth.widen(wt["W2"]), w.act)
    H.assert_y_close(w, st["y_perm"][:n].numpy(), yp_ref, "y_perm")


def test_deterministic_and_stream_independent():
    w = SMALL["zipf_small"]
    wt, tk = H.prepare(w)
    dw, dt = H.device_weights(w, wt), H.device_tokens(w, tk)
    a = H.run_forward(w, dw, dt)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = H.run_forward(w, dw, dt, stream=s)
    c = H.run_forward(w, dw, dt)
    for key in a:
        assert torch.equal(a[key], b[key]) and torch.equal(a[key], c[key]), key


# ---------------------------------------------------------------- edge cases

def _edge(**kw):
    base = dict(name="edge", T=96, d=64, d_ff=128, E=8, k=2, gate="renorm", cf=0.0,
                act="swiglu", dtype="bf16")
    base.update(kw)
    return synth.Workload(**base)


@pytest.mark.parametrize("w", [
    _edge(name="T1", T=1),
    _edge(name="T1_f32", T=1, dtype="f32", d=5, d_ff=7),
    _edge(name="dense_E1", E=1, k=1),
    _edge(name="k_eq_E_renorm", E=4, k=4),
    _edge(name="k_eq_E_switch", E=4, k=4, gate="switch"),
    _edge(name="min_width", d=8, d_ff=8, T=40),
    _edge(name="cf_tiny", cf=1e-6, T=80),
    _edge(name="E128_k8", E=128, k=8, T=300, cf=2.0, act="gelu"),
    _edge(name="gelu_f32", dtype="f32", act="gelu", T=50, d=20, d_ff=30, E=5, k=2, cf=1.0),
], ids=lambda w: w.name)
def test_edge_shapes(w):
    print(f"[edge] {w.name}", flush=True)
    wt, tk = H.prepare(w)
    _check_all(w, wt, tk)


def test_all_tokens_on_one_expert():
    """A dominant router bias sends every token's first choice to expert 0;
    with cf = 1 only C of them fit, the rest are dropped in token order."""
    w = _edge(name="collapse", T=256, cf=1.0, k=1, E=8, gate="switch")
    wt = synth.make_weights(w)
    wt["bias"] = np.zeros(w.E, np.float32)
    wt["bias"][0] = 40.0
    wt, tk = H.prepare(w, weights=wt)
    ref, got = _check_all(w, wt, tk)
    assert ref["routed"][0] == w.T and ref["kept"][0] == 32
    assert ref["dropped"].sum() == w.T - 32
    np.testing.assert_allclose(got["stats"][2 * w.E].item(), w.E, rtol=1e-5)


def test_empty_experts():
    w = _edge(name="empty", T=300, E=16, k=2)
    wt = synth.make_weights(w)
    wt["bias"] = np.where(np.arange(w.E) % 2 == 1, -60.0, 0.0).astype(np.float32)
    wt, tk = H.prepare(w, weights=wt)
    ref, got = _check_all(w, wt, tk)
    assert (ref["routed"][1::2] == 0).all()


def test_exact_ties_go_to_lower_index():
    """Duplicated router rows give bit-identical logits on both sides; the
    lower expert index must come first everywhere."""
    w = _edge(name="ties", T=400, E=8, k=3, cf=1.5)
    wt = synth.make_weights(w)
    wt["Wr"][5] = wt["Wr"][2]
    wt, tk = H.prepare(w, weights=wt, ignore=(5,))
    ref, got = _check_all(w, wt, tk)
    idx = ref["idx"]
    both = (idx == 2).any(1) & (idx == 5).any(1)
    assert both.sum() > 10
    pos2 = np.argmax(idx == 2, axis=1)
    pos5 = np.argmax(idx == 5, axis=1)
    assert (pos2[both] + 1 == pos5[both]).all()


def test_workspace_too_small_raises_before_launch():
    w = SMALL["tiny"]
    desc = B.desc_for(w)
    ws = torch.empty(B.moe_workspace_size(desc) - 1, dtype=torch.uint8, device="cuda")
    wt, tk = H.prepare(w)
    dw, dt = H.device_weights(w, wt), H.device_tokens(w, tk)
    out = B.alloc_outputs(desc)
    with pytest.raises(B.MoeError) as ei:
        B.moe_forward(desc, dt["x"], dw["Wr"], None, None, dw["W1"], None, dw["W2"], out["y"], ws)
    assert ei.value.code == -4


@pytest.mark.parametrize("T,E,k,cf", [(100, 5, 2, 0.5), (300, 6, 2, 0.8), (3000, 16, 3, 1.0),
                                      (12000, 16, 3, 1.0), (9000, 128, 4, 1.25)])
def test_dispatch_drops_invalid_indices(T, E, k, cf):
    """moe_dispatch on caller indices that include entries outside [0, E)
    and experts repeated within a token: those entries count nowhere and
    come back dropped; the valid ones are ranked in token order against the
    capacity as usual (checked against a plain sequential fill).  The larger
    shapes span several dispatch chunks, of 256 and of 1024 assignments; with
    k = 3 some tokens begin in one chunk and end in the next."""
    rng = np.random.default_rng(7)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    bad = rng.random((T, k)) < 0.1
    idx[bad] = rng.choice([-1, E, E + 5, -7], size=int(bad.sum()))
    rep = np.nonzero(rng.random(T) < 0.1)[0]
    idx[rep, k - 1] = idx[rep, 0]                      # a repeat of slot 0's expert
    desc = B.make_desc(T, 64, 64, E, k, gate="renorm", act="relu", dtype="bf16", cf=cf)
    C = B.moe_capacity(desc)
    # expected: assignments in token-major order, an invalid one skipped
    routed = np.zeros(E, np.int64)
    rank = np.full((T, k), -1, np.int64)
    for t in range(T):
        for s in range(k):
            e = int(idx[t, s])
            if e < 0 or e >= E or e in idx[t, :s]:
                continue
            rank[t, s] = routed[e]
            routed[e] += 1
    kept = routed if C is None else np.minimum(routed, C)
    offs = np.concatenate([[0], np.cumsum(kept)])
    keep = (rank >= 0) & ((rank < C) if C is not None else True)
    rows_exp = np.where(keep, offs[np.where(rank >= 0, idx, 0)] + rank, -1)
    x = torch.randn((T, 64), device="cuda").to(torch.bfloat16)
    i32 = dict(dtype=torch.int32, device="cuda")
    out = dict(routed=torch.empty(E, **i32), kept=torch.empty(E, **i32),
               offsets=torch.empty(E + 1, **i32), rows=torch.empty((T, k), **i32),
               tok=torch.empty(T * k, **i32),
               dropped=torch.empty((T, k), dtype=torch.uint8, device="cuda"),
               x_perm=torch.empty((T * k, 64), dtype=torch.bfloat16, device="cuda"))
    B.moe_dispatch(desc, x, torch.from_numpy(idx).cuda(), out["routed"], out["kept"],
                   out["offsets"], out["rows"], out["tok"], out["dropped"], out["x_perm"],
                   B.workspace(desc))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out["routed"].cpu().numpy(), routed)
    np.testing.assert_array_equal(out["kept"].cpu().numpy(), kept)
    np.testing.assert_array_equal(out["offsets"].cpu().numpy(), offs)
    np.testing.assert_array_equal(out["rows"].cpu().numpy(), rows_exp)
    np.testing.assert_array_equal(out["dropped"].cpu().numpy(), (rows_exp < 0).astype(np.uint8))
    tok = out["tok"].cpu().numpy()
    n = int(offs[-1])
    r_t, r_s = np.nonzero(rows_exp >= 0)
    exp_tok = np.full(T * k, -1, np.int64)
    exp_tok[rows_exp[r_t, r_s]] = r_t
    np.testing.assert_array_equal(tok, exp_tok)
    np.testing.assert_array_equal(out["x_perm"][:n].view(torch.int16).cpu().numpy(),
                                  x[torch.from_numpy(tok[:n]).long().cuda()].view(torch.int16).cpu().numpy())
