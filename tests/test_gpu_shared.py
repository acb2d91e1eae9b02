"""GPU parity of the shared experts and the block residual against the CPU
oracle, through the C ABI (moe_forward_shared and the staged
moe_shared_ffn / moe_combine_shared).

Section "Total versus active parameters" of the page names DeepSeek-V3's
layer (many small routed experts plus shared experts every token visits);
the Implementation section's block adds the layer output to its hidden
state.  The S shared experts run as one dense layer (up with N = S*d_ff,
down with K = S*d_ff against a repacked W2).  Cases cover every GEMM path
that layer can take (64/128-row tiles, the 256-row kernel with and without
the dual accumulator, a K split of the down projection, the
weight-streaming kernel with two and three 16-row tiles, the fp32
kernels), the W2 repack (S > 1, 16- and 4-byte rows), the combine's vector
and scalar forms, one to three shared experts, residual only, shared
experts only, and capacity drops (a dropped token keeps its residual and
its shared experts).
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_mixture_experts_03_amd import binding as B
from sparse_mixture_experts_03_amd import synth

import harness as H

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
SHARED = {
    # 128-row tiles (K = 520 not a multiple of 64), one shared expert
    "sh_mixtral_small": W["mixtral_prefill"].with_(name="sh_mixtral_small", T=700, d=520, d_ff=1000,
                                                   n_shared=1, residual=True),
    # Zipf-skewed top-4 of 32 with capacity drops, two shared experts
    "sh_zipf_small": W["finegrained_zipf"].with_(name="sh_zipf_small", T=1500, d=264, d_ff=200, E=32,
                                                 n_shared=2, residual=True),
    # 256-row kernel, SwiGLU; the shared down projection splits K in two
    # (its halves are added in the combine)
    "sh_big_splitk": W["mixtral_prefill"].with_(name="sh_big_splitk", T=1024, d=320, d_ff=4096,
                                                n_shared=1, residual=True),
    # 256-row kernel without the dual accumulator (GELU), half-width pieces,
    # three shared experts, drops
    "sh_big_gelu": W["switch"].with_(name="sh_big_gelu", T=1000, d=320, d_ff=384, E=4, cf=1.05,
                                     noise_std=0.25, n_shared=3, residual=True),
    # weight-streaming kernel, two 16-row tiles (T = 32), single-block routing
    "sh_decode_small": W["mixtral_decode"].with_(name="sh_decode_small", d=512, d_ff=768,
                                                 n_shared=2, residual=True),
    # weight-streaming kernel, three 16-row tiles (T = 40), GELU, drops
    "sh_skinny_mt3": W["switch"].with_(name="sh_skinny_mt3", T=40, d=256, d_ff=384, E=4, cf=0.8,
                                       noise_std=0.25, n_shared=1, residual=True),
    # fp32 kernels, vector combine
    "sh_tiny_f32": W["tiny"].with_(name="sh_tiny_f32", n_shared=2, residual=True),
    # fp32, width not a multiple of 4: the scalar combine; W2 rows of 88
    # bytes (the 4-byte repack copy)
    "sh_f32_scalar": W["tiny"].with_(name="sh_f32_scalar", T=50, d=30, d_ff=22, E=5, cf=1.0,
                                     act="gelu", n_shared=2, residual=True),
    # the residual alone, and shared experts without a residual
    "sh_residual_only": W["mixtral_prefill"].with_(name="sh_residual_only", T=300, d=128, d_ff=192,
                                                   cf=0.8, residual=True),
    "sh_no_residual": W["mixtral_prefill"].with_(name="sh_no_residual", T=300, d=128, d_ff=192,
                                                 E=6, k=3, n_shared=2),
}

EXPECT_DROPS = {"sh_zipf_small", "sh_big_gelu", "sh_skinny_mt3", "sh_residual_only"}


def _shared_sum_ref(w, wt, tk):
    """The oracle's shared experts on every token (each output row fp32),
    summed over the experts in float64."""
    T, S = w.T, w.n_shared
    W3 = None if wt["Ws3"] is None else synth.widen(wt["Ws3"])
    rows = oracle.expert_ffn(np.tile(np.arange(T), S), np.repeat(np.arange(S), T),
                             synth.widen(tk["x"]), synth.widen(wt["Ws1"]), W3,
                             synth.widen(wt["Ws2"]), w.act)
    return rows.astype(np.float64).reshape(S, T, w.d).sum(axis=0)


@pytest.mark.parametrize("name", sorted(SHARED))
def test_forward_shared_matches_oracle(name):
    w = SHARED[name]
    print(f"[shared] {name} T={w.T} d={w.d} d_ff={w.d_ff} E={w.E} k={w.k} S={w.n_shared} "
          f"residual={w.residual}", flush=True)
    wt, tk = H.prepare(w)
    ref = H.reference(w, wt, tk)
    got = H.run_forward(w, H.device_weights(w, wt), H.device_tokens(w, tk))
    H.assert_routing_exact(w, got, ref)
    H.assert_gates_close(got, ref)
    H.assert_stats_close(w, got, ref)
    y = H.y_float(got["y"])
    H.assert_y_close(w, y, ref["y"])
    full = (ref["row_of_slot"] < 0).all(axis=1)
    if name in EXPECT_DROPS:
        assert ref["dropped"].sum() > 0
    if full.any():
        # tokens dropped from every routed expert: residual + shared only,
        # not zero
        H.assert_y_close(w, y[full], ref["y"][full], "y of fully dropped tokens")
        assert (np.abs(ref["y"][full]) > 0).any()


@pytest.mark.parametrize("name", ["sh_zipf_small", "sh_big_splitk", "sh_decode_small",
                                  "sh_tiny_f32", "sh_residual_only"])
def test_staged_shared_entry_points(name):
    """route, dispatch, expert_ffn, shared_ffn and combine_shared one by one:
    the shared experts' summed output matches the oracle's, and every output
    equals moe_forward_shared's bit for bit."""
    w = SHARED[name]
    wt, tk = H.prepare(w)
    dw, dt = H.device_weights(w, wt), H.device_tokens(w, tk)
    st = H.run_staged(w, dw, dt)
    fw = H.run_forward(w, dw, dt)
    for key in fw:
        assert torch.equal(st[key], fw[key]), key
    if w.n_shared:
        H.assert_y_close(w, st["y_shared"].numpy(), _shared_sum_ref(w, wt, tk), "y_shared")


def test_no_shared_no_residual_equals_forward():
    """moe_forward_shared with S = 0 and no residual is moe_forward, bit for bit."""
    w = W["finegrained_zipf"].with_(name="plain", T=1500, d=264, d_ff=200, E=32)
    wt, tk = H.prepare(w)
    dw, dt = H.device_weights(w, wt), H.device_tokens(w, tk)
    a = H.run_forward(w, dw, dt)
    b = H.run_forward(w, dw, dt, force_shared=True)
    for key in a:
        assert torch.equal(a[key], b[key]), key


def test_forward_shared_deterministic():
    w = SHARED["sh_big_gelu"]
    wt, tk = H.prepare(w)
    dw, dt = H.device_weights(w, wt), H.device_tokens(w, tk)
    a = H.run_forward(w, dw, dt)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = H.run_forward(w, dw, dt, stream=s)
    for key in a:
        assert torch.equal(a[key], b[key]), key


def test_shared_workspace_too_small_raises_before_launch():
    w = SHARED["sh_tiny_f32"]
    desc = B.desc_for(w)
    wt, tk = H.prepare(w)
    dw, dt = H.device_weights(w, wt), H.device_tokens(w, tk)
    need = B.moe_workspace_size_shared(desc, H.shared_arg(w, desc, dw, dt))
    assert need > B.moe_workspace_size(desc)
    ws = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    out = B.alloc_outputs(desc)
    with pytest.raises(B.MoeError) as ei:
        B.moe_forward_shared(desc, H.shared_arg(w, desc, dw, dt), dt["x"], dw["Wr"], None, None,
                             dw["W1"], None, dw["W2"], out["y"], ws)
    assert ei.value.code == -4
