"""GPU parity of the layer's backward (moe_backward) against the oracle's
backward, through the C ABI.

The GPU forward's routing (bit-exact with the oracle's, checked first) is
held fixed; dy is a seeded bf16 tensor; the loss adds the load-balancing
and z terms with weights 0.3 and 0.05.  Every gradient (dx, dW_r, dbias,
dW1, dW3, dW2) must be within 2e-2 * max|ref| (bf16 operands, fp32
accumulation).  Cases: several row and column tiles with ragged tails,
capacity drops, both gate conventions, SwiGLU / GELU / ReLU, an expert
without rows, a decode-sized batch (the streaming kernels), and the
256-row tiles with a K split in the recomputed down projection (and
those tiles for every GEMM of a ReLU layer in b_big_relu); and the
full-size Mixtral prefill layer (sampled dx against the oracle, exact
scaling in dy, reproducibility).  fp32 layers (the tiny layer and two
more) are held to 1e-5 of the largest reference gradient.
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
BWD = {
    "b_mixtral_small": W["mixtral_prefill"].with_(name="b_mixtral_small", T=300, d=200, d_ff=328),
    "b_zipf_drops": W["finegrained_zipf"].with_(name="b_zipf_drops", T=500, d=136, d_ff=96, E=16),
    "b_switch_gelu": W["switch"].with_(name="b_switch_gelu", T=400, d=128, d_ff=192, E=8,
                                       noise_std=0.1),
    "b_relu_k3": W["tiny"].with_(name="b_relu_k3", T=160, d=64, d_ff=136, E=6, k=3, cf=0.8,
                                 dtype="bf16"),
    "b_decode": W["mixtral_decode"].with_(name="b_decode", d=256, d_ff=384),
    "b_big_splitk": W["mixtral_prefill"].with_(name="b_big_splitk", T=1024, d=320, d_ff=4096, E=4),
    # E >= 16, T a multiple of 8 and d of 64: the router's logits and dW_r
    # on matrix cores; capacity drops
    "b_router_mfma": W["finegrained_zipf"].with_(name="b_router_mfma", T=256, d=192, d_ff=64, E=32),
    # 256-row tiles for every GEMM of a ReLU layer
    "b_big_relu": W["mixtral_prefill"].with_(name="b_big_relu", T=512, d=128, d_ff=264, E=2, k=1,
                                             act="relu"),
    # fp32 layers: the tiny layer as specified, SwiGLU with capacity drops,
    # GELU with the Switch gate, noise and 40 experts (the blocked logits)
    "b_tiny_f32": W["tiny"],
    "b_f32_swiglu_drops": W["tiny"].with_(name="b_f32_swiglu_drops", T=200, d=48, d_ff=80, E=6,
                                          act="swiglu", cf=0.8),
    "b_f32_switch_gelu": W["tiny"].with_(name="b_f32_switch_gelu", T=150, d=40, d_ff=72, E=40, k=1,
                                         gate="switch", act="gelu", noise_std=0.05),
}
# fp32 layers: fp32 operands and accumulation against the oracle's float64
# (sums of at most a few hundred terms): within 1e-5 of the largest
# reference gradient, the bar for the fp32 layer's output
TOL = {"bf16": 2e-2, "f32": 1e-5}


def _run(w, wt=None, alpha_aux=0.3, alpha_z=0.05):
    wt, tk = H.prepare(w, weights=wt)
    dw, dt = H.device_weights(w, wt), H.device_tokens(w, tk)
    desc = B.desc_for(w)
    fwd = B.alloc_outputs(desc)
    ws = B.workspace(desc)
    B.moe_forward(desc, dt["x"], dw["Wr"], dw["bias"], dt["noise"], dw["W1"], dw["W3"], dw["W2"],
                  fwd["y"], ws, **{k: fwd[k] for k in fwd if k != "y"})
    dy_f = np.random.default_rng(9).standard_normal((w.T, w.d)).astype(np.float32)
    dy_bits = synth.to_bf16(dy_f) if w.dtype == "bf16" else dy_f
    dy = B.to_device(dy_bits, w.dtype)
    grads = B.alloc_grads(desc, bias=dw["bias"] is not None)
    bws = B.backward_workspace(desc)
    B.moe_backward(desc, dt["x"], dw["Wr"], dw["bias"], dt["noise"], dw["W1"], dw["W3"], dw["W2"],
                   fwd, dy, grads, bws, alpha_aux, alpha_z)
    torch.cuda.synchronize()
    got = {k: (None if v is None else v.cpu().numpy()) for k, v in grads.items()}
    fw = {k: v.cpu() for k, v in fwd.items()}
    ref_fw = H.reference(w, wt, tk, tokens=np.zeros(0, np.int64))
    H.assert_routing_exact(w, fw, ref_fw)
    wid = lambda a: None if a is None else synth.widen(a)
    ref = oracle.backward(synth.widen(tk["x"]), wt["Wr"], wid(wt["W1"]), wid(wt["W3"]), wid(wt["W2"]),
                          w.k, w.gate, w.cf, w.act, synth.widen(dy_bits), alpha_aux, alpha_z,
                          wt["bias"], tk["noise"], rows=ref_fw["row_of_slot"])
    return got, ref, ref_fw


def _check(got, ref, tol=2e-2):
    for key, rkey in (("dx", "dx"), ("dW_r", "dWr"), ("dbias", "dbias"), ("dW1", "dW1"),
                      ("dW3", "dW3"), ("dW2", "dW2")):
        if ref[rkey] is None:
            assert got[key] is None, key
            continue
        g, r = got[key], ref[rkey]
        assert np.isfinite(g).all(), key
        scale = float(np.abs(r).max())
        err = float(np.abs(g.astype(np.float64) - r).max())
        print(f"    {key}: max|err| / max|ref| = {err / max(scale, 1e-300):.2e}", flush=True)
        assert err <= tol * scale, f"{key}: max|err| {err:.3e} > {tol} * {scale:.3e}"


@pytest.mark.parametrize("name", sorted(BWD))
def test_backward_matches_oracle(name):
    w = BWD[name]
    print(f"[bwd] {name} T={w.T} d={w.d} d_ff={w.d_ff} E={w.E} k={w.k} act={w.act} gate={w.gate}",
          flush=True)
    got, ref, ref_fw = _run(w)
    _check(got, ref, TOL[w.dtype])
    if name in ("b_zipf_drops", "b_f32_swiglu_drops"):
        assert ref_fw["dropped"].sum() > 0


def test_backward_expert_without_rows():
    """An expert no token reaches gets zero weight gradients."""
    w = W["mixtral_prefill"].with_(name="b_empty", T=200, d=64, d_ff=128, E=6, x_rmsnorm=False)
    wt = synth.make_weights(w)
    wt["bias"] = np.zeros(w.E, np.float32)
    wt["bias"][5] = -60.0
    got, ref, ref_fw = _run(w, wt=wt)
    assert ref_fw["routed"][5] == 0
    _check(got, ref)
    assert (got["dW1"][5] == 0).all() and (got["dW2"][5] == 0).all() and (got["dW3"][5] == 0).all()


def test_backward_deterministic():
    w = BWD["b_zipf_drops"]
    a, _, _ = _run(w)
    b, _, _ = _run(w)
    for key in a:
        if a[key] is not None:
            assert np.array_equal(a[key], b[key]), key


def test_full_size_backward_mixtral():
    """The Mixtral prefill layer at full size (T=4096, d=4096, d_ff=14336,
    E=8, top-2, no capacity limit), in the launch configuration of
    `bench.py --backward`, with the load-balancing and z weights at 0: then
    each token's dx depends on that token alone, so the oracle's backward on
    8 sampled tokens (their own routing, all kept) gives their dx exactly.
    Every gradient of dy scaled by 2 must be exactly twice that of dy (a
    power-of-two scale passes every bf16 and fp32 step unchanged), and the
    call must repeat bit for bit.  The busiest expert's weight gradients are
    compared on 16 hidden units (rows of dW1, dW3, columns of dW2)."""
    w = W["mixtral_prefill"]
    print(f"[bwd] full size {w.name}", flush=True)
    wt, tk = H.prepare(w)
    dw, dt = H.device_weights(w, wt), H.device_tokens(w, tk)
    desc = B.desc_for(w)
    fwd = B.alloc_outputs(desc)
    B.moe_forward(desc, dt["x"], dw["Wr"], dw["bias"], dt["noise"], dw["W1"], dw["W3"], dw["W2"],
                  fwd["y"], B.workspace(desc), **{k: fwd[k] for k in fwd if k != "y"})
    dy_bits = synth.to_bf16(np.random.default_rng(9).standard_normal((w.T, w.d)).astype(np.float32))
    bws = B.backward_workspace(desc)
    out = []
    for scale in (1.0, 2.0, 1.0):
        grads = B.alloc_grads(desc, bias=False)
        dy = B.to_device(synth.to_bf16(synth.widen(dy_bits) * scale), "bf16")
        B.moe_backward(desc, dt["x"], dw["Wr"], None, dt["noise"], dw["W1"], dw["W3"], dw["W2"],
                       fwd, dy, grads, bws, 0.0, 0.0)
        torch.cuda.synchronize()
        out.append({k: v.cpu().numpy() for k, v in grads.items() if v is not None})
    for key in out[0]:
        assert np.isfinite(out[0][key]).all(), key
        assert np.array_equal(out[0][key], out[2][key]), f"{key}: not reproducible"
        assert np.array_equal(out[1][key], 2 * out[0][key]), f"{key}: dy * 2 does not double it"
    # dx of sampled tokens against the oracle on those tokens alone
    sample = H.sample_tokens(w.T, 8, seed=3)
    ref_fw = H.reference(w, wt, tk, tokens=np.zeros(0, np.int64))
    H.assert_routing_exact(w, {k: v.cpu() for k, v in fwd.items()}, ref_fw)
    rows = ref_fw["row_of_slot"][sample]
    assert (rows >= 0).all()
    ref = oracle.backward(synth.widen(tk["x"][sample]), wt["Wr"], synth.widen(wt["W1"]),
                          synth.widen(wt["W3"]), synth.widen(wt["W2"]), w.k, w.gate, w.cf, w.act,
                          synth.widen(dy_bits[sample]), 0.0, 0.0, None, None, rows=rows)
    g, r = out[0]["dx"][sample], ref["dx"]
    scale = float(np.abs(r).max())
    err = float(np.abs(g.astype(np.float64) - r).max())
    assert err <= 2e-2 * scale, f"dx: max|err| {err:.3e} > 2e-2 * {scale:.3e}"
    # weight gradients of the busiest expert: 16 rows of dW1 and dW3 and 16
    # columns of dW2 (hidden units spread over d_ff, the first and the last
    # included) against the oracle's one-expert gradients over all its rows
    e = int(np.argmax(ref_fw["kept"]))
    lo, hi = int(ref_fw["offsets"][e]), int(ref_fw["offsets"][e + 1])
    tok = ref_fw["token_of_row"][lo:hi]
    t_s = np.nonzero((ref_fw["idx"] == e) & (ref_fw["row_of_slot"] >= 0))
    gate = np.zeros(hi - lo)
    gate[ref_fw["row_of_slot"][t_s] - lo] = ref_fw["gates"][t_s]
    fsel = np.unique(np.concatenate([[0, w.d_ff - 1],
                                     np.random.default_rng(4).choice(w.d_ff, 14, replace=False)]))
    print(f"[bwd] oracle weight gradients of expert {e} ({hi - lo} rows, {len(fsel)} hidden units)", flush=True)
    wg = oracle.expert_wgrad_sel(synth.widen(tk["x"]), synth.widen(wt["W1"][e]), synth.widen(wt["W3"][e]),
                                 synth.widen(wt["W2"][e]), tok, gate, synth.widen(dy_bits), w.act, fsel)
    for key, got_k, ref_k in (("dW1", out[0]["dW1"][e][fsel], wg["dW1"]),
                              ("dW3", out[0]["dW3"][e][fsel], wg["dW3"]),
                              ("dW2", out[0]["dW2"][e][:, fsel], wg["dW2"])):
        scale = float(np.abs(ref_k).max())
        err = float(np.abs(got_k.astype(np.float64) - ref_k).max())
        assert err <= 2e-2 * scale, f"{key}[{e}]: max|err| {err:.3e} > 2e-2 * {scale:.3e}"
