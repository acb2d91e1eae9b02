"""GPU tests of the streaming tile layout (moe_pack_stream) and of the layer
on packed expert weights (moe_forward_packed, moe_expert_ffn_packed),
through the C ABI.

The layout is a permutation of 16-byte units, defined in include/moe.h:
the packed bytes must equal that definition, written in the test harness
once with loops over (row, column) and once as a reshape / transpose (the
two pinned to each other on the CPU).  The streaming kernels multiply the
same values in the same order on packed as on row-major weights, so
moe_forward_packed must equal moe_forward (bf16 weights) or
moe_forward_fp8 (e4m3 codes) bit for bit, and match the oracle at the
bf16 tolerance.  Cases: SwiGLU / GELU / ReLU, two and three 16-row tiles,
K split over four waves, capacity drops with the Switch gate, T = 1, the
staged entry point, and the full-size decode and Switch layers.
"""
import numpy as np
import pytest
import torch

from sparse_mixture_experts_03_amd import binding as B
from sparse_mixture_experts_03_amd import synth

import harness as H

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _random(shape, dtype):
    g = torch.Generator().manual_seed(7)
    if dtype == torch.uint8:
        return torch.randint(0, 256, shape, dtype=torch.uint8, generator=g)
    return torch.randint(-32768, 32768, shape, dtype=torch.int32, generator=g).to(torch.int16).view(torch.bfloat16)


def _host_bits(t):
    return t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.numpy()


@pytest.mark.parametrize("shape", [(16, 128), (48, 384), (3, 32, 256), (2, 64, 1024)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.uint8], ids=["bf16", "e4m3"])
def test_pack_stream_layout(shape, dtype):
    print(f"[packed] layout {shape} {dtype}", flush=True)
    Wt = _random(shape, dtype)
    dev = Wt.cuda()
    out = torch.empty_like(dev)
    B.moe_pack_stream(dev, out)
    torch.cuda.synchronize()
    got = _host_bits(out.cpu()).reshape(-1, shape[-1])
    want = H.pack_reshape(_host_bits(Wt).reshape(-1, shape[-1]))
    np.testing.assert_array_equal(got, want)
    if Wt.numel() <= 16 * 128 * 3:
        np.testing.assert_array_equal(got, H.pack_loops(_host_bits(Wt).reshape(-1, shape[-1])))


CASES = {
    # decode shape: two 16-row tiles per expert, top-2 of 8, SwiGLU
    "p_decode": W["mixtral_decode"].with_(name="p_decode", d=512, d_ff=768),
    # the up projection's K (= d = 8192) split over four waves
    "p_splitk": W["mixtral_decode"].with_(name="p_splitk", T=24, d=8192, d_ff=512, E=4),
    # three 16-row tiles (up to 40 rows per expert), GELU, 128 weight rows per wave
    "p_gelu_mt3": W["switch"].with_(name="p_gelu_mt3", T=40, d=256, d_ff=384, E=4, cf=0.0, noise_std=0.25),
    # Switch gate, k = 1, capacity 38 with drops, 16 experts
    "p_switch": W["switch"].with_(name="p_switch", T=600, d=256, d_ff=384, E=16, cf=1.0),
    # ReLU, top-3 of 6, ragged counts
    "p_relu": W["tiny"].with_(name="p_relu", T=28, d=384, d_ff=256, E=6, k=3, dtype="bf16"),
    # a single token
    "p_T1": W["mixtral_decode"].with_(name="p_T1", T=1, d=256, d_ff=512),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_packed_bf16_equals_row_major(name):
    w = CASES[name]
    print(f"[packed] bf16 {name} T={w.T} d={w.d} d_ff={w.d_ff} E={w.E} k={w.k} act={w.act}", flush=True)
    wt, tk = H.prepare(w)
    dw, dt = H.device_weights(w, wt), H.device_tokens(w, tk)
    got = H.run_forward_packed(w, dw, dt)
    H.assert_outputs_identical(got, H.run_forward(w, dw, dt))
    ref = H.reference(w, wt, tk)
    H.assert_routing_exact(w, got, ref)
    H.assert_stats_close(w, got, ref)
    H.assert_y_close(w, H.y_float(got["y"]), ref["y"])
    if name == "p_switch":
        assert ref["dropped"].sum() > 0


@pytest.mark.parametrize("name", sorted(CASES))
def test_packed_e4m3_equals_row_major(name):
    w = CASES[name]
    print(f"[packed] e4m3 {name} T={w.T} d={w.d} d_ff={w.d_ff} E={w.E} k={w.k} act={w.act}", flush=True)
    wt, tk = H.prepare(w)
    dw, dt = H.device_weights(w, wt), H.device_tokens(w, tk)
    f8 = H.device_fp8(dw)
    got = H.run_forward_packed(w, dw, dt, f8)
    H.assert_outputs_identical(got, H.run_forward_fp8(w, dw, dt, f8))
    qref = H.quantize_ref(wt)
    H.assert_fp8_equal(f8, qref)
    ref = H.reference_fp8(w, wt, tk, qref)
    H.assert_routing_exact(w, got, ref)
    H.assert_y_close(w, H.y_float(got["y"]), ref["y"])


@pytest.mark.parametrize("fmt", ["bf16", "e4m3"])
def test_staged_packed_equals_row_major(fmt):
    """moe_expert_ffn_packed on the permuted rows of moe_dispatch equals the
    row-major entry point (moe_expert_ffn, or moe_expert_ffn_fp8) bit for bit."""
    w = CASES["p_gelu_mt3"]
    wt, tk = H.prepare(w)
    dw, dt = H.device_weights(w, wt), H.device_tokens(w, tk)
    desc = B.desc_for(w)
    out = B.alloc_outputs(desc)
    ws = B.workspace(desc)
    B.moe_route(desc, dt["x"], dw["Wr"], dw["bias"], dt["noise"], out["topk_idx"], out["gates"],
                out["stats"], ws)
    x_perm = torch.zeros((w.T * w.k, w.d), dtype=torch.bfloat16, device="cuda")
    B.moe_dispatch(desc, dt["x"], out["topk_idx"], out["routed_counts"], out["kept_counts"], out["offsets"],
                   out["row_of_slot"], out["token_of_row"], out["dropped"], x_perm, ws)
    y_row = torch.zeros((w.T * w.k, w.d), dtype=torch.float32, device="cuda")
    y_pk = torch.zeros_like(y_row)
    f8 = H.device_fp8(dw) if fmt == "e4m3" else None
    tensors, pk = H.device_packed(w, desc, dw, f8)
    if f8 is None:
        B.moe_expert_ffn(desc, x_perm, out["offsets"], dw["W1"], dw["W3"], dw["W2"], y_row, ws)
    else:
        fp8 = B.make_fp8(desc, f8["q1"], f8["q3"], f8["q2"], f8["s1"], f8["s3"], f8["s2"])
        B.moe_expert_ffn_fp8(desc, x_perm, out["offsets"], fp8, y_row, ws)
    B.moe_expert_ffn_packed(desc, x_perm, out["offsets"], pk, y_pk, ws)
    torch.cuda.synchronize()
    n = int(out["offsets"][-1].item())
    assert n > 0
    assert torch.equal(y_pk[:n].view(torch.int32), y_row[:n].view(torch.int32))
    del tensors


def test_full_size_packed_decode():
    """The Mixtral-shape decode layer at full size (T = 32, d = 4096, d_ff =
    14336, 8 experts): packed bf16 weights give moe_forward's outputs bit for
    bit, packed e4m3 codes moe_forward_fp8's (both of which the full-size
    tests compare with the oracle)."""
    w = W["mixtral_decode"]
    print("[packed] mixtral_decode: generating inputs", flush=True)
    wt, tk = H.prepare(w)
    dw, dt = H.device_weights(w, wt), H.device_tokens(w, tk)
    del wt
    print("[packed] mixtral_decode: bf16", flush=True)
    H.assert_outputs_identical(H.run_forward_packed(w, dw, dt), H.run_forward(w, dw, dt))
    print("[packed] mixtral_decode: e4m3", flush=True)
    f8 = H.device_fp8(dw)
    H.assert_outputs_identical(H.run_forward_packed(w, dw, dt, f8), H.run_forward_fp8(w, dw, dt, f8))


def test_full_size_packed_switch():
    """The Switch-shape layer at full size (T = 4096, E = 128, capacity 40):
    packed bf16 weights give moe_forward's outputs bit for bit."""
    w = W["switch"]
    print("[packed] switch: generating inputs", flush=True)
    wt, tk = H.prepare(w)
    dw, dt = H.device_weights(w, wt), H.device_tokens(w, tk)
    print("[packed] switch: forward", flush=True)
    H.assert_outputs_identical(H.run_forward_packed(w, dw, dt), H.run_forward(w, dw, dt))


def test_full_size_packed_switch_fp8():
    """The Switch-shape layer at full size with e4m3 expert weights: the
    library's codes and scales equal the oracle's bit for bit, packed codes
    give moe_forward_fp8's outputs bit for bit, routing is exact on every
    token and y matches the oracle on a sample of 64 tokens (with the fully
    dropped ones, whose output is exactly 0)."""
    w = W["switch_fp8"]
    print("[packed] switch_fp8: generating inputs", flush=True)
    wt, tk = H.prepare(w)
    dw, dt = H.device_weights(w, wt), H.device_tokens(w, tk)
    f8 = H.device_fp8(dw)
    print("[packed] switch_fp8: oracle quantisation", flush=True)
    qref = H.quantize_ref(wt)
    H.assert_fp8_equal(f8, qref)
    print("[packed] switch_fp8: forward", flush=True)
    got = H.run_forward_packed(w, dw, dt, f8)
    H.assert_outputs_identical(got, H.run_forward_fp8(w, dw, dt, f8))
    route_ref = H.reference_fp8(w, wt, tk, qref, tokens=np.zeros(0, np.int64))
    full_drop = np.nonzero((route_ref["row_of_slot"] < 0).all(axis=1))[0]
    sel = H.sample_tokens(w.T, 64, seed=1, must=full_drop[:4])
    print(f"[packed] switch_fp8: oracle FFN on {len(sel)} tokens", flush=True)
    ref = H.reference_fp8(w, wt, tk, qref, tokens=sel)
    H.assert_routing_exact(w, got, ref)
    H.assert_stats_close(w, got, ref)
    y = H.y_float(got["y"])
    H.assert_y_close(w, y[sel], ref["y"])
    assert (y[full_drop] == 0).all()
