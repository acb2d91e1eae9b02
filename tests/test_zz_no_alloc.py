"""moe_forward_noalloc (the forward whose workspace is the library's static
device scratch) against moe_forward with a caller workspace, through the C
ABI: two calls in a row, the second on a smaller layer, so the second call
runs on scratch that still holds the first call's contents.  Same kernels,
so every output must match bit for bit (routing, counts, permutation and
drops are integer; y and the statistics are bitwise reproducible).  Then
the oracle checks the no-alloc results to the parity bar."""
import numpy as np
import pytest
import torch

import harness as H
from sparse_mixture_experts_03_amd import binding as B
from sparse_mixture_experts_03_amd import synth

pytestmark = pytest.mark.gpu

BIG = synth.WORKLOADS["finegrained_zipf"].with_(name="noalloc_big", T=1536, d=512, d_ff=384, E=24)
SMALL = synth.WORKLOADS["switch"].with_(name="noalloc_small", T=200, d=256, d_ff=512, E=10)


def _run_both(w):
    wt, tk = H.prepare(w)
    dw, dt = H.device_weights(w, wt), H.device_tokens(w, tk)
    desc = B.desc_for(w)
    assert B.moe_workspace_size(desc) <= B.NOALLOC_SCRATCH_BYTES
    ref_out = H.run_forward(w, dw, dt)
    out = B.alloc_outputs(desc)
    B.moe_forward_noalloc(desc, dt["x"], dw["Wr"], dw["bias"], dt["noise"], dw["W1"], dw["W3"],
                          dw["W2"], out["y"], topk_idx=out["topk_idx"], gates=out["gates"],
                          routed_counts=out["routed_counts"], kept_counts=out["kept_counts"],
                          offsets=out["offsets"], row_of_slot=out["row_of_slot"],
                          token_of_row=out["token_of_row"], dropped=out["dropped"],
                          stats=out["stats"])
    torch.cuda.synchronize()
    got = {k: v.cpu() for k, v in out.items()}
    for key in ref_out:
        a, b = got[key], ref_out[key]
        if a.dtype in (torch.bfloat16, torch.float32):   # compare the bits
            a, b = a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32), \
                b.view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32)
        np.testing.assert_array_equal(a.numpy(), b.numpy(), err_msg=f"{w.name}: {key}")
    ref = H.reference(w, wt, tk)
    H.assert_routing_exact(w, got, ref)
    H.assert_stats_close(w, got, ref)
    H.assert_y_close(w, H.y_float(got["y"]), ref["y"])
    return got


def test_noalloc_matches_forward_twice_then_smaller():
    assert B.moe_workspace_size(B.desc_for(SMALL)) < B.moe_workspace_size(B.desc_for(BIG))
    first = _run_both(BIG)
    assert int(first["dropped"].sum()) > 0          # the capacity path ran
    _run_both(SMALL)


def test_noalloc_rejects_a_layer_past_the_scratch():
    w = synth.WORKLOADS["mixtral_prefill"]
    desc = B.desc_for(w)
    assert B.moe_workspace_size(desc) > B.NOALLOC_SCRATCH_BYTES
    lib = B.load()
    import ctypes
    fake = [ctypes.c_void_p(0x1000)] * 17
    assert lib.moe_forward_noalloc(ctypes.byref(desc), *fake, None) == -5
