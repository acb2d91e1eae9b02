"""Pins of the oracle's backward (training gradients) against what does not
share its code: torch's autograd in float64 on the layer's forward written
with torch operations, the routing decisions (top-k, capacity drops) taken
from the oracle's forward and held fixed, and a closed form for the
load-balancing term.  Page "Mixture of experts" (rayaq.ca), Mechanics.
"""
import numpy as np
import pytest
import scipy.special as sps
import torch
import torch.nn.functional as F

import oracle


def _inputs(seed, T, d, d_ff, E, act, bias=True, noise=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d)).astype(np.float32)
    Wr = (rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    b = (rng.standard_normal(E) * 0.3).astype(np.float32) if bias else None
    n = (rng.standard_normal((T, E)) * 0.1).astype(np.float32) if noise else None
    W1 = (rng.standard_normal((E, d_ff, d)) / np.sqrt(d)).astype(np.float32)
    W3 = (rng.standard_normal((E, d_ff, d)) / np.sqrt(d)).astype(np.float32) if act == "swiglu" else None
    W2 = (rng.standard_normal((E, d, d_ff)) / np.sqrt(d_ff)).astype(np.float32)
    dy = rng.standard_normal((T, d)).astype(np.float32)
    return x, Wr, b, n, W1, W3, W2, dy


def _autograd(x, Wr, b, n, W1, W3, W2, dy, idx, rows, k, mode, act, a_aux, a_z):
    """Gradients of sum <dy, y> + a_aux aux + a_z z by torch autograd (float64)."""
    t64 = lambda a: None if a is None else torch.tensor(a, dtype=torch.float64, requires_grad=True)
    X, WR, B, W1t, W3t, W2t = t64(x), t64(Wr), t64(b), t64(W1), t64(W3), t64(W2)
    T, E = x.shape[0], Wr.shape[0]
    h = X @ WR.T
    if B is not None:
        h = h + B
    if n is not None:
        h = h + torch.tensor(n, dtype=torch.float64)
    p = torch.softmax(h, dim=1)
    lse = torch.logsumexp(h, dim=1)
    I = torch.tensor(idx, dtype=torch.int64)
    g = torch.softmax(h.gather(1, I), dim=1) if mode == "renorm" else p.gather(1, I)
    ys = []
    for t in range(T):
        yt = torch.zeros(x.shape[1], dtype=torch.float64)
        for s in range(k):
            if rows[t, s] < 0:
                continue
            e = int(idx[t, s])
            a1 = W1t[e] @ X[t]
            if act == "swiglu":
                H = F.silu(a1) * (W3t[e] @ X[t])
            elif act == "gelu":
                H = F.gelu(a1)
            else:
                H = F.relu(a1)
            yt = yt + g[t, s] * (W2t[e] @ H)
        ys.append(yt)
    y = torch.stack(ys)
    f = torch.tensor(np.bincount(idx[:, 0], minlength=E) / T, dtype=torch.float64)
    aux = E * (f * p.mean(0)).sum()
    z = (lse ** 2).mean()
    L = (y * torch.tensor(dy, dtype=torch.float64)).sum() + a_aux * aux + a_z * z
    L.backward()
    grad = lambda a: None if a is None else a.grad.numpy()
    return dict(dx=grad(X), dWr=grad(WR), dbias=grad(B), dW1=grad(W1t), dW3=grad(W3t), dW2=grad(W2t))


def _close(a, b, rtol, what):
    scale = float(np.abs(b).max())
    err = float(np.abs(a.astype(np.float64) - b).max())
    assert err <= rtol * scale, f"{what}: {err:.3e} > {rtol} * {scale:.3e}"


@pytest.mark.parametrize("mode,act,cf,k", [("renorm", "swiglu", 0.0, 2), ("renorm", "swiglu", 0.5, 2),
                                           ("switch", "gelu", 1.0, 1), ("switch", "swiglu", 0.0, 2),
                                           ("renorm", "relu", 0.7, 3), ("renorm", "gelu", 0.0, 4)])
def test_backward_matches_autograd(mode, act, cf, k):
    T, d, d_ff, E = 24, 12, 16, 4
    x, Wr, b, n, W1, W3, W2, dy = _inputs(5 + k, T, d, d_ff, E, act)
    fw = oracle.forward(x, Wr, W1, W3, W2, k, mode, cf, act, b, n)
    if cf == 0.5:
        assert (fw["row_of_slot"] < 0).any()
    o = oracle.backward(x, Wr, W1, W3, W2, k, mode, cf, act, dy, 0.3, 0.05, b, n,
                        rows=fw["row_of_slot"])
    ref = _autograd(x, Wr, b, n, W1, W3, W2, dy, fw["idx"], fw["row_of_slot"], k, mode, act, 0.3, 0.05)
    for key in ("dx", "dWr", "dbias", "dW1", "dW3", "dW2"):
        if ref[key] is None:
            assert o[key] is None
            continue
        _close(o[key], ref[key], 1e-6, key)


def test_aux_gradient_closed_form():
    """With dy = 0 and only the load-balancing term, d aux / d P_i = E f_i, so
    the router bias gradient is sum_t p_t (a - <p_t, a>), a_i = E f_i / T
    (p from scipy's softmax, f from the top choices)."""
    T, d, d_ff, E, k = 40, 8, 8, 5, 2
    x, Wr, b, n, W1, W3, W2, dy = _inputs(11, T, d, d_ff, E, "swiglu", noise=False)
    dy[:] = 0.0
    o = oracle.backward(x, Wr, W1, W3, W2, k, "renorm", 0.0, "swiglu", dy, 1.0, 0.0, b, None)
    h = (x.astype(np.float64) @ Wr.astype(np.float64).T + b).astype(np.float32).astype(np.float64)
    p = sps.softmax(h, axis=1)
    top = np.argmax(h, axis=1)
    a = E * np.bincount(top, minlength=E) / T / T
    ref = (p * (a[None, :] - (p @ a)[:, None])).sum(axis=0)
    np.testing.assert_allclose(o["dbias"], ref, rtol=1e-6, atol=1e-9)
    assert np.abs(o["dW1"]).max() == 0.0 and np.abs(o["dW2"]).max() == 0.0


def test_z_gradient_closed_form():
    """Only the z term: d z / d h_t = (2 / T) lse_t p_t (scipy), so dbias is its sum."""
    T, d, d_ff, E, k = 30, 8, 8, 6, 2
    x, Wr, b, n, W1, W3, W2, dy = _inputs(12, T, d, d_ff, E, "relu", noise=False)
    dy[:] = 0.0
    o = oracle.backward(x, Wr, W1, W3, W2, k, "switch", 0.0, "relu", dy, 0.0, 1.0, b, None)
    h = (x.astype(np.float64) @ Wr.astype(np.float64).T + b).astype(np.float32).astype(np.float64)
    ref = (2.0 / T * sps.logsumexp(h, axis=1)[:, None] * sps.softmax(h, axis=1)).sum(axis=0)
    np.testing.assert_allclose(o["dbias"], ref, rtol=1e-6)


@pytest.mark.parametrize("mode,act,cf,k", [("renorm", "swiglu", 0.5, 2), ("switch", "gelu", 1.0, 1),
                                           ("renorm", "relu", 0.0, 3)])
def test_selected_weight_gradients_match_autograd(mode, act, cf, k):
    """The one-expert, selected-hidden-unit weight gradients (used where the
    whole backward is too large) against torch autograd: rows of dW1 and dW3
    and columns of dW2 of every expert, for a spread of hidden units, with
    the expert's kept rows in token order from the oracle's routing."""
    T, d, d_ff, E = 30, 12, 16, 4
    x, Wr, b, n, W1, W3, W2, dy = _inputs(21 + k, T, d, d_ff, E, act)
    fw = oracle.forward(x, Wr, W1, W3, W2, k, mode, cf, act, b, n)
    ref = _autograd(x, Wr, b, n, W1, W3, W2, dy, fw["idx"], fw["row_of_slot"], k, mode, act, 0.0, 0.0)
    fsel = np.array([0, 5, 6, 15])
    for e in range(E):
        lo, hi = fw["offsets"][e], fw["offsets"][e + 1]
        tok = fw["token_of_row"][lo:hi]
        t_s = np.nonzero((fw["idx"] == e) & (fw["row_of_slot"] >= 0))
        gate = np.zeros(hi - lo)
        gate[fw["row_of_slot"][t_s] - lo] = fw["gates"][t_s]
        got = oracle.expert_wgrad_sel(x, W1[e], None if W3 is None else W3[e], W2[e], tok, gate, dy, act, fsel)
        _close(got["dW1"], ref["dW1"][e][fsel], 1e-6, f"dW1[{e}]")
        _close(got["dW2"], ref["dW2"][e][:, fsel], 1e-6, f"dW2[{e}]")
        if act == "swiglu":
            _close(got["dW3"], ref["dW3"][e][fsel], 1e-6, f"dW3[{e}]")
