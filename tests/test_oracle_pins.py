"""Pins of the CPU oracle against what the page and the mathematics fix.

Nothing here compares the oracle with itself: every check is against a
library routine on a special case, a closed form, an identity stated on
the page, a brute-force enumeration, or a fixture reconstructed from the
page's worked example.  Page: "Mixture of experts" (rayaq.ca).
"""
import itertools
import json
import os

import numpy as np
import pytest
import scipy.special as sps
import scipy.stats as sst

import oracle
from oracle.margin import tight_tokens

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _layer(rng, T, d, d_ff, E, act="swiglu"):
    x = rng.standard_normal((T, d)).astype(np.float32)
    Wr = (rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    W1 = (rng.standard_normal((E, d_ff, d)) / np.sqrt(d)).astype(np.float32)
    W3 = (rng.standard_normal((E, d_ff, d)) / np.sqrt(d)).astype(np.float32) if act == "swiglu" else None
    W2 = (rng.standard_normal((E, d, d_ff)) / np.sqrt(d_ff)).astype(np.float32)
    return x, Wr, W1, W3, W2


def _act64(act, a1, a3):
    # Library routines for the activations: ReLU by np.maximum, exact GELU
    # as a * Phi(a) with scipy's normal CDF, SiLU as a * expit(a).
    if act == "relu":
        return np.maximum(a1, 0.0)
    if act == "gelu":
        return a1 * sst.norm.cdf(a1)
    return a1 * sps.expit(a1) * a3


def _dense_expert64(x, W1, W3, W2, e, act):
    """E_e(x) by float64 matrix products; hidden rounded to fp32 like a stored tensor."""
    x = x.astype(np.float64)
    a1 = x @ W1[e].astype(np.float64).T
    a3 = x @ W3[e].astype(np.float64).T if act == "swiglu" else None
    H = _act64(act, a1, a3).astype(np.float32).astype(np.float64)
    return H @ W2[e].astype(np.float64).T


# ---------------------------------------------------------------- router

@pytest.mark.parametrize("T,d,E,bias,noise", [(37, 48, 5, False, False), (64, 96, 16, True, True),
                                             (9, 8, 1, True, False)])
def test_router_equals_float64_matmul(T, d, E, bias, noise):
    """h = W_r x (+b +n) ("Replacing the feed-forward block"), a matrix
    product: numpy's float64 matmul rounded once to fp32 must agree to 1 ulp."""
    rng = _rng(1)
    x = rng.standard_normal((T, d)).astype(np.float32)
    Wr = rng.standard_normal((E, d)).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32) if bias else None
    n = rng.standard_normal((T, E)).astype(np.float32) if noise else None
    h = oracle.router_logits(x, Wr, b, n)
    ref = x.astype(np.float64) @ Wr.astype(np.float64).T
    if b is not None:
        ref = ref + b
    if n is not None:
        ref = ref + n
    ref = ref.astype(np.float32)
    ulp = np.abs(h.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert ulp.max() <= 1
    assert (ulp == 0).mean() > 0.9


# ---------------------------------------------------------------- softmax / lse

def test_softmax_and_lse_match_scipy():
    rng = _rng(2)
    h = (3 * rng.standard_normal((50, 13))).astype(np.float32)
    _, _, p, lse = oracle.gate(h, 2, "renorm")
    np.testing.assert_allclose(p, sps.softmax(h.astype(np.float64), axis=1), rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(lse, sps.logsumexp(h.astype(np.float64), axis=1), rtol=1e-14)
    np.testing.assert_allclose(p.sum(1), 1.0, rtol=0, atol=1e-14)


@pytest.mark.parametrize("E", [1, 4, 7, 128])
def test_equal_logits_closed_form(E):
    """Equal logits c: p = 1/E, lse = c + ln E, z = (c + ln E)^2."""
    c = 0.75
    h = np.full((6, E), c, np.float32)
    k = min(2, E)
    idx, g, p, lse = oracle.gate(h, k, "renorm")
    np.testing.assert_allclose(p, 1.0 / E, rtol=1e-15)
    np.testing.assert_allclose(lse, c + np.log(E), rtol=1e-15)
    # all tied: lower indices first
    assert (idx == np.arange(k)).all()
    np.testing.assert_allclose(g, 1.0 / k, rtol=1e-15)
    f, P, aux, z = oracle.stats(idx, p, lse)
    np.testing.assert_allclose(z, (c + np.log(E)) ** 2, rtol=1e-14)


# ---------------------------------------------------------------- top-k

def _brute_topk(hrow, k):
    """The ordered k-tuple of distinct experts whose key sequence
    (logit, -index) is lexicographically largest: the k largest logits,
    largest first, ties to the lower index."""
    E = len(hrow)
    best, best_key = None, None
    for perm in itertools.permutations(range(E), k):
        key = tuple((float(hrow[i]), -i) for i in perm)
        if best_key is None or key > best_key:
            best, best_key = perm, key
    return list(best)


@pytest.mark.parametrize("E,k", [(1, 1), (3, 1), (4, 2), (5, 3), (6, 2), (6, 6)])
def test_topk_brute_force_with_ties(E, k):
    rng = _rng(3 + E * 10 + k)
    # small integer-valued logits make exact ties frequent
    h = rng.integers(-2, 3, size=(200, E)).astype(np.float32)
    idx, _, _, _ = oracle.gate(h, k, "renorm")
    for t in range(h.shape[0]):
        assert list(idx[t]) == _brute_topk(h[t], k), (t, h[t])
    # numpy's stable argsort of -h is the same order
    assert (idx == np.argsort(-h, axis=1, kind="stable")[:, :k]).all()


def test_duplicated_router_rows_tie_to_lower_index():
    """Identical router rows give bit-identical logits; the lower index wins."""
    rng = _rng(4)
    d, E = 64, 8
    x = rng.standard_normal((40, d)).astype(np.float32)
    Wr = rng.standard_normal((E, d)).astype(np.float32)
    Wr[5] = Wr[2]
    Wr[7] = Wr[2]
    h = oracle.router_logits(x, Wr)
    assert (h[:, 5] == h[:, 2]).all() and (h[:, 7] == h[:, 2]).all()
    idx, _, _, _ = oracle.gate(h, 3, "renorm")
    for t in range(40):
        pos = {e: list(idx[t]).index(e) for e in (2, 5, 7) if e in idx[t]}
        if 5 in pos:
            assert 2 in pos and pos[2] < pos[5]
        if 7 in pos:
            assert 5 in pos and pos[5] < pos[7]


# ---------------------------------------------------------------- gates

def test_renorm_gate_identities():
    """Renormalised top-k ("Top-k gating"): gates sum to 1 and equal the
    full-softmax probabilities divided by their selected sum."""
    rng = _rng(5)
    h = (2 * rng.standard_normal((300, 9))).astype(np.float32)
    for k in (1, 2, 4, 9):
        idx, g, p, _ = oracle.gate(h, k, "renorm")
        np.testing.assert_allclose(g.sum(1), 1.0, rtol=0, atol=1e-14)
        psel = np.take_along_axis(p, idx, 1)
        np.testing.assert_allclose(g, psel / psel.sum(1, keepdims=True), rtol=1e-13)
        assert (np.diff(g, axis=1) <= 0).all()   # largest first
    idx, g, _, _ = oracle.gate(h, 1, "renorm")
    assert (g == 1.0).all()


def test_switch_gate_is_full_softmax_prob_below_one():
    """Switch ("Top-k gating", k = 1): argmax h, gate = its full-softmax p < 1."""
    rng = _rng(6)
    h = rng.standard_normal((300, 16)).astype(np.float32)
    idx, g, p, _ = oracle.gate(h, 1, "switch")
    assert (idx[:, 0] == np.argmax(h, axis=1)).all()
    np.testing.assert_allclose(g[:, 0], sps.softmax(h.astype(np.float64), axis=1).max(1), rtol=1e-13)
    assert (g < 1.0).all()


# ---------------------------------------------------------------- capacity and dispatch

@pytest.mark.parametrize("T,E,k,cf,C", [(4096, 128, 1, 1.25, 40), (16384, 128, 4, 1.0, 512),
                                        (10, 4, 1, 1.0, 3), (8, 4, 1, 1.0, 2), (8, 4, 1, 2.0, 4),
                                        (64, 4, 2, 0.0, None), (5, 3, 2, 1e-9, 1)])
def test_capacity_values(T, E, k, cf, C):
    assert oracle.capacity(T, E, k, cf) == C


def _brute_dispatch(idx, E, C):
    """Fill slots by streaming tokens in position order with one counter per
    expert ("Capacity and dropped tokens": slots fill in position order)."""
    T, k = idx.shape
    fill = [[] for _ in range(E)]
    routed = np.zeros(E, np.int64)
    dropped = np.zeros((T, k), np.uint8)
    for t in range(T):
        for s in range(k):
            e = idx[t, s]
            routed[e] += 1
            if C is None or len(fill[e]) < C:
                fill[e].append((t, s))
            else:
                dropped[t, s] = 1
    kept = np.array([len(f) for f in fill])
    offsets = np.concatenate([[0], np.cumsum(kept)])
    row_of_slot = np.full((T, k), -1)
    token_of_row = np.full(T * k, -1)
    for e in range(E):
        for r, (t, s) in enumerate(fill[e]):
            row_of_slot[t, s] = offsets[e] + r
            token_of_row[offsets[e] + r] = t
    return routed, kept, offsets, row_of_slot, token_of_row, dropped


@pytest.mark.parametrize("T,E,k,cf,skew", [(50, 4, 2, 1.0, 0.0), (200, 8, 2, 0.5, 2.0),
                                           (128, 16, 4, 1.25, 3.0), (64, 4, 2, 0.0, 1.0),
                                           (33, 5, 5, 1.0, 0.0), (1, 1, 1, 1.0, 0.0),
                                           (300, 6, 1, 1e-6, 2.0)])
def test_dispatch_equals_sequential_fill(T, E, k, cf, skew):
    rng = _rng(7 + T)
    h = (rng.standard_normal((T, E)) + skew * np.linspace(1, 0, E)).astype(np.float32)
    idx, _, _, _ = oracle.gate(h, k, "renorm")
    C = oracle.capacity(T, E, k, cf)
    o = oracle.dispatch(idx, E, C)
    routed, kept, offsets, ros, tor, dropped = _brute_dispatch(idx, E, C)
    assert (o["routed"] == routed).all() and (o["kept"] == kept).all()
    assert (o["offsets"] == offsets).all() and (o["row_of_slot"] == ros).all()
    assert (o["token_of_row"] == tor).all() and (o["dropped"] == dropped).all()
    # invariants: kept counts sum to T*k minus dropped; none exceeds C; dropless when cf = 0
    assert o["kept"].sum() == T * k - o["dropped"].sum()
    if C is not None:
        assert o["kept"].max() <= C
    else:
        assert o["dropped"].sum() == 0


def test_worked_example_reconstruction():
    with open(os.path.join(GOLDEN, "worked_example_capacity.json")) as fh:
        ex = json.load(fh)
    T, E, k = ex["T"], ex["E"], ex["k"]
    top = np.array(ex["top_expert_of_token"])
    h = np.zeros((T, E), np.float32)
    h[np.arange(T), top] = 1.0
    idx, _, _, _ = oracle.gate(h, k, "renorm")
    assert (idx[:, 0] == top).all()
    for case in ex["cases"]:
        C = oracle.capacity(T, E, k, case["cf"])
        assert C == case["capacity"]
        o = oracle.dispatch(idx, E, C)
        assert list(o["kept"]) == case["kept"]
        assert list(np.nonzero(o["dropped"][:, 0])[0]) == case["dropped_tokens"]
        if "empty_fraction_experts_0_to_2" in case:
            assert all(1 - o["kept"][e] / C == case["empty_fraction_experts_0_to_2"] for e in range(3))
    n1 = len(ex["cases"][0]["dropped_tokens"])
    n2 = len(ex["cases"][1]["dropped_tokens"])
    assert n1 - n2 == 2   # doubling the factor saves two


# ---------------------------------------------------------------- expert FFN and combine

@pytest.mark.parametrize("act", ["relu", "gelu", "swiglu"])
def test_single_expert_is_dense_ffn(act):
    """E = 1, k = 1: the layer is the dense FFN (gate 1, nothing dropped)."""
    rng = _rng(8)
    T, d, d_ff = 21, 24, 40
    x, Wr, W1, W3, W2 = _layer(rng, T, d, d_ff, 1, act)
    o = oracle.forward(x, Wr, W1, W3, W2, 1, "renorm", 0.0, act)
    ref = _dense_expert64(x, W1, W3, W2, 0, act)
    assert np.abs(o["y"] - ref).max() <= 1e-6 * np.abs(ref).max()


def test_activation_values():
    """GELU(1) = Phi(1), GELU(-1) = -Phi(-1), silu(1) = 1/(1+e^-1): textbook values."""
    x = np.array([[1.0], [-1.0]], np.float32)
    W1 = np.ones((1, 1, 1), np.float32)
    W2 = np.ones((1, 1, 1), np.float32)
    tok = np.array([0, 1])
    ex = np.array([0, 0])
    g = oracle.expert_ffn(tok, ex, x, W1, None, W2, "gelu")[:, 0]
    np.testing.assert_allclose(g, [0.8413447460685429, -0.15865525393145707], rtol=1e-7)
    s = oracle.expert_ffn(tok, ex, x, W1, W1, W2, "swiglu")[:, 0]
    np.testing.assert_allclose(s, [0.7310585786300049, 0.2689414213699951], rtol=1e-7)
    r = oracle.expert_ffn(tok, ex, x, W1, None, W2, "relu")[:, 0]
    assert list(r) == [1.0, 0.0]


@pytest.mark.parametrize("mode", ["renorm", "switch"])
def test_k_equals_E_is_full_softmax_mixture(mode):
    """k = E: every expert is chosen and both gate conventions give the full
    softmax p, so y = sum_i p_i E_i(x)."""
    rng = _rng(9)
    T, d, d_ff, E = 17, 16, 24, 5
    x, Wr, W1, W3, W2 = _layer(rng, T, d, d_ff, E)
    o = oracle.forward(x, Wr, W1, W3, W2, E, mode, 0.0, "swiglu")
    h = (x.astype(np.float64) @ Wr.astype(np.float64).T).astype(np.float32)
    p = sps.softmax(h.astype(np.float64), axis=1)
    ref = sum(p[:, [e]] * _dense_expert64(x, W1, W3, W2, e, "swiglu") for e in range(E))
    assert np.abs(o["y"] - ref).max() <= 1e-6 * np.abs(ref).max()


def _dense_moe64(x, top, gates, C, W1, W3, W2, act):
    """The layer output written as the equations state it, on dense [T][E]
    matrices: y_t = sum_i G[t, i] K[t, i] E_i(x_t) ("Replacing the
    feed-forward block"), with G[t, i] the gate of expert i for token t (0
    when i is not among its top k) and K[t, i] = 1 while the number of tokens
    up to and including t that chose i is at most C ("Capacity and dropped
    tokens": slots filled in position order).  Every expert is applied to
    every token (float64), then one contraction over experts."""
    T, k = top.shape
    E = W1.shape[0]
    A = np.zeros((T, E))
    G = np.zeros((T, E))
    rows = np.repeat(np.arange(T), k)
    A[rows, top.ravel()] = 1.0
    G[rows, top.ravel()] = gates.ravel()
    K = np.ones((T, E)) if C is None else (np.cumsum(A, axis=0) <= C).astype(np.float64)
    Y = np.stack([_dense_expert64(x, W1, W3, W2, e, act) for e in range(E)])   # [E][T][d]
    return np.einsum("te,etd->td", G * K * A, Y)


@pytest.mark.parametrize("cf", [0.0, 1.0, 0.4])
def test_matches_dense_equations(cf):
    """The oracle's dispatch + per-row FFN + slot-ordered combine equals the
    equations on dense [T][E] gate and capacity matrices."""
    rng = _rng(10)
    T, d, d_ff, E, k = 40, 16, 32, 6, 2
    x, Wr, W1, W3, W2 = _layer(rng, T, d, d_ff, E)
    o = oracle.forward(x, Wr, W1, W3, W2, k, "renorm", cf, "swiglu")
    h = (x.astype(np.float64) @ Wr.astype(np.float64).T).astype(np.float32)
    top = np.argsort(-h, axis=1, kind="stable")[:, :k]
    tl = np.take_along_axis(h, top, 1).astype(np.float64)
    gates = sps.softmax(tl, axis=1)
    C = None if cf == 0 else int(np.ceil(cf * T * k / E))
    out = _dense_moe64(x, top, gates, C, W1, W3, W2, "swiglu")
    assert np.abs(o["y"] - out).max() <= 1e-6 * np.abs(out).max()
    if cf == 0.4:
        assert o["dropped"].sum() > 0
        full = o["row_of_slot"].max(axis=1) < 0
        assert (o["y"][full] == 0).all()


def test_sampled_tokens_equal_full_forward():
    rng = _rng(11)
    T, d, d_ff, E, k = 30, 16, 24, 4, 2
    x, Wr, W1, W3, W2 = _layer(rng, T, d, d_ff, E)
    full = oracle.forward(x, Wr, W1, W3, W2, k, "renorm", 0.6, "swiglu")
    sel = np.array([29, 0, 7, 7, 13])
    part = oracle.forward(x, Wr, W1, W3, W2, k, "renorm", 0.6, "swiglu", tokens=sel)
    assert (part["y"] == full["y"][sel]).all()


# ---------------------------------------------------------------- shared experts and residual

def _shared(rng, S, d, d_ff, act):
    Ws1 = (rng.standard_normal((S, d_ff, d)) / np.sqrt(d)).astype(np.float32)
    Ws3 = (rng.standard_normal((S, d_ff, d)) / np.sqrt(d)).astype(np.float32) if act == "swiglu" else None
    Ws2 = (rng.standard_normal((S, d, d_ff)) / np.sqrt(d_ff)).astype(np.float32)
    return Ws1, Ws3, Ws2


@pytest.mark.parametrize("act,cf", [("swiglu", 0.0), ("gelu", 0.3), ("relu", 0.3)])
def test_shared_experts_are_ungated_dense_ffns(act, cf):
    """With the routed experts' outputs zero (W2 = 0), the layer output is the
    sum of the shared experts' dense FFNs on every token -- dropped tokens
    included -- each with weight 1 (section "Total versus active
    parameters": shared experts every token visits)."""
    rng = _rng(30)
    T, d, d_ff, E, k, S = 29, 16, 24, 4, 2, 3
    x, Wr, W1, W3, W2 = _layer(rng, T, d, d_ff, E, act)
    W2 = np.zeros_like(W2)
    sh = _shared(rng, S, d, d_ff, act)
    o = oracle.forward(x, Wr, W1, W3, W2, k, "renorm", cf, act, shared=sh)
    ref = sum(_dense_expert64(x, sh[0], sh[1], sh[2], j, act) for j in range(S))
    assert np.abs(o["y"] - ref).max() <= 1e-6 * np.abs(ref).max()
    if cf > 0:
        assert (o["row_of_slot"].max(axis=1) < 0).any()   # some token lost every slot


def test_shared_expert_equals_routed_expert_with_gate_one():
    """One shared expert gives, bit for bit, what the same weights give as the
    only routed expert of an E = 1, k = 1 layer (gate exactly 1, nothing
    dropped): a shared expert is an expert with weight 1 on every token."""
    rng = _rng(31)
    T, d, d_ff = 23, 24, 40
    x, Wr, W1, W3, W2 = _layer(rng, T, d, d_ff, 3)
    sh = _shared(rng, 1, d, d_ff, "swiglu")
    routed = oracle.forward(x, Wr[:1], sh[0], sh[1], sh[2], 1, "renorm", 0.0, "swiglu")
    shared = oracle.forward(x, Wr, W1, W3, np.zeros_like(W2), 2, "renorm", 0.0, "swiglu", shared=sh)
    assert (routed["gates"] == 1.0).all()
    assert (shared["y"] == routed["y"]).all()


@pytest.mark.parametrize("cf", [0.0, 0.4])
def test_shared_and_residual_match_dense_equations(cf):
    """y = h + moe_out (the Implementation section's block), moe_out being the
    routed experts by the dense gate and capacity matrices plus the shared
    experts; a token dropped from every routed expert keeps its residual and
    its shared experts ("Capacity and dropped tokens")."""
    rng = _rng(32)
    T, d, d_ff, E, k, S = 40, 16, 32, 6, 2, 2
    x, Wr, W1, W3, W2 = _layer(rng, T, d, d_ff, E)
    sh = _shared(rng, S, d, d_ff, "swiglu")
    res = rng.standard_normal((T, d)).astype(np.float32)
    o = oracle.forward(x, Wr, W1, W3, W2, k, "renorm", cf, "swiglu", shared=sh, residual=res)
    h = (x.astype(np.float64) @ Wr.astype(np.float64).T).astype(np.float32)
    top = np.argsort(-h, axis=1, kind="stable")[:, :k]
    gates = sps.softmax(np.take_along_axis(h, top, 1).astype(np.float64), axis=1)
    C = None if cf == 0 else int(np.ceil(cf * T * k / E))
    out = res.astype(np.float64) + _dense_moe64(x, top, gates, C, W1, W3, W2, "swiglu")
    for j in range(S):
        out += _dense_expert64(x, sh[0], sh[1], sh[2], j, "swiglu")
    err = np.abs(o["y"] - out).max(axis=1)
    assert (err <= 1e-6 * np.abs(out).max(axis=1)).all()
    if cf > 0:
        full = o["row_of_slot"].max(axis=1) < 0
        assert full.any()
        alone = res[full].astype(np.float64) + sum(
            _dense_expert64(x[full], sh[0], sh[1], sh[2], j, "swiglu") for j in range(S))
        assert np.abs(o["y"][full] - alone).max() <= 1e-6 * np.abs(alone).max()


def test_residual_passes_exactly():
    """With every expert weight zero the layer adds nothing: y is the residual,
    bit for bit, also for tokens dropped by capacity."""
    rng = _rng(33)
    T, d, d_ff, E, k = 25, 8, 16, 3, 2
    x, Wr, W1, W3, W2 = _layer(rng, T, d, d_ff, E)
    sh = _shared(rng, 2, d, d_ff, "swiglu")
    res = rng.standard_normal((T, d)).astype(np.float32)
    o = oracle.forward(x, Wr, W1, W3, np.zeros_like(W2), k, "renorm", 0.5, "swiglu",
                       shared=(sh[0], sh[1], np.zeros_like(sh[2])), residual=res)
    assert (o["y"] == res).all()
    sel = np.array([24, 3, 3])
    part = oracle.forward(x, Wr, W1, W3, W2, k, "renorm", 0.5, "swiglu", tokens=sel, shared=sh,
                          residual=res)
    full = oracle.forward(x, Wr, W1, W3, W2, k, "renorm", 0.5, "swiglu", shared=sh, residual=res)
    assert (part["y"] == full["y"][sel]).all()


# ---------------------------------------------------------------- e4m3 weights

import torch  # noqa: E402  (the library routine for OCP e4m3: torch.float8_e4m3fn)


def _torch_e4m3_value(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def _torch_e4m3_encode(v):
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_values_match_library():
    """Every code's value equals torch's float8_e4m3fn (the OCP E4M3 format);
    closed forms: 0x38 = 1, 0x7E = 448 (largest), 0x08 = 2^-6 (smallest
    normal), 0x01 = 2^-9 (smallest subnormal), 0x7F and 0xFF are NaN."""
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = _torch_e4m3_value(codes)
    fin = np.isfinite(ref)
    assert (np.isnan(ours) == ~fin).all()
    assert (ours[fin] == ref[fin]).all()
    assert (np.signbit(ours[fin]) == np.signbit(ref[fin])).all()
    assert oracle.e4m3_value(0x38) == 1.0 and oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0xFE) == -448.0 and oracle.e4m3_value(0x08) == 2.0 ** -6
    assert oracle.e4m3_value(0x01) == 2.0 ** -9 and oracle.e4m3_value(0x07) == 7 * 2.0 ** -9
    assert np.isnan(oracle.e4m3_value(0x7F)) and np.isnan(oracle.e4m3_value(0xFF))


def _e4m3_sweep():
    codes = np.arange(256, dtype=np.uint8)
    fin = np.unique(_torch_e4m3_value(codes)[np.isfinite(_torch_e4m3_value(codes))])
    mids = ((fin[:-1].astype(np.float64) + fin[1:]) / 2).astype(np.float32)   # exact ties
    near = np.concatenate([np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(-np.inf))])
    rnd = np.clip(_rng(40).standard_normal(3000).astype(np.float32) * 50, -448, 448)
    tiny = np.array([0.0, -0.0, 1e-30, -1e-30, 2.0 ** -10, -(2.0 ** -10), 3 * 2.0 ** -11], np.float32)
    return np.concatenate([fin, mids, near, rnd, tiny]).astype(np.float32)


def test_e4m3_encode_matches_library():
    """Round to nearest e4m3, ties to the even mantissa, sign kept: equals
    torch's conversion to float8_e4m3fn on every finite value, every exact
    midpoint between neighbours, the floats next to each midpoint, random
    values and signed zeros / underflows."""
    v = _e4m3_sweep()
    assert (oracle.e4m3_encode(v) == _torch_e4m3_encode(v)).all()


def test_e4m3_encode_saturates():
    assert oracle.e4m3_encode(np.array([460.0, 1e6, -470.0], np.float32)).tolist() == [0x7E, 0x7E, 0xFE]


def _nearest_code_brute(v):
    """Brute force over the 252 finite nonzero codes and zero: the nearest
    value, a tie to the code with the even low bit."""
    vals = {c: oracle.e4m3_value(c) for c in range(0x7F)}
    a = abs(float(v))
    best = min(vals, key=lambda c: (abs(vals[c] - a), c & 1))
    return best | (0x80 if np.signbit(v) else 0)


def test_quantize_rows_brute_force():
    """Per row: s = fl32(amax / 448) (1 for a zero row), code = the e4m3 value
    nearest fl32(w / s) by brute force, the largest magnitude lands on
    +-448, and s * value(q) is within half a grid step of w."""
    rng = _rng(41)
    W = (rng.standard_normal((6, 40)) * np.array([[1.0], [0.02], [300.0], [1e-3], [0.0], [5.0]])).astype(np.float32)
    W[5, 7] = -W[5].__abs__().max() * 1.5           # the row's extreme is negative
    q, s = oracle.quantize_e4m3(W)
    for i in range(W.shape[0]):
        amax = np.float32(np.abs(W[i]).max())
        si = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
        assert s[i] == si
        for j in range(W.shape[1]):
            v = np.clip(np.float32(W[i, j] / si), -448, 448)
            assert q[i, j] == _nearest_code_brute(v), (i, j)
        if amax > 0:
            jmax = int(np.argmax(np.abs(W[i])))
            assert q[i, jmax] == (0xFE if W[i, jmax] < 0 else 0x7E)
            deq = s[i].astype(np.float64) * oracle.e4m3_decode(q[i]).astype(np.float64)
            # half a step: 2^-4 relative in the normal range, 2^-10 * s below 2^-6 * s
            bound = np.maximum(np.abs(W[i]) * 2.0 ** -4, 2.0 ** -10 * s[i]) * (1 + 1e-6)
            assert (np.abs(deq - W[i]) <= bound).all()
    assert s[4] == 1.0 and (q[4] & 0x7F == 0).all()


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_row_scaled_ffn_equals_dequantised_dense(act):
    """Row-scaled weights: the FFN with scales equals the dense FFN on the
    dequantised weights s * value(q) formed in float64."""
    rng = _rng(42)
    T, d, d_ff, E = 19, 32, 48, 3
    x, Wr, W1, W3, W2 = _layer(rng, T, d, d_ff, E, act)
    q1, s1 = oracle.quantize_e4m3(W1)
    q2, s2 = oracle.quantize_e4m3(W2)
    q3, s3 = oracle.quantize_e4m3(W3) if act == "swiglu" else (None, None)
    dec = lambda q: None if q is None else oracle.e4m3_decode(q)
    o = oracle.forward(x, Wr, dec(q1), dec(q3), dec(q2), 1, "renorm", 0.0, act,
                       scales=(s1, s3, s2))
    D = lambda q, sc: None if q is None else sc[..., None].astype(np.float64) * dec(q).astype(np.float64)
    W1d, W3d, W2d = D(q1, s1), D(q3, s3), D(q2, s2)
    e = o["idx"][:, 0]
    ref = np.stack([_dense_expert64(x[t:t + 1], W1d, W3d, W2d, e[t], act)[0] for t in range(T)])
    assert np.abs(o["y"] - ref).max() <= 1e-6 * np.abs(ref).max()
    # and the quantised layer stays close to the unquantised one (not a parity bound)
    o32 = oracle.forward(x, Wr, W1, W3, W2, 1, "renorm", 0.0, act)
    assert np.abs(o["y"] - o32["y"]).max() <= 0.1 * np.abs(o32["y"]).max()


# ---------------------------------------------------------------- statistics

def test_aux_is_one_when_balanced():
    """Uniform f gives E * sum f_i P_i = sum P_i = 1 ("The load-balancing loss")."""
    rng = _rng(12)
    E, m = 8, 7
    T = m * E
    h = rng.standard_normal((T, E)).astype(np.float32)
    h[np.arange(T), np.arange(T) % E] = 10.0     # distinct top choice per residue class
    idx, _, p, lse = oracle.gate(h, 2, "renorm")
    f, P, aux, z = oracle.stats(idx, p, lse)
    np.testing.assert_allclose(f, 1.0 / E, rtol=1e-15)
    np.testing.assert_allclose(aux, 1.0, rtol=1e-13)
    np.testing.assert_allclose(P.sum(), 1.0, rtol=1e-13)


def test_aux_tends_to_E_when_collapsed():
    E, T = 16, 50
    h = np.zeros((T, E), np.float32)
    h[:, 3] = 60.0
    idx, _, p, lse = oracle.gate(h, 1, "switch")
    f, P, aux, z = oracle.stats(idx, p, lse)
    assert f[3] == 1.0 and f.sum() == 1.0
    np.testing.assert_allclose(aux, E, rtol=1e-12)


def test_stats_match_library_on_random_logits():
    rng = _rng(13)
    T, E, k = 120, 10, 3
    h = (2 * rng.standard_normal((T, E))).astype(np.float32)
    idx, _, p, lse = oracle.gate(h, k, "renorm")
    f, P, aux, z = oracle.stats(idx, p, lse)
    h64 = h.astype(np.float64)
    fref = np.bincount(np.argmax(h, axis=1), minlength=E) / T
    Pref = sps.softmax(h64, axis=1).mean(0)
    np.testing.assert_allclose(f, fref, rtol=1e-15)
    np.testing.assert_allclose(P, Pref, rtol=1e-13)
    np.testing.assert_allclose(aux, E * (fref * Pref).sum(), rtol=1e-13)
    np.testing.assert_allclose(z, (sps.logsumexp(h64, axis=1) ** 2).mean(), rtol=1e-13)


def test_f_counts_top_choice_before_drops():
    rng = _rng(14)
    T, d, d_ff, E, k = 64, 8, 8, 4, 2
    x, Wr, W1, W3, W2 = _layer(rng, T, d, d_ff, E)
    a = oracle.forward(x, Wr, W1, W3, W2, k, "renorm", 0.0, "swiglu")
    b = oracle.forward(x, Wr, W1, W3, W2, k, "renorm", 0.3, "swiglu")
    assert b["dropped"].sum() > 0
    assert (a["f"] == b["f"]).all() and (a["P"] == b["P"]).all() and a["z"] == b["z"]


# ---------------------------------------------------------------- margin filter

def test_tight_tokens_detects_small_gaps():
    h = np.array([[3.0, 2.0, 1.0, 0.0],
                  [3.0, 3.00001, 1.0, 0.0],     # gap inside top-2 too small
                  [3.0, 2.0, 1.99995, 0.0],     # gap between 2nd and 3rd too small
                  [3.0, 2.0, 1.0, 0.99999]],    # gap outside the top 3: fine
                 np.float32)
    assert list(tight_tokens(h, 2, 1e-4)) == [1, 2]
    assert list(tight_tokens(h, 4, 1e-4)) == [1, 2, 3]
