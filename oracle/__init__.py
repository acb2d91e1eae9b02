"""CPU oracle for the sparse-MoE FFN layer forward -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never uses it, and
it uses nothing from the GPU library.

Thin numpy/ctypes wrapper over ``moe_oracle.c``; the arithmetic lives in
the C file (fp32 storage, fp64 sequential sums).  Each function states the
passage of the page "Mixture of experts" (rayaq.ca) it follows.

Integer codes used here are the oracle's own:
  gate: "renorm" (softmax over the k chosen logits) | "switch" (full-softmax p)
  act:  "relu" | "gelu" | "swiglu"
"""
import ctypes
import os

import numpy as np

from . import build as _build

_GATE = {"renorm": 0, "switch": 1}
_ACT = {"relu": 0, "gelu": 1, "swiglu": 2}

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("MOE_ORACLE_LIB")   # a planted-mistake build, in the mutation test
    if path is None:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build()
    lib = ctypes.CDLL(path)
    i64, ip, fp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    lib.orc_router_logits.argtypes = [i64, i64, i64, fp, fp, fp, fp, fp]
    lib.orc_router_logits.restype = None
    lib.orc_gate.argtypes = [i64, i64, i64, ctypes.c_int, fp, ip, dp, dp, dp]
    lib.orc_gate.restype = ctypes.c_int
    lib.orc_capacity.argtypes = [i64, i64, i64, ctypes.c_double]
    lib.orc_capacity.restype = i64
    lib.orc_dispatch.argtypes = [i64, i64, i64, i64, ip, ip, ip, ip, ip, ip, ip]
    lib.orc_dispatch.restype = None
    lib.orc_expert_ffn.argtypes = [i64, ip, ip, i64, i64, ctypes.c_int, fp, fp, fp, fp, fp, fp, fp, fp]
    lib.orc_expert_ffn.restype = ctypes.c_int
    lib.orc_combine.argtypes = [i64, i64, i64, dp, ip, fp, fp]
    lib.orc_combine.restype = None
    lib.orc_combine_shared.argtypes = [i64, i64, i64, i64, dp, ip, fp, fp, fp, fp]
    lib.orc_combine_shared.restype = None
    lib.orc_stats.argtypes = [i64, i64, i64, ip, dp, dp, dp, dp, dp, dp]
    lib.orc_stats.restype = None
    lib.orc_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_value.restype = ctypes.c_double
    lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_quantize_e4m3.argtypes = [i64, i64, fp, ip, fp]
    lib.orc_quantize_e4m3.restype = None
    lib.orc_e4m3_decode.argtypes = [i64, ip, fp]
    lib.orc_e4m3_decode.restype = None
    lib.orc_backward.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int, fp, fp, fp, fp,
                                 fp, fp, fp, ip, fp, ctypes.c_double, ctypes.c_double, fp, fp, fp,
                                 fp, fp, fp]
    lib.orc_backward.restype = ctypes.c_int
    lib.orc_expert_wgrad_sel.argtypes = [i64, ip, dp, i64, i64, ctypes.c_int, fp, fp, fp, fp, fp, i64, ip,
                                         fp, fp, fp]
    lib.orc_expert_wgrad_sel.restype = ctypes.c_int
    lib.orc_threads.argtypes = []
    lib.orc_threads.restype = ctypes.c_int
    lib.orc_set_threads.argtypes = [ctypes.c_int]
    lib.orc_set_threads.restype = None
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def router_logits(x, Wr, bias=None, noise=None):
    """h = W_r x (+ b + n), fp32 ("Replacing the feed-forward block"; noise per
    "Top-k gating"; float32 router per "Implementation")."""
    x, Wr, bias, noise = _f32(x), _f32(Wr), _f32(bias), _f32(noise)
    T, d = x.shape
    E = Wr.shape[0]
    assert Wr.shape == (E, d)
    assert bias is None or bias.shape == (E,)
    assert noise is None or noise.shape == (T, E)
    h = np.empty((T, E), np.float32)
    _load().orc_router_logits(T, d, E, _p(x), _p(Wr), _p(bias), _p(noise), _p(h))
    return h


def gate(h, k, mode):
    """Softmax, top-k (largest first, ties to the lower index) and gates
    ("Top-k gating").  Returns idx int32 [T,k], gates f64 [T,k],
    p f64 [T,E], lse f64 [T]."""
    h = _f32(h)
    T, E = h.shape
    idx = np.empty((T, k), np.int32)
    g = np.empty((T, k), np.float64)
    p = np.empty((T, E), np.float64)
    lse = np.empty((T,), np.float64)
    rc = _load().orc_gate(T, E, k, _GATE[mode], _p(h), _p(idx), _p(g), _p(p), _p(lse))
    if rc != 0:
        raise ValueError("orc_gate: bad arguments")
    return idx, g, p, lse


def capacity(T, E, k, cf):
    """ceil(cf*T*k/E), or None for no limit ("Capacity and dropped tokens")."""
    c = _load().orc_capacity(T, E, k, float(cf))
    return None if c < 0 else int(c)


def dispatch(idx, E, C):
    """Token-ordered per-expert lists cut at capacity C (None = no limit)
    ("Capacity and dropped tokens"; the listing's nonzero + [:capacity])."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    out = dict(
        routed=np.empty(E, np.int32), kept=np.empty(E, np.int32),
        offsets=np.empty(E + 1, np.int32), row_of_slot=np.empty((T, k), np.int32),
        token_of_row=np.empty(T * k, np.int32), dropped=np.empty((T, k), np.uint8))
    _load().orc_dispatch(T, E, k, -1 if C is None else int(C), _p(idx),
                         _p(out["routed"]), _p(out["kept"]), _p(out["offsets"]),
                         _p(out["row_of_slot"]), _p(out["token_of_row"]), _p(out["dropped"]))
    return out


def expert_ffn(tok, ex, x, W1, W3, W2, act, scales=None):
    """E_e(x_t) for each (t, e) pair ("Implementation": SwiGLU expert; ReLU/GELU
    experts d -> d_ff -> d).  Weights: W1, W3 [E][d_ff][d], W2 [E][d][d_ff].
    ``scales``: None, or per-row scales (S1 [E][d_ff], S3 [E][d_ff] or None,
    S2 [E][d]) of row-scaled weights (weight row = scale * stored row)."""
    tok = np.ascontiguousarray(tok, dtype=np.int32)
    ex = np.ascontiguousarray(ex, dtype=np.int32)
    x, W1, W2 = _f32(x), _f32(W1), _f32(W2)
    W3 = _f32(W3) if act == "swiglu" else None
    if act == "swiglu" and W3 is None:
        raise ValueError("swiglu needs W3")
    n = tok.shape[0]
    d = x.shape[1]
    d_ff = W1.shape[1]
    assert W1.shape[2] == d and W2.shape[1:] == (d, d_ff)
    S1 = S3 = S2 = None
    if scales is not None:
        S1, S3, S2 = (_f32(a) for a in scales)
        assert S1.shape == W1.shape[:2] and S2.shape == W2.shape[:2]
        assert S3 is None or S3.shape == W1.shape[:2]
    out = np.empty((n, d), np.float32)
    rc = _load().orc_expert_ffn(n, _p(tok), _p(ex), d, d_ff, _ACT[act], _p(x), _p(W1),
                                _p(W3), _p(W2), _p(S1), _p(S3), _p(S2), _p(out))
    if rc != 0:
        raise MemoryError("orc_expert_ffn: could not allocate its per-thread scratch")
    return out


def combine(gates, rows, ys):
    """y_t = sum over kept slots, in slot order, of g_s * ys[row] (Eq. for y in
    "Replacing the feed-forward block"; fully dropped tokens give 0)."""
    gates = np.ascontiguousarray(gates, dtype=np.float64)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    ys = _f32(ys)
    n, k = gates.shape
    d = ys.shape[1]
    y = np.empty((n, d), np.float32)
    _load().orc_combine(n, k, d, _p(gates), _p(rows), _p(ys), _p(y))
    return y


def combine_shared(gates, rows, ys, ysh, res):
    """y_t = fl32(res_t + routed slots in slot order + shared experts in order)
    (section "Total versus active parameters": shared experts every token
    visits; Implementation: the block adds the layer output to its hidden
    state).  ysh [S*n][d]: shared expert j on token t is row j*n + t;
    res [n][d] or None."""
    gates = np.ascontiguousarray(gates, dtype=np.float64)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    ys, ysh, res = _f32(ys), _f32(ysh), _f32(res)
    n, k = gates.shape
    d = ys.shape[1] if ys.shape[0] else ysh.shape[1]
    S = ysh.shape[0] // n if n else 0
    assert ysh.shape == (S * n, d)
    assert res is None or res.shape == (n, d)
    y = np.empty((n, d), np.float32)
    _load().orc_combine_shared(n, k, d, S, _p(gates), _p(rows), _p(ys), _p(ysh), _p(res), _p(y))
    return y


def e4m3_value(code):
    """Value of one e4m3 code (OCP 8-bit floating point, E4M3; NaN for 0x7F, 0xFF)."""
    return float(_load().orc_e4m3_value(int(code)))


def e4m3_encode(v):
    """Nearest e4m3 codes (ties to even mantissa, saturating at 448) of fp32 values."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    lib = _load()
    return np.array([lib.orc_e4m3_encode(float(a)) for a in v.ravel()], np.uint8).reshape(v.shape)


def e4m3_decode(q):
    """fp32 values of e4m3 codes."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    out = np.empty(q.shape, np.float32)
    _load().orc_e4m3_decode(q.size, _p(q), _p(out))
    return out


def quantize_e4m3(W):
    """Row-wise post-training quantisation of W [..., cols] (fp32): codes q
    (uint8, same shape) and scales s [...] with W ~= s[..., None] * value(q)
    (the model quantization entry of the inference-optimization glossary
    page "Mixture of Experts (MoE)": post-training quantisation of a trained
    model's weights)."""
    W = _f32(W)
    cols = W.shape[-1]
    rows = W.size // cols
    q = np.empty(W.shape, np.uint8)
    s = np.empty(W.shape[:-1], np.float32)
    _load().orc_quantize_e4m3(rows, cols, _p(W), _p(q), _p(s))
    return q, s


def stats(idx, p, lse):
    """f, P, aux = E*sum f P, z = mean lse^2 ("The load-balancing loss")."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    p = np.ascontiguousarray(p, dtype=np.float64)
    lse = np.ascontiguousarray(lse, dtype=np.float64)
    T, k = idx.shape
    E = p.shape[1]
    f = np.empty(E, np.float64)
    P = np.empty(E, np.float64)
    aux = np.zeros(1, np.float64)
    z = np.zeros(1, np.float64)
    _load().orc_stats(T, E, k, _p(idx), _p(p), _p(lse), _p(f), _p(P), _p(aux), _p(z))
    return f, P, float(aux[0]), float(z[0])


def backward(x, Wr, W1, W3, W2, k, mode, cf, act, dy, alpha_aux=0.0, alpha_z=0.0, bias=None,
             noise=None, rows=None):
    """Gradients of L = sum <dy, y> + alpha_aux aux + alpha_z z for the routing
    the forward takes (held fixed): dx, dWr, dbias (or None), dW1, dW3 (or
    None), dW2 (the Mechanics equations differentiated; see moe_oracle.c).
    ``rows``: the forward's row_of_slot (computed here if None)."""
    x, Wr, W1, W2, dy = _f32(x), _f32(Wr), _f32(W1), _f32(W2), _f32(dy)
    W3 = _f32(W3) if act == "swiglu" else None
    bias, noise = _f32(bias), _f32(noise)
    T, d = x.shape
    E, d_ff = W1.shape[0], W1.shape[1]
    if rows is None:
        fw = forward(x, Wr, W1, W3, W2, k, mode, cf, act, bias, noise, tokens=np.zeros(0, np.int64))
        rows = fw["row_of_slot"]
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    out = dict(dx=np.empty((T, d), np.float32), dWr=np.empty((E, d), np.float32),
               dbias=np.empty(E, np.float32) if bias is not None else None,
               dW1=np.empty(W1.shape, np.float32),
               dW3=np.empty(W1.shape, np.float32) if W3 is not None else None,
               dW2=np.empty(W2.shape, np.float32))
    rc = _load().orc_backward(T, d, d_ff, E, k, _GATE[mode], _ACT[act], _p(x), _p(Wr), _p(bias),
                              _p(noise), _p(W1), _p(W3), _p(W2), _p(rows), _p(dy),
                              float(alpha_aux), float(alpha_z), _p(out["dx"]), _p(out["dWr"]),
                              _p(out["dbias"]), _p(out["dW1"]), _p(out["dW3"]), _p(out["dW2"]))
    if rc != 0:
        raise ValueError("orc_backward failed")
    return out


def expert_wgrad_sel(x, W1e, W3e, W2e, tok, gate, dy, act, fsel):
    """Weight gradients of one expert for the hidden units ``fsel`` (the
    backward's rows of dW1 and dW3 and columns of dW2, see
    orc_expert_wgrad_sel): x, dy [T][d]; W1e, W3e [d_ff][d] (W3e only for
    SwiGLU), W2e [d][d_ff] of that expert; tok, gate [n] its kept rows in
    token order.  Returns dW1 [nf][d], dW3 [nf][d] or None, dW2 [d][nf]."""
    x, W1e, W2e, dy = _f32(x), _f32(W1e), _f32(W2e), _f32(dy)
    W3e = _f32(W3e) if act == "swiglu" else None
    tok = np.ascontiguousarray(tok, dtype=np.int32)
    gate = np.ascontiguousarray(gate, dtype=np.float64)
    fsel = np.ascontiguousarray(fsel, dtype=np.int32)
    d_ff, d = W1e.shape
    assert W2e.shape == (d, d_ff) and x.shape[1] == d and dy.shape == x.shape
    nf = len(fsel)
    dW1 = np.empty((nf, d), np.float32)
    dW3 = np.empty((nf, d), np.float32) if W3e is not None else None
    dW2 = np.empty((d, nf), np.float32)
    rc = _load().orc_expert_wgrad_sel(len(tok), _p(tok), _p(gate), d, d_ff, _ACT[act], _p(x), _p(W1e),
                                      _p(W3e), _p(W2e), _p(dy), nf, _p(fsel), _p(dW1), _p(dW3), _p(dW2))
    if rc != 0:
        raise MemoryError("orc_expert_wgrad_sel: could not allocate its scratch")
    return dict(dW1=dW1, dW3=dW3, dW2=dW2)


def threads():
    """Host threads the oracle's parallel loops use."""
    return int(_load().orc_threads())


def set_threads(n):
    """Sets the host threads of the oracle's parallel loops (results do not
    depend on it: threads split tokens and rows, never a sum)."""
    _load().orc_set_threads(int(n))


def route(x, Wr, k, mode, bias=None, noise=None):
    """Router + gate + statistics for all tokens."""
    h = router_logits(x, Wr, bias, noise)
    idx, g, p, lse = gate(h, k, mode)
    f, P, aux, z = stats(idx, p, lse)
    return dict(h=h, idx=idx, gates=g, p=p, lse=lse, f=f, P=P, aux=aux, z=z)


def forward(x, Wr, W1, W3, W2, k, mode, cf, act, bias=None, noise=None, tokens=None,
            shared=None, residual=None, scales=None):
    """Whole layer forward.  Routing, dispatch and statistics always cover
    every token (capacity couples tokens through their order); the expert
    FFN and the combine run for ``tokens`` only (all tokens if None), and
    ``y`` then holds those tokens' rows in the order given.

    ``shared``: None, or (Ws1, Ws3, Ws2) with S shared experts of the
    routed experts' shape ([S][d_ff][d], [S][d_ff][d] or None, [S][d][d_ff]),
    run on every selected token with weight 1; ``residual``: None or [T][d],
    added to the layer output (section "Total versus active parameters";
    Implementation's h + moe_out).  ``scales``: None, or the per-row scales
    (S1, S3, S2) of row-scaled routed expert weights (see expert_ffn)."""
    x = _f32(x)
    T, d = x.shape
    E = Wr.shape[0]
    r = route(x, Wr, k, mode, bias, noise)
    C = capacity(T, E, k, cf)
    disp = dispatch(r["idx"], E, C)
    sel = np.arange(T, dtype=np.int64) if tokens is None else np.asarray(tokens, np.int64)
    kept = disp["row_of_slot"][sel] >= 0                       # [n, k]
    pair_t = np.repeat(sel, k).reshape(len(sel), k)[kept]
    pair_e = r["idx"][sel][kept]
    ys = expert_ffn(pair_t, pair_e, x, W1, W3, W2, act, scales) if len(pair_t) else \
        np.zeros((0, d), np.float32)
    rows = np.full((len(sel), k), -1, np.int32)
    rows[kept] = np.arange(int(kept.sum()), dtype=np.int32)
    if shared is None and residual is None:
        y = combine(r["gates"][sel], rows, ys)
    else:
        if shared is None:
            ysh = np.zeros((0, d), np.float32)
        else:
            Ws1, Ws3, Ws2 = shared
            S = np.asarray(Ws1).shape[0]
            sh_t = np.tile(sel, S)                                  # row j*n + t'
            sh_e = np.repeat(np.arange(S), len(sel))
            ysh = expert_ffn(sh_t, sh_e, x, Ws1, Ws3, Ws2, act) if len(sh_t) else \
                np.zeros((0, d), np.float32)
        res = None if residual is None else _f32(residual)[sel]
        y = combine_shared(r["gates"][sel], rows, ys, ysh, res)
    out = dict(r)
    out.update(disp)
    out.update(C=C, y=y, tokens=sel)
    return out
