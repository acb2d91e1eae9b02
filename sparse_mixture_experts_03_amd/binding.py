"""Python binding of libmoe's C ABI (``include/moe.h``).

Argument marshalling only: every function checks that the torch tensors it
is given have the dtype, shape and device the ABI expects, then passes raw
device pointers and the current HIP stream to the library.  Every step of
the layer runs in the library's HIP kernels; there is no fallback path, and
loading fails loudly when the library cannot be found or built.

Names match the ABI: moe_workspace_size, moe_capacity, moe_route,
moe_dispatch, moe_expert_ffn, moe_combine, moe_forward, and for shared
experts plus the block residual moe_workspace_size_shared, moe_shared_ffn,
moe_combine_shared, moe_forward_shared, and for E4M3 expert weights
moe_quantize_e4m3, moe_expert_ffn_fp8, moe_forward_fp8, and for expert weights in
the streaming tile layout moe_pack_stream, moe_expert_ffn_packed,
moe_forward_packed, and for training
moe_backward_workspace_size, moe_backward, and the forward without a
workspace argument (its workspace is a static device array in the library)
moe_forward_noalloc.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

GATE = {"renorm": 0, "switch": 1}
ACT = {"relu": 0, "gelu": 1, "swiglu": 2}
DTYPE = {"f32": 0, "bf16": 1}
TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}
FORWARD_STAGES = 7
STAGE_NAMES = ("route", "route_finalize", "dispatch", "gather", "expert_up", "expert_down", "combine")
FORWARD_SHARED_STAGES = 8
STAGE_NAMES_SHARED = ("route", "route_finalize", "dispatch", "gather", "expert_up", "expert_down",
                      "shared", "combine")
MAX_SHARED = 16

MOE_OK = 0
STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED", -3: "MOE_ERR_HIP",
          -4: "MOE_ERR_WORKSPACE", -5: "MOE_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 64 << 20


class MoeError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        super().__init__(f"{fn} returned {code} ({STATUS.get(code, 'unknown')})")


class MoeDesc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("gate", ctypes.c_int32),
                ("act", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("capacity_factor", ctypes.c_double),
                ("stage_events", ctypes.POINTER(ctypes.c_void_p)),
                ("n_stage_events", ctypes.c_int32)]


class MoeShared(ctypes.Structure):
    _fields_ = [("n_shared", ctypes.c_int32), ("W1", ctypes.c_void_p), ("W3", ctypes.c_void_p),
                ("W2", ctypes.c_void_p), ("residual", ctypes.c_void_p)]


class MoeFp8Experts(ctypes.Structure):
    _fields_ = [("W1", ctypes.c_void_p), ("W3", ctypes.c_void_p), ("W2", ctypes.c_void_p),
                ("s1", ctypes.c_void_p), ("s3", ctypes.c_void_p), ("s2", ctypes.c_void_p)]


class MoePackedExperts(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("W1", ctypes.c_void_p), ("W3", ctypes.c_void_p),
                ("W2", ctypes.c_void_p), ("s1", ctypes.c_void_p), ("s3", ctypes.c_void_p),
                ("s2", ctypes.c_void_p)]


WEIGHTS = {"bf16": 1, "e4m3": 2}


def make_desc(T, d, d_ff, E, k, gate="renorm", act="swiglu", dtype="bf16", cf=0.0) -> MoeDesc:
    return MoeDesc(int(T), int(d), int(d_ff), int(E), int(k), GATE[gate], ACT[act], DTYPE[dtype],
                   float(cf), None, 0)


def desc_for(w, T=None) -> MoeDesc:
    """Description of a synth.Workload (optionally with another T)."""
    return make_desc(w.T if T is None else T, w.d, w.d_ff, w.E, w.k, w.gate, w.act, w.dtype, w.cf)


_lib = None


def load(build_if_missing: bool = True):
    """Load libmoe.so; build it first if it is not there."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        if not build_if_missing:
            raise RuntimeError(f"libmoe not built: {LIB_PATH} is missing")
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    D = ctypes.POINTER(MoeDesc)
    sz = ctypes.c_size_t
    lib.moe_workspace_size.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_capacity.argtypes = [D, ctypes.POINTER(ctypes.c_int64)]
    lib.moe_route.argtypes = [D, P, P, P, P, P, P, P, P, sz, P]
    lib.moe_dispatch.argtypes = [D, P, P, P, P, P, P, P, P, P, P, sz, P]
    lib.moe_expert_ffn.argtypes = [D, P, P, P, P, P, P, P, sz, P]
    lib.moe_combine.argtypes = [D, P, P, P, P, P]
    lib.moe_forward.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, sz, P]
    lib.moe_forward_noalloc.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P]
    SH = ctypes.POINTER(MoeShared)
    lib.moe_workspace_size_shared.argtypes = [D, SH, ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_shared_ffn.argtypes = [D, SH, P, P, P, sz, P]
    lib.moe_combine_shared.argtypes = [D, P, P, P, P, P, P, P]
    lib.moe_forward_shared.argtypes = [D, SH, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                       sz, P]
    F8 = ctypes.POINTER(MoeFp8Experts)
    lib.moe_quantize_e4m3.argtypes = [ctypes.c_int32, P, ctypes.c_int64, ctypes.c_int64, P, P, P]
    lib.moe_expert_ffn_fp8.argtypes = [D, P, P, F8, P, P, sz, P]
    lib.moe_forward_fp8.argtypes = [D, P, P, P, P, F8, P, P, P, P, P, P, P, P, P, P, P, sz, P]
    PK = ctypes.POINTER(MoePackedExperts)
    lib.moe_pack_stream.argtypes = [ctypes.c_int32, P, ctypes.c_int64, ctypes.c_int64, P, P]
    lib.moe_expert_ffn_packed.argtypes = [D, P, P, PK, P, P, sz, P]
    lib.moe_forward_packed.argtypes = [D, P, P, P, P, PK, P, P, P, P, P, P, P, P, P, P, P, sz, P]
    lib.moe_backward_workspace_size.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_backward.argtypes = [D] + [P] * 14 + [ctypes.c_float, ctypes.c_float] + [P] * 7 + [sz, P]
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    for fn in ("moe_workspace_size", "moe_capacity", "moe_route", "moe_dispatch",
               "moe_expert_ffn", "moe_combine", "moe_forward", "moe_workspace_size_shared",
               "moe_shared_ffn", "moe_combine_shared", "moe_forward_shared", "moe_quantize_e4m3",
               "moe_expert_ffn_fp8", "moe_forward_fp8", "moe_backward_workspace_size", "moe_backward",
               "moe_forward_noalloc", "moe_pack_stream", "moe_expert_ffn_packed", "moe_forward_packed"):
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(fn, rc):
    if rc != MOE_OK:
        raise MoeError(fn, rc)


def _ptr(t, dtype=None, shape=None, name="tensor", optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _act_dtype(desc):
    return torch.float32 if desc.dtype == DTYPE["f32"] else torch.bfloat16


def moe_workspace_size(desc: MoeDesc) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_workspace_size", load().moe_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def moe_capacity(desc: MoeDesc):
    c = ctypes.c_int64(0)
    _check("moe_capacity", load().moe_capacity(ctypes.byref(desc), ctypes.byref(c)))
    return None if c.value < 0 else c.value


def workspace(desc: MoeDesc, device="cuda", n_shared=None) -> torch.Tensor:
    """Workspace for desc (n_shared given: for the shared-expert entry points)."""
    n = moe_workspace_size(desc) if n_shared is None else \
        moe_workspace_size_shared(desc, MoeShared(int(n_shared), None, None, None, None))
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def make_shared(desc, Ws1=None, Ws3=None, Ws2=None, residual=None) -> MoeShared:
    """A moe_shared over device tensors (S = Ws1.shape[0], or 0 without Ws1);
    the tensors must outlive every call that is given the result."""
    T, d, d_ff = desc.T, desc.d, desc.d_ff
    dt = _act_dtype(desc)
    S = 0 if Ws1 is None else int(Ws1.shape[0])
    return MoeShared(S, _ptr(Ws1, dt, (S, d_ff, d), "Ws1", True),
                     _ptr(Ws3, dt, (S, d_ff, d), "Ws3", True),
                     _ptr(Ws2, dt, (S, d, d_ff), "Ws2", S == 0),
                     _ptr(residual, dt, (T, d), "residual", True))


def moe_workspace_size_shared(desc: MoeDesc, shared: MoeShared) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_workspace_size_shared",
           load().moe_workspace_size_shared(ctypes.byref(desc), ctypes.byref(shared), ctypes.byref(n)))
    return n.value


def moe_route(desc, x, W_r, bias, noise, topk_idx, gates, stats, ws, stream=None):
    T, d, E, k = desc.T, desc.d, desc.E, desc.k
    rc = load().moe_route(
        ctypes.byref(desc), _ptr(x, _act_dtype(desc), (T, d), "x"),
        _ptr(W_r, torch.float32, (E, d), "W_r"), _ptr(bias, torch.float32, (E,), "bias", True),
        _ptr(noise, torch.float32, (T, E), "noise", True),
        _ptr(topk_idx, torch.int32, (T, k), "topk_idx"), _ptr(gates, torch.float32, (T, k), "gates"),
        _ptr(stats, torch.float32, (2 * E + 2,), "stats"), _ptr(ws, torch.uint8, None, "ws"),
        ws.numel(), _stream(stream))
    _check("moe_route", rc)


def moe_dispatch(desc, x, topk_idx, routed_counts, kept_counts, offsets, row_of_slot, token_of_row,
                 dropped, x_perm, ws, stream=None):
    T, d, E, k = desc.T, desc.d, desc.E, desc.k
    rc = load().moe_dispatch(
        ctypes.byref(desc), _ptr(x, _act_dtype(desc), (T, d), "x"),
        _ptr(topk_idx, torch.int32, (T, k), "topk_idx"),
        _ptr(routed_counts, torch.int32, (E,), "routed_counts"),
        _ptr(kept_counts, torch.int32, (E,), "kept_counts"),
        _ptr(offsets, torch.int32, (E + 1,), "offsets"),
        _ptr(row_of_slot, torch.int32, (T, k), "row_of_slot"),
        _ptr(token_of_row, torch.int32, (T * k,), "token_of_row"),
        _ptr(dropped, torch.uint8, (T, k), "dropped"),
        _ptr(x_perm, _act_dtype(desc), (T * k, d), "x_perm"),
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream(stream))
    _check("moe_dispatch", rc)


def moe_expert_ffn(desc, x_perm, offsets, W1, W3, W2, y_perm, ws, stream=None):
    T, d, d_ff, E, k = desc.T, desc.d, desc.d_ff, desc.E, desc.k
    dt = _act_dtype(desc)
    rc = load().moe_expert_ffn(
        ctypes.byref(desc), _ptr(x_perm, dt, (T * k, d), "x_perm"),
        _ptr(offsets, torch.int32, (E + 1,), "offsets"), _ptr(W1, dt, (E, d_ff, d), "W1"),
        _ptr(W3, dt, (E, d_ff, d), "W3", True), _ptr(W2, dt, (E, d, d_ff), "W2"),
        _ptr(y_perm, torch.float32, (T * k, d), "y_perm"), _ptr(ws, torch.uint8, None, "ws"),
        ws.numel(), _stream(stream))
    _check("moe_expert_ffn", rc)


def moe_combine(desc, y_perm, row_of_slot, gates, y, stream=None):
    T, d, k = desc.T, desc.d, desc.k
    rc = load().moe_combine(
        ctypes.byref(desc), _ptr(y_perm, torch.float32, (T * k, d), "y_perm"),
        _ptr(row_of_slot, torch.int32, (T, k), "row_of_slot"),
        _ptr(gates, torch.float32, (T, k), "gates"), _ptr(y, _act_dtype(desc), (T, d), "y"),
        _stream(stream))
    _check("moe_combine", rc)


def moe_forward(desc, x, W_r, bias, noise, W1, W3, W2, y, ws, topk_idx=None, gates=None,
                routed_counts=None, kept_counts=None, offsets=None, row_of_slot=None,
                token_of_row=None, dropped=None, stats=None, stream=None):
    T, d, d_ff, E, k = desc.T, desc.d, desc.d_ff, desc.E, desc.k
    dt = _act_dtype(desc)
    rc = load().moe_forward(
        ctypes.byref(desc), _ptr(x, dt, (T, d), "x"), _ptr(W_r, torch.float32, (E, d), "W_r"),
        _ptr(bias, torch.float32, (E,), "bias", True),
        _ptr(noise, torch.float32, (T, E), "noise", True),
        _ptr(W1, dt, (E, d_ff, d), "W1"), _ptr(W3, dt, (E, d_ff, d), "W3", True),
        _ptr(W2, dt, (E, d, d_ff), "W2"), _ptr(y, dt, (T, d), "y"),
        _ptr(topk_idx, torch.int32, (T, k), "topk_idx", True),
        _ptr(gates, torch.float32, (T, k), "gates", True),
        _ptr(routed_counts, torch.int32, (E,), "routed_counts", True),
        _ptr(kept_counts, torch.int32, (E,), "kept_counts", True),
        _ptr(offsets, torch.int32, (E + 1,), "offsets", True),
        _ptr(row_of_slot, torch.int32, (T, k), "row_of_slot", True),
        _ptr(token_of_row, torch.int32, (T * k,), "token_of_row", True),
        _ptr(dropped, torch.uint8, (T, k), "dropped", True),
        _ptr(stats, torch.float32, (2 * E + 2,), "stats", True),
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream(stream))
    _check("moe_forward", rc)


def moe_forward_noalloc(desc, x, W_r, bias, noise, W1, W3, W2, y, topk_idx=None, gates=None,
                        routed_counts=None, kept_counts=None, offsets=None, row_of_slot=None,
                        token_of_row=None, dropped=None, stats=None, stream=None):
    """moe_forward with the library's static device scratch as its workspace
    (no workspace argument; calls on one device must not overlap)."""
    T, d, d_ff, E, k = desc.T, desc.d, desc.d_ff, desc.E, desc.k
    dt = _act_dtype(desc)
    rc = load().moe_forward_noalloc(
        ctypes.byref(desc), _ptr(x, dt, (T, d), "x"), _ptr(W_r, torch.float32, (E, d), "W_r"),
        _ptr(bias, torch.float32, (E,), "bias", True),
        _ptr(noise, torch.float32, (T, E), "noise", True),
        _ptr(W1, dt, (E, d_ff, d), "W1"), _ptr(W3, dt, (E, d_ff, d), "W3", True),
        _ptr(W2, dt, (E, d, d_ff), "W2"), _ptr(y, dt, (T, d), "y"),
        _ptr(topk_idx, torch.int32, (T, k), "topk_idx", True),
        _ptr(gates, torch.float32, (T, k), "gates", True),
        _ptr(routed_counts, torch.int32, (E,), "routed_counts", True),
        _ptr(kept_counts, torch.int32, (E,), "kept_counts", True),
        _ptr(offsets, torch.int32, (E + 1,), "offsets", True),
        _ptr(row_of_slot, torch.int32, (T, k), "row_of_slot", True),
        _ptr(token_of_row, torch.int32, (T * k,), "token_of_row", True),
        _ptr(dropped, torch.uint8, (T, k), "dropped", True),
        _ptr(stats, torch.float32, (2 * E + 2,), "stats", True), _stream(stream))
    _check("moe_forward_noalloc", rc)


def moe_shared_ffn(desc, shared: MoeShared, x, y_shared, ws, stream=None):
    T, d, S = desc.T, desc.d, shared.n_shared
    rc = load().moe_shared_ffn(
        ctypes.byref(desc), ctypes.byref(shared), _ptr(x, _act_dtype(desc), (T, d), "x"),
        _ptr(y_shared, torch.float32, (T, d), "y_shared", S == 0), _ptr(ws, torch.uint8, None, "ws"),
        ws.numel(), _stream(stream))
    _check("moe_shared_ffn", rc)


def moe_combine_shared(desc, y_perm, row_of_slot, gates, y_shared, residual, y, stream=None):
    T, d, k = desc.T, desc.d, desc.k
    dt = _act_dtype(desc)
    rc = load().moe_combine_shared(
        ctypes.byref(desc), _ptr(y_perm, torch.float32, (T * k, d), "y_perm"),
        _ptr(row_of_slot, torch.int32, (T, k), "row_of_slot"),
        _ptr(gates, torch.float32, (T, k), "gates"),
        _ptr(y_shared, torch.float32, (T, d), "y_shared", True),
        _ptr(residual, dt, (T, d), "residual", True), _ptr(y, dt, (T, d), "y"), _stream(stream))
    _check("moe_combine_shared", rc)


def moe_forward_shared(desc, shared: MoeShared, x, W_r, bias, noise, W1, W3, W2, y, ws,
                       topk_idx=None, gates=None, routed_counts=None, kept_counts=None,
                       offsets=None, row_of_slot=None, token_of_row=None, dropped=None,
                       stats=None, stream=None):
    T, d, d_ff, E, k = desc.T, desc.d, desc.d_ff, desc.E, desc.k
    dt = _act_dtype(desc)
    rc = load().moe_forward_shared(
        ctypes.byref(desc), ctypes.byref(shared), _ptr(x, dt, (T, d), "x"),
        _ptr(W_r, torch.float32, (E, d), "W_r"),
        _ptr(bias, torch.float32, (E,), "bias", True),
        _ptr(noise, torch.float32, (T, E), "noise", True),
        _ptr(W1, dt, (E, d_ff, d), "W1"), _ptr(W3, dt, (E, d_ff, d), "W3", True),
        _ptr(W2, dt, (E, d, d_ff), "W2"), _ptr(y, dt, (T, d), "y"),
        _ptr(topk_idx, torch.int32, (T, k), "topk_idx", True),
        _ptr(gates, torch.float32, (T, k), "gates", True),
        _ptr(routed_counts, torch.int32, (E,), "routed_counts", True),
        _ptr(kept_counts, torch.int32, (E,), "kept_counts", True),
        _ptr(offsets, torch.int32, (E + 1,), "offsets", True),
        _ptr(row_of_slot, torch.int32, (T, k), "row_of_slot", True),
        _ptr(token_of_row, torch.int32, (T * k,), "token_of_row", True),
        _ptr(dropped, torch.uint8, (T, k), "dropped", True),
        _ptr(stats, torch.float32, (2 * E + 2,), "stats", True),
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream(stream))
    _check("moe_forward_shared", rc)


def moe_quantize_e4m3(W, q, scales, stream=None):
    """Row-wise E4M3 quantisation of W [..., cols] (bf16 or fp32) into q
    (uint8, W's shape) and scales (fp32, W.shape[:-1])."""
    if W.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("W must be bf16 or fp32")
    cols = int(W.shape[-1])
    rows = W.numel() // cols if cols else 0
    dt = DTYPE["bf16"] if W.dtype == torch.bfloat16 else DTYPE["f32"]
    rc = load().moe_quantize_e4m3(dt, _ptr(W, None, None, "W"), rows, cols,
                                  _ptr(q, torch.uint8, tuple(W.shape), "q"),
                                  _ptr(scales, torch.float32, tuple(W.shape[:-1]), "scales"),
                                  _stream(stream))
    _check("moe_quantize_e4m3", rc)


def quantize_experts(W1, W3, W2, stream=None) -> dict:
    """E4M3 codes and row scales of expert weights (device tensors):
    q1, q3, q2 (uint8) and s1, s3, s2 (fp32); W3 may be None."""
    out = {}
    for name, W in (("1", W1), ("3", W3), ("2", W2)):
        if W is None:
            out["q" + name] = out["s" + name] = None
            continue
        q = torch.empty(W.shape, dtype=torch.uint8, device=W.device)
        sc = torch.empty(W.shape[:-1], dtype=torch.float32, device=W.device)
        moe_quantize_e4m3(W, q, sc, stream)
        out["q" + name], out["s" + name] = q, sc
    return out


def make_fp8(desc, q1, q3, q2, s1, s3, s2) -> MoeFp8Experts:
    """A moe_fp8_experts over device tensors (they must outlive its use)."""
    d, d_ff, E = desc.d, desc.d_ff, desc.E
    return MoeFp8Experts(_ptr(q1, torch.uint8, (E, d_ff, d), "q1"),
                         _ptr(q3, torch.uint8, (E, d_ff, d), "q3", True),
                         _ptr(q2, torch.uint8, (E, d, d_ff), "q2"),
                         _ptr(s1, torch.float32, (E, d_ff), "s1"),
                         _ptr(s3, torch.float32, (E, d_ff), "s3", True),
                         _ptr(s2, torch.float32, (E, d), "s2"))


def moe_expert_ffn_fp8(desc, x_perm, offsets, fp8: MoeFp8Experts, y_perm, ws, stream=None):
    T, d, E, k = desc.T, desc.d, desc.E, desc.k
    rc = load().moe_expert_ffn_fp8(
        ctypes.byref(desc), _ptr(x_perm, _act_dtype(desc), (T * k, d), "x_perm"),
        _ptr(offsets, torch.int32, (E + 1,), "offsets"), ctypes.byref(fp8),
        _ptr(y_perm, torch.float32, (T * k, d), "y_perm"), _ptr(ws, torch.uint8, None, "ws"),
        ws.numel(), _stream(stream))
    _check("moe_expert_ffn_fp8", rc)


def moe_forward_fp8(desc, fp8: MoeFp8Experts, x, W_r, bias, noise, y, ws, topk_idx=None,
                    gates=None, routed_counts=None, kept_counts=None, offsets=None,
                    row_of_slot=None, token_of_row=None, dropped=None, stats=None, stream=None):
    T, d, E, k = desc.T, desc.d, desc.E, desc.k
    dt = _act_dtype(desc)
    rc = load().moe_forward_fp8(
        ctypes.byref(desc), _ptr(x, dt, (T, d), "x"), _ptr(W_r, torch.float32, (E, d), "W_r"),
        _ptr(bias, torch.float32, (E,), "bias", True),
        _ptr(noise, torch.float32, (T, E), "noise", True), ctypes.byref(fp8),
        _ptr(y, dt, (T, d), "y"),
        _ptr(topk_idx, torch.int32, (T, k), "topk_idx", True),
        _ptr(gates, torch.float32, (T, k), "gates", True),
        _ptr(routed_counts, torch.int32, (E,), "routed_counts", True),
        _ptr(kept_counts, torch.int32, (E,), "kept_counts", True),
        _ptr(offsets, torch.int32, (E + 1,), "offsets", True),
        _ptr(row_of_slot, torch.int32, (T, k), "row_of_slot", True),
        _ptr(token_of_row, torch.int32, (T * k,), "token_of_row", True),
        _ptr(dropped, torch.uint8, (T, k), "dropped", True),
        _ptr(stats, torch.float32, (2 * E + 2,), "stats", True),
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream(stream))
    _check("moe_forward_fp8", rc)


def moe_pack_stream(W, out, stream=None):
    """W [..., cols] (bf16, or uint8 e4m3 codes) viewed as [rows][cols] ->
    out (same dtype and shape) in the streaming tile layout."""
    if W.dtype not in (torch.bfloat16, torch.uint8):
        raise TypeError("W must be bf16 or uint8 (e4m3 codes)")
    cols = int(W.shape[-1])
    rows = W.numel() // cols if cols else 0
    rc = load().moe_pack_stream(2 if W.dtype == torch.bfloat16 else 1, _ptr(W, None, None, "W"), rows, cols,
                                _ptr(out, W.dtype, tuple(W.shape), "out"), _stream(stream))
    _check("moe_pack_stream", rc)


def pack_experts(W1, W3, W2, stream=None) -> dict:
    """Packed copies p1, p3, p2 of expert weights or codes (W3 may be None)."""
    out = {}
    for name, W in (("1", W1), ("3", W3), ("2", W2)):
        if W is None:
            out["p" + name] = None
            continue
        pk = torch.empty_like(W)
        moe_pack_stream(W, pk, stream)
        out["p" + name] = pk
    return out


def make_packed(desc, fmt, p1, p3, p2, s1=None, s3=None, s2=None) -> MoePackedExperts:
    """A moe_packed_experts over device tensors (they must outlive its use);
    fmt "bf16" (no scales) or "e4m3" (codes with row scales)."""
    d, d_ff, E = desc.d, desc.d_ff, desc.E
    wt = torch.bfloat16 if fmt == "bf16" else torch.uint8
    return MoePackedExperts(WEIGHTS[fmt],
                            _ptr(p1, wt, (E, d_ff, d), "p1"),
                            _ptr(p3, wt, (E, d_ff, d), "p3", True),
                            _ptr(p2, wt, (E, d, d_ff), "p2"),
                            _ptr(s1, torch.float32, (E, d_ff), "s1", True),
                            _ptr(s3, torch.float32, (E, d_ff), "s3", True),
                            _ptr(s2, torch.float32, (E, d), "s2", True))


def moe_expert_ffn_packed(desc, x_perm, offsets, pk: MoePackedExperts, y_perm, ws, stream=None):
    T, d, E, k = desc.T, desc.d, desc.E, desc.k
    rc = load().moe_expert_ffn_packed(
        ctypes.byref(desc), _ptr(x_perm, _act_dtype(desc), (T * k, d), "x_perm"),
        _ptr(offsets, torch.int32, (E + 1,), "offsets"), ctypes.byref(pk),
        _ptr(y_perm, torch.float32, (T * k, d), "y_perm"), _ptr(ws, torch.uint8, None, "ws"),
        ws.numel(), _stream(stream))
    _check("moe_expert_ffn_packed", rc)


def moe_forward_packed(desc, pk: MoePackedExperts, x, W_r, bias, noise, y, ws, topk_idx=None,
                       gates=None, routed_counts=None, kept_counts=None, offsets=None,
                       row_of_slot=None, token_of_row=None, dropped=None, stats=None, stream=None):
    T, d, E, k = desc.T, desc.d, desc.E, desc.k
    dt = _act_dtype(desc)
    rc = load().moe_forward_packed(
        ctypes.byref(desc), _ptr(x, dt, (T, d), "x"), _ptr(W_r, torch.float32, (E, d), "W_r"),
        _ptr(bias, torch.float32, (E,), "bias", True),
        _ptr(noise, torch.float32, (T, E), "noise", True), ctypes.byref(pk),
        _ptr(y, dt, (T, d), "y"),
        _ptr(topk_idx, torch.int32, (T, k), "topk_idx", True),
        _ptr(gates, torch.float32, (T, k), "gates", True),
        _ptr(routed_counts, torch.int32, (E,), "routed_counts", True),
        _ptr(kept_counts, torch.int32, (E,), "kept_counts", True),
        _ptr(offsets, torch.int32, (E + 1,), "offsets", True),
        _ptr(row_of_slot, torch.int32, (T, k), "row_of_slot", True),
        _ptr(token_of_row, torch.int32, (T * k,), "token_of_row", True),
        _ptr(dropped, torch.uint8, (T, k), "dropped", True),
        _ptr(stats, torch.float32, (2 * E + 2,), "stats", True),
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream(stream))
    _check("moe_forward_packed", rc)


def moe_backward_workspace_size(desc: MoeDesc) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_backward_workspace_size",
           load().moe_backward_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def backward_workspace(desc: MoeDesc, device="cuda") -> torch.Tensor:
    return torch.empty(max(moe_backward_workspace_size(desc), 1), dtype=torch.uint8, device=device)


def alloc_grads(desc, bias=False, device="cuda") -> dict:
    T, d, d_ff, E = desc.T, desc.d, desc.d_ff, desc.E
    f32 = dict(dtype=torch.float32, device=device)
    return dict(dx=torch.empty((T, d), **f32), dW_r=torch.empty((E, d), **f32),
                dbias=torch.empty((E,), **f32) if bias else None,
                dW1=torch.empty((E, d_ff, d), **f32),
                dW3=torch.empty((E, d_ff, d), **f32) if desc.act == ACT["swiglu"] else None,
                dW2=torch.empty((E, d, d_ff), **f32))


def moe_backward(desc, x, W_r, bias, noise, W1, W3, W2, fwd: dict, dy, grads: dict, ws,
                 alpha_aux=0.0, alpha_z=0.0, stream=None):
    """Gradients for the routing of a moe_forward call whose outputs are in
    ``fwd`` (topk_idx, gates, offsets, row_of_slot, token_of_row, stats)."""
    T, d, d_ff, E, k = desc.T, desc.d, desc.d_ff, desc.E, desc.k
    dt = _act_dtype(desc)
    rc = load().moe_backward(
        ctypes.byref(desc), _ptr(x, dt, (T, d), "x"), _ptr(W_r, torch.float32, (E, d), "W_r"),
        _ptr(bias, torch.float32, (E,), "bias", True),
        _ptr(noise, torch.float32, (T, E), "noise", True),
        _ptr(W1, dt, (E, d_ff, d), "W1"), _ptr(W3, dt, (E, d_ff, d), "W3", True),
        _ptr(W2, dt, (E, d, d_ff), "W2"),
        _ptr(fwd["topk_idx"], torch.int32, (T, k), "topk_idx"),
        _ptr(fwd["gates"], torch.float32, (T, k), "gates"),
        _ptr(fwd["offsets"], torch.int32, (E + 1,), "offsets"),
        _ptr(fwd["row_of_slot"], torch.int32, (T, k), "row_of_slot"),
        _ptr(fwd["token_of_row"], torch.int32, (T * k,), "token_of_row"),
        _ptr(fwd["stats"], torch.float32, (2 * E + 2,), "stats"),
        _ptr(dy, dt, (T, d), "dy"), float(alpha_aux), float(alpha_z),
        _ptr(grads["dx"], torch.float32, (T, d), "dx"),
        _ptr(grads["dW_r"], torch.float32, (E, d), "dW_r"),
        _ptr(grads.get("dbias"), torch.float32, (E,), "dbias", True),
        _ptr(grads["dW1"], torch.float32, (E, d_ff, d), "dW1"),
        _ptr(grads.get("dW3"), torch.float32, (E, d_ff, d), "dW3", True),
        _ptr(grads["dW2"], torch.float32, (E, d, d_ff), "dW2"),
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream(stream))
    _check("moe_backward", rc)


def status_string(code: int) -> str:
    return load().moe_status_string(int(code)).decode()


# ---- helpers for callers holding synth inputs (host numpy arrays) ----------

def to_device(a, dtype_name, device="cuda"):
    """A synth array (uint16 bf16 bits or float32) as a device tensor of the
    matching torch dtype (bf16 bits are reinterpreted, not converted)."""
    import numpy as np
    if a is None:
        return None
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)


def alloc_outputs(desc, device="cuda") -> dict:
    T, d, E, k = desc.T, desc.d, desc.E, desc.k
    dt = _act_dtype(desc)
    i32 = dict(dtype=torch.int32, device=device)
    return dict(
        y=torch.empty((T, d), dtype=dt, device=device),
        topk_idx=torch.empty((T, k), **i32), gates=torch.empty((T, k), dtype=torch.float32, device=device),
        routed_counts=torch.empty((E,), **i32), kept_counts=torch.empty((E,), **i32),
        offsets=torch.empty((E + 1,), **i32), row_of_slot=torch.empty((T, k), **i32),
        token_of_row=torch.empty((T * k,), **i32),
        dropped=torch.empty((T, k), dtype=torch.uint8, device=device),
        stats=torch.empty((2 * E + 2,), dtype=torch.float32, device=device))
