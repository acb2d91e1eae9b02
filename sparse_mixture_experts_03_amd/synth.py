"""Seeded synthetic inputs for the sparse-MoE layer.

This module only draws random numbers and lays them out; it holds none of
the layer's arithmetic.  Both the CPU oracle side and the GPU side take
their inputs from here, so that both see the same values.

Recipe (workload shapes follow the configurations the layer is measured
on; the distributions are stated per tensor):
  * every tensor comes from its own Philox4x32 stream keyed by
    (seed, crc32(tensor name), step[, row, attempt]) through numpy's
    SeedSequence, so any tensor or single row can be regenerated alone;
  * router W_r [E][d] fp32 ~ N(0, std 1/sqrt(d));
  * experts W1, W3 [E][d_ff][d] ~ N(0, std 1/sqrt(d)),
    W2 [E][d][d_ff] ~ N(0, std 1/sqrt(d_ff)); stored as bf16 (round to
    nearest even from the fp32 draw) for bf16 workloads, fp32 otherwise;
  * tokens x [T][d] ~ N(0, 1); for the Mixtral-shape workloads each row is
    RMS-normalised (divided by sqrt(mean_j x_j^2), no epsilon, no gain),
    then stored like the weights;
  * logit noise [T][E] fp32 ~ N(0, std noise_std) where the workload asks
    for it (the Switch-style layer: std 1/E);
  * router bias [E] fp32 for the Zipf workload: b_i = 2 ln w_{i+1}, with
    w_r = r^-s / sum_{j=1..E} j^-s (s = 1.1), expert i at rank i+1;
  * shared experts (workloads with n_shared > 0): Ws1, Ws3 [S][d_ff][d],
    Ws2 [S][d][d_ff], drawn and stored like the routed experts' weights;
  * block residual h [T][d] (workloads with residual): N(0, 1), stored
    like x, not normalised.
A row that has to be drawn again (rejection of near-tied logits is done by
the caller) comes from the stream (seed, name, step, row, attempt).

bf16 tensors are numpy uint16 arrays holding the bf16 bit patterns; use
``widen`` for their exact fp32 values.
"""
from __future__ import annotations

import os
import zlib
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    d_ff: int
    E: int
    k: int
    gate: str            # "renorm" | "switch"
    cf: float            # capacity factor, 0 = no limit
    act: str             # "relu" | "gelu" | "swiglu"
    dtype: str           # "f32" | "bf16" (experts and activations; router is fp32)
    x_rmsnorm: bool = False
    noise_std: float = 0.0
    zipf_s: float = 0.0  # > 0: Zipf router bias
    steps: int = 1       # decode: fresh x per step
    n_shared: int = 0    # shared experts every token visits
    residual: bool = False  # block residual added to the layer output
    weights: str = "act"    # "act": experts in the act dtype; "e4m3": quantised from those

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # Tiny fp32 layer: T=64, d=32, E=4, top-2 renormalised, ReLU d->64->d, no capacity.
    "tiny": Workload("tiny", 64, 32, 64, 4, 2, "renorm", 0.0, "relu", "f32"),
    # Switch-style: T=4096, d=768, d_ff=3072, E=128, k=1, full-softmax gate, cf=1.25,
    # GELU, bf16, logit noise std 1/E.
    "switch": Workload("switch", 4096, 768, 3072, 128, 1, "switch", 1.25, "gelu", "bf16",
                       noise_std=1.0 / 128),
    # Mixtral-8x7B-shape layer, prefill: T=4096, d=4096, d_ff=14336, E=8, top-2, SwiGLU.
    "mixtral_prefill": Workload("mixtral_prefill", 4096, 4096, 14336, 8, 2, "renorm", 0.0,
                                "swiglu", "bf16", x_rmsnorm=True),
    # Same layer, decode: 32 sequences x 1 token, 100 steps with fresh x.
    "mixtral_decode": Workload("mixtral_decode", 32, 4096, 14336, 8, 2, "renorm", 0.0,
                               "swiglu", "bf16", x_rmsnorm=True, steps=100),
    # Fine-grained, Zipf-skewed routing: T=16384, d=2048, d_ff=768, E=128, top-4, cf=1.0.
    "finegrained_zipf": Workload("finegrained_zipf", 16384, 2048, 768, 128, 4, "renorm", 1.0,
                                 "swiglu", "bf16", zipf_s=1.1),
    # Shared-expert variants (section "Total versus active parameters": many
    # small routed experts plus shared experts every token visits), with the
    # block residual: the fine-grained layer with two shared experts of its
    # own expert shape, and the Mixtral-shape prefill layer with one.
    "finegrained_zipf_shared": Workload("finegrained_zipf_shared", 16384, 2048, 768, 128, 4,
                                        "renorm", 1.0, "swiglu", "bf16", zipf_s=1.1,
                                        n_shared=2, residual=True),
    "mixtral_prefill_shared": Workload("mixtral_prefill_shared", 4096, 4096, 14336, 8, 2,
                                       "renorm", 0.0, "swiglu", "bf16", x_rmsnorm=True,
                                       n_shared=1, residual=True),
    # The Mixtral-shape decode layer with its expert weights quantised row
    # by row to e4m3 (from the bf16 draws; the quantisation itself is the
    # library's or the oracle's, not this module's).
    "mixtral_decode_fp8": Workload("mixtral_decode_fp8", 32, 4096, 14336, 8, 2, "renorm", 0.0,
                                   "swiglu", "bf16", x_rmsnorm=True, steps=100, weights="e4m3"),
    # The Switch-shape layer with e4m3 expert weights (at most 40 rows per
    # expert: the weight-streaming kernels).
    "switch_fp8": Workload("switch_fp8", 4096, 768, 3072, 128, 1, "switch", 1.25, "gelu", "bf16",
                           noise_std=1.0 / 128, weights="e4m3"),
}


def _stream(seed: int, name: str, *more: int) -> np.random.Generator:
    ss = np.random.SeedSequence([int(seed), zlib.crc32(name.encode())] + [int(m) for m in more])
    return np.random.Generator(np.random.Philox(ss))


def to_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def widen(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp32 values; fp32 passes through."""
    if bits.dtype == np.float32:
        return bits
    assert bits.dtype == np.uint16
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _store(w: Workload, a32: np.ndarray) -> np.ndarray:
    return to_bf16(a32) if w.dtype == "bf16" else np.ascontiguousarray(a32, np.float32)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def make_weights(w: Workload, seed: int = 0, experts: int | None = None) -> dict:
    """Router and expert weights of workload ``w``.  ``experts`` (default E)
    limits how many experts' FFN weights are drawn (expert e always comes
    from the same stream, so a prefix is a prefix of the full set)."""
    E = w.E if experts is None else experts
    out = {"Wr": _normal(_stream(seed, "Wr"), (w.E, w.d), 1.0 / np.sqrt(w.d))}
    if w.zipf_s > 0:
        r = np.arange(1, w.E + 1, dtype=np.float64)
        pmf = r ** (-w.zipf_s)
        pmf /= pmf.sum()
        out["bias"] = (2.0 * np.log(pmf)).astype(np.float32)
    else:
        out["bias"] = None
    names = [("W1", (w.d_ff, w.d), 1.0 / np.sqrt(w.d)), ("W2", (w.d, w.d_ff), 1.0 / np.sqrt(w.d_ff))]
    if w.act == "swiglu":
        names.append(("W3", (w.d_ff, w.d), 1.0 / np.sqrt(w.d)))
    sdt = np.uint16 if w.dtype == "bf16" else np.float32
    for name, shape, std in names:
        out[name] = np.empty((E,) + shape, sdt)

    def one(job):
        name, shape, std, e = job
        out[name][e] = _store(w, _normal(_stream(seed, name, e), shape, std))

    jobs = [(n, s, sd, e) for (n, s, sd) in names for e in range(E)]
    S = w.n_shared
    if S > 0:
        for name, shape, std in names:
            out["Ws" + name[1:]] = np.empty((S,) + shape, sdt)
        jobs += [("Ws" + n[1:], s, sd, j) for (n, s, sd) in names for j in range(S)]
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, jobs))
    if "W3" not in out:
        out["W3"] = None
    for name in ("Ws1", "Ws3", "Ws2"):
        out.setdefault(name, None)
    return out


def _x_rows(w: Workload, rng: np.random.Generator, n: int) -> np.ndarray:
    x = rng.standard_normal((n, w.d), dtype=np.float32)
    if w.x_rmsnorm:
        rms = np.sqrt(np.mean(x.astype(np.float64) ** 2, axis=1, keepdims=True))
        x = (x / rms).astype(np.float32)
    return x


def make_tokens(w: Workload, seed: int = 0, step: int = 0) -> dict:
    """Tokens x (stored dtype) and logit noise (fp32 or None) for one step."""
    x = _store(w, _x_rows(w, _stream(seed, "x", step), w.T))
    noise = None
    if w.noise_std > 0:
        noise = _normal(_stream(seed, "noise", step), (w.T, w.E), w.noise_std)
    res = _store(w, _normal(_stream(seed, "res", step), (w.T, w.d), 1.0)) if w.residual else None
    return {"x": x, "noise": noise, "res": res}


def redraw_token(w: Workload, seed: int, step: int, t: int, attempt: int):
    """A fresh draw of token row t (and its noise row) for retry ``attempt`` >= 1."""
    x = _store(w, _x_rows(w, _stream(seed, "x", step, t, attempt), 1))[0]
    noise = None
    if w.noise_std > 0:
        noise = _normal(_stream(seed, "noise", step, t, attempt), (w.E,), w.noise_std)
    return x, noise
