"""Benchmark of the sparse-MoE layer forward on one MI355X.

One step = one moe_forward call (router, top-k, dispatch with capacity,
gather, grouped expert GEMMs, combine, statistics) over one batch of
seeded synthetic tokens, inputs resident in HBM before the timed region.

Default workload: the Mixtral-8x7B-shape layer in prefill (T=4096, d=4096,
d_ff=14336, E=8, top-2, SwiGLU, bf16 experts, fp32 router); the same layer
in decode (T=32, 100 steps with fresh tokens each step) is measured in the
same run and reported in the "decode" object.  Prints one JSON line.

Timing: W untimed warm-up steps, then exactly K steps between two device
synchronisations.  The dominant kernel's duration comes from two HIP
events that the library records on the launch stream around it (the
descriptor's stage-event hook), over the same timed steps.

The default line also carries "decode_fp8": the decode layer with its
expert weights quantised row by row to e4m3 (one fp32 scale per row) before
timing (weights 1 byte, activations bf16).

The weight-streaming layers (decode, decode_fp8 and the Switch layer, whose
experts hold at most 48 rows) are timed on expert weights re-ordered once,
before timing, into the streaming tile layout (moe_pack_stream; then
moe_forward_packed), which gives the same results bit for bit as row-major
weights; each of their objects carries the row-major entry point's
(moe_forward, moe_forward_fp8) figures beside, under "row_major".
"switch_fp8" is the Switch layer again with its expert weights quantised
to e4m3 and packed before timing, against 8 TB/s over its bytes (1-byte
codes plus a 4-byte scale per weight row).

Roofline of the dominant kernel (the expert up-projection, a grouped GEMM
on bf16 MFMA): algorithmic FLOPs per launch = N_kept * 2 * n_up * d * d_ff
(n_up = 2 matrices for SwiGLU) over its mean event-timed duration, against
the 2.5 PFLOP/s dense bf16 peak.  Decode is bound by HBM: algorithmic bytes
per launch = the touched experts' W1 and W3 (2 * d * d_ff * 2 bytes each)
plus the permuted activations in and H out, against 8 TB/s.

Shared-expert workloads (--workload finegrained_zipf_shared or
mixtral_prefill_shared) run moe_forward_shared: the same stages plus the
shared experts on every token and the block residual fused into the
combine.  Their FLOPs add S * T * 2 * n_mat * d * d_ff, and the line adds a
"shared_stage" object: those FLOPs over the event-timed shared stage.

CPU baseline: the CPU oracle (test infrastructure; fp64 sums) timed on this
host on a bounded sample: routing, dispatch and statistics over all T
tokens plus the expert FFN and combine on S sampled tokens; tokens/s is
1 / (t_route / T + t_ffn / S).

The default line also carries "switch" and "finegrained_zipf": the
Switch-style and fine-grained Zipf layers, HBM-bound, each timed over
--layer-steps steps with the last-level cache flushed (a 512 MB device
fill) before every step (median, minimum, 90th percentile), against 8 TB/s
over their algorithmic bytes: the touched experts' weights (from the run's
kept counts) + x + y + W_r (+ the noise input); plus their dominant
kernel's event-timed rate.  "sclk" samples the shader clock and socket
power (amdsmi; each refresh of its metrics table counted once) while
prefill steps run back to back for about three seconds; "cpu_baseline_1thread"
times the oracle on one host thread for the tiny layer and the decode
layer.

--backward times moe_backward (training gradients, routing of one forward
held fixed) on the workload instead, and prints its own JSON line; --cold
flushes the last-level cache (a 512 MB device fill) before every forward
step and reports per-step median, minimum and 90th percentile;
--library-gemm times torch's own GEMM (hipBLASLt) on the up projection's
FLOPs for context.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-cpu] [--no-decode] [--backward] [--cold]
                       [--library-gemm] [--packed]
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s + % bf16 MFMA peak (prefill) / % HBM BW (decode), Mixtral-shape"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
STAGES = ("route", "route_finalize", "dispatch", "gather", "expert_up", "expert_down", "combine")
STAGES_SHARED = ("route", "route_finalize", "dispatch", "gather", "expert_up", "expert_down",
                 "shared", "combine")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
LAYOUT_PACKED = ("streaming tile layout (moe_pack_stream once before timing; moe_forward_packed; "
                 "the same values and results bit for bit as row-major)")
GEMM_SRCS = [os.path.join(ROOT, "sparse_mixture_experts_03_amd", "csrc", f)
             for f in ("expert_gemm.hip", "expert_fp8.hip")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles from the HIP runtime (the library records them)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n, keep=None):
        """An array of n event handles; slots outside ``keep`` stay NULL."""
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            if keep is not None and i not in keep:
                continue
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            arr[i] = e
        return arr

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value

    def destroy(self, arr):
        for e in arr:
            if e:
                self.hip.hipEventDestroy(e)


def source_sha():
    """Hash of the GEMM kernel sources (the bf16 and the e4m3 ones)."""
    h = hashlib.sha256()
    for path in GEMM_SRCS:
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(workload, kernel, launches_per_step=1):
    """HBM bytes per launch of ``kernel`` from the committed rocprofv3 counter
    summary, or None when absent or taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("gemm_source_sha") != source_sha():
        return None
    ent = rec.get("kernels", {}).get(f"{workload}/{kernel}")
    if not ent:
        return None
    return ent["hbm_bytes_per_launch"]


def pack_weights(w, desc, dw, f8):
    """The expert weights of a weight-streaming layer (bf16 values, or the
    e4m3 codes f8) re-ordered once into the streaming tile layout
    (moe_pack_stream), before any timing; the row-major copies are freed.
    Returns the moe_packed_experts and the tensors it points to."""
    from sparse_mixture_experts_03_amd import binding as B

    if f8 is not None:
        t = B.pack_experts(f8["q1"], f8["q3"], f8["q2"])
        t.update(s1=f8["s1"], s3=f8["s3"], s2=f8["s2"])
        pk = B.make_packed(desc, "e4m3", t["p1"], t["p3"], t["p2"], t["s1"], t["s3"], t["s2"])
        for key in ("q1", "q3", "q2"):
            f8[key] = None
    else:
        t = B.pack_experts(dw["W1"], dw["W3"], dw["W2"])
        pk = B.make_packed(desc, "bf16", t["p1"], t["p3"], t["p2"])
        for key in ("W1", "W3", "W2"):
            dw[key] = None
    return pk, t


def run_workload(w, steps, warmup, fresh_x_steps=0, seed=0, sclk_seconds=0.0, packed=False):
    """Times ``steps`` forward steps of workload w. Returns a result dict
    (with sclk_seconds > 0 also the shader clock sampled afterwards while
    steps run back to back for that long, outside the timed region).
    packed: expert weights in the streaming tile layout, moe_forward_packed."""
    import torch
    from sparse_mixture_experts_03_amd import binding as B
    from sparse_mixture_experts_03_amd import synth

    t0 = time.time()
    wt = synth.make_weights(w, seed)
    dw = {k: B.to_device(v, w.dtype) for k, v in wt.items()}
    del wt
    f8 = None
    if w.weights == "e4m3":
        # post-training quantisation of the expert weights, before timing
        f8 = B.quantize_experts(dw["W1"], dw["W3"], dw["W2"])
        for key in ("W1", "W3", "W2"):
            dw[key] = None
        torch.cuda.synchronize()
    n_x = max(1, fresh_x_steps)
    xs, noises, ress = [], [], []
    for s in range(n_x):
        tk = synth.make_tokens(w, seed, s)
        xs.append(B.to_device(tk["x"], w.dtype))
        noises.append(B.to_device(tk["noise"], w.dtype))
        ress.append(B.to_device(tk["res"], w.dtype))
    log(f"[bench] {w.name}: inputs ready in {time.time() - t0:.1f}s")

    desc = B.desc_for(w)
    # shared experts and/or the block residual: moe_forward_shared
    with_shared = w.n_shared > 0 or w.residual
    stages = STAGES_SHARED if with_shared else STAGES
    ws = B.workspace(desc, n_shared=w.n_shared if with_shared else None)
    shs = [B.make_shared(desc, dw["Ws1"], dw["Ws3"], dw["Ws2"], ress[j]) for j in range(n_x)] \
        if with_shared else None
    out = B.alloc_outputs(desc)
    pk = None
    if packed:
        pk, pk_tensors = pack_weights(w, desc, dw, f8)  # noqa: F841  (kept alive for the steps)
        f8 = None
        torch.cuda.synchronize()
    fp8 = B.make_fp8(desc, f8["q1"], f8["q3"], f8["q2"], f8["s1"], f8["s3"], f8["s2"]) if f8 else None
    ev = HipEvents()
    nev = len(stages) + 1
    stream = torch.cuda.current_stream()

    def step(i, events=None):
        j = i % n_x
        if events is not None:
            desc.stage_events = ctypes.cast(events, ctypes.POINTER(ctypes.c_void_p))
            desc.n_stage_events = nev
        else:
            desc.stage_events = None
            desc.n_stage_events = 0
        # only the two events around the expert up-projection (the dominant
        # kernel) are recorded: each recorded event separates the kernels
        # around it by a few us
        if pk is not None:
            B.moe_forward_packed(desc, pk, xs[j], dw["Wr"], dw["bias"], noises[j], out["y"], ws,
                                 kept_counts=out["kept_counts"], stats=out["stats"], stream=stream)
        elif fp8 is not None:
            B.moe_forward_fp8(desc, fp8, xs[j], dw["Wr"], dw["bias"], noises[j], out["y"], ws,
                              kept_counts=out["kept_counts"], stats=out["stats"], stream=stream)
        elif with_shared:
            B.moe_forward_shared(desc, shs[j], xs[j], dw["Wr"], dw["bias"], noises[j], dw["W1"],
                                 dw["W3"], dw["W2"], out["y"], ws, kept_counts=out["kept_counts"],
                                 stats=out["stats"], stream=stream)
        else:
            B.moe_forward(desc, xs[j], dw["Wr"], dw["bias"], noises[j], dw["W1"], dw["W3"],
                          dw["W2"], out["y"], ws, kept_counts=out["kept_counts"],
                          stats=out["stats"], stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    up = stages.index("expert_up")
    keep = (up, up + 1)
    if not with_shared:
        # the combine's launch is timestamped like expert-up's (moe_forward)
        cb = stages.index("combine")
        keep = keep + (cb, cb + 1)
    if with_shared and w.n_shared > 0:
        sh = stages.index("shared")
        keep = keep + (sh, sh + 1)
    # the expert-up launch (and the shared stage, if any) is timed with
    # events on every `every`-th timed step (about ten samples): an
    # event-timed launch is separated from its neighbours by a few us, which
    # would otherwise be charged to every step
    every = max(1, steps // 10)
    sampled = list(range(0, steps, every))
    evsets = [ev.create(nev, keep=keep) for _ in sampled]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(steps):
        step(warmup + i, evsets[i // every] if i % every == 0 else None)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start

    stage_ms = np.array([[ev.elapsed_ms(es[j], es[j + 1]) if es[j] and es[j + 1] else np.nan
                          for j in range(nev - 1)] for es in evsets])
    for es in evsets:
        ev.destroy(es)
    kept = out["kept_counts"].cpu().numpy().astype(np.int64)
    n_kept = int(kept.sum())
    touched = int((kept > 0).sum())
    sclk = sample_sclk(lambda: step(warmup), sclk_seconds) if sclk_seconds > 0 else None
    return dict(elapsed=elapsed, steps=steps, stage_ms=stage_ms.mean(0), stage_ms_all=stage_ms,
                n_kept=n_kept, touched=touched, event_steps=len(sampled), stages=stages, sclk=sclk)


def cpu_baseline(w, seed=0, target_s=22.0):
    """The oracle on this host's cores on a bounded sample of workload w."""
    import oracle
    from oracle.margin import reject_near_ties  # noqa: F401  (inputs are used unfiltered here)
    from sparse_mixture_experts_03_amd import synth

    wt = synth.make_weights(w, seed)
    tk = synth.make_tokens(w, seed, 0)
    x = synth.widen(tk["x"])
    W1 = synth.widen(wt["W1"])
    W3 = None if wt["W3"] is None else synth.widen(wt["W3"])
    W2 = synth.widen(wt["W2"])
    extra = {}
    if w.n_shared > 0:
        extra["shared"] = (synth.widen(wt["Ws1"]),
                           None if wt["Ws3"] is None else synth.widen(wt["Ws3"]),
                           synth.widen(wt["Ws2"]))
    if w.residual:
        extra["residual"] = synth.widen(tk["res"])
    t0 = time.perf_counter()
    r = oracle.forward(x, wt["Wr"], W1, W3, W2, w.k, w.gate, w.cf, w.act, wt["bias"], tk["noise"],
                       tokens=np.zeros(0, np.int64), **extra)
    t_route = time.perf_counter() - t0
    rng = np.random.default_rng(1)

    def ffn_time(S):
        sel = np.sort(rng.choice(w.T, size=S, replace=False))
        t1 = time.perf_counter()
        oracle.forward(x, wt["Wr"], W1, W3, W2, w.k, w.gate, w.cf, w.act, wt["bias"], tk["noise"],
                       tokens=sel, **extra)
        return time.perf_counter() - t1 - t_route  # the call re-routes every token

    S = 4
    t_ffn = max(ffn_time(S), 1e-6)
    S = int(min(w.T, max(S, round(S * target_s / t_ffn))))
    t_ffn = max(ffn_time(S), 1e-6)
    per_token = t_route / w.T + t_ffn / S
    return {"value": 1.0 / per_token, "unit": "tokens/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": (f"{w.name}: router, gate, dispatch and statistics on all {w.T} tokens "
                       f"({t_route:.2f}s); expert FFN{' (routed and shared)' if w.n_shared else ''} "
                       f"and combine on {S} sampled tokens ({t_ffn:.2f}s); fp64 sums")}


def run_cold(w, steps, warmup, seed=0, flush_bytes=512 << 20, packed=False):
    """Per-step times of moe_forward (packed: moe_forward_packed) with the
    last-level cache flushed before every step (a device fill of
    ``flush_bytes``, outside the timed events): each step is bracketed by
    its own events on the launch stream.  Returns the median, minimum and
    90th percentile."""
    import torch
    from sparse_mixture_experts_03_amd import binding as B
    from sparse_mixture_experts_03_amd import synth

    wt = synth.make_weights(w, seed)
    dw = {k: B.to_device(v, w.dtype) for k, v in wt.items()}
    del wt
    tk = synth.make_tokens(w, seed, 0)
    x, noise = B.to_device(tk["x"], w.dtype), B.to_device(tk["noise"], w.dtype)
    desc = B.desc_for(w)
    ws = B.workspace(desc)
    out = B.alloc_outputs(desc)
    f8 = None
    if w.weights == "e4m3":
        # post-training quantisation of the expert weights, before timing
        f8 = B.quantize_experts(dw["W1"], dw["W3"], dw["W2"])
        for key in ("W1", "W3", "W2"):
            dw[key] = None
    pk = pack_weights(w, desc, dw, f8)[0] if packed else None
    fp8 = B.make_fp8(desc, f8["q1"], f8["q3"], f8["q2"], f8["s1"], f8["s3"], f8["s2"]) if f8 and not packed else None
    scratch = torch.empty(flush_bytes // 4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    times = []
    for i in range(warmup + steps):
        scratch.fill_(float(i))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        if pk is not None:
            B.moe_forward_packed(desc, pk, x, dw["Wr"], dw["bias"], noise, out["y"], ws, stream=stream)
        elif fp8 is not None:
            B.moe_forward_fp8(desc, fp8, x, dw["Wr"], dw["bias"], noise, out["y"], ws, stream=stream)
        else:
            B.moe_forward(desc, x, dw["Wr"], dw["bias"], noise, dw["W1"], dw["W3"], dw["W2"], out["y"], ws,
                          stream=stream)
        b.record(stream)
        if i >= warmup:
            times.append((a, b))
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in times])
    med = float(np.median(ms))
    return {"metric": METRIC, "workload": w.name, "mode": "last-level cache flushed before each step",
            "value": round(w.T / (med * 1e-3), 1), "unit": "tokens/s", "steps": steps,
            "ms_per_step_median_min_p90": [round(med, 4), round(float(ms.min()), 4),
                                           round(float(np.percentile(ms, 90)), 4)],
            "flush_bytes": flush_bytes}


def layer_bytes(w, n_kept, touched):
    """Algorithmic HBM bytes of one forward step of workload w: the touched
    experts' weights, x in, y out, the router matrix (and bias), and the
    noise input when the workload has one."""
    n_mat = 3 if w.act == "swiglu" else 2
    eb = 2 if w.dtype == "bf16" else 4
    wb = 1 if w.weights == "e4m3" else eb      # e4m3: 1-byte codes, a 4-byte scale per weight row
    b = touched * n_mat * w.d * w.d_ff * wb + 2 * w.T * w.d * eb + w.E * w.d * 4
    if w.weights == "e4m3":
        b += touched * ((n_mat - 1) * w.d_ff + w.d) * 4
    if w.noise_std > 0:
        b += w.T * w.E * 4
    if w.zipf_s > 0:
        b += w.E * 4
    return int(b)


def kernel_bytes(w, stage, n_kept, touched):
    """Algorithmic bytes of one expert GEMM launch: its touched weights, the
    rows of A it reads and the rows it writes."""
    eb = 2 if w.dtype == "bf16" else 4
    f8 = w.weights == "e4m3"
    wb = 1 if f8 else eb
    if stage == "expert_up":
        n_up = 2 if w.act == "swiglu" else 1
        return int(touched * n_up * w.d_ff * (w.d * wb + (4 if f8 else 0)) + n_kept * (w.d + w.d_ff) * eb)
    return int(touched * w.d * (w.d_ff * wb + (4 if f8 else 0)) + n_kept * w.d_ff * eb + n_kept * w.d * 4)


def hbm_layer_object(w, steps, warmup=5, packed=False):
    """An HBM-bound layer (Switch, fine-grained Zipf) in the default line:
    per-step median, minimum and p90 with the last-level cache flushed
    before every step, against 8 TB/s over the algorithmic bytes; the warm
    back-to-back rate and the dominant kernel's event-timed rate beside.
    packed: weights in the streaming tile layout (moe_forward_packed)."""
    res = run_workload(w, steps, warmup, packed=packed)
    cold = run_cold(w, steps, 3, packed=packed)
    med, mn, p90 = cold["ms_per_step_median_min_p90"]
    nbytes = layer_bytes(w, res["n_kept"], res["touched"])
    gbs = nbytes / (med * 1e-3) / 1e9
    stages = {n: float(v) for n, v in zip(res["stages"], res["stage_ms"]) if np.isfinite(v)}
    dom = max(("expert_up", "expert_down"), key=lambda n: stages.get(n, 0.0))
    kb = kernel_bytes(w, dom, res["n_kept"], res["touched"])
    kgbs = kb / (stages[dom] * 1e-3) / 1e9
    ms_warm = res["elapsed"] * 1e3 / res["steps"]
    return {
        "workload": w.name, "T": w.T, "d": w.d, "d_ff": w.d_ff, "E": w.E, "k": w.k,
        "gate": w.gate, "act": w.act, "capacity_factor": w.cf,
        "kept_rows": res["n_kept"], "touched_experts": res["touched"],
        "weights": "e4m3" if w.weights == "e4m3" else "bf16",
        "weight_layout": LAYOUT_PACKED if packed else "row-major (moe_forward)",
        "value": round(w.T / (med * 1e-3), 1), "unit": "tokens/s", "steps": steps,
        "cache": "last-level cache flushed (512 MB device fill) before every timed step",
        "ms_per_step_median_min_p90": [med, mn, p90],
        "ms_per_step_warm": round(ms_warm, 4),
        "stage_ms_warm": {n: round(v, 4) for n, v in stages.items()},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "algorithmic_per_step": nbytes, "traffic": None},
        "dominant_kernel": {"stage": dom, "mean_launch_ms": round(stages[dom], 4),
                            "algorithmic_per_launch": kb, "achieved": round(kgbs, 1),
                            "unit": "GB/s", "frac": round(kgbs / PEAK_HBM_GBS, 4),
                            "traffic": traffic_for(w.name + ("_packed" if packed else ""), dom)},
    }


def sample_sclk(step, seconds=2.0, period_s=0.002):
    """The shader clock (and socket power) while ``step`` runs back to back
    for about ``seconds``, from amdsmi's GPU metrics polled from a second
    thread.  The firmware refreshes that table only every few hundred ms,
    so consecutive polls mostly return the same snapshot: a snapshot counts
    once (a new value of the accumulated gfx activity marks a refresh), and
    the first one seen after the steps start is left out (it may predate
    them).  Returns the median and range over those snapshots (None if
    amdsmi is not usable here)."""
    import threading

    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        h = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception as e:  # noqa: BLE001 -- reported, never fatal
        return {"mhz": None, "reason": f"amdsmi unavailable: {e}"[:160]}

    def num(v):
        return float(v) if isinstance(v, (int, float)) else None

    def read():
        m = amdsmi.amdsmi_get_gpu_metrics_info(h)
        clk = None
        v = m.get("current_gfxclks")
        if isinstance(v, (list, tuple)):
            v = [c for c in v if isinstance(c, (int, float)) and 0 < c < 10000]
            if v:
                clk = float(np.mean(v))
        if clk is None:
            c = num(m.get("current_gfxclk"))
            clk = c if c is not None and 0 < c < 10000 else None
        return clk, num(m.get("current_socket_power")), m.get("gfx_activity_acc")

    snaps, stop = [], threading.Event()
    started = threading.Event()

    def poll():
        last = None
        while not stop.is_set():
            try:
                clk, pw, acc = read()
            except Exception:  # noqa: BLE001
                clk, pw, acc = None, None, None
            key = (acc, clk, pw)
            if clk is not None and key != last:
                snaps.append((started.is_set(), clk, pw))
                last = key
            time.sleep(period_s)

    th = threading.Thread(target=poll, daemon=True)
    th.start()
    time.sleep(0.01)
    started.set()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
        n += 20
    stop.set()
    th.join()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:  # noqa: BLE001
        pass
    # snapshots refreshed after the steps began, less the first of them
    during = [(c, p) for after, c, p in snaps if after][1:]
    if not during:
        return {"mhz": None, "reason": "no refreshed clock snapshot from amdsmi during the steps"}
    clk = np.array([c for c, _ in during])
    pw = np.array([p for _, p in during if p is not None])
    out = {"mhz": round(float(np.median(clk)), 1), "min": round(float(clk.min()), 1),
           "max": round(float(clk.max()), 1), "snapshots": len(during), "steps": n,
           "source": "amdsmi gpu metrics (current_gfxclks, mean over XCDs); each refresh of the table "
                     "counted once, the first after the steps began left out"}
    if len(pw):
        out["socket_power_w"] = round(float(np.median(pw)), 1)
    return out


def cpu_one_thread(seed=0):
    """The oracle on one host thread: the tiny layer (all 64 tokens) and the
    Mixtral-shape decode layer (routing of all 32 tokens, expert FFN and
    combine for 4 of them; tokens/s = 1 / (t_route / T + t_ffn / 4))."""
    import oracle
    from sparse_mixture_experts_03_amd import synth

    n0 = oracle.threads()
    oracle.set_threads(1)
    out = {}
    try:
        for name, n_ffn in (("tiny", None), ("mixtral_decode", 4)):
            w = synth.WORKLOADS[name]
            wt = synth.make_weights(w, seed)
            tk = synth.make_tokens(w, seed, 0)
            x = synth.widen(tk["x"])
            W1, W2 = synth.widen(wt["W1"]), synth.widen(wt["W2"])
            W3 = None if wt["W3"] is None else synth.widen(wt["W3"])
            args = (x, wt["Wr"], W1, W3, W2, w.k, w.gate, w.cf, w.act, wt["bias"], tk["noise"])
            t0 = time.perf_counter()
            oracle.forward(*args, tokens=np.zeros(0, np.int64))
            t_route = time.perf_counter() - t0
            sel = np.arange(w.T) if n_ffn is None else np.arange(n_ffn)
            t1 = time.perf_counter()
            oracle.forward(*args, tokens=sel)
            t_ffn = max(time.perf_counter() - t1 - t_route, 1e-9)
            out[name] = {"value": round(1.0 / (t_route / w.T + t_ffn / len(sel)), 2),
                         "unit": "tokens/s", "cores": 1, "kind": "oracle",
                         "sample": f"{name}: routing of all {w.T} tokens, expert FFN and combine "
                                   f"of {len(sel)}"}
    finally:
        oracle.set_threads(n0)
    return out


def run_backward(w, steps, warmup, seed=0):
    """Times ``steps`` moe_backward calls of workload w (after one forward
    that fixes the routing); loss weights 0.01 (aux) and 0.001 (z), the
    page's.  FLOPs: the recomputed expert forward (n_mat GEMMs) plus dgrad
    (n_mat) and wgrad (n_mat) over the kept rows, and 2 T E d for each of
    the router's logits, dx and dW_r."""
    import torch
    from sparse_mixture_experts_03_amd import binding as B
    from sparse_mixture_experts_03_amd import synth

    wt = synth.make_weights(w, seed)
    dw = {k: B.to_device(v, w.dtype) for k, v in wt.items()}
    del wt
    tk = synth.make_tokens(w, seed, 0)
    x, noise = B.to_device(tk["x"], w.dtype), B.to_device(tk["noise"], w.dtype)
    desc = B.desc_for(w)
    fwd = B.alloc_outputs(desc)
    ws = B.workspace(desc)
    B.moe_forward(desc, x, dw["Wr"], dw["bias"], noise, dw["W1"], dw["W3"], dw["W2"], fwd["y"], ws,
                  **{k: fwd[k] for k in fwd if k != "y"})
    del ws
    dy = B.to_device(synth.to_bf16(np.random.default_rng(seed + 1).standard_normal(
        (w.T, w.d)).astype(np.float32)), "bf16")
    grads = B.alloc_grads(desc, bias=dw["bias"] is not None)
    bws = B.backward_workspace(desc)

    def step():
        B.moe_backward(desc, x, dw["Wr"], dw["bias"], noise, dw["W1"], dw["W3"], dw["W2"], fwd, dy,
                       grads, bws, 0.01, 0.001)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    n_kept = int(fwd["kept_counts"].sum().item())
    n_mat = 3 if w.act == "swiglu" else 2
    flops = 3 * n_kept * 2.0 * n_mat * w.d * w.d_ff + 3 * 2.0 * w.T * w.E * w.d
    ms = elapsed * 1e3 / steps
    tf = flops / (ms * 1e-3) / 1e12
    return {"metric": "MoE layer backward tokens/s (training gradients)", "value": round(w.T / (ms * 1e-3), 1),
            "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
            "ms_per_step": round(ms, 4), "higher_is_better": True, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": w.name, "T": w.T, "d": w.d, "d_ff": w.d_ff, "E": w.E, "k": w.k,
                       "gate": w.gate, "act": w.act, "capacity_factor": w.cf, "pass": "backward"},
            "tflops": round(tf, 2), "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "flops_per_step": flops}


def gather_object(w, launches=20, seed=0):
    """The gather of the staged moe_dispatch (the copy of the kept rows of x
    into expert order), which moe_forward folds into the up projection's
    loads: its launch timed by the stage-event hook (the launch's own start
    and end timestamps), against 8 TB/s over the kept rows read and
    written plus their row indices."""
    import torch
    from sparse_mixture_experts_03_amd import binding as B
    from sparse_mixture_experts_03_amd import synth

    wt = synth.make_weights(w, seed, experts=1)
    tk = synth.make_tokens(w, seed, 0)
    desc = B.desc_for(w)
    x = B.to_device(tk["x"], w.dtype)
    out = B.alloc_outputs(desc)
    ws = B.workspace(desc)
    B.moe_route(desc, x, B.to_device(wt["Wr"], "f32"), B.to_device(wt["bias"], "f32"),
                B.to_device(tk["noise"], "f32"), out["topk_idx"], out["gates"], out["stats"], ws)
    x_perm = torch.empty((w.T * w.k, w.d), dtype=x.dtype, device=x.device)
    ev = HipEvents()

    def disp(events=None):
        desc.stage_events = ctypes.cast(events, ctypes.POINTER(ctypes.c_void_p)) if events else None
        desc.n_stage_events = 2 if events else 0
        B.moe_dispatch(desc, x, out["topk_idx"], out["routed_counts"], out["kept_counts"], out["offsets"],
                       out["row_of_slot"], out["token_of_row"], out["dropped"], x_perm, ws)

    for _ in range(3):
        disp()
    sets = [ev.create(2) for _ in range(launches)]
    torch.cuda.synchronize()
    for es in sets:
        disp(es)
    torch.cuda.synchronize()
    ms = np.array([ev.elapsed_ms(es[0], es[1]) for es in sets])
    for es in sets:
        ev.destroy(es)
    desc.stage_events, desc.n_stage_events = None, 0
    n_kept = int(out["kept_counts"].sum().item())
    eb = 2 if w.dtype == "bf16" else 4
    nbytes = 2 * n_kept * w.d * eb + n_kept * 4
    gbs = nbytes / (float(ms.mean()) * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_per_launch": nbytes,
            "mean_launch_ms": round(float(ms.mean()), 4), "launches": launches,
            "entry_point": "moe_dispatch (staged path)"}


def combine_object(w, res):
    """The combine's HBM rate over its event-timed launches: algorithmic bytes
    = kept rows of y_perm (fp32) + gates and row indices + y (act dtype),
    against 8 TB/s (a K-split down projection's second partial, when read,
    is extra traffic not counted)."""
    if "combine" not in res["stages"]:
        return None
    cb = res["stages"].index("combine")
    ms = float(res["stage_ms"][cb])
    if not np.isfinite(ms) or ms <= 0:
        return None
    ab = 2 if w.dtype == "bf16" else 4
    nbytes = res["n_kept"] * w.d * 4 + w.T * w.k * 8 + w.T * w.d * ab
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_per_launch": int(nbytes),
            "mean_launch_ms": round(ms, 4)}


def decode_object(wd, rd, packed=False):
    """Throughput and HBM roofline of a decode workload's run: the expert
    up-projection (weight streaming) against 8 TB/s, algorithmic bytes =
    the touched experts' W1 and W3 (bf16: 2 B per weight; e4m3: 1 B plus a
    4-byte scale per row) + permuted rows in + H out."""
    ms_d = rd["elapsed"] * 1e3 / rd["steps"]
    up = rd["stages"].index("expert_up")
    up_ms_d = float(rd["stage_ms"][up])
    wbytes = 1 if wd.weights == "e4m3" else 2
    sbytes = 4 if wd.weights == "e4m3" else 0
    up_bytes = (rd["touched"] * 2 * wd.d_ff * (wd.d * wbytes + sbytes)
                + rd["n_kept"] * (wd.d + wd.d_ff) * 2)
    step_bytes = (rd["touched"] * (3 * wd.d * wd.d_ff * wbytes + (2 * wd.d_ff + wd.d) * sbytes)
                  + wd.T * wd.d * 4 + wd.E * wd.d * 4)
    gbs = up_bytes / (up_ms_d * 1e-3) / 1e9
    return {
        "workload": wd.name, "weights": "e4m3" if wd.weights == "e4m3" else "bf16",
        "weight_layout": LAYOUT_PACKED if packed else "row-major",
        "value": round(wd.T * rd["steps"] / rd["elapsed"], 1),
        "unit": "tokens/s", "steps": rd["steps"], "ms_per_step": round(ms_d, 4),
        "step_hbm_gbs": round(step_bytes / (ms_d * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(step_bytes / (ms_d * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "stage_ms": {n: round(float(v), 4) for n, v in zip(rd["stages"], rd["stage_ms"]) if np.isfinite(v)},
        "combine": combine_object(wd, rd),
        "roofline": {"bound": "hbm", "kernel": "expert_up", "achieved": round(gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic_for(wd.name + ("_packed" if packed else ""), "expert_up"),
                     "algorithmic_per_launch": up_bytes, "mean_launch_ms": round(up_ms_d, 4),
                     "event_timed_launches": rd["event_steps"]},
    }


def run_library_gemm(w, steps, warmup, seed=0):
    """The up projection's FLOPs through torch's own GEMM (hipBLASLt), for
    context: X [N][d] times the stacked [W1; W3] of one expert, transposed
    (torch.nn.functional.linear, weights [n_up*d_ff][d] as stored), once as one
    dense call over all N = T*k rows and once as E calls of N/E rows each
    (the balanced grouped problem as separate library calls).  bf16 in, fp32
    accumulation, bf16 out, as in the layer's own kernel."""
    import torch
    import torch.nn.functional as F

    n_up = 2 if w.act == "swiglu" else 1
    N = w.T * w.k
    g = torch.Generator(device="cuda").manual_seed(seed)
    X = torch.randn((N, w.d), generator=g, device="cuda").to(torch.bfloat16)
    Wt = [(torch.randn((n_up * w.d_ff, w.d), generator=g, device="cuda") * w.d ** -0.5)
          .to(torch.bfloat16) for _ in range(w.E)]
    rows = N // w.E
    flops = 2.0 * N * w.d * n_up * w.d_ff

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        return {"ms": round(ms, 4), "tflops": round(flops / ms * 1e-9, 1),
                "frac_bf16_peak": round(flops / ms * 1e-9 / PEAK_BF16_TFLOPS, 4)}

    dense = timed(lambda: F.linear(X, Wt[0]))
    per_expert = timed(lambda: [F.linear(X[e * rows:(e + 1) * rows], Wt[e]) for e in range(w.E)])
    return {"library_gemm": "torch.nn.functional.linear (hipBLASLt)", "workload": w.name,
            "shape": {"rows": N, "K": w.d, "N": n_up * w.d_ff, "E": w.E},
            "gflop": round(flops * 1e-9, 1), "steps": steps, "warmup": warmup,
            "dense_one_call": dense, "per_expert_calls": per_expert}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_prefill")
    ap.add_argument("--decode-steps", type=int, default=100)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-layers", action="store_true",
                    help="leave out the Switch and fine-grained Zipf layers of the default line")
    ap.add_argument("--layer-steps", type=int, default=50)
    ap.add_argument("--packed", action="store_true",
                    help="expert weights in the streaming tile layout (moe_forward_packed; "
                         "weight-streaming shapes: decode batches, the Switch layer)")
    ap.add_argument("--backward", action="store_true",
                    help="time moe_backward on the workload instead of the forward")
    ap.add_argument("--cold", action="store_true",
                    help="flush the last-level cache before every step and time each step alone")
    ap.add_argument("--library-gemm", action="store_true",
                    help="only time torch's GEMM (hipBLASLt) on the up projection's FLOPs, "
                         "one dense call and one call per expert, for context")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (a kernel of "
                         "known traffic, to calibrate rocprofv3's FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the layer runs on a single MI355X with every expert "
              "resident in its HBM (no expert parallelism, no collectives). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_mixture_experts_03_amd import binding as B
    from sparse_mixture_experts_03_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": src.numel() * 4, "launches": 3}))
        return
    w = synth.WORKLOADS[args.workload]
    if args.library_gemm:
        print(json.dumps(run_library_gemm(w, args.steps, args.warmup)), flush=True)
        return
    B.load(build_if_missing=False)
    if args.backward:
        print(json.dumps(run_backward(w, args.steps, args.warmup)), flush=True)
        return
    if args.cold:
        print(json.dumps(run_cold(w, args.steps, args.warmup)), flush=True)
        return
    if w.steps > 1:
        # a decode workload on its own: fresh tokens every step, HBM roofline
        res = run_workload(w, args.steps, args.warmup, fresh_x_steps=args.steps, packed=args.packed)
        obj = decode_object(w, res, packed=args.packed)
        line = {
            "metric": METRIC, "value": obj["value"], "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": obj["ms_per_step"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": w.name, "T": w.T, "d": w.d, "d_ff": w.d_ff, "E": w.E, "k": w.k,
                       "gate": w.gate, "act": w.act, "capacity_factor": w.cf, "router": "fp32",
                       "expert_weights": obj["weights"], "parallelism": "single_gpu"},
            "stage_ms": obj["stage_ms"], "step_hbm_frac": obj["step_hbm_frac"],
            "weight_layout": obj["weight_layout"], "roofline": obj["roofline"],
        }
        print(json.dumps(line), flush=True)
        return
    res = run_workload(w, args.steps, args.warmup,
                       sclk_seconds=3.0 if w.name == "mixtral_prefill" else 0.0, packed=args.packed)
    ms_step = res["elapsed"] * 1e3 / res["steps"]
    tokens_s = w.T * res["steps"] / res["elapsed"]
    n_up = 2 if w.act == "swiglu" else 1
    n_mat = n_up + 1
    # active-parameter FLOPs: router, kept routed rows, and every token on
    # each shared expert
    shared_flops = w.n_shared * w.T * 2.0 * n_mat * w.d * w.d_ff
    flops_step = 2.0 * w.T * w.E * w.d + res["n_kept"] * 2.0 * n_mat * w.d * w.d_ff + shared_flops
    up = res["stages"].index("expert_up")
    up_ms = float(res["stage_ms"][up])
    up_flops = res["n_kept"] * 2.0 * n_up * w.d * w.d_ff
    achieved = up_flops / (up_ms * 1e-3) / 1e12
    up_all = res["stage_ms_all"][:, up]
    stages = {n: round(float(v), 4) for n, v in zip(res["stages"], res["stage_ms"]) if np.isfinite(v)}
    log(f"[bench] {w.name}: {ms_step:.3f} ms/step, stages(ms) {stages}")
    line = {
        "metric": METRIC, "value": round(tokens_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "d_ff": w.d_ff, "E": w.E, "k": w.k,
                   "gate": w.gate, "act": w.act, "capacity_factor": w.cf, "router": "fp32",
                   "parallelism": "single_gpu",
                   **({"n_shared": w.n_shared, "residual": w.residual}
                      if (w.n_shared or w.residual) else {})},
        "tflops_per_step": round(flops_step / (ms_step * 1e-3) / 1e12, 2),
        "stage_ms": stages,
        "roofline": {"bound": "mfma", "kernel": "expert_up (grouped GEMM, SwiGLU epilogue)",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_for(w.name, "expert_up"),
                     "algorithmic_per_launch": up_flops, "mean_launch_ms": round(up_ms, 4),
                     "launch_ms_median_min_p90": [round(float(np.median(up_all)), 4),
                                                  round(float(np.min(up_all)), 4),
                                                  round(float(np.percentile(up_all, 90)), 4)],
                     "event_timed_launches": res["event_steps"]},
    }
    # per-step distribution of the same layer with the last-level cache
    # flushed before each step (its 2.8 GB of weights never fit it anyway)
    cold = run_cold(w, max(args.steps, 20), 3, packed=args.packed)
    line["step_ms_median_min_p90"] = cold["ms_per_step_median_min_p90"]
    line["step_ms_mode"] = "each step timed alone by its own events, last-level cache flushed before it"
    line["combine"] = combine_object(w, res)
    line["gather"] = gather_object(w) if w.n_shared == 0 and not w.residual else None
    line["gather_in_forward"] = ("folded into the expert up-projection's loads (rows of x read through "
                                 "token_of_row): its bytes are part of that kernel's traffic")
    if w.n_shared > 0:
        # the shared stage: the row map, then the shared experts' up and
        # down projections (dense GEMMs of all T tokens), against the MFMA peak
        sh_ms = float(res["stage_ms"][res["stages"].index("shared")])
        sh_tf = shared_flops / (sh_ms * 1e-3) / 1e12
        line["shared_stage"] = {"bound": "mfma", "achieved": round(sh_tf, 2),
                                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                "frac": round(sh_tf / PEAK_BF16_TFLOPS, 4),
                                "algorithmic_per_stage": shared_flops, "mean_stage_ms": round(sh_ms, 4)}
    if not args.no_decode and w.name == "mixtral_prefill":
        # weight-streaming layers run on packed weights (the library's
        # fastest form for them); the row-major entry point is timed beside
        for key, name in (("decode", "mixtral_decode"), ("decode_fp8", "mixtral_decode_fp8")):
            wd = synth.WORKLOADS[name]
            rd = run_workload(wd, args.decode_steps, 10, fresh_x_steps=args.decode_steps, packed=True)
            line[key] = decode_object(wd, rd, packed=True)
            rr = decode_object(wd, run_workload(wd, args.decode_steps, 10, fresh_x_steps=args.decode_steps))
            line[key]["row_major"] = {
                "entry_point": "moe_forward_fp8" if wd.weights == "e4m3" else "moe_forward",
                "ms_per_step": rr["ms_per_step"], "step_hbm_frac": rr["step_hbm_frac"],
                "stage_ms": rr["stage_ms"], "expert_up_frac": rr["roofline"]["frac"]}
            log(f"[bench] {wd.name}: {line[key]['ms_per_step']:.3f} ms/step packed, "
                f"{rr['ms_per_step']:.3f} row-major")
    if not args.no_layers and w.name == "mixtral_prefill":
        for name in ("switch", "finegrained_zipf"):
            log(f"[bench] {name}: {args.layer_steps} warm + {args.layer_steps} cold steps ...")
            # the Switch layer's experts hold at most 40 rows: weight streaming,
            # on packed weights; the row-major entry point beside
            packed = name == "switch"
            line[name] = hbm_layer_object(synth.WORKLOADS[name], args.layer_steps, packed=packed)
            if packed:
                rr = hbm_layer_object(synth.WORKLOADS[name], args.layer_steps)
                line[name]["row_major"] = {
                    "entry_point": "moe_forward", "ms_per_step_median_min_p90": rr["ms_per_step_median_min_p90"],
                    "ms_per_step_warm": rr["ms_per_step_warm"], "stage_ms_warm": rr["stage_ms_warm"],
                    "frac": rr["roofline"]["frac"]}
            log(f"[bench] {name}: median {line[name]['ms_per_step_median_min_p90'][0]:.4f} ms/step "
                f"(cold), {line[name]['roofline']['frac']:.3f} of HBM")
        # the Switch layer with e4m3 expert weights (quantised and packed
        # before timing), against 8 TB/s over its bytes (1-byte codes + scales)
        log(f"[bench] switch_fp8: {args.layer_steps} warm + {args.layer_steps} cold steps ...")
        line["switch_fp8"] = hbm_layer_object(synth.WORKLOADS["switch_fp8"], args.layer_steps, packed=True)
        log(f"[bench] switch_fp8: median {line['switch_fp8']['ms_per_step_median_min_p90'][0]:.4f} ms/step "
            f"(cold), {line['switch_fp8']['roofline']['frac']:.3f} of HBM")
    if res["sclk"] is not None:
        line["sclk"] = res["sclk"]
    if not args.no_cpu:
        log("[bench] CPU oracle baseline ...")
        line["cpu_baseline"] = cpu_baseline(w)
        if w.name == "mixtral_prefill":
            line["cpu_baseline_1thread"] = cpu_one_thread()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
