"""Benchmark of the Key-only GLA token mixer (libgtrscan) on one MI355X.

One step = one full mixer call (every phase of the chunkwise scan, epilogue
and grid-order store) on the 16.4K-token workload: B=1, 128x128 grid
(16384 tokens), H=12, dk=dv=64, fp16 I/O, chunk 64.  Inputs are seeded
synthetic arrays already resident in HBM; consecutive steps rotate over
enough buffer sets (>= 512 MB in total) that the 256 MB Infinity Cache cannot
serve one step from the previous one.

Prints one JSON line (see the keys below); progress goes to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gated_token_recurrence_amd as g  # noqa: E402
from gated_token_recurrence_amd import _lib, workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0 # dense bf16/fp16 MFMA


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------- HIP events --
class Hip:
    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def events(self, n):
        arr = (ctypes.c_void_p * n)()
        base = ctypes.addressof(arr)
        for i in range(n):
            if self.lib.hipEventCreate(base + i * ctypes.sizeof(ctypes.c_void_p)) != 0:
                raise RuntimeError("hipEventCreate failed")
        return arr

    def record(self, ev, stream):
        if self.lib.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        self.lib.hipEventSynchronize(b)
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, arr):
        for e in arr:
            self.lib.hipEventDestroy(e)


# ----------------------------------------------------------------- inputs --
TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def device_sets(w: W.Workload, n_sets: int, dev):
    x = W.make_inputs(w)
    base = {}
    for key in ("q", "k", "v", "z"):
        a = x[key]
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if w.dtype == "bf16" \
            else torch.from_numpy(a)
        base[key] = t
    base["log_g"] = torch.from_numpy(x["log_g"])
    base["rms_w"] = torch.from_numpy(x["rms_w"])
    sets = []
    for _ in range(n_sets):
        s = {key: val.to(dev) for key, val in base.items()}
        s["out"] = torch.empty_like(s["v"])
        sets.append(s)
    torch.cuda.synchronize(dev)
    return x, sets


def call(lib, w, s, direction, chunk, path, stream, events=None, n_events=0, nl=None):
    args = (s["q"].data_ptr(), s["k"].data_ptr(), s["v"].data_ptr(), s["log_g"].data_ptr(),
            s["z"].data_ptr(), s["rms_w"].data_ptr(), s["out"].data_ptr(), w.B, w.H, w.grid_h,
            w.grid_w, w.dk, w.dv, direction, chunk, W.DTYPE_CODE[w.dtype], path)
    if events is None:
        st = lib.gtr_gla_fwd_path(*args, stream)
    else:
        st = lib.gtr_gla_fwd_events(*args, events, n_events, nl, stream)
    _lib.check(st)


def time_workload(w, dev, hip, stream_ptr, steps, warmup, path, chunk, direction=0,
                  per_kernel=True, graph=True):
    """Returns a dict of timings for one workload (rotating buffer sets)."""
    lib = _lib.load()
    per_set = w.compulsory_bytes()
    n_sets = W.rotation_sets(per_set)
    x, sets = device_sets(w, n_sets, dev)
    res = {"n_sets": n_sets, "set_mb": per_set / 1e6}
    for i in range(warmup):
        call(lib, w, sets[i % n_sets], direction, chunk, path, stream_ptr)
    torch.cuda.synchronize(dev)

    # Whole-call timing: events at the ends of the region, rotating sets.
    ev = hip.events(2)
    hip.record(ev[0], stream_ptr)
    for i in range(steps):
        call(lib, w, sets[i % n_sets], direction, chunk, path, stream_ptr)
    hip.record(ev[1], stream_ptr)
    total_ms = hip.elapsed_ms(ev[0], ev[1])
    torch.cuda.synchronize(dev)
    res["us_per_call"] = total_ms * 1e3 / steps
    hip.destroy(ev)

    # Hot: the same set every time (cache-resident inputs), labelled as such.
    ev = hip.events(2)
    hip.record(ev[0], stream_ptr)
    for i in range(steps):
        call(lib, w, sets[0], direction, chunk, path, stream_ptr)
    hip.record(ev[1], stream_ptr)
    res["us_per_call_hot"] = hip.elapsed_ms(ev[0], ev[1]) * 1e3 / steps
    torch.cuda.synchronize(dev)
    hip.destroy(ev)

    if per_kernel:
        # Per-launch timing: events between the launches of every call.
        nl = ctypes.c_int(0)
        probe = hip.events(8)
        call(lib, w, sets[0], direction, chunk, path, stream_ptr, probe, 8, ctypes.byref(nl))
        torch.cuda.synchronize(dev)
        hip.destroy(probe)
        n_ev = nl.value + 1
        evs = [hip.events(n_ev) for _ in range(steps)]
        for i in range(steps):
            call(lib, w, sets[i % n_sets], direction, chunk, path, stream_ptr, evs[i], n_ev,
                 None)
        torch.cuda.synchronize(dev)
        per = [[hip.elapsed_ms(e[j], e[j + 1]) * 1e3 for j in range(n_ev - 1)] for e in evs]
        for e in evs:
            hip.destroy(e)
        res["launch_us_mean"] = [statistics.fmean(p[j] for p in per) for j in range(n_ev - 1)]
        res["launch_us_median"] = [statistics.median(p[j] for p in per) for j in range(n_ev - 1)]
        calls = [sum(p) for p in per]
        res["us_per_call_evented_median"] = statistics.median(calls)
        res["us_per_call_evented_p10"] = float(np.percentile(calls, 10))
        res["us_per_call_evented_p90"] = float(np.percentile(calls, 90))

    if graph:
        try:
            res["us_per_call_graph"] = graph_time(lib, w, sets, n_sets, dev, direction, chunk,
                                                  path, steps, warmup)
        except Exception as exc:  # e.g. a launch kind that stream capture does not take
            res["us_per_call_graph"] = None
            res["graph_error"] = str(exc)[:200]
            torch.cuda.synchronize(dev)
    del sets
    torch.cuda.empty_cache()
    return x, res


def _io_tensor(a, dtype):
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if dtype == "bf16" \
        else torch.from_numpy(a)


def time_lowrank(w, dev, hip, stream_ptr, steps, warmup, chunk, direction=0, rank=16):
    """Whole-call and per-launch timing of gtr_gla_lowrank_fwd on the workload's shapes
    with rank-r gate features (rotating buffer sets, as for the main workload)."""
    lib = _lib.load()
    x = W.make_lowrank_inputs(w, rank=rank)
    per_set = w.compulsory_bytes_lowrank(rank)
    n_sets = W.rotation_sets(per_set)
    base = {key: _io_tensor(x[key], w.dtype) for key in ("q", "k", "v", "z", "feat", "gate_w")}
    base["gate_b"] = torch.from_numpy(x["gate_b"])
    base["rms_w"] = torch.from_numpy(x["rms_w"])
    sets = []
    for _ in range(n_sets):
        st = {key: val.to(dev) for key, val in base.items()}
        st["out"] = torch.empty_like(st["v"])
        sets.append(st)
    torch.cuda.synchronize(dev)

    def run(s, events=None, n_events=0, nl=None):
        st = lib.gtr_gla_lowrank_fwd(
            s["q"].data_ptr(), s["k"].data_ptr(), s["v"].data_ptr(), s["feat"].data_ptr(),
            s["gate_w"].data_ptr(), s["gate_b"].data_ptr(), x["tau"], rank, s["z"].data_ptr(),
            s["rms_w"].data_ptr(), s["out"].data_ptr(), w.B, w.H, w.grid_h, w.grid_w, w.dk,
            w.dv, direction, chunk, W.DTYPE_CODE[w.dtype], g.PATH_AUTO, events, n_events, nl,
            stream_ptr)
        _lib.check(st)

    for i in range(warmup):
        run(sets[i % n_sets])
    torch.cuda.synchronize(dev)
    ev = hip.events(2)
    hip.record(ev[0], stream_ptr)
    for i in range(steps):
        run(sets[i % n_sets])
    hip.record(ev[1], stream_ptr)
    us = hip.elapsed_ms(ev[0], ev[1]) * 1e3 / steps
    torch.cuda.synchronize(dev)
    hip.destroy(ev)
    nl = ctypes.c_int(0)
    probe = hip.events(8)
    run(sets[0], probe, 8, ctypes.byref(nl))
    torch.cuda.synchronize(dev)
    hip.destroy(probe)
    n_ev = nl.value + 1
    evs = [hip.events(n_ev) for _ in range(steps)]
    for i in range(steps):
        run(sets[i % n_sets], evs[i], n_ev, None)
    torch.cuda.synchronize(dev)
    per = [[hip.elapsed_ms(e[j], e[j + 1]) * 1e3 for j in range(n_ev - 1)] for e in evs]
    for e in evs:
        hip.destroy(e)
    del sets
    torch.cuda.empty_cache()
    return {"us_per_call": us, "n_sets": n_sets, "launches": nl.value,
            "launch_us_mean": [statistics.fmean(p[j] for p in per) for j in range(n_ev - 1)]}


def time_sswiglu(ws, dev, hip, stream_ptr, steps, warmup):
    """Timing of gtr_sswiglu_mix on a Spatial SwiGLU workload (rotating buffer sets)."""
    lib = _lib.load()
    x = W.make_sswiglu_inputs(ws)
    per_set = ws.compulsory_bytes()
    n_sets = W.rotation_sets(per_set)
    u0 = _io_tensor(x["u"], ws.dtype)
    wc, bc = torch.from_numpy(x["w_conv"]).to(dev), torch.from_numpy(x["b_conv"]).to(dev)
    sets = []
    for _ in range(n_sets):
        u = u0.to(dev)
        sets.append((u, torch.empty(u.shape[:-1] + (ws.F,), dtype=u.dtype, device=dev)))
    torch.cuda.synchronize(dev)

    def run(i):
        u, m = sets[i % n_sets]
        _lib.check(lib.gtr_sswiglu_mix(u.data_ptr(), wc.data_ptr(), bc.data_ptr(), m.data_ptr(),
                                       ws.B, ws.grid_h, ws.grid_w, ws.F, ws.k,
                                       W.DTYPE_CODE[ws.dtype], stream_ptr))

    for i in range(warmup):
        run(i)
    torch.cuda.synchronize(dev)
    ev = hip.events(2)
    hip.record(ev[0], stream_ptr)
    for i in range(steps):
        run(i)
    hip.record(ev[1], stream_ptr)
    us = hip.elapsed_ms(ev[0], ev[1]) * 1e3 / steps
    torch.cuda.synchronize(dev)
    hip.destroy(ev)
    del sets
    torch.cuda.empty_cache()
    return {"us_per_call": us, "n_sets": n_sets}


def time_stack(dev, hip, stream_ptr, steps, warmup):
    """gtr_gla_stack_fwd on the 12-block stack workload (B = 8, 64 x 64, H = 12, dk = 64,
    dv = 128, bf16).  Inputs are drawn on the device from a seeded generator with the
    workload's distributions (~6 GB; parity of this configuration is tested on host-drawn
    inputs): q, k, v, z ~ N(0, 1)/8, log_g = logsigmoid(N(0, 1))/16, rms_w ~ 1 + 0.1 N(0, 1)."""
    w = W.WORKLOADS["stack_1024"]
    nb = w.n_blocks
    gen = torch.Generator(device=dev).manual_seed(1000 * w.wid)
    qk = (nb, w.B, w.grid_h, w.grid_w, w.H, w.dk)
    vz = (nb, w.B, w.grid_h, w.grid_w, w.H, w.dv)

    def io(shape):
        return (torch.randn(shape, generator=gen, device=dev) * w.scale).to(torch.bfloat16)

    q, k, v, z = io(qk), io(qk), io(vz), io(vz)
    log_g = torch.nn.functional.logsigmoid(torch.randn(qk, generator=gen, device=dev)) / 16.0
    rms_w = 1.0 + 0.1 * torch.randn((nb, w.dv), generator=gen, device=dev)
    out = torch.empty_like(v)
    torch.cuda.synchronize(dev)
    for _ in range(warmup):
        g.gla_stack_fwd(q, k, v, log_g, z, rms_w, 0, w.chunk, out=out)
    torch.cuda.synchronize(dev)
    ev = hip.events(2)
    hip.record(ev[0], stream_ptr)
    for _ in range(steps):
        g.gla_stack_fwd(q, k, v, log_g, z, rms_w, 0, w.chunk, out=out)
    hip.record(ev[1], stream_ptr)
    ms = hip.elapsed_ms(ev[0], ev[1]) / steps
    torch.cuda.synchronize(dev)
    hip.destroy(ev)
    th = w.B * w.L * w.H
    per_th = (2 * w.dk + 3 * w.dv) * 2 + 4 * w.dk  # 16-bit I/O
    nbytes = th * per_th * nb + th * w.dv * 2 * (nb - 1)  # + the residual read of blocks 1..
    del q, k, v, z, log_g, rms_w, out
    torch.cuda.empty_cache()
    return w, ms, nbytes


def time_backbone(dev, steps):
    """12-block random-weight backbone at 640 x 640, batch 1: eager and HIP-graph replay."""
    from gated_token_recurrence_amd import backbone as bb
    cfg = bb.BackboneConfig()
    net = bb.Backbone(cfg, dev, seed=1)
    image = torch.randn(cfg.batch, 3, cfg.image, cfg.image,
                        generator=torch.Generator().manual_seed(2)).to(dev)
    stream = torch.cuda.Stream(dev)
    with torch.cuda.stream(stream):
        for _ in range(3):
            net.forward(image)
    torch.cuda.synchronize(dev)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        t0.record(stream)
        for _ in range(steps):
            net.forward(image)
        t1.record(stream)
    torch.cuda.synchronize(dev)
    eager_ms = t0.elapsed_time(t1) / steps
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        net.forward(image)
    graph.replay()
    torch.cuda.synchronize(dev)
    with torch.cuda.stream(stream):
        t0.record(stream)
        for _ in range(steps):
            graph.replay()
        t1.record(stream)
    torch.cuda.synchronize(dev)
    graph_ms = t0.elapsed_time(t1) / steps
    del graph
    return cfg, eager_ms, graph_ms


def time_backward(w, dev, hip, stream_ptr, steps, warmup):
    """gtr_gla_bwd on the workload's inputs (one buffer set; the call moves about twice
    the forward's bytes, so two sets already exceed the last-level cache)."""
    lib = _lib.load()
    x, sets = device_sets(w, 2, dev)
    rng = np.random.default_rng(5)
    grads = []
    for s_ in sets:
        dy = torch.from_numpy(W.cast_io(rng.standard_normal(x["v"].shape), w.dtype))
        s_["dy"] = (dy.view(torch.bfloat16) if w.dtype == "bf16" else dy).to(dev)
        grads.append({k: torch.empty_like(s_[src]) for k, src in
                      (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dlog_g", "log_g"), ("dz", "z"),
                       ("drms_w", "rms_w"))})
    # the forward's segment states of each set (gtr_gla_fwd_states), for the variant
    # that takes them instead of recomputing
    nbytes = lib.gtr_gla_states_bytes(w.B, w.H, w.grid_h, w.grid_w, w.dk, w.dv, w.chunk,
                                      W.DTYPE_CODE[w.dtype])
    states = []
    for s_ in sets if nbytes else []:
        buf = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
        out = torch.empty_like(s_["v"])
        _lib.check(lib.gtr_gla_fwd_states(
            s_["q"].data_ptr(), s_["k"].data_ptr(), s_["v"].data_ptr(), s_["log_g"].data_ptr(),
            s_["z"].data_ptr(), s_["rms_w"].data_ptr(), out.data_ptr(), w.B, w.H, w.grid_h,
            w.grid_w, w.dk, w.dv, 0, w.chunk, W.DTYPE_CODE[w.dtype], buf.data_ptr(), nbytes,
            stream_ptr))
        states.append(buf)
    torch.cuda.synchronize(dev)

    def run(i, events=None, n_events=0, nl=None, with_states=False):
        s_, g_ = sets[i % 2], grads[i % 2]
        st = states[i % 2] if with_states else None
        _lib.check(lib.gtr_gla_bwd_states(
            s_["q"].data_ptr(), s_["k"].data_ptr(), s_["v"].data_ptr(), s_["log_g"].data_ptr(),
            s_["z"].data_ptr(), s_["rms_w"].data_ptr(), s_["dy"].data_ptr(), g_["dq"].data_ptr(),
            g_["dk"].data_ptr(), g_["dv"].data_ptr(), g_["dlog_g"].data_ptr(), g_["dz"].data_ptr(),
            g_["drms_w"].data_ptr(), w.B, w.H, w.grid_h, w.grid_w, w.dk, w.dv, 0, w.chunk,
            W.DTYPE_CODE[w.dtype], None if st is None else st.data_ptr(),
            0 if st is None else nbytes, events, n_events, nl, stream_ptr))

    def timed(with_states):
        for i in range(warmup):
            run(i, with_states=with_states)
        torch.cuda.synchronize(dev)
        ev = hip.events(2)
        hip.record(ev[0], stream_ptr)
        for i in range(steps):
            run(i, with_states=with_states)
        hip.record(ev[1], stream_ptr)
        t = hip.elapsed_ms(ev[0], ev[1]) * 1e3 / steps
        torch.cuda.synchronize(dev)
        hip.destroy(ev)
        return t

    us = timed(False)
    us_states = timed(True) if states else None
    evs = hip.events(16)
    nl = ctypes.c_int(0)
    per = []
    for i in range(5):
        run(i, evs, 16, ctypes.byref(nl))
        torch.cuda.synchronize(dev)
        per.append([hip.elapsed_ms(evs[j], evs[j + 1]) * 1e3 for j in range(min(nl.value, 15))])
    hip.destroy(evs)
    del sets, grads, states
    torch.cuda.empty_cache()
    return us, [statistics.fmean(p[j] for p in per) for j in range(len(per[0]))], us_states


def graph_time(lib, w, sets, n_sets, dev, direction, chunk, path, steps, warmup=2):
    """hipGraph replay of one call per buffer set (the pages' own kernel benchmark
    used graph launch); microseconds per call.  Warmed up with as many calls as the
    eager timing."""
    s = torch.cuda.Stream(device=dev)
    sp = s.cuda_stream
    with torch.cuda.stream(s):
        for i in range(n_sets):
            call(lib, w, sets[i], direction, chunk, path, sp)
    torch.cuda.synchronize(dev)
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=s):
        for i in range(n_sets):
            call(lib, w, sets[i], direction, chunk, path, sp)
    torch.cuda.synchronize(dev)
    reps = max(1, steps // n_sets)
    for _ in range(max(2, warmup // n_sets)):
        gr.replay()
    torch.cuda.synchronize(dev)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        gr.replay()
    t1.record()
    torch.cuda.synchronize(dev)
    out = t0.elapsed_time(t1) * 1e3 / (reps * n_sets)
    del gr
    return out


# ----------------------------------------------------------- CPU baseline --
def cpu_baseline(w: W.Workload, x: dict, target_s: float = 12.0, single_s: float = 4.0):
    """The fp64 oracle (test infrastructure, untuned) on a bounded sample of the
    same workload, on every host thread and on one: whole calls repeated for about
    target_s seconds (at least three), or, when one call would take longer, the
    first (batch, head) sequences that fit, run three times; the median run is
    reported.  The one-thread figure samples fewer sequences (single_s seconds)."""
    import oracle
    oracle.build(force=False)
    f = {key: W.io_to_f64(x[key], w.dtype) for key in ("q", "k", "v", "z")}
    lg = x["log_g"].astype(np.float64)
    rw = x["rms_w"].astype(np.float64)
    n_seq = w.B * w.H

    def one(bh):
        t0 = time.perf_counter()
        oracle.fwd(f["q"], f["k"], f["v"], lg, f["z"], rw, 0, bh=bh)
        return time.perf_counter() - t0

    def measure(budget_s):
        t_one = one([0])
        if t_one * n_seq * 3 <= budget_s:  # whole calls
            times = []
            t0 = time.perf_counter()
            while len(times) < 3 or time.perf_counter() - t0 < budget_s:
                times.append(one(None))
            per_call = statistics.median(times)
            return per_call, f"{len(times)} whole calls of {w.name} (LR scan), median"
        n = max(1, min(n_seq, int(budget_s / 3 / t_one)))
        times = [one(list(range(n))) for _ in range(3)]
        per_call = statistics.median(times) / n * n_seq
        return per_call, (f"{n} of {n_seq} (batch, head) sequences of {w.name} (LR scan), "
                          f"median of 3 runs, scaled to the whole call")

    all_threads = oracle.threads()
    per_call, sample = measure(target_s)
    oracle.set_threads(1)
    try:
        per_one, sample_one = measure(single_s)
    finally:
        oracle.set_threads(all_threads)
    return {"value": w.tokens / per_call, "unit": "tokens/s", "cores": all_threads,
            "kind": "oracle", "sample": sample, "us_per_call": per_call * 1e6,
            "cpu_model": cpu_model(),
            "single_thread": {"value": w.tokens / per_one, "unit": "tokens/s", "cores": 1,
                              "sample": sample_one, "us_per_call": per_one * 1e6}}


# --------------------------------------------------------------- roofline --
def kernel_sources_hash():
    """Hash of the kernel sources' code: comments and whitespace are left out, so a change
    to the documentation alone keeps a traffic record valid."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "gated_token_recurrence_amd", "csrc", "*"))):
        with open(p, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)   # block comments
        text = re.sub(r"//[^\n]*", " ", text)                # line comments
        h.update(os.path.basename(p).encode())
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


PATH_NAMES = {g.PATH_AUTO: "auto", g.PATH_MFMA: "mfma", g.PATH_FAST: "fast",
              g.PATH_SERIAL: "serial"}
LAUNCH_NAMES = {
    "mfma": ["segment_summary", "state_scan", "chunk_output"],
    "serial": ["chunk_summary", "state_scan", "chunk_output"],
    "fast": ["fast_single_launch"],
}
# launches a call may leave out: the matrix-core path has no scan launch when its output
# kernel folds the incoming states itself (few segments per sequence)
OPTIONAL_LAUNCHES = {"mfma": ("state_scan",)}


def launch_names(pname, n):
    """Names of the n launches of a call on path pname."""
    names = LAUNCH_NAMES[pname]
    if n < len(names):
        names = [x for x in names if x not in OPTIONAL_LAUNCHES.get(pname, ())]
    if len(names) != n:
        raise SystemExit(f"{n} launches on the {pname} path: expected {len(LAUNCH_NAMES[pname])}")
    return names


def resolve_path(w, requested, chunk=0):
    """The path the library runs: the requested one, or the one AUTO selects."""
    if requested != g.PATH_AUTO:
        return requested
    p = _lib.load().gtr_gla_auto_path(w.B, w.H, w.grid_h, w.grid_w, w.dk, w.dv, chunk,
                                      W.DTYPE_CODE[w.dtype])
    if p < 0:
        raise _lib.GtrError(p, _lib.last_error())
    return p


COPY_BYTES = 256 << 20


def profile_run(w, dev, sp, steps, path, chunk):
    """Workload calls for counter collection, preceded by a copy of known size."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize(dev)
    dst.copy_(src)                      # calibration: reads and writes COPY_BYTES
    torch.cuda.synchronize(dev)
    del src, dst
    lib = _lib.load()
    n_sets = W.rotation_sets(w.compulsory_bytes())
    _, sets = device_sets(w, n_sets, dev)
    for i in range(steps):
        call(lib, w, sets[i % n_sets], 0, chunk, path, sp)
    torch.cuda.synchronize(dev)
    log(f"profile run: {steps} calls of {w.name} ({PATH_NAMES[path]} path), "
        f"calibration copy {COPY_BYTES} bytes")


KERNEL_KEYS = {  # launch name -> test on the kernel symbol
    "segment_summary": lambda n: "k_sum<" in n or ("k_chunk<" in n and "true>" in n),
    "chunk_output": lambda n: "k_rows<" in n or ("k_chunk<" in n and "false>" in n),
    "state_scan": lambda n: "scan" in n,
    "fast_single_launch": lambda n: "k_fast" in n,
}

# SQ and GRBM counters taken in one pass (the hardware collects at most 8 SQ
# counters at once): instruction mix, matrix-core and VALU activity, GPU busy
# cycles for the utilisation fractions.
SQ_COUNTERS = ("SQ_WAVES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_LDS "
               "SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_BUSY_CYCLES GRBM_GUI_ACTIVE")
CU_COUNT, SIMDS_PER_CU, XCD_COUNT = 256, 4, 8


def _counter_values(csv_path):
    """Per (kernel, counter) list of per-dispatch values from a rocprofv3
    counter-collection CSV (FETCH_SIZE / WRITE_SIZE are in KiB)."""
    import csv
    vals = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            vals.setdefault((r["Kernel_Name"], r["Counter_Name"]), []).append(
                float(r["Counter_Value"]))
    return vals


def _find(vals, counter, key, reduce):
    match = key if callable(key) else (lambda n: key in n)
    hits = [v for (kn, c), v in vals.items() if c == counter and match(kn)]
    if len(hits) != 1:
        raise SystemExit(f"expected one kernel matching {key!r} for {counter}, found {len(hits)}")
    return reduce(hits[0])


def _mean(v):
    return sum(v) / len(v)


def present_launches(csv_path, path_name):
    """The path's launches whose kernel appears in a counter CSV (an optional launch
    the call left out is dropped; a missing required one stays, for ingest to report)."""
    kernels = {kn for kn, _ in _counter_values(csv_path)}
    return [n for n in LAUNCH_NAMES[path_name]
            if n not in OPTIONAL_LAUNCHES.get(path_name, ()) or
            any(KERNEL_KEYS[n](kn) for kn in kernels)]


def ingest_counters(fetch_csv, write_csv, sq_csv, workload, path_name, launches, out_dir=None):
    """Writes profiles/counters_<path>_<workload>.json from three counter runs of
    ``bench.py --profile-run`` (FETCH_SIZE; WRITE_SIZE; the SQ/GRBM set above).
    FETCH_SIZE and WRITE_SIZE are scaled by the ratio of the calibration copy's
    known bytes to what the same counter read for it; per launch of the call and
    summed over the call.  Utilisation: matrix-core busy cycles over the GPU's busy
    cycles times its SIMDs (rocprofv3's MfmaUtil); VALU: the VALU-active count over
    the busy cycles times the CUs (rocprofv3's VALUBusy)."""
    fetch, write = _counter_values(fetch_csv), _counter_values(write_csv)
    sq = _counter_values(sq_csv) if sq_csv else {}
    copy_f = _find(fetch, "FETCH_SIZE", "copyBuffer", max) * 1024
    copy_w = _find(write, "WRITE_SIZE", "copyBuffer", max) * 1024
    f_scale, w_scale = COPY_BYTES / copy_f, COPY_BYTES / copy_w
    per = {}
    for name in launches:
        key = KERNEL_KEYS[name]
        kf = _find(fetch, "FETCH_SIZE", key, _mean) * 1024 * f_scale
        kw = _find(write, "WRITE_SIZE", key, _mean) * 1024 * w_scale
        rec = {"fetch_bytes": round(kf), "write_bytes": round(kw), "bytes": round(kf + kw)}
        if sq:
            c = {cn: _find(sq, cn, key, _mean) for cn in SQ_COUNTERS.split()}
            waves = c["SQ_WAVES"]
            # GRBM_GUI_ACTIVE comes summed over the XCDs: per XCD it is the kernel's
            # busy clock count (rocprofv3's MfmaUtil and VALUBusy take its maximum)
            gui = c["GRBM_GUI_ACTIVE"] / XCD_COUNT
            rec.update({
                "valu_insts_per_wave": round(c["SQ_INSTS_VALU"] / waves, 1),
                "trans_insts_per_wave": round(c["SQ_INSTS_VALU_TRANS_F32"] / waves, 1),
                "mfma_insts_per_wave": round(c["SQ_INSTS_MFMA"] / waves, 1),
                "lds_insts_per_wave": round(c["SQ_INSTS_LDS"] / waves, 1),
                "busy_us_at_2400mhz": round(gui / 2400.0, 2),
                # rocprofv3's MfmaUtil and VALUBusy, as fractions
                "mfma_busy_frac": round(c["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * CU_COUNT * SIMDS_PER_CU), 4),
                "valu_busy_frac": round(c["SQ_ACTIVE_INST_VALU"] / (gui * CU_COUNT), 4),
                "raw": {cn: round(v, 1) for cn, v in c.items()}})
        per[name] = rec
    out = {"workload": workload, "path": path_name, "launches": per,
           "call_fetch_bytes": sum(r["fetch_bytes"] for r in per.values()),
           "call_write_bytes": sum(r["write_bytes"] for r in per.values()),
           "call_bytes": sum(r["bytes"] for r in per.values()),
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "calibration_copy_bytes": COPY_BYTES, "sources_hash": kernel_sources_hash(),
           "csv": [os.path.relpath(p, ROOT) for p in (fetch_csv, write_csv, sq_csv) if p]}
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"counters_{path_name}_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))
    return out


def counters_record(path_name, workload, out_dir=None):
    p = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"counters_{path_name}_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    if rec.get("sources_hash") != kernel_sources_hash():
        return None  # the kernels changed since the counters were taken
    return rec


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def roofline_record(comp, us, launch_us, names, cr, flops):
    """The JSON line's roofline object.  comp: the call's algorithmic bytes; us: the
    call's mean duration; launch_us: mean duration of each launch (names); cr: the
    counter record of this path and workload (or None); flops: the call's algorithmic
    flops.  The dominant kernel (chunk outputs) reads every input and writes the
    output, so its algorithmic bytes per launch are the call's; "frac" is that
    kernel's fraction of the HBM peak, and the call as a whole (the bar the method is
    judged on) is reported under "whole_call"."""
    dom = int(np.argmax(launch_us))
    dom_us = launch_us[dom]
    achieved = comp / (dom_us * 1e-6) / 1e9
    call_achieved = comp / (us * 1e-6) / 1e9
    traffic = call_traffic = None
    mfma_meas = valu_meas = mfma_call = None
    if cr is not None:
        lr = cr["launches"]
        if names[dom] in lr:
            traffic = lr[names[dom]]["bytes"]
            mfma_meas = lr[names[dom]].get("mfma_busy_frac")
            valu_meas = lr[names[dom]].get("valu_busy_frac")
        call_traffic = cr["call_bytes"]
        if all("mfma_busy_frac" in lr.get(n, {}) for n in names):
            mfma_call = sum(lr[n]["mfma_busy_frac"] * t for n, t in zip(names, launch_us)) / sum(launch_us)
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": names[dom], "kernel_us": round(dom_us, 3),
            "frac_of": f"the dominant kernel ({names[dom]}); the whole call: whole_call_frac",
            "algorithmic_bytes": comp,
            "whole_call": {"us": round(us, 3), "achieved": round(call_achieved, 1),
                           "frac": round(call_achieved / HBM_PEAK_GBS, 4),
                           "traffic": call_traffic},
            "whole_call_frac": round(call_achieved / HBM_PEAK_GBS, 4),
            "mfma_util": {"measured_kernel": mfma_meas,
                          "measured_call": round(mfma_call, 4) if mfma_call is not None else None,
                          "algorithmic_call": round(flops / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5),
                          "peak_tflops": MFMA_BF16_PEAK_TFLOPS},
            "valu_busy_kernel": valu_meas}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # Measured on MI355X: the first few hundred calls of a workload run ~10% slower than the
    # steady state (75 vs 69 us per call at 16.4K tokens after 20 vs 500 warm-up calls;
    # loading the GPU with copies or matrix products first does not shorten it), so the
    # default warms up for 1000 calls (~0.1 s at 16.4K tokens).
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default="mixer_2048")
    ap.add_argument("--path", type=int, default=g.PATH_AUTO)
    ap.add_argument("--chunk", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--profile-run", action="store_true",
                    help="for rocprofv3 counter passes: a plain 256 MiB device copy (the "
                         "calibration kernel), then --steps calls of the workload; no timing")
    ap.add_argument("--ingest-counters", nargs="+", metavar="CSV",
                    help="write the counter record for --workload from the rocprofv3 counter "
                         "CSVs of --profile-run: FETCH_SIZE, WRITE_SIZE and optionally the SQ "
                         "set (bench.SQ_COUNTERS); no GPU needed")
    args = ap.parse_args()
    if args.ingest_counters:
        if len(args.ingest_counters) not in (2, 3):
            raise SystemExit("--ingest-counters takes FETCH_CSV WRITE_CSV [SQ_CSV]")
        wi = W.WORKLOADS[args.workload]
        pn = PATH_NAMES[resolve_path(wi, args.path, args.chunk or wi.chunk)]
        f_csv, w_csv = args.ingest_counters[:2]
        sq_csv = args.ingest_counters[2] if len(args.ingest_counters) == 3 else None
        ingest_counters(f_csv, w_csv, sq_csv, args.workload, pn, present_launches(f_csv, pn))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hip = Hip()
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    w = W.WORKLOADS[args.workload]
    chunk = args.chunk or w.chunk
    path = resolve_path(w, args.path, chunk)
    if args.profile_run:
        profile_run(w, dev, sp, args.steps, path, chunk)
        return
    pname = PATH_NAMES[path]
    log(f"workload {w.name}: B={w.B} grid {w.grid_h}x{w.grid_w} H={w.H} dk={w.dk} dv={w.dv} "
        f"{w.dtype} chunk {chunk} path {pname}")
    x, res = time_workload(w, dev, hip, sp, args.steps, args.warmup, path, chunk)
    log(f"  {res['us_per_call']:.2f} us/call (rotating {res['n_sets']} sets), "
        f"hot {res['us_per_call_hot']:.2f}, graph {res.get('us_per_call_graph')}, "
        f"launches {['%.2f' % t for t in res['launch_us_mean']]}")

    comp = w.compulsory_bytes()
    us = res["us_per_call"]
    value = w.tokens / (us * 1e-6)
    launch_us = res["launch_us_mean"]
    names = launch_names(pname, len(launch_us))
    roofline = roofline_record(comp, us, launch_us, names, counters_record(pname, w.name),
                               w.algorithmic_flops(chunk))
    extra = {}
    if not args.no_extra:
        for name in ("mixer_640", "mixer_640_wide"):
            we = W.WORKLOADS[name]
            pa = resolve_path(we, args.path, we.chunk)
            for pe in dict.fromkeys([pa, g.PATH_MFMA, g.PATH_FAST]):
                key = name if pe == pa else f"{name}@{PATH_NAMES[pe]}"
                try:
                    _, r = time_workload(we, dev, hip, sp, args.steps, args.warmup, pe, we.chunk,
                                         per_kernel=False)
                except Exception as exc:  # report, do not hide
                    extra[key] = {"error": str(exc)}
                    continue
                extra[key] = {"us_per_call": round(r["us_per_call"], 3),
                              "us_per_call_graph": (round(r["us_per_call_graph"], 3)
                                                    if r["us_per_call_graph"] else None),
                              "us_per_call_hot": round(r["us_per_call_hot"], 3),
                              "tokens_per_s": round(we.tokens / (r["us_per_call"] * 1e-6)),
                              "hbm_frac": round(we.compulsory_bytes() / (r["us_per_call"] * 1e-6)
                                                / 1e9 / HBM_PEAK_GBS, 4),
                              "path": PATH_NAMES[pe]}
                log(f"  {key}: {r['us_per_call']:.2f} us/call, graph {r['us_per_call_graph']}"
                    f"{' (' + r['graph_error'] + ')' if r.get('graph_error') else ''}")
    directions = {}
    if not args.no_extra:
        # the other scan orders on the same workload (TB and BT gather columns with a stride
        # of grid_w rows)
        directions["LR"] = {"us_per_call": round(us, 3), "hbm_frac": roofline["whole_call_frac"]}
        for d, dn in ((1, "RL"), (2, "TB"), (3, "BT")):
            try:
                _, r = time_workload(w, dev, hip, sp, args.steps, args.warmup, path, chunk,
                                     direction=d, per_kernel=False, graph=False)
            except Exception as exc:  # report, do not hide
                directions[dn] = {"error": str(exc)[:300]}
                continue
            directions[dn] = {"us_per_call": round(r["us_per_call"], 3),
                              "hbm_frac": round(comp / (r["us_per_call"] * 1e-6) / 1e9
                                                / HBM_PEAK_GBS, 4)}
            log(f"  direction {dn}: {r['us_per_call']:.2f} us/call")
    lowrank = None
    if not args.no_extra and w.dtype != "f32":
        # the same shapes with the gate formed from rank-16 features inside the kernels
        try:
            r = time_lowrank(w, dev, hip, sp, args.steps, args.warmup, chunk)
            lb = w.compulsory_bytes_lowrank(16)
            # the gate formed in the kernels: the plain call's launches; written out
            # first: one more
            lnames = (names if r["launches"] == len(names)
                      else ("gate_projection",) + tuple(names))
            lowrank = {"workload": f"{w.name} shapes, log_g formed from rank-16 fp16 gate "
                                   f"features (tau 16) in the kernels",
                       "us_per_call": round(r["us_per_call"], 3),
                       "tokens_per_s": round(w.tokens / (r["us_per_call"] * 1e-6), 1),
                       "algorithmic_bytes": lb,
                       "whole_call_frac": round(lb / (r["us_per_call"] * 1e-6) / 1e9
                                                / HBM_PEAK_GBS, 4),
                       "launch_us_mean": {n: round(t, 3) for n, t in
                                          zip(lnames, r["launch_us_mean"])},
                       "rotating_sets": r["n_sets"]}
            log(f"  lowrank gate: {r['us_per_call']:.2f} us/call, launches "
                f"{['%.2f' % t for t in r['launch_us_mean']]}")
        except Exception as exc:  # report, do not hide
            lowrank = {"error": str(exc)[:300]}
    sswiglu = {}
    if not args.no_extra:
        for name, ws in W.SSWIGLU_WORKLOADS.items():
            try:
                r = time_sswiglu(ws, dev, hip, sp, args.steps, args.warmup)
            except Exception as exc:  # report, do not hide
                sswiglu[name] = {"error": str(exc)[:300]}
                continue
            gbs = ws.compulsory_bytes() / (r["us_per_call"] * 1e-6) / 1e9
            sswiglu[name] = {"workload": f"B={ws.B}, grid {ws.grid_h}x{ws.grid_w}, F={ws.F}, "
                                         f"{ws.k}x{ws.k} depthwise, {ws.dtype}",
                             "us_per_call": round(r["us_per_call"], 3),
                             "tokens_per_s": round(ws.tokens / (r["us_per_call"] * 1e-6), 1),
                             "algorithmic_bytes": ws.compulsory_bytes(),
                             "achieved_GBs": round(gbs, 1),
                             "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                             "rotating_sets": r["n_sets"]}
            log(f"  {name}: {r['us_per_call']:.2f} us/call, {gbs:.0f} GB/s")
    backward = None
    if not args.no_extra:
        try:
            bus, blaunch, bus_states = time_backward(w, dev, hip, sp, max(10, args.steps // 4), 3)
            s_io = W.DTYPE_BYTES[w.dtype]
            bbytes = w.tokens * w.H * ((2 * w.dk + 3 * w.dv) * s_io + 4 * w.dk      # reads
                                       + (2 * w.dk + 2 * w.dv) * s_io + 4 * w.dk)   # writes
            if w.dtype != "f32" and w.dk == 64 and w.dv == 64 and w.chunk <= 64:  # matrix-core gradients
                names_b = ("forward_segment_summary", "forward_segment_scan", "chunk_do_and_summary_mfma",
                           "fallback_do_and_summary_rms_w", "reverse_state_scan", "chunk_gradients_mfma",
                           "fallback_gradients")
            else:
                names_b = ("forward_chunk_summary", "forward_state_scan", "forward_walk_dq",
                           "reverse_chunk_summary", "reverse_state_scan", "reverse_walk_dk_dv",
                           "gate_total_scan", "gate_offsets", "rms_w_sum")
            backward = {"workload": f"{w.name}: backward of one call (matrix cores, bf16 hi+lo operands, fp32 accumulation)",
                        "us_per_call": round(bus, 3),
                        "tokens_per_s": round(w.tokens / (bus * 1e-6), 1),
                        "algorithmic_bytes": bbytes,
                        "hbm_frac": round(bbytes / (bus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                        "launch_us_mean": {n: round(t, 2) for n, t in zip(names_b, blaunch)}}
            if bus_states is not None:  # given the forward's segment states (gtr_gla_bwd_states)
                backward["us_per_call_with_forward_states"] = round(bus_states, 3)
            log(f"  backward: {bus:.1f} us/call, launches {['%.1f' % t for t in blaunch]}, "
                f"with forward states {bus_states}")
        except Exception as exc:  # report, do not hide
            backward = {"error": str(exc)[:300]}
    backbone = None
    if not args.no_extra:
        try:
            cfg, eager_ms, graph_ms = time_backbone(dev, max(10, args.steps // 4))
            backbone = {"workload": f"{cfg.blocks}-block backbone, {cfg.image}x{cfg.image} "
                                    f"image (grid {cfg.grid}x{cfg.grid}), width {cfg.width}, "
                                    f"{cfg.heads} heads, S-SwiGLU hidden {cfg.hidden}, fp16, "
                                    f"random weights",
                        "ms_per_image_graph": round(graph_ms, 4),
                        "ms_per_image_eager": round(eager_ms, 4)}
            log(f"  backbone: graph {graph_ms:.3f} ms, eager {eager_ms:.3f} ms per image")
        except Exception as exc:  # report, do not hide
            backbone = {"error": str(exc)[:300]}
    stack = None
    if not args.no_extra:
        try:
            ws, ms, sbytes = time_stack(dev, hip, sp, 5, 2)
            stack = {"workload": f"{ws.name}: {ws.n_blocks}-block stack, B = {ws.B}, grid "
                                 f"{ws.grid_h}x{ws.grid_w}, H = {ws.H}, dk = {ws.dk}, dv = {ws.dv}, "
                                 f"{ws.dtype}, inputs drawn on the device",
                     "ms_per_stack": round(ms, 4),
                     "us_per_block": round(ms * 1e3 / ws.n_blocks, 2),
                     "algorithmic_bytes": sbytes,
                     "hbm_frac": round(sbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            log(f"  stack: {ms:.3f} ms ({ms * 1e3 / ws.n_blocks:.1f} us per block)")
        except Exception as exc:  # report, do not hide
            stack = {"error": str(exc)[:300]}
    cpu = None
    if not args.no_cpu:
        log("  timing the fp64 oracle on the host (bounded sample)")
        cpu = cpu_baseline(w, x)
        log(f"  oracle: {cpu['value']:.3e} tokens/s on {cpu['cores']} threads")

    line = {
        "metric": "GLA-scan tokens/s + µs/call at 1.6K & 16.4K tokens; % of HBM/MFMA roofline",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if pname == "serial" else "bf16x2-f32acc",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B={w.B}, grid {w.grid_h}x{w.grid_w} ({w.L} tokens), "
                               f"H={w.H}, dk={w.dk}, dv={w.dv}, {w.dtype} I/O, chunk {chunk}, "
                               f"direction LR",
                   "path": pname, "global_batch": w.B, "seq_len": w.L, "parallelism": "none"},
        "us_per_call": round(us, 3),
        "us_per_call_hot": round(res["us_per_call_hot"], 3),
        "us_per_call_graph": (round(res["us_per_call_graph"], 3)
                              if res["us_per_call_graph"] else None),
        "us_per_call_p10_p50_p90": [round(res["us_per_call_evented_p10"], 3),
                                    round(res["us_per_call_evented_median"], 3),
                                    round(res["us_per_call_evented_p90"], 3)],
        "launch_us_mean": {n: round(t, 3) for n, t in zip(names, res["launch_us_mean"])},
        "rotating_sets": res["n_sets"],
        "roofline": roofline,
        "cpu_baseline": cpu,
        "directions": directions,
        "extra_1p6k": extra,
        "lowrank_gate": lowrank,
        "sswiglu_mix": sswiglu,
        "backbone_640": backbone,
        "stack_1024": stack,
        "backward": backward,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
