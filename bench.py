#!/usr/bin/env python3
"""Throughput of speculative verification over the vocabulary on one MI355X.

One step = one full verification call (all kernels of the path) over one
batch of synthetic logits already resident in HBM.  The headline workload is
the largest chain configuration that fits one GPU: chain verification over a
speculation cache, 32 requests x 8 anticipated outcomes = 256 blocks,
gamma=16, V=151936, bf16 logits, T=0.6.  The other workloads (the B=1 fp32
chain, the B=64 bf16 chain, greedy and stochastic tree verification,
point-mass chains, outcome scoring and tree construction) are reported in the
same JSON line under "per_config", each with its own roofline block.

Timing: the K timed steps are captured once in a HIP graph (rotating through
enough input copies that the working set is at least 512 MiB, twice the
Infinity Cache) and replayed between two events, with a device synchronise on
both sides; a spin kernel queued ahead of the start event covers the host's
submission of the graph, so the events bracket the K steps themselves.  The dominant kernel's average duration comes from HIP events the
library records around it on the same stream, over K eager steps.  The CPU
baseline is the fp64 oracle on a bounded sample of the same workload.

Prints exactly one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBPS = 8000.0  # MI355X HBM3E peak, GB/s
METRIC = "logit bytes verified/s (HBM GB/s, % peak) + verify rounds/s at B×γ×V"
CACHE_BYTES = 512 << 20
HEADLINE_CFG = 5


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch already loaded."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.lib.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a),
                                        ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.lib.hipEventDestroy(ctypes.c_void_p(e))


def source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_draft_verification_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel_key)
    if not rec or rec.get("source_digest") != source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------- workloads --

def synth_rows(W, N):
    return sum(W ** d for d in range(N))


class Workload:
    """Device-resident input copies plus a direct C-ABI call per step."""

    def __init__(self, cfg, seed, torch, sv):
        import numpy as np

        import synth

        self.cfg = cfg
        if cfg == "outcome":
            self.spec = dict(synth.OUTCOME_CONFIG, kind="outcome")
            self.bytes = synth.outcome_config_bytes()
            t0 = time.time()
            d = synth.outcome_config_inputs(seed=seed)
        elif cfg == "stree":
            self.spec = dict(synth.STREE_CONFIG, kind="stree")
            self.bytes = synth.stree_config_bytes()
            t0 = time.time()
            d = synth.stree_config_inputs(seed=seed)
        elif cfg == "treebuild":
            self.spec = dict(synth.TREEBUILD_CONFIG, kind="treebuild")
            self.bytes = synth.treebuild_config_bytes()
            t0 = time.time()
            d = synth.treebuild_config_inputs(seed=seed)
        elif isinstance(cfg, str) and cfg.startswith("pm"):
            base = int(cfg[2:])
            self.spec = dict(synth.POINTMASS_CONFIGS[base], kind="pointmass")
            self.bytes = synth.pointmass_config_bytes(base)
            t0 = time.time()
            d = synth.pointmass_config_inputs(base, seed=seed)
        else:
            self.spec = dict(synth.CONFIGS[cfg])
            self.bytes = synth.config_bytes(cfg)
            t0 = time.time()
            d = synth.config_inputs(cfg, seed=seed)
        self.kind = self.spec["kind"]
        log(f"[bench] config {cfg}: inputs drawn in {time.time() - t0:.1f}s")
        self.host = d
        self.nsets = max(2, math.ceil(CACHE_BYTES / self.bytes))
        dev = torch.device("cuda:0")
        dt = self.spec["dtype"]

        def logits(a):
            if dt == "f32":
                return torch.from_numpy(a).to(dev)
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

        self.lib = sv.load_library()
        self.code = sv.SV_DTYPE_F32 if dt == "f32" else sv.SV_DTYPE_BF16
        P = ctypes.c_void_p
        if self.kind == "outcome":
            R, g, V, nc = d["R"], d["gamma"], d["V"], d["ncache"]
            t0g = logits(d["target"])
            tok = torch.from_numpy(d["draft_tokens"]).to(dev)
            self.sets = []
            for i in range(self.nsets):
                lg = t0g if i == 0 else t0g.clone()
                k = torch.empty((R, nc), dtype=torch.int32, device=dev)
                a = torch.empty((R, nc), dtype=torch.int32, device=dev)
                pr = torch.empty((R, nc), dtype=torch.float64, device=dev)
                hit = torch.empty(R, dtype=torch.float64, device=dev)
                self.sets.append((lg, tok, k, a, pr, hit))
            nbytes = sv.spec_outcome_topk_workspace_bytes(R, g, V, self.code, nc)
            self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
            self.args = [(P(lg.data_ptr()), self.code, P(tk.data_ptr()), R, g, V, float(d["T"]), nc,
                          P(k_.data_ptr()), P(a_.data_ptr()), P(p_.data_ptr()), P(h_.data_ptr()),
                          P(self.ws.data_ptr()), nbytes)
                         for lg, tk, k_, a_, p_, h_ in self.sets]
            self.n_events = 2
            self.shape = dict(R=R, gamma=g, V=V, ncache=nc)
        elif self.kind == "stree":
            B, n, V = d["B"], d["n"], d["V"]
            t0g, d0g = logits(d["target"]), logits(d["draft"])
            par = torch.from_numpy(d["parents"]).to(dev)
            tok = torch.from_numpy(d["tokens"]).to(dev)
            uni = torch.from_numpy(d["uniforms"]).to(dev)
            self.sets = []
            for i in range(self.nsets):
                tg = t0g if i == 0 else t0g.clone()
                dr = d0g if i == 0 else d0g.clone()
                acc = torch.empty(B, dtype=torch.int32, device=dev)
                node = torch.empty(B, dtype=torch.int32, device=dev)
                out = torch.empty((B, n), dtype=torch.int32, device=dev)
                self.sets.append((tg, dr, acc, node, out))
            nbytes = sv.spec_verify_tree_stochastic_workspace_bytes(B, n, V, self.code)
            self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
            self.args = [(P(tg.data_ptr()), P(dr.data_ptr()), self.code, P(par.data_ptr()),
                          P(tok.data_ptr()), P(uni.data_ptr()), B, n, V, float(d["T"]),
                          P(ac.data_ptr()), P(no.data_ptr()), P(ou.data_ptr()), None,
                          P(self.ws.data_ptr()), nbytes)
                         for tg, dr, ac, no, ou in self.sets]
            self.n_events = 3
            self.shape = dict(B=B, n=n, V=V)
        elif self.kind == "treebuild":
            R, M, V, W, N, nb = d["R"], d["M"], d["V"], d["W"], d["N"], d["budget"]
            z0 = logits(d["logits"])
            self.sets = []
            for i in range(self.nsets):
                lg = z0 if i == 0 else z0.clone()
                outs = [torch.empty((R, nb), dtype=torch.int32, device=dev) for _ in range(3)]
                sc = torch.empty((R, nb), dtype=torch.float64, device=dev)
                n = torch.empty(R, dtype=torch.int32, device=dev)
                self.sets.append((lg, *outs, sc, n))
            nbytes = sv.spec_tree_build_workspace_bytes(R, M, V, self.code, W, N, nb)
            self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
            self.args = [(P(lg.data_ptr()), self.code, None, R, M, V, float(d["T"]), W, N, nb,
                          P(pa.data_ptr()), P(tk.data_ptr()), P(ro.data_ptr()), P(sc.data_ptr()),
                          P(n.data_ptr()), P(self.ws.data_ptr()), nbytes)
                         for lg, pa, tk, ro, sc, n in self.sets]
            self.n_events = 2
            self.shape = dict(R=R, M=M, V=V, W=W, N=N, budget=nb)
        elif self.kind == "pointmass":
            B, g, V = d["B"], d["gamma"], d["V"]
            t0g = logits(d["target"])
            tok = torch.from_numpy(d["draft_tokens"]).to(dev)
            uni = torch.from_numpy(d["uniforms"]).to(dev)
            self.sets = []
            for i in range(self.nsets):
                tg = t0g if i == 0 else t0g.clone()
                acc = torch.empty(B, dtype=torch.int32, device=dev)
                out = torch.empty((B, g + 1), dtype=torch.int32, device=dev)
                self.sets.append((tg, tok, uni, acc, out))
            nbytes = sv.spec_verify_chain_pointmass_workspace_bytes(B, g, V, self.code)
            self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
            self.args = [(P(tg.data_ptr()), self.code, P(tk.data_ptr()), P(un.data_ptr()), B, g, V,
                          float(d["T"]), P(ac.data_ptr()), P(ou.data_ptr()), None,
                          P(self.ws.data_ptr()), nbytes)
                         for tg, tk, un, ac, ou in self.sets]
            self.n_events = 3
            self.shape = dict(B=B, gamma=g, V=V)
        elif self.kind == "chain":
            B, g, V = d["B"], d["gamma"], d["V"]
            t0g, d0g = logits(d["target"]), logits(d["draft"])
            tok = torch.from_numpy(d["draft_tokens"]).to(dev)
            uni = torch.from_numpy(d["uniforms"]).to(dev)
            self.sets = []
            for i in range(self.nsets):
                tg = t0g if i == 0 else t0g.clone()
                dr = d0g if i == 0 else d0g.clone()
                acc = torch.empty(B, dtype=torch.int32, device=dev)
                out = torch.empty((B, g + 1), dtype=torch.int32, device=dev)
                self.sets.append((tg, dr, tok, uni, acc, out))
            nbytes = sv.spec_verify_chain_workspace_bytes(B, g, V, self.code)
            self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
            self.args = [(P(tg.data_ptr()), P(dr.data_ptr()), self.code, P(tk.data_ptr()),
                          P(un.data_ptr()), B, g, V, float(d["T"]), P(ac.data_ptr()),
                          P(ou.data_ptr()), None, P(self.ws.data_ptr()), nbytes)
                         for tg, dr, tk, un, ac, ou in self.sets]
            self.n_events = 3
            self.shape = dict(B=B, gamma=g, V=V)
        else:
            B, n, V = d["B"], d["n"], d["V"]
            t0g = logits(d["target"])
            par = torch.from_numpy(d["parents"]).to(dev)
            tok = torch.from_numpy(d["tokens"]).to(dev)
            self.sets = []
            for i in range(self.nsets):
                tg = t0g if i == 0 else t0g.clone()
                acc = torch.empty(B, dtype=torch.int32, device=dev)
                node = torch.empty(B, dtype=torch.int32, device=dev)
                out = torch.empty((B, n), dtype=torch.int32, device=dev)
                self.sets.append((tg, par, tok, acc, node, out))
            nbytes = sv.spec_verify_tree_greedy_workspace_bytes(B, n, V, self.code)
            self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
            self.args = [(P(tg.data_ptr()), self.code, P(pa.data_ptr()), P(tk.data_ptr()), B, n,
                          V, P(ac.data_ptr()), P(no.data_ptr()), P(ou.data_ptr()),
                          P(self.ws.data_ptr()), nbytes)
                         for tg, pa, tk, ac, no, ou in self.sets]
            self.n_events = 2
            self.shape = dict(B=B, n=n, V=V)
        torch.cuda.synchronize()

    ENTRY = {"chain": "spec_verify_chain", "pointmass": "spec_verify_chain_pointmass",
             "outcome": "spec_outcome_topk", "treebuild": "spec_tree_build",
             "stree": "spec_verify_tree_stochastic", "tree": "spec_verify_tree_greedy"}

    def step(self, i, stream_handle, events=None):
        """One library call; with events, its instrumented twin (the same
        kernels, plus event records around the dominant kernel)."""
        a = self.args[i % self.nsets]
        name = self.ENTRY[self.kind]
        if events is None:
            st = getattr(self.lib, name)(*a, stream_handle)
        else:
            arr = (ctypes.c_void_p * len(events))(*events)
            st = getattr(self.lib, name + "_timed")(*a, stream_handle,
                                                    ctypes.cast(arr, ctypes.c_void_p))
        if st != 0:
            raise RuntimeError(f"library call failed with status {st}")

    def outputs(self):
        keep = {"treebuild": 5, "stree": 3}.get(self.kind, 2)  # every output tensor of the call
        return [tuple(t.cpu().clone() for t in s[-keep:]) for s in self.sets]

    def describe(self):
        s = self.spec
        if self.kind == "outcome":
            return (f"outcome scoring + cache of {s['ncache']} R={s['R']} gamma={s['gamma']} "
                    f"V={s['V']} {s['dtype']} T={s['T']} (decoder rows {s['target'][0]}x"
                    f"{s['target'][1]}; draft token = row argmax w.p. {s['p_match']} else uniform)")
        if self.kind == "stree":
            return (f"stochastic tree verify B={s['B']} n={s['n']} V={s['V']} {s['dtype']} "
                    f"T={s['T']} (target {s['target'][0]}x{s['target'][1]}, draft = target + "
                    f"N(0,{s['noise']}^2) per node, depth<={s['max_depth']}, "
                    f"branching<={s['max_children']}, node tokens ~ q at the parent, "
                    f"seeded uniforms)")
        if self.kind == "treebuild":
            return (f"draft-tree construction R={s['R']} W={s['W']} N={s['N']} "
                    f"budget={s['budget']} V={s['V']} {s['dtype']} T={s['T']} (one draft row per "
                    f"potential node of the complete {s['W']}-ary tree above depth {s['N']}: "
                    f"{synth_rows(s['W'], s['N'])} rows of {s['logits'][0]}x{s['logits'][1]})")
        if self.kind == "pointmass":
            tgt = f"{s['target'][0]}x{s['target'][1]}"
            extra = f", +{s['boost'][1]:g} on {s['boost'][0]} ids/row" if s.get("boost") else ""
            return (f"point-mass chain verify B={s['B']} gamma={s['gamma']} V={s['V']} "
                    f"{s['dtype']} T={s['T']} (target {tgt}{extra}; draft token = target "
                    f"argmax w.p. {s['p_match']} else uniform; no draft logits; seeded uniforms)")
        if self.kind == "chain":
            tgt = f"{s['target'][0]}x{s['target'][1]}"
            extra = f", +{s['boost'][1]:g} on {s['boost'][0]} ids/row" if s.get("boost") else ""
            return (f"chain verify B={s['B']} gamma={s['gamma']} V={s['V']} {s['dtype']} "
                    f"T={s['T']} (target {tgt}{extra}, draft = target + N(0,{s['noise']}^2), "
                    f"draft tokens ~ q, seeded uniforms)")
        return (f"greedy tree verify B={s['B']} n={s['n']} V={s['V']} {s['dtype']} "
                f"(target N(0,{s['sigma']}^2), depth<={s['max_depth']}, "
                f"branching<={s['max_children']}, tokens = parent argmax w.p. {s['p_match']})")


def measure(w, steps, warmup, torch, hip):
    """Graph-replayed throughput plus per-kernel event timing."""
    cur = torch.cuda.current_stream()
    h = ctypes.c_void_p(cur.cuda_stream)
    for i in range(max(warmup, w.nsets)):
        w.step(i, h)
    torch.cuda.synchronize()
    eager = w.outputs()

    # capture the K timed steps once
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap):
        hc = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for i in range(steps):
            w.step(i, hc)
    g.replay()  # untimed warm replay
    torch.cuda.synchronize()
    for a, b in zip(eager, w.outputs()):
        for x, y in zip(a, b):
            if not torch.equal(x, y):
                raise RuntimeError("graph replay disagrees with eager results")

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)

    def timed_replay(graph):
        """ms between events around one replay of the K captured steps.  The
        host needs about 15 us per step to submit the graph's kernels; a spin
        kernel ahead of the start event (at least about 5 ms) keeps the GPU
        busy meanwhile and at its working clock after the host-side checks,
        so the events bracket the K steps running back to back rather than
        the submission (which would add about 300 us to 20 config-5 steps)."""
        torch.cuda.synchronize()
        torch.cuda._sleep(min(max(steps * 120_000, 12_000_000), 400_000_000))
        start.record()
        graph.replay()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end)

    g.replay()  # a second untimed replay, just ahead of the timed one
    ms = timed_replay(g)
    for a, b in zip(eager, w.outputs()):
        for x, y in zip(a, b):
            if not torch.equal(x, y):
                raise RuntimeError("timed replay disagrees with eager results")
    del g

    # dominant-kernel duration from events recorded around it by the library
    n_ev = min(steps, 400)
    evs = hip.create(w.n_events * n_ev)
    torch.cuda.synchronize()
    # The host needs about 30 us to enqueue one call, longer than a small
    # workload's step: a spin kernel ahead of the calls (about 60 us of GPU
    # time per call) lets all of them be queued first, so that they run back
    # to back as in the graph instead of one by one on an idling GPU.
    torch.cuda._sleep(n_ev * 150_000)
    for i in range(n_ev):
        w.step(i, h, evs[i * w.n_events:(i + 1) * w.n_events])
    torch.cuda.synchronize()
    k1 = [hip.elapsed_ms(evs[i * w.n_events], evs[i * w.n_events + 1]) for i in range(n_ev)]
    k2 = ([hip.elapsed_ms(evs[i * 3 + 1], evs[i * 3 + 2]) for i in range(n_ev)]
          if w.n_events == 3 else None)
    hip.destroy(evs)
    k1_ms = sum(k1) / len(k1)

    # the same K steps captured again and replayed 5 more times: the spread of
    # the measurement (reported beside the one bracketed run above)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        hc = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for i in range(steps):
            w.step(i, hc)
    reps = []
    for _ in range(5):
        reps.append(timed_replay(g) * 1e3 / steps)
    del g
    reps.sort()
    res = dict(ms_per_step=ms / steps, gbps=w.bytes * steps / (ms * 1e-3) / 1e9,
               rounds_per_s=steps / (ms * 1e-3), dominant_ms=k1_ms,
               dominant_gbps=w.bytes / (k1_ms * 1e-3) / 1e9,
               repeats=dict(n=len(reps), median_us_per_step=round(reps[len(reps) // 2], 3),
                            min_us_per_step=round(reps[0], 3), max_us_per_step=round(reps[-1], 3)))
    if k2 is not None:
        res["final_kernel_ms"] = sum(k2) / len(k2)
    return res


def cpu_baseline(w, budget_s):
    """The oracle on the host cores, on whole rounds of the workload (or, for
    the single-threaded outcome and tree-construction oracles, on rounds of
    its first few requests), for about budget_s seconds."""
    import oracle

    d = w.host
    threads = min(16, os.cpu_count() or 1)
    units, used = d.get("B", d.get("R")), None
    if w.kind in ("outcome", "treebuild", "stree"):
        used = min(4, units)
        threads = 1
    rounds, t0 = 0, time.time()
    while True:
        if w.kind == "chain":
            oracle.chain(d["target"], d["draft"], d["draft_tokens"], d["uniforms"], d["T"],
                         dtype=d["dtype"], threads=threads)
        elif w.kind == "pointmass":
            oracle.chain_pointmass(d["target"], d["draft_tokens"], d["uniforms"], d["T"],
                                   dtype=d["dtype"], threads=threads)
        elif w.kind == "outcome":
            oracle.outcome_topk(d["target"][:used], d["draft_tokens"][:used], d["T"], d["ncache"],
                                dtype=d["dtype"])
        elif w.kind == "treebuild":
            oracle.tree_build(d["logits"][:used], d["T"], d["W"], d["N"], d["budget"],
                              dtype=d["dtype"])
        elif w.kind == "stree":
            oracle.tree_stochastic(d["target"][:used], d["draft"][:used], d["parents"][:used],
                                   d["tokens"][:used], d["uniforms"][:used], d["T"],
                                   dtype=d["dtype"])
        else:
            oracle.tree_greedy(d["target"], d["parents"], d["tokens"], dtype=d["dtype"],
                               threads=threads)
        rounds += 1
        if time.time() - t0 >= budget_s:
            break
    dt = time.time() - t0
    frac = 1.0 if used is None else used / units
    n = units if used is None else used
    if used is None:
        sample = (f"{rounds} full rounds of the workload ({units} block(s), "
                  f"{min(threads, units)} thread(s)) in {dt:.1f}s (fp64 oracle)")
    else:
        sample = (f"{rounds} rounds of the first {used} of the workload's {units} requests "
                  f"on one thread in {dt:.1f}s (fp64 oracle), scaled to bytes per second")
    return {"value": round(w.bytes * frac * rounds / dt / 1e9, 4), "unit": "GB/s",
            "cores": min(threads, n), "kind": "oracle",
            "rounds_per_s": round(rounds / dt, 3), "sample": sample, "host": host_cpu()}


def host_cpu():
    """The host's logical CPU count and model name (as /proc/cpuinfo gives it)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"logical_cpus": os.cpu_count(), "model": model}


def copy_calibration(nbytes, reps, torch):
    """A plain device copy of known size, for scaling rocprofv3 counters."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


def stream_reference(nbytes, reps, torch):
    """Reference rates for reading nbytes of bf16 logits once, with torch's own
    reduction kernels (a max and an fp32 sum over the whole tensor): the
    bandwidth a general-purpose streaming kernel reaches on the same box, to
    set beside the statistics kernels.  Prints one JSON line."""
    x = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    x.normal_()
    ops = {"amax": lambda: torch.amax(x), "sum_fp32": lambda: torch.sum(x, dtype=torch.float32)}
    out = {"stream_reference_bytes": x.numel() * 2, "reps": reps}
    for name, fn in ops.items():
        for _ in range(3):
            fn()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for _ in range(reps):
            fn()
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / reps
        out[name] = {"us": round(ms * 1e3, 2), "gbps": round(x.numel() * 2 / (ms * 1e-3) / 1e9, 1)}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: about 0.2 s of GPU time)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=str, default=str(HEADLINE_CFG),
                    help="workload for the headline line (1-5; pm3 / pm5 for the point-mass "
                         "workloads with the shapes of configs 3 and 5; outcome for outcome "
                         "scoring; treebuild for draft-tree construction; stree for stochastic "
                         "tree verification)")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the other workloads in the per_config field")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    ap.add_argument("--stream-reference", type=int, default=0, metavar="BYTES",
                    help="time torch's own reductions over BYTES of bf16 (a bandwidth reference)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the verification kernels run on a single "
              "device and the library has no multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 5, torch)
        return
    if args.stream_reference:
        stream_reference(args.stream_reference, 20, torch)
        return
    import exact_draft_verification_amd as sv

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    hip = HipEvents()
    default_steps = {1: 2000, 2: 2000, 3: 200, 4: 100, 5: 50, "pm3": 200, "pm5": 50,
                     "outcome": 200, "treebuild": 100, "stree": 30}
    cfg_arg = int(args.config) if args.config.isdigit() else args.config

    def run(cfg, steps):
        if cfg == "outcome":
            seed = 8077
        elif cfg == "treebuild":
            seed = 9077
        elif cfg == "stree":
            seed = 9177
        else:
            seed = 1000 * int(cfg[2:]) + 77 if isinstance(cfg, str) else 1000 * cfg + 7
        w = Workload(cfg, seed=seed, torch=torch, sv=sv)
        k = steps or default_steps[cfg]
        r = measure(w, k, args.warmup, torch, hip)
        log(f"[bench] config {cfg}: {r['gbps']:.1f} GB/s over {k} steps, "
            f"{r['ms_per_step'] * 1e3:.2f} us/step; dominant kernel {r['dominant_ms'] * 1e3:.2f} us")
        return w, k, r

    w, K, r = run(cfg_arg, args.steps)
    line = {
        "metric": METRIC,
        "value": round(r["gbps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic type: every kernel widens its logits (bf16 or fp32) to
        # fp32 for the per-element work and accumulates and decides in fp64
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.describe(), **w.shape, "config_index": cfg_arg,
                   "logits_dtype": w.spec["dtype"], "bytes_per_step": w.bytes,
                   "input_sets": w.nsets, "timing": "hip graph replay"},
        "pct_peak": round(100.0 * r["gbps"] / PEAK_GBPS, 2),
        "rounds_per_s": round(r["rounds_per_s"], 1),
        "repeats": r["repeats"],
        "roofline": roofline(w, r, args.config),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    del w
    torch.cuda.empty_cache()
    if not args.no_per_config:
        per = {}
        for cfg in (2, 3, 4, 5, "pm3", "pm5", "outcome", "treebuild", "stree"):
            if cfg == cfg_arg:
                continue
            try:
                wc, kc, rc = run(cfg, None)
                per[f"config{cfg}"] = {
                    "workload": wc.describe(), "steps": kc,
                    "gbps": round(rc["gbps"], 2), "pct_peak": round(100 * rc["gbps"] / PEAK_GBPS, 2),
                    "step_frac": round(rc["gbps"] / PEAK_GBPS, 4),
                    "rounds_per_s": round(rc["rounds_per_s"], 1),
                    "us_per_step": round(rc["ms_per_step"] * 1e3, 3),
                    "bytes_per_step": wc.bytes,
                    "repeats": rc["repeats"],
                    "roofline": roofline(wc, rc, str(cfg))}
                del wc
                torch.cuda.empty_cache()
            except Exception as e:  # keep the headline line even if one extra workload fails
                per[f"config{cfg}"] = {"error": repr(e)}
        line["per_config"] = per
    print(json.dumps(line), flush=True)


def dominant_kernel(w):
    """rocprofv3's name stem of the kernel that streams every logit once."""
    stem = {"tree": "tree_argmax_kernel", "outcome": "outcome_stats_kernel",
            "treebuild": "outcome_stats_kernel"}.get(w.kind, "chain_stats_kernel")
    return stem + ("<F32>" if w.spec["dtype"] == "f32" else "<BF16>")


def roofline(w, r, cfg_name):
    """Roofline block of one workload: the dominant kernel's algorithmic
    bytes per launch over its event-timed duration, against the HBM peak,
    plus the whole step's fraction and, for the verification chains, the
    draw phase that follows the statistics pass (the step's limiter where it
    takes longer than that pass)."""
    kernel = dominant_kernel(w)
    out = {"bound": "hbm", "kernel": kernel,
           "achieved": round(r["dominant_gbps"], 2), "peak": PEAK_GBPS, "unit": "GB/s",
           "frac": round(r["dominant_gbps"] / PEAK_GBPS, 4),
           "traffic": measured_traffic(f"{kernel} config{cfg_name}"),
           "avg_kernel_us": round(r["dominant_ms"] * 1e3, 3),
           "algorithmic_bytes_per_launch": w.bytes,
           "step_us": round(r["ms_per_step"] * 1e3, 3),
           "step_frac": round(r["gbps"] / PEAK_GBPS, 4)}
    if "final_kernel_ms" in r:
        draw = r["final_kernel_ms"] * 1e3
        out["draw_phase_us"] = round(draw, 3)
        out["step_limiter"] = ("draw phase (decision, chunk sums and selection kernels)"
                               if draw > r["dominant_ms"] * 1e3 else
                               "statistics pass (" + kernel + ")")
    return out


if __name__ == "__main__":
    main()
