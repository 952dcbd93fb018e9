#!/usr/bin/env python3
"""Benchmark of the BRA forward pass on one MI355X.

One step = one pass of the whole path (region mean-pool, affinity + top-k
routing, fused gather + attention) over one batch of synthetic input that is
already resident in HBM. Steps are replayed from HIP graphs and rotate over
several copies of the inputs, so that the 256 MB Infinity Cache cannot hold a
step's working set between two uses of the same copy.

Prints ONE JSON line. Its top-level fields are the headline workload (the
56x56, S = 7 stage-1 shape): whole-job tokens/s, per-step time, TFLOP/s, the
roofline of the dominant kernel (fused gather + attention) from HIP events on
the stream it runs on, and the CPU oracle timed on a bounded sample. The
``configs`` list repeats the measurement for each of the five synthetic
workloads: per-phase times (pool, route, attention) by HIP events, tokens/s,
TFLOP/s, the fraction of the binding roofline (HBM for the stage shapes, the
bf16 matrix cores for the dense map), the pool + route phase against HBM, and
the oracle on one host thread and on all the host cores the run may use. The
``peaks`` object holds what a plain bf16 matrix-core loop and a plain
streaming copy reach on this part, beside the published peaks; the
``detection`` list measures two detection-shaped maps at S = 16 (256
regions) the same way.

Side measurements of the headline workload (not its value): ``with_lce``
(the module output with the local context term, a seeded synthetic 5x5
depthwise filter), ``train`` (routing, attention and the backward pass for a
seeded output gradient, routing held fixed) and ``from_input`` (the QKV
projection with the region pooling fused into it, routing from the fused
means, attention; seeded synthetic projection weights).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--only]
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "BRA forward tokens/sec and TFLOP/s (% of MFMA/HBM roofline) at 56×56,S=7"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
F32_PEAK_TFLOPS = 157.3     # MI355X dense fp32 matrix, published
CACHE_DEFEAT_BYTES = 640 << 20  # rotate input copies over more than the 256 MB MALL
CPU_WORKERS_MAX = 16        # host cores a one-GPU run may use
ATTEND_SOURCES = ["attend.hip", "attn_common.h", "lce_tile.h", "bra_internal.h"]  # what the attention kernels are built from
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "attend_stage1_b64_56x56_pmc.md")


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None, help="workload of the top-level line (default: the 56x56, S=7 shape)")
    ap.add_argument("--only", action="store_true", help="measure only that workload (no configs list, no peaks)")
    ap.add_argument("--sets", type=int, default=0, help="input copies to rotate over (0 = enough to exceed the MALL)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="single-thread oracle sample, top-level workload")
    ap.add_argument("--cpu-seconds-other", type=float, default=2.5,
                    help="oracle sample per thread setting for the other workloads and the all-core run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the matrix-core loop and copy probes")
    ap.add_argument("--peaks-only", action="store_true", help="only run the matrix-core loop and copy probes")
    ap.add_argument("--no-lce", action="store_true", help="skip the side measurement with the local context term")
    ap.add_argument("--no-train", action="store_true", help="skip the side measurement of the training step")
    ap.add_argument("--no-proj", action="store_true", help="skip the side measurement from the block input")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration) and exit")
    return ap.parse_args(argv)


def attention_kernel_name(w):
    """The attention kernel the library launches for workload w (the
    library's own dispatch decision, bra_attend_kernel)."""
    import vision_transformer_dynamic_amd as bra

    return bra.attend_kernel(w.B, w.H, w.W, w.C, w.heads, w.S, w.topk, w.torch_dtype)


def attend_source_sha() -> str:
    h = hashlib.sha256()
    for name in ATTEND_SOURCES:
        with open(os.path.join(ROOT, "vision_transformer_dynamic_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profiled_traffic():
    """HBM bytes per attention launch at the headline shape from the
    committed counter summary, if it was taken on the current attention
    kernel source; else None."""
    if not os.path.exists(PROFILE_TRAFFIC):
        return None
    text = open(PROFILE_TRAFFIC).read()
    sha = re.search(r"attend_source_sha:\s*([0-9a-f]+)", text)
    tb = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not sha or not tb or sha.group(1) != attend_source_sha():
        return None
    return float(tb.group(1))


# ---------------------------------------------------------------------------
# CPU oracle leg. It runs before the GPU is touched, so the worker processes
# (forked, one host thread each) start from a process without GPU state.

_CPU = {}  # workload name -> (w, q, k, v) on the host, inherited by forked workers


def _oracle_images(name, start, step, seconds):
    """Oracle over images start, start + step, ... of a workload (one host
    thread) until `seconds` have passed; returns the number of images."""
    from threadpoolctl import threadpool_limits

    from oracle import bra_oracle as O
    from vision_transformer_dynamic_amd.workloads import to_f64

    w, q, k, v = _CPU[name]
    done = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        b = start % w.B
        while True:
            O.bra(to_f64(q[b:b + 1]), to_f64(k[b:b + 1]), to_f64(v[b:b + 1]), w.heads, w.S, w.topk)
            done += 1
            b = (b + step) % w.B
            if time.perf_counter() - t0 >= seconds:
                break
    return done


def _oracle_worker(a):
    return _oracle_images(*a)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, q, k, v, seconds_single, seconds_all):
    """The oracle as it stands (fp64 numpy, image by image) on one host
    thread, then on every host core the run may use (forked processes of one
    thread each, images dealt round-robin). Each is timed over a bounded
    sample; the value is tokens/s."""
    import multiprocessing as mp

    _CPU[w.name] = (w, q, k, v)
    hw = w.H * w.W
    t0 = time.perf_counter()
    n1 = _oracle_images(w.name, 0, 1, seconds_single)
    el1 = time.perf_counter() - t0
    workers = max(1, min(CPU_WORKERS_MAX, os.cpu_count() or 1))
    ctx = mp.get_context("fork")
    with ctx.Pool(workers) as pool:
        t0 = time.perf_counter()
        counts = pool.map(_oracle_worker, [(w.name, i, workers, seconds_all) for i in range(workers)])
        el_all = time.perf_counter() - t0
    nall = sum(counts)
    single = {"value": n1 * hw / el1, "unit": "tokens/s", "cores": 1, "kind": "oracle",
              "sample": f"{n1} images of {w.name}, one at a time, fp64 numpy, one thread, {el1:.1f} s"}
    return {
        "value": nall * hw / el_all,
        "unit": "tokens/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{nall} images of {w.name} on {workers} forked processes of one thread each "
                  f"(images dealt round-robin), fp64 numpy, {el_all:.1f} s wall including the fork",
        "single_thread": single,
        "cpu_model": cpu_model(),
        "os_cpu_count": os.cpu_count(),
    }


# ---------------------------------------------------------------------------
# GPU leg

def calibrate_copy(mib: int) -> None:
    import torch

    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": n, "launches": 5}))


class Step:
    """Pre-bound C-ABI calls for one input copy (no per-call allocation)."""

    def __init__(self, w, q, k, v, lce_w=None, lce_b=None, grad=None):
        import torch
        import vision_transformer_dynamic_amd as bra

        self.bra = bra
        self.w = w
        self.q, self.k, self.v = q, k, v
        self.lce_w, self.lce_b = lce_w, lce_b
        self.grad = grad
        self.grads = None
        self.bws = None
        self.out = torch.empty_like(q)
        self.idx = torch.empty((w.B, w.R, w.topk), dtype=torch.int32, device=q.device)
        self.idx2 = torch.empty_like(self.idx)
        self.qr = torch.empty((w.B, w.R, w.C), dtype=torch.float32, device=q.device)
        self.kr = torch.empty_like(self.qr)
        nbytes = bra.workspace_bytes(w.B, w.H, w.W, w.C, w.S, w.topk)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
        # the routing table bra_forward_ws leaves in its workspace ([Q^r | K^r | idx], 256-byte aligned parts)
        pooled = -(-4 * w.B * w.R * w.C // 256) * 256
        self.tab = self.ws[2 * pooled: 2 * pooled + 4 * w.B * w.R * w.topk].view(torch.int32).view(w.B, w.R, w.topk)

    def route(self):
        self.bra.route_ws(self.q, self.k, self.w.S, self.w.topk, self.ws, out=self.idx)

    def pool(self):
        self.bra.pool(self.q, self.k, self.w.S, out=(self.qr, self.kr))

    def route_pooled(self):
        self.bra.route_pooled(self.qr, self.kr, self.w.S, self.w.topk, out=self.idx2)

    def attend(self):
        self.bra.attend(self.q, self.k, self.v, self.idx, self.w.heads, self.w.S, out=self.out)

    def attend_lce(self):
        self.bra.attend_lce(self.q, self.k, self.v, self.idx, self.lce_w, self.lce_b, self.w.heads, self.w.S,
                            out=self.out)

    def step_lce(self):
        self.route()
        self.attend_lce()

    def backward(self):
        import torch

        if self.grads is None:
            w = self.w
            self.grads = tuple(torch.empty_like(self.q) for _ in range(3))
            n = self.bra.backward_workspace_bytes(w.B, w.H, w.W, w.C, w.heads, w.S, w.topk)
            self.bws = torch.empty(n, dtype=torch.uint8, device=self.q.device)
        self.bra.attend_backward(self.q, self.k, self.v, self.out, self.grad, self.tab, self.w.heads, self.w.S,
                                 out=self.grads, workspace=self.bws)

    def step_train(self):
        self()
        self.backward()

    def __call__(self):
        """The forward step: bra_forward_ws (pool, routing, attention; the
        table stays in the workspace)."""
        self.bra.forward_ws(self.q, self.k, self.v, self.w.heads, self.w.S, self.w.topk, self.ws, out=self.out)


def capture(fns):
    import torch

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    return g


class Timer:
    """A phase (one call per input copy, `fns[i]` for copy i) captured as HIP
    graphs of exactly `warmup` and exactly `steps` calls, the copies taken in
    rotation, and timed with HIP events on the stream the graphs run on: one
    graph launch for the whole timed run, so no host launch gap sits between
    its calls."""

    def __init__(self, stream, steps, warmup):
        self.stream, self.steps, self.warmup = stream, steps, warmup

    def graphs(self, fns):
        import torch

        for f in fns:
            f()
        torch.cuda.synchronize()
        with torch.cuda.stream(self.stream):
            gw = capture([fns[i % len(fns)] for i in range(max(1, self.warmup))])
            gk = capture([fns[i % len(fns)] for i in range(self.steps)])
        torch.cuda.synchronize()
        return gw, gk

    def run(self, fns):
        """(events us per call, wall-clock us per call) of `steps` calls."""
        import torch

        gw, gk = self.graphs(fns)
        with torch.cuda.stream(self.stream):
            gw.replay()
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            a.record(self.stream)
            gk.replay()
            b.record(self.stream)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
        return a.elapsed_time(b) * 1e3 / self.steps, (t1 - t0) * 1e6 / self.steps

    def us(self, fns):
        """Average microseconds of one call of the phase (HIP events)."""
        return self.run(fns)[0]


def hbm(nbytes, us):
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"algorithmic_bytes": nbytes, "GB/s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


def work_figures(w):
    """Algorithmic flops and compulsory bytes of the phases (2 flop per
    multiply-add; attention reads Q, K, V once and writes O)."""
    esz = 4 if w.dtype == "f32" else 2
    T = w.tokens
    return {
        "esz": esz,
        "attn_flop": 4.0 * T * w.kv * w.C,
        "aff_flop": 2.0 * w.B * w.R * w.R * w.C,
        "attn_bytes": 4.0 * T * w.C * esz,
        "pool_bytes": 2.0 * T * w.C * esz + 2.0 * w.B * w.R * w.C * 4,
        "route_bytes": 2.0 * w.B * w.R * w.C * 4 + 4.0 * w.B * w.R * w.topk,
    }


def roofline(w, attend_us):
    f = work_figures(w)
    peak_tf = BF16_PEAK_TFLOPS if w.dtype == "bf16" else F32_PEAK_TFLOPS
    ridge = peak_tf * 1e12 / (HBM_PEAK_GBS * 1e9)
    tflops = f["attn_flop"] / (attend_us * 1e-6) / 1e12
    if f["attn_flop"] / f["attn_bytes"] < ridge:
        achieved = f["attn_bytes"] / (attend_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak_tf, "unit": "TFLOP/s",
                "frac": round(tflops / peak_tf, 4)}
    # the matrix-core fraction whatever binds (a bound of 32 / 312 flop per
    # byte on the stage shapes)
    roof["mfma_frac_raw"] = round(tflops / peak_tf, 4)
    return roof


def measure(w, args, dev, stream, side=False):
    """Every phase of workload w on the GPU; `side` adds the headline's side
    measurements. Returns (config entry, extras for the top-level line)."""
    import torch

    import vision_transformer_dynamic_amd as bra
    from vision_transformer_dynamic_amd import workloads as wl

    q, k, v = wl.make_inputs(w)
    f = work_figures(w)
    set_bytes = 4 * w.tokens * w.C * f["esz"]
    nsets = args.sets or max(1, min(32, math.ceil(CACHE_DEFEAT_BYTES / set_bytes)))
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    lw, lb = (t.to(dev) for t in wl.make_lce_params(w))
    gd = wl.make_grad_output(w).to(dev)
    steps = [Step(w, qd.clone(), kd.clone(), vd.clone(), lw, lb, gd) for _ in range(nsets)]
    torch.cuda.synchronize()
    for s in steps:  # eager warm-up of every copy (also the first-launch code loading)
        s()
    torch.cuda.synchronize()
    tm = Timer(stream, args.steps, args.warmup)

    # ---- timed region: exactly K whole steps (one graph of K steps, the
    # input copies in rotation), bracketed by synchronisations
    ev_us, wall_us = tm.run(steps)
    step_us = max(wall_us, ev_us)

    # ---- the same launches one phase at a time
    pool_route_us = tm.us([s.route for s in steps])  # (also leaves each copy's table for the attention phase)
    attend_us = tm.us([s.attend for s in steps])
    pool_us = tm.us([s.pool for s in steps])
    route_us = tm.us([s.route_pooled for s in steps])
    # a plain streaming kernel with the attention kernel's traffic (read three
    # tensors of Q's shape and dtype, write a fourth: torch.addcmul)
    ref_outs = [torch.empty_like(s_.q) for s_ in steps]
    stream_us = tm.us([lambda s_=s_, o_=o_: torch.addcmul(s_.q, s_.k, s_.v, out=o_) for s_, o_ in zip(steps, ref_outs)])
    del ref_outs
    # the backward of the attention (routing held fixed) from the timed
    # steps' outputs: dQ, dK, dV
    backward_us = None if args.no_train else tm.us([s_.backward for s_ in steps])

    # the timed steps computed the real thing: spot-check one copy, and the
    # phase-by-phase routing against the fused one
    ref = bra.forward(qd, kd, vd, w.heads, w.S, w.topk)
    torch.cuda.synchronize()
    if not torch.equal(ref, steps[0].out):
        raise RuntimeError(f"{w.name}: benchmark output differs from bra_forward")
    if not torch.equal(steps[0].idx, steps[0].idx2):
        raise RuntimeError(f"{w.name}: bra_pool + bra_route_pooled differs from bra_route")
    if not torch.equal(steps[0].idx, steps[0].tab):
        raise RuntimeError(f"{w.name}: the routing table of bra_forward_ws differs from bra_route")

    roof = roofline(w, attend_us)
    roof["kernel"] = attention_kernel_name(w)
    roof["algorithmic_bytes_per_launch"] = f["attn_bytes"]
    roof["algorithmic_flop_per_launch"] = f["attn_flop"]
    roof["launch_us"] = round(attend_us, 2)
    roof["stream_reference_us"] = round(stream_us, 2)
    roof["frac_of_stream_reference"] = round(stream_us / attend_us, 4)
    entry = {
        "workload": w.name,
        "B": w.B, "H": w.H, "W": w.W, "C": w.C, "heads": w.heads, "S": w.S, "topk": w.topk, "dtype": w.dtype,
        "tokens_per_step": w.tokens,
        "input_copies": nsets,
        "us": {"pool": round(pool_us, 2), "route": round(route_us, 2), "pool_route": round(pool_route_us, 2),
               "attend": round(attend_us, 2), "step": round(step_us, 3), "step_wall": round(wall_us, 2),
               "step_events": round(ev_us, 2)},
        "tokens_per_s": round(w.tokens / (step_us * 1e-6), 1),
        "tflops": round((f["attn_flop"] + f["aff_flop"]) / (step_us * 1e-6) / 1e12, 3),
        "attend_tflops": round(f["attn_flop"] / (attend_us * 1e-6) / 1e12, 3),
        "roofline": roof,
        "phase_hbm": {"pool": hbm(f["pool_bytes"], pool_us), "route": hbm(f["route_bytes"], route_us),
                      "pool_route": hbm(f["pool_bytes"] + f["route_bytes"], pool_route_us)},
    }
    if backward_us is not None:
        entry["us"]["backward"] = round(backward_us, 2)
    extras = {"step_us": step_us, "wall_us": wall_us, "ev_us": ev_us, "nsets": nsets}

    if side and not args.no_lce:
        step_lce_us = tm.us([s_.step_lce for s_ in steps])
        alce_us = tm.us([s_.attend_lce for s_ in steps])
        ref_lce = bra.forward_lce(qd, kd, vd, lw, lb, w.heads, w.S, w.topk)
        torch.cuda.synchronize()
        if not torch.equal(ref_lce, steps[0].out):
            raise RuntimeError("benchmark output with the local context term differs from bra_forward_lce")
        extras["with_lce"] = {"value": round(w.tokens / (step_lce_us * 1e-6), 1), "unit": "tokens/s",
                              "us_per_step": round(step_lce_us, 2), "attend_lce_us": round(alce_us, 2),
                              "attend_lce_kernel": bra.attend_kernel(w.B, w.H, w.W, w.C, w.heads, w.S, w.topk,
                                                                     w.torch_dtype, with_lce=True),
                              "filter": "seeded synthetic 5x5 depthwise weights and bias"}
        for s_ in steps:  # leave the plain outputs in place for the backward
            s_()
        torch.cuda.synchronize()

    if side and not args.no_train:
        train_us = tm.us([s_.step_train for s_ in steps])
        bw_us = tm.us([s_.backward for s_ in steps])
        s0 = steps[0]
        refg = bra.attend_backward(s0.q, s0.k, s0.v, s0.out, gd, s0.tab, w.heads, w.S)
        torch.cuda.synchronize()
        if not all(torch.equal(a, b) for a, b in zip(refg, s0.grads)):
            raise RuntimeError("benchmark gradients differ from bra_attend_backward")
        extras["train"] = {"value": round(w.tokens / (train_us * 1e-6), 1), "unit": "tokens/s",
                           "us_per_step": round(train_us, 2), "backward_us": round(bw_us, 2),
                           "step": "pool + route + attention + backward (dQ, dK, dV), routing held fixed"}

    if side and not args.no_proj and w.C % 32 == 0 and w.C <= (256 if w.dtype == "bf16" else 128):
        xh, wq, bq = wl.make_projection(w)
        wq, bq = wq.to(dev), bq.to(dev)
        xs = [xh.to(dev) for _ in range(nsets)]
        outs = [tuple(torch.empty_like(xs[0]) for _ in range(4)) for _ in range(nsets)]
        pouts = [tuple(torch.empty_like(xs[0]) for _ in range(3)) + tuple(
            torch.empty((w.B, w.R, w.C), dtype=torch.float32, device=dev) for _ in range(2)) for _ in range(nsets)]
        fws = [torch.empty(bra.workspace_bytes(w.B, w.H, w.W, w.C, w.S, w.topk), dtype=torch.uint8, device=dev)
               for _ in range(nsets)]
        fx_us = tm.us([lambda i=i: bra.forward_qkv(xs[i], wq, bq, w.heads, w.S, w.topk, out=outs[i],
                                                   workspace=fws[i]) for i in range(nsets)])
        pj_us = tm.us([lambda i=i: bra.qkv_pool(xs[i], wq, bq, w.S, out=pouts[i]) for i in range(nsets)])
        o0, q0, k0, v0 = outs[0]
        if not torch.equal(o0, bra.forward(q0, k0, v0, w.heads, w.S, w.topk)):
            raise RuntimeError("output from the block input differs from bra_forward on its projections")
        extras["from_input"] = {"value": round(w.tokens / (fx_us * 1e-6), 1), "unit": "tokens/s",
                                "us_per_step": round(fx_us, 2), "qkv_pool_us": round(pj_us, 2),
                                "step": "QKV projection with fused region pooling + route + attention, "
                                        "seeded synthetic weights"}
        del xs, outs, pouts, fws

    del steps, qd, kd, vd, gd
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return entry, extras


def measure_peaks(dev, stream):
    """A plain bf16 matrix-core loop and a plain streaming copy (libbra_peak.so),
    timed with HIP events: what this part reaches, beside the published peaks."""
    import torch

    from vision_transformer_dynamic_amd import build as bra_build

    lib = ctypes.CDLL(bra_build.PEAK_LIB_PATH)
    lib.bra_peak_mfma.restype = ctypes.c_int
    lib.bra_peak_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.bra_peak_mfma_flops.restype = ctypes.c_double
    lib.bra_peak_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.bra_peak_copy.restype = ctypes.c_int
    lib.bra_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    sp = ctypes.c_void_p(stream.cuda_stream)

    def timed(fn, reps):
        with torch.cuda.stream(stream):
            fn()
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / reps  # seconds

    blocks, iters = 256 * 8, 2000  # 8 waves per SIMD
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)

    def mfma():
        if lib.bra_peak_mfma(ctypes.c_void_p(out.data_ptr()), blocks, iters, sp) != 0:
            raise RuntimeError("matrix-core probe launch failed")

    t_mfma = timed(mfma, 5)
    tflops = lib.bra_peak_mfma_flops(blocks, iters) / t_mfma / 1e12
    nbytes = 512 << 20
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)

    def copy():
        if lib.bra_peak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes, sp) != 0:
            raise RuntimeError("copy probe launch failed")

    t_copy = timed(copy, 10)
    torch.cuda.synchronize()
    if not torch.equal(src[:1024], dst[:1024]):
        raise RuntimeError("copy probe gave wrong data")
    gbs = 2 * nbytes / t_copy / 1e9
    del src, dst, out
    torch.cuda.empty_cache()
    return {
        "mfma_bf16": {"achieved": round(tflops, 1), "unit": "TFLOP/s", "published": BF16_PEAK_TFLOPS,
                      "frac_of_published": round(tflops / BF16_PEAK_TFLOPS, 4),
                      "probe": f"{blocks} workgroups of 4 waves, {iters} x 8 independent "
                               "v_mfma_f32_16x16x32_bf16 per wave"},
        "hbm_copy": {"achieved": round(gbs, 1), "unit": "GB/s", "published": HBM_PEAK_GBS,
                     "frac_of_published": round(gbs / HBM_PEAK_GBS, 4),
                     "probe": "copy of 512 MiB (read + write counted), 16-byte vectors"},
    }


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by image with no exchange; see the design notes)", file=sys.stderr)
        return 2

    import torch

    if args.calibrate_copy_mib:
        calibrate_copy(args.calibrate_copy_mib)
        return 0

    import vision_transformer_dynamic_amd as bra
    from vision_transformer_dynamic_amd import workloads as wl

    bra.load_library()
    head = wl.BY_NAME[args.workload] if args.workload else wl.HEADLINE
    todo = [head] if args.only else [head] + [w for w in wl.WORKLOADS + wl.DETECTION if w is not head]

    # ---- CPU oracle first, before anything touches the GPU
    cpu = {}
    if not args.no_cpu_baseline and not args.peaks_only:
        for w in todo:
            q, k, v = wl.make_inputs(w)
            single = args.cpu_seconds if w is head else args.cpu_seconds_other
            cpu[w.name] = cpu_baseline(w, q, k, v, single, args.cpu_seconds_other)
            print(f"[bench] oracle {w.name}: {cpu[w.name]['single_thread']['value']:.0f} tokens/s on one thread, "
                  f"{cpu[w.name]['value']:.0f} on {cpu[w.name]['cores']}", file=sys.stderr, flush=True)
        _CPU.clear()

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream()
    if args.peaks_only:
        print(json.dumps({"peaks": measure_peaks(dev, stream)}))
        return 0
    peaks = None if (args.no_peaks or args.only) else measure_peaks(dev, stream)

    entries = {}
    extras = None
    for w in todo:
        entry, ex = measure(w, args, dev, stream, side=w is head)
        if w.name in cpu:
            entry["cpu_baseline"] = cpu[w.name]
        entries[w.name] = entry
        if w is head:
            extras = ex
        print(f"[bench] {w.name}: step {entry['us']['step']:.2f} us, attention {entry['us']['attend']:.2f} us "
              f"({entry['roofline']['bound']} frac {entry['roofline']['frac']})", file=sys.stderr, flush=True)

    e = entries[head.name]
    f = work_figures(head)
    ms_per_step = extras["step_us"] * 1e-3
    roof = dict(e["roofline"])
    # HBM bytes per launch by the FETCH_SIZE / WRITE_SIZE counters, scaled by
    # a plain copy's readings, from the committed summary (null once the
    # attention source has changed since it was taken)
    roof["traffic"] = profiled_traffic() if head is wl.HEADLINE else None
    result = {
        "metric": METRIC,
        "value": e["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head.dtype,
        "data": "synthetic",
        "config": {"workload": head.name, "B": head.B, "H": head.H, "W": head.W, "C": head.C,
                   "heads": head.heads, "S": head.S, "topk": head.topk, "global_batch": head.B,
                   "tokens_per_step": head.tokens, "input_copies": extras["nsets"], "parallelism": "single-gpu"},
        "tflops": round((f["attn_flop"] + f["aff_flop"]) / (ms_per_step * 1e-3) / 1e12, 3),
        "phases_us": {"pool": e["us"]["pool"], "route": e["us"]["route"], "pool_route": e["us"]["pool_route"],
                      "attend": e["us"]["attend"], "step_wall": round(extras["wall_us"], 2),
                      "step_events": round(extras["ev_us"], 2)},
        "phase_hbm": e["phase_hbm"],
        "roofline": roof,
    }
    for key in ("from_input", "with_lce", "train"):
        if key in extras:
            result[key] = extras[key]
    if head.name in cpu:
        result["cpu_baseline"] = cpu[head.name]
    if peaks is not None:
        result["peaks"] = peaks
    if not args.only:
        result["configs"] = [entries[w.name] for w in wl.WORKLOADS if w.name in entries]
        # detection-shaped maps at S = 16 (256 regions), beside the five
        result["detection"] = [entries[w.name] for w in wl.DETECTION if w.name in entries]
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
