#!/usr/bin/env python3
"""Benchmark of the BRA forward pass on one MI355X.

One step = one pass of the whole path (region mean-pool, affinity + top-k
routing, fused gather + attention) over one batch of synthetic input that is
already resident in HBM. Steps are replayed from HIP graphs and rotate over
several copies of the inputs, so that the 256 MB Infinity Cache cannot hold a
step's working set between two uses of the same copy.

Prints ONE JSON line: whole-job tokens/s, per-step time, TFLOP/s, the
roofline of the dominant kernel (fused gather + attention) from HIP events on
the stream it runs on, and the CPU oracle timed on a bounded sample. The
``with_lce`` object times the module output with the local context term
(5x5 depthwise convolution of V, seeded synthetic filter) the same way; it is
a side measurement, not the headline value. The ``train`` object times a
training step of the same operator the same way: routing, attention and the
backward pass (dQ, dK, dV for a seeded output gradient, routing held fixed).
The ``from_input`` object times the module from its block input X: the QKV
projection with the region pooling fused into it, routing from the fused
means, and attention (seeded synthetic projection weights).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

from __future__ import annotations

import argparse
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
ATTEND_SOURCES = ["attend.hip", "attn_common.h", "lce_tile.h", "bra_internal.h"]  # what the attention kernels are built from
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "attend_stage1_b64_56x56_pmc.md")


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None, help="workload name (default: the 56x56, S=7 stage-1 shape)")
    ap.add_argument("--sets", type=int, default=0, help="input copies to rotate over (0 = enough to exceed the MALL)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU oracle sample budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-lce", action="store_true", help="skip the side measurement with the local context term")
    ap.add_argument("--no-train", action="store_true", help="skip the side measurement of the training step")
    ap.add_argument("--no-proj", action="store_true", help="skip the side measurement from the block input")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration) and exit")
    return ap.parse_args(argv)


def attend_source_sha() -> str:
    h = hashlib.sha256()
    for name in ATTEND_SOURCES:
        with open(os.path.join(ROOT, "vision_transformer_dynamic_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def attention_kernel_name(w):
    """The attention kernel the library launches for workload w (its dispatch
    rule: more than 64 keys per query take the chunked kernel; bf16 regions of
    a multiple of 4 tokens with at least 128 (image, head) pairs, at most 64
    units of 16 query columns and an image's head slice within 160 KB of LDS
    take the image-resident kernel; the rest the per-region kernel). The LDS
    bound here takes the largest row pad the library may choose."""
    n = (w.H // w.S) * (w.W // w.S)
    R, HW = w.S * w.S, w.H * w.W
    if n * w.topk > 64:
        return "attend_kernel"
    if w.dtype == "bf16" and n % 4 == 0 and w.B * w.heads >= 128:
        qr = 4 if n == 4 else 2 if n == 8 else 1
        units = -(-R // qr) if qr > 1 else R * -(-n // 16)
        lds = 2 * HW * 40 + 2 * 32 * (-(-HW // 32) * 32 + 56) + 4 * R * w.topk
        if units <= 64 and lds <= 160 * 1024:
            return "attend_image_kernel"
    return "attend_head_kernel"


def profiled_traffic():
    """HBM bytes per attention launch from the committed counter summary, if it
    was taken on the current attention kernel source; else None."""
    if not os.path.exists(PROFILE_TRAFFIC):
        return None
    text = open(PROFILE_TRAFFIC).read()
    sha = re.search(r"attend_source_sha:\s*([0-9a-f]+)", text)
    tb = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not sha or not tb or sha.group(1) != attend_source_sha():
        return None
    return float(tb.group(1))


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
        nbytes = bra.workspace_bytes(w.B, w.H, w.W, w.C, w.S, w.topk)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)

    def route(self):
        self.bra.route(self.q, self.k, self.w.S, self.w.topk, out=self.idx, workspace=self.ws)

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
        self.bra.attend_backward(self.q, self.k, self.v, self.out, self.grad, self.idx, self.w.heads, self.w.S,
                                 out=self.grads, workspace=self.bws)

    def step_train(self):
        self.route()
        self.attend()
        self.backward()

    def __call__(self):
        self.route()
        self.attend()


def capture(fns):
    import torch

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    return g


def run_graphs(cycle, singles, nsets, count):
    """Replay exactly `count` steps: whole cycles, then single-set graphs."""
    full, rem = divmod(count, nsets)
    for _ in range(full):
        cycle.replay()
    for s in range(rem):
        singles[s].replay()


def cpu_baseline(w, q, k, v, seconds):
    """Time the oracle, single-threaded, image by image (passes over the batch
    repeat) until `seconds` of CPU work have been done."""
    from threadpoolctl import threadpool_limits

    from oracle import bra_oracle as O
    from vision_transformer_dynamic_amd.workloads import to_f64

    done = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            b = done % w.B
            O.bra(to_f64(q[b:b + 1]), to_f64(k[b:b + 1]), to_f64(v[b:b + 1]), w.heads, w.S, w.topk)
            done += 1
            if time.perf_counter() - t0 >= seconds:
                break
        el = time.perf_counter() - t0
    return {
        "value": done * w.H * w.W / el,
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{done} images ({done / w.B:.1f} passes over the {w.B}-image batch) of {w.name}, "
                  f"one image at a time, fp64 numpy, single thread, {el:.1f} s",
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
    w = wl.BY_NAME[args.workload] if args.workload else wl.HEADLINE
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = wl.make_inputs(w)
    esz = 4 if w.dtype == "f32" else 2
    set_bytes = 4 * w.tokens * w.C * esz
    nsets = args.sets or max(1, min(32, math.ceil(CACHE_DEFEAT_BYTES / set_bytes)))
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    lw, lb = (t.to(dev) for t in wl.make_lce_params(w))
    gd = wl.make_grad_output(w).to(dev)
    steps = [Step(w, qd.clone(), kd.clone(), vd.clone(), lw, lb, gd) for _ in range(nsets)]
    torch.cuda.synchronize()

    # eager warm-up of every copy (also the first-launch code loading)
    for s in steps:
        s()
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        cycle = capture(steps)
        singles = [capture([s]) for s in steps]
        attend_cycle = capture([s.attend for s in steps])
        attend_singles = [capture([s.attend]) for s in steps]
        route_cycle = capture([s.route for s in steps])
        route_singles = [capture([s.route]) for s in steps]
    torch.cuda.synchronize()

    # ---- timed region: K whole steps
    with torch.cuda.stream(stream):
        run_graphs(cycle, singles, nsets, args.warmup)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        run_graphs(cycle, singles, nsets, args.steps)
        e1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3 / args.steps
    ev_ms = e0.elapsed_time(e1) / args.steps
    ms_per_step = max(wall_ms, ev_ms)

    # ---- per-kernel durations: the same launches, one phase at a time, HIP
    # events on the stream the kernels run on
    def phase_us(cyc, sing):
        with torch.cuda.stream(stream):
            run_graphs(cyc, sing, nsets, max(nsets, args.warmup))
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            run_graphs(cyc, sing, nsets, args.steps)
            b.record(stream)
            torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / args.steps

    attend_us = phase_us(attend_cycle, attend_singles)
    route_us = phase_us(route_cycle, route_singles)

    # a plain streaming reference with the attention kernel's traffic: read
    # three tensors of Q's shape and dtype, write a fourth (torch.addcmul),
    # over the same input copies and timed the same way
    ref_outs = [torch.empty_like(s_.q) for s_ in steps]
    stream_fns = [lambda s_=s_, o_=o_: torch.addcmul(s_.q, s_.k, s_.v, out=o_) for s_, o_ in zip(steps, ref_outs)]
    for f in stream_fns:
        f()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        stream_cycle = capture(stream_fns)
        stream_singles = [capture([f]) for f in stream_fns]
    torch.cuda.synchronize()
    stream_us = phase_us(stream_cycle, stream_singles)
    del ref_outs

    with_lce = None
    if not args.no_lce:
        for s_ in steps:
            s_.step_lce()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            lce_cycle = capture([s_.step_lce for s_ in steps])
            lce_singles = [capture([s_.step_lce]) for s_ in steps]
            alce_cycle = capture([s_.attend_lce for s_ in steps])
            alce_singles = [capture([s_.attend_lce]) for s_ in steps]
        torch.cuda.synchronize()
        lce_step_us = phase_us(lce_cycle, lce_singles)
        alce_us = phase_us(alce_cycle, alce_singles)
        ref_lce = bra.forward_lce(qd, kd, vd, lw, lb, w.heads, w.S, w.topk)
        torch.cuda.synchronize()
        if not torch.equal(ref_lce, steps[0].out):
            raise RuntimeError("benchmark output with the local context term differs from bra_forward_lce")
        with_lce = {"value": round(w.tokens / (lce_step_us * 1e-6), 1), "unit": "tokens/s",
                    "us_per_step": round(lce_step_us, 2), "attend_lce_us": round(alce_us, 2),
                    "filter": "seeded synthetic 5x5 depthwise weights and bias"}
        for s_ in steps:  # leave the plain outputs in place for the check below
            s_()
        torch.cuda.synchronize()

    train = None
    if not args.no_train:
        for s_ in steps:
            s_.step_train()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            tr_cycle = capture([s_.step_train for s_ in steps])
            tr_singles = [capture([s_.step_train]) for s_ in steps]
            bw_cycle = capture([s_.backward for s_ in steps])
            bw_singles = [capture([s_.backward]) for s_ in steps]
        torch.cuda.synchronize()
        train_us = phase_us(tr_cycle, tr_singles)
        bw_us = phase_us(bw_cycle, bw_singles)
        s0 = steps[0]
        ref = bra.attend_backward(s0.q, s0.k, s0.v, s0.out, gd, s0.idx, w.heads, w.S)
        torch.cuda.synchronize()
        if not all(torch.equal(a, b) for a, b in zip(ref, s0.grads)):
            raise RuntimeError("benchmark gradients differ from bra_attend_backward")
        train = {"value": round(w.tokens / (train_us * 1e-6), 1), "unit": "tokens/s",
                 "us_per_step": round(train_us, 2), "backward_us": round(bw_us, 2),
                 "step": "pool + route + attention + backward (dQ, dK, dV), routing held fixed"}

    from_input = None
    if not args.no_proj and w.C % 32 == 0 and w.C <= (256 if w.dtype == "bf16" else 128):
        xh, wq, bq = wl.make_projection(w)
        wq, bq = wq.to(dev), bq.to(dev)
        xs = [xh.to(dev) for _ in range(nsets)]
        outs = [tuple(torch.empty_like(xs[0]) for _ in range(4)) for _ in range(nsets)]
        pouts = [tuple(torch.empty_like(xs[0]) for _ in range(3)) + tuple(
            torch.empty((w.B, w.R, w.C), dtype=torch.float32, device=dev) for _ in range(2)) for _ in range(nsets)]
        fws = [torch.empty(bra.workspace_bytes(w.B, w.H, w.W, w.C, w.S, w.topk), dtype=torch.uint8, device=dev)
               for _ in range(nsets)]
        fwd_x = [lambda i=i: bra.forward_qkv(xs[i], wq, bq, w.heads, w.S, w.topk, out=outs[i], workspace=fws[i])
                 for i in range(nsets)]
        proj = [lambda i=i: bra.qkv_pool(xs[i], wq, bq, w.S, out=pouts[i]) for i in range(nsets)]
        for f in fwd_x + proj:
            f()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            fx_cycle = capture(fwd_x)
            fx_singles = [capture([f]) for f in fwd_x]
            pj_cycle = capture(proj)
            pj_singles = [capture([f]) for f in proj]
        torch.cuda.synchronize()
        fx_us = phase_us(fx_cycle, fx_singles)
        pj_us = phase_us(pj_cycle, pj_singles)
        o0, q0, k0, v0 = outs[0]
        if not torch.equal(o0, bra.forward(q0, k0, v0, w.heads, w.S, w.topk)):
            raise RuntimeError("output from the block input differs from bra_forward on its projections")
        from_input = {"value": round(w.tokens / (fx_us * 1e-6), 1), "unit": "tokens/s", "us_per_step": round(fx_us, 2),
                      "qkv_pool_us": round(pj_us, 2),
                      "step": "QKV projection with fused region pooling + route + attention, seeded synthetic weights"}
        del xs, outs, pouts, fws

    # the timed steps computed the real thing: spot-check one copy
    ref = bra.forward(qd, kd, vd, w.heads, w.S, w.topk)
    torch.cuda.synchronize()
    if not torch.equal(ref, steps[0].out):
        raise RuntimeError("benchmark output differs from bra_forward")

    tokens = w.tokens
    attn_flop = 4.0 * tokens * w.kv * w.C
    aff_flop = 2.0 * w.B * w.R * w.R * w.C
    attn_bytes = 4.0 * tokens * w.C * esz  # read Q, K, V once, write O
    pr_bytes = 2.0 * tokens * w.C * esz + 4.0 * w.B * w.R * w.C * 4 + 4.0 * w.B * w.R * w.topk
    peak_tf = BF16_PEAK_TFLOPS if w.dtype == "bf16" else F32_PEAK_TFLOPS
    ridge = peak_tf * 1e12 / (HBM_PEAK_GBS * 1e9)
    if attn_flop / attn_bytes < ridge:
        achieved = attn_bytes / (attend_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = attn_flop / (attend_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak_tf, "unit": "TFLOP/s",
                "frac": round(achieved / peak_tf, 4)}
    traffic = profiled_traffic() if w is wl.HEADLINE else None
    roof["traffic"] = traffic
    roof["kernel"] = attention_kernel_name(w)
    roof["algorithmic_bytes_per_launch"] = attn_bytes
    roof["launch_us"] = round(attend_us, 2)
    # the same bytes moved by a plain streaming kernel on this GPU, and the
    # attention kernel's rate as a fraction of that
    roof["stream_reference_us"] = round(stream_us, 2)
    roof["frac_of_stream_reference"] = round(stream_us / attend_us, 4)

    result = {
        "metric": METRIC,
        "value": round(tokens / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "W": w.W, "C": w.C, "heads": w.heads,
                   "S": w.S, "topk": w.topk, "global_batch": w.B, "tokens_per_step": tokens,
                   "input_copies": nsets, "parallelism": "single-gpu"},
        "tflops": round((attn_flop + aff_flop) / (ms_per_step * 1e-3) / 1e12, 3),
        "phases_us": {"pool_route": round(route_us, 2), "attend": round(attend_us, 2),
                      "step_wall": round(wall_ms * 1e3, 2), "step_events": round(ev_ms * 1e3, 2)},
        # the pool + route phase against the HBM peak: its algorithmic bytes
        # (read Q and K once, the region means written and read back, the
        # table written) over its measured time, both launches and the gap
        # between them included
        "phase_hbm": {"pool_route": {"algorithmic_bytes": pr_bytes, "GB/s": round(pr_bytes / (route_us * 1e-6) / 1e9, 1),
                                     "frac_of_peak": round(pr_bytes / (route_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}},
        "roofline": roof,
    }
    if from_input is not None:
        result["from_input"] = from_input
    if with_lce is not None:
        result["with_lce"] = with_lce
    if train is not None:
        result["train"] = train
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_seconds)
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
