"""Every entry point captured in a HIP graph and replayed: each replay must give
exactly the eager call's result.

The kernels are deterministic (fixed summation orders, no atomics on values)
and none records a memset into the graph, so replays are compared bit for bit.
Between replays the program does eager work of its own (a fresh eager call on
other inputs and a synchronisation), as a graph in a training or serving loop
would see.
"""

import pytest
import torch

import vision_transformer_dynamic_amd as bra
from vision_transformer_dynamic_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

SHAPES = [
    wl.custom(2, 28, 28, 64, 2, 7, 2, "bf16", seed=60),   # single-chunk attention, n = 16
    wl.custom(2, 16, 16, 64, 2, 2, 2, "bf16", seed=61),   # chunked attention: n = 64, 128 keys per query
    wl.custom(1, 16, 16, 32, 1, 4, 2, "f32", seed=62),    # fp32
    wl.custom(32, 14, 14, 128, 4, 7, 8, "bf16", seed=63), # image-resident attention
]

REPLAYS = 3


def _inputs(w, seed_shift=0):
    q, k, v = (t.to(DEV) for t in wl.make_inputs(wl.custom(w.B, w.H, w.W, w.C, w.heads, w.S, w.topk, w.dtype,
                                                                 seed=w.seed + seed_shift)))
    return q, k, v


def _replay_and_check(capture_fn, eager_fn, outs, other_eager):
    """capture_fn() enqueues the calls writing `outs`; eager_fn() returns the
    reference tensors computed eagerly; other_eager() is unrelated eager work
    run between replays."""
    ref = [t.clone() for t in eager_fn()]
    torch.cuda.synchronize()
    capture_fn()  # warm-up outside the graph (first-launch code loading)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g):
            capture_fn()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        for t in outs:
            t.fill_(float("nan") if t.is_floating_point() else -7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (got, want) in enumerate(zip(outs, ref)):
            assert torch.equal(got, want), f"replay {r}: output {i} differs from the eager call"
        other_eager()
        torch.cuda.synchronize()


@pytest.mark.parametrize("w", SHAPES, ids=[w.name for w in SHAPES])
def test_forward_and_route_in_graph(w):
    q, k, v = _inputs(w)
    q2, k2, v2 = _inputs(w, 100)
    nbytes = bra.workspace_bytes(w.B, w.H, w.W, w.C, w.S, w.topk)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    o = torch.empty_like(q)
    idx = torch.empty((w.B, w.R, w.topk), dtype=torch.int32, device=DEV)

    def cap():
        bra.route(q, k, w.S, w.topk, out=idx, workspace=ws)
        bra.forward(q, k, v, w.heads, w.S, w.topk, out=o, workspace=ws)

    _replay_and_check(cap, lambda: (bra.forward(q, k, v, w.heads, w.S, w.topk), bra.route(q, k, w.S, w.topk)),
                      [o, idx], lambda: bra.forward(q2, k2, v2, w.heads, w.S, w.topk))


@pytest.mark.parametrize("w", [s for s in SHAPES if s.dtype == "bf16"], ids=lambda s: s.name)
def test_forward_with_local_context_in_graph(w):
    q, k, v = _inputs(w)
    lw, lb = (t.to(DEV) for t in wl.make_lce_params(w))
    nbytes = bra.workspace_bytes(w.B, w.H, w.W, w.C, w.S, w.topk)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    o = torch.empty_like(q)

    def cap():
        bra.forward_lce(q, k, v, lw, lb, w.heads, w.S, w.topk, out=o, workspace=ws)

    _replay_and_check(cap, lambda: (bra.forward_lce(q, k, v, lw, lb, w.heads, w.S, w.topk),), [o],
                      lambda: bra.forward(q, k, v, w.heads, w.S, w.topk))


@pytest.mark.parametrize("w", SHAPES, ids=[w.name for w in SHAPES])
def test_backward_in_graph(w):
    q, k, v = _inputs(w)
    do = wl.make_grad_output(w).to(DEV)
    idx = bra.route(q, k, w.S, w.topk)
    o = bra.attend(q, k, v, idx, w.heads, w.S)
    n = bra.backward_workspace_bytes(w.B, w.H, w.W, w.C, w.heads, w.S, w.topk)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    grads = tuple(torch.empty_like(q) for _ in range(3))

    def cap():
        bra.attend_backward(q, k, v, o, do, idx, w.heads, w.S, out=grads, workspace=ws)

    _replay_and_check(cap, lambda: bra.attend_backward(q, k, v, o, do, idx, w.heads, w.S), list(grads),
                      lambda: bra.attend(q, k, v, idx, w.heads, w.S))


@pytest.mark.parametrize("w", [s for s in SHAPES if s.dtype == "bf16"], ids=lambda s: s.name)
def test_projection_forward_in_graph(w):
    x, wq, bq = (t.to(DEV) for t in wl.make_projection(w))
    nbytes = bra.workspace_bytes(w.B, w.H, w.W, w.C, w.S, w.topk)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    outs = tuple(torch.empty_like(x) for _ in range(4))  # O, Q, K, V

    def cap():
        bra.forward_qkv(x, wq, bq, w.heads, w.S, w.topk, out=outs, workspace=ws)

    _replay_and_check(cap, lambda: bra.forward_qkv(x, wq, bq, w.heads, w.S, w.topk), list(outs),
                      lambda: bra.qkv_pool(x, wq, bq, w.S))
