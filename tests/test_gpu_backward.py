"""GPU parity of the backward pass (routing held fixed) through the C ABI,
against the fp64 oracle's explicit gradients.

The GPU's own routing table and forward output are used, as in training; the
oracle recomputes the softmax from the exact (upcast) inputs. Full-size
workloads run the whole batch on the GPU and check sampled images (gradients
never cross images).
"""

import numpy as np
import pytest
import torch

import vision_transformer_dynamic_amd as bra
from vision_transformer_dynamic_amd import workloads as wl
from oracle import bra_oracle as O
from tests import parity
from tests.test_gpu_parity import EDGE, PAGE_SCHEDULES, _sample_images

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _f64(t):
    return wl.to_f64(t)


def _run(w, q, k, v, g):
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    idx = bra.route(qd, kd, w.S, w.topk)
    o = bra.attend(qd, kd, vd, idx, w.heads, w.S)
    dq, dk, dv = bra.attend_backward(qd, kd, vd, o, gd, idx, w.heads, w.S)
    torch.cuda.synchronize()
    return idx, o, dq, dk, dv


def _check_backward(w, images=None):
    print(f"\n[bwd case] {w.name}", flush=True)
    q, k, v = wl.make_inputs(w)
    g = wl.make_grad_output(w)
    idx, _, dq, dk, dv = _run(w, q, k, v, g)
    images = images if images is not None else _sample_images(w.B)
    ref = O.attend_backward(_f64(q[images]), _f64(k[images]), _f64(v[images]), idx.cpu().numpy()[images],
                            _f64(g[images]), w.heads, w.S)
    errs = []
    for name, out, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        errs.append(parity.assert_grad_close(_f64(out.cpu()[images]), r, w.dtype, f"{w.name} {name}"))
    print(f"[bwd case] {w.name}: " + ", ".join(f"d{n} max-abs {a:.2e} mean-rel {m:.2e}"
                                             for n, (a, m) in zip("QKV", errs)), flush=True)


@pytest.mark.parametrize("w", wl.WORKLOADS, ids=[w.name for w in wl.WORKLOADS])
def test_workload_backward(w):
    _check_backward(w)


@pytest.mark.parametrize("w", EDGE, ids=[w.name for w in EDGE])
def test_edge_shapes_backward(w):
    _check_backward(w, images=list(range(w.B)))


@pytest.mark.parametrize("w", PAGE_SCHEDULES[4:], ids=[w.name for w in PAGE_SCHEDULES[4:]])
def test_page_schedules_backward(w):
    _check_backward(w, images=list(range(w.B)))


def test_backward_is_deterministic_and_sums_hold():
    w = wl.custom(2, 28, 28, 128, 4, 7, 4, "f32", seed=80)
    q, k, v = wl.make_inputs(w)
    g = wl.make_grad_output(w)
    _, _, dq, dk, dv = _run(w, q, k, v, g)
    _, _, dq2, dk2, dv2 = _run(w, q, k, v, g)
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    # per image and channel: sum(dK) = 0, sum(dV) = sum(dO) (softmax rows sum to one)
    sk = dk.double().sum(dim=(1, 2)).cpu()
    sv = dv.double().sum(dim=(1, 2)).cpu()
    sg = g.double().sum(dim=(1, 2))
    assert sk.abs().max().item() <= 1e-3
    assert (sv - sg).abs().max().item() <= 1e-3


def test_unrouted_tokens_get_zero_key_and_value_gradients():
    """Planted routing: every region routes to itself only except region 0,
    which routes to region 1; region 0's keys are then routed to by nobody."""
    w = wl.custom(1, 16, 16, 64, 2, 4, 1, "bf16", seed=81)
    q, k, v = (t.to(DEV) for t in wl.make_inputs(w))
    g = wl.make_grad_output(w).to(DEV)
    idx = torch.arange(16, dtype=torch.int32, device=DEV).reshape(1, 16, 1).contiguous()
    idx[0, 0, 0] = 1
    o = bra.attend(q, k, v, idx, w.heads, w.S)
    dq, dk, dv = bra.attend_backward(q, k, v, o, g, idx, w.heads, w.S)
    torch.cuda.synchronize()
    assert torch.all(dk[0, :4, :4] == 0) and torch.all(dv[0, :4, :4] == 0)
    ref = O.attend_backward(_f64(q.cpu()), _f64(k.cpu()), _f64(v.cpu()), idx.cpu().numpy(), _f64(g.cpu()),
                            w.heads, w.S)
    for name, out, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        parity.assert_grad_close(_f64(out.cpu()), r, "bf16", name)


def test_bad_route_entry_gives_nan_dq_of_its_region_only():
    w = wl.custom(1, 14, 14, 64, 2, 7, 2, "bf16", seed=82)
    q, k, v = (t.to(DEV) for t in wl.make_inputs(w))
    g = wl.make_grad_output(w).to(DEV)
    idx = bra.route(q, k, w.S, w.topk)
    o = bra.attend(q, k, v, idx, w.heads, w.S)
    bad = idx.clone()
    bad[0, 5, 1] = 49
    dq, dk, dv = bra.attend_backward(q, k, v, o, g, bad, w.heads, w.S)
    torch.cuda.synchronize()
    rq = dq.float().cpu().reshape(1, 7, 2, 7, 2, 64).permute(0, 1, 3, 2, 4, 5).reshape(1, 49, 4, 64)
    assert torch.isnan(rq[0, 5]).all()
    keep = [r for r in range(49) if r != 5]
    assert not torch.isnan(rq[0, keep]).any()
    assert not torch.isnan(dk).any() and not torch.isnan(dv).any()
    # the bad region's queries are left out of dK, dV: the oracle without them
    routes = bad.cpu().numpy().copy()
    ref = O.attend_backward(_f64(q.cpu()), _f64(k.cpu()), _f64(v.cpu()), idx.cpu().numpy(),
                            _f64(g.cpu()) * _region_mask(w, 5), w.heads, w.S)
    for name, out, r in zip(("dK", "dV"), (dk, dv), ref[1:]):
        parity.assert_grad_close(_f64(out.cpu()), r, "bf16", name)


def _region_mask(w, region):
    m = np.ones((1, w.H, w.W, 1))
    ys, xs = O.region_token_coords(w.H, w.W, w.S, region)
    m[0, ys, xs, 0] = 0.0
    return m
