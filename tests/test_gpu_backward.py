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


@pytest.mark.parametrize("w", wl.DETECTION, ids=[w.name for w in wl.DETECTION])
def test_detection_backward(w):
    _check_backward(w, images=list(range(w.B)))


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


BAD_ROWS = [wl.custom(1, 14, 14, 64, 2, 7, 2, "bf16", seed=82),   # at most 64 keys per query
            wl.custom(1, 28, 28, 64, 2, 7, 6, "bf16", seed=83)]   # several 64-key chunks


@pytest.mark.parametrize("w", BAD_ROWS, ids=[w.name for w in BAD_ROWS])
@pytest.mark.parametrize("kind", ["out_of_range", "repeated"])
def test_bad_route_row_gives_nan_dq_of_its_region_only(w, kind):
    """A routing row with an entry outside [0, S*S), or with a repeated entry
    (which bra_route never writes), gives NaN dQ for its region's queries and
    leaves them out of dK and dV."""
    q, k, v = (t.to(DEV) for t in wl.make_inputs(w))
    g = wl.make_grad_output(w).to(DEV)
    idx = bra.route(q, k, w.S, w.topk)
    o = bra.attend(q, k, v, idx, w.heads, w.S)
    bad = idx.clone()
    bad[0, 5, 1] = w.R if kind == "out_of_range" else bad[0, 5, 0]
    dq, dk, dv = bra.attend_backward(q, k, v, o, g, bad, w.heads, w.S)
    torch.cuda.synchronize()
    ys, xs = (torch.as_tensor(a) for a in O.region_token_coords(w.H, w.W, w.S, 5))
    dqf = dq.float().cpu()
    assert torch.isnan(dqf[0, ys, xs]).all()
    dqf[0, ys, xs] = 0
    assert not torch.isnan(dqf).any()
    assert not torch.isnan(dk).any() and not torch.isnan(dv).any()
    # the bad region's queries are left out of dK, dV: the oracle without them
    ref = O.attend_backward(_f64(q.cpu()), _f64(k.cpu()), _f64(v.cpu()), idx.cpu().numpy(),
                            _f64(g.cpu()) * _region_mask(w, 5), w.heads, w.S)
    for name, out, r in zip(("dK", "dV"), (dk, dv), ref[1:]):
        parity.assert_grad_close(_f64(out.cpu()), r, "bf16", name)


def _region_mask(w, region):
    m = np.ones((1, w.H, w.W, 1))
    ys, xs = O.region_token_coords(w.H, w.W, w.S, region)
    m[0, ys, xs, 0] = 0.0
    return m


# Shapes the one-launch image-resident backward takes (bf16, regions of 4, 8
# or 16 tokens, at most 64 regions, at least 128 (image, head) pairs): every
# region size, full and ragged key sets (kv < 64), H != W.
IMAGE_BWD = [
    wl.custom(64, 8, 8, 64, 2, 4, 16, "bf16", seed=90),     # n = 4, kv = 64
    wl.custom(32, 14, 14, 128, 4, 7, 8, "bf16", seed=91),   # n = 4, kv = 32
    wl.custom(32, 8, 16, 128, 4, 4, 8, "bf16", seed=92),    # n = 8 (2 x 4), kv = 64, H != W
    wl.custom(32, 14, 28, 128, 4, 7, 3, "bf16", seed=93),   # n = 8 (2 x 4), kv = 24, H != W
    wl.custom(32, 16, 16, 128, 4, 4, 4, "bf16", seed=94),   # n = 16, kv = 64
    wl.custom(32, 16, 16, 128, 4, 4, 2, "bf16", seed=95, content="clustered"),  # n = 16, kv = 32
    # K, V and then Q, dO in the same LDS (the four row arrays do not fit together)
    wl.custom(32, 28, 28, 128, 4, 7, 2, "bf16", seed=98),   # n = 16, kv = 32
    wl.custom(32, 16, 32, 128, 4, 8, 8, "bf16", seed=99),   # n = 8 (2 x 4), kv = 64, 64 regions
]


@pytest.mark.parametrize("w", IMAGE_BWD, ids=[w.name for w in IMAGE_BWD])
def test_image_resident_backward(w):
    _check_backward(w)


def test_image_resident_backward_is_deterministic():
    w = IMAGE_BWD[1]
    q, k, v = wl.make_inputs(w)
    g = wl.make_grad_output(w)
    _, _, dq, dk, dv = _run(w, q, k, v, g)
    _, _, dq2, dk2, dv2 = _run(w, q, k, v, g)
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)


def test_image_resident_unrouted_tokens_get_zero_key_and_value_gradients():
    """As above on 64 images (the image-resident backward): every region
    routes to itself except region 0, which routes to region 1."""
    w = wl.custom(64, 16, 16, 64, 2, 4, 1, "bf16", seed=96)
    q, k, v = (t.to(DEV) for t in wl.make_inputs(w))
    g = wl.make_grad_output(w).to(DEV)
    idx = torch.arange(16, dtype=torch.int32, device=DEV).reshape(1, 16, 1).repeat(w.B, 1, 1).contiguous()
    idx[:, 0, 0] = 1
    o = bra.attend(q, k, v, idx, w.heads, w.S)
    dq, dk, dv = bra.attend_backward(q, k, v, o, g, idx, w.heads, w.S)
    torch.cuda.synchronize()
    assert torch.all(dk[:, :4, :4] == 0) and torch.all(dv[:, :4, :4] == 0)
    sel = [0, w.B - 1]
    ref = O.attend_backward(_f64(q.cpu()[sel]), _f64(k.cpu()[sel]), _f64(v.cpu()[sel]), idx.cpu().numpy()[sel],
                            _f64(g.cpu()[sel]), w.heads, w.S)
    for name, out, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        parity.assert_grad_close(_f64(out.cpu()[sel]), r, "bf16", name)


@pytest.mark.parametrize("kind", ["out_of_range", "repeated"])
def test_image_resident_bad_route_row(kind):
    """The bad-row rule on the image-resident backward (64 images, 2 x 2
    regions, kv = 16): NaN dQ for the bad region's queries only, which are left
    out of dK and dV; the other images are untouched."""
    w = wl.custom(64, 14, 14, 64, 2, 7, 4, "bf16", seed=97)
    q, k, v = (t.to(DEV) for t in wl.make_inputs(w))
    g = wl.make_grad_output(w).to(DEV)
    idx = bra.route(q, k, w.S, w.topk)
    o = bra.attend(q, k, v, idx, w.heads, w.S)
    bad = idx.clone()
    bad[0, 5, 1] = w.R if kind == "out_of_range" else bad[0, 5, 0]
    dq, dk, dv = bra.attend_backward(q, k, v, o, g, bad, w.heads, w.S)
    dq0, dk0, dv0 = bra.attend_backward(q, k, v, o, g, idx, w.heads, w.S)
    torch.cuda.synchronize()
    ys, xs = (torch.as_tensor(a) for a in O.region_token_coords(w.H, w.W, w.S, 5))
    dqf = dq.float().cpu()
    assert torch.isnan(dqf[0, ys, xs]).all()
    dqf[0, ys, xs] = 0
    assert not torch.isnan(dqf).any()
    assert not torch.isnan(dk).any() and not torch.isnan(dv).any()
    # images other than 0 are those of the good table, bit for bit
    assert torch.equal(dq[1:], dq0[1:]) and torch.equal(dk[1:], dk0[1:]) and torch.equal(dv[1:], dv0[1:])
    ref = O.attend_backward(_f64(q.cpu()[:1]), _f64(k.cpu()[:1]), _f64(v.cpu()[:1]), idx.cpu().numpy()[:1],
                            _f64(g.cpu()[:1]) * _region_mask(w, 5), w.heads, w.S)
    for name, out, r in zip(("dK", "dV"), (dk, dv), ref[1:]):
        parity.assert_grad_close(_f64(out.cpu()[:1]), r, "bf16", name)


# Shapes the one-launch top-1 backward takes (bf16, top-k = 1, regions of 16
# to 64 tokens): full and ragged regions, one to four 16-row tiles, an odd
# head count (the last pair has one head), more than 64 regions (several
# ballot steps of the routing column), H != W.
TOP1_BWD = [
    wl.custom(2, 56, 56, 64, 2, 7, 1, "bf16", seed=110),    # n = 64, 49 regions (the first stage's shape)
    wl.custom(2, 56, 56, 96, 3, 8, 1, "bf16", seed=111),    # n = 49, three heads
    wl.custom(1, 72, 72, 64, 2, 9, 1, "bf16", seed=112),    # n = 64, 81 regions
    wl.custom(2, 24, 24, 128, 4, 4, 1, "bf16", seed=113),   # n = 36, two pairs of heads
    wl.custom(1, 64, 64, 32, 1, 16, 1, "bf16", seed=114),   # n = 16, one head, 256 regions
    wl.custom(2, 40, 60, 64, 2, 5, 1, "bf16", seed=115, content="clustered"),  # n = 8 x 12 = 96: not taken
    wl.custom(2, 35, 42, 64, 2, 7, 1, "bf16", seed=116),    # n = 5 x 6 = 30, H != W
]


@pytest.mark.parametrize("w", TOP1_BWD, ids=[w.name for w in TOP1_BWD])
def test_top1_backward(w):
    _check_backward(w, images=list(range(w.B)))


def test_top1_backward_is_deterministic():
    w = TOP1_BWD[1]
    q, k, v = wl.make_inputs(w)
    g = wl.make_grad_output(w)
    _, _, dq, dk, dv = _run(w, q, k, v, g)
    _, _, dq2, dk2, dv2 = _run(w, q, k, v, g)
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)


def test_top1_backward_one_popular_region():
    """Planted routing: every query region of image 0 routes to region 3 (a
    list of all 49 regions for one workgroup, every other key region
    unrouted); image 1 keeps its own routing."""
    w = TOP1_BWD[0]
    q, k, v = (t.to(DEV) for t in wl.make_inputs(w))
    g = wl.make_grad_output(w).to(DEV)
    idx = bra.route(q, k, w.S, w.topk)
    idx[0] = 3
    o = bra.attend(q, k, v, idx, w.heads, w.S)
    dq, dk, dv = bra.attend_backward(q, k, v, o, g, idx, w.heads, w.S)
    torch.cuda.synchronize()
    ys, xs = (torch.as_tensor(a) for a in O.region_token_coords(w.H, w.W, w.S, 3))
    keep = torch.zeros(w.H, w.W, dtype=torch.bool)
    keep[ys, xs] = True
    assert torch.all(dk[0].cpu()[~keep] == 0) and torch.all(dv[0].cpu()[~keep] == 0)
    ref = O.attend_backward(_f64(q.cpu()), _f64(k.cpu()), _f64(v.cpu()), idx.cpu().numpy(), _f64(g.cpu()),
                            w.heads, w.S)
    for name, out, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        parity.assert_grad_close(_f64(out.cpu()), r, "bf16", name)


def test_top1_bad_route_row():
    """The bad-row rule on the top-1 backward: an entry outside [0, S*S) in
    row 5 gives NaN dQ for region 5's queries only, which are left out of dK
    and dV; image 1 is that of the good table, bit for bit."""
    w = TOP1_BWD[0]
    q, k, v = (t.to(DEV) for t in wl.make_inputs(w))
    g = wl.make_grad_output(w).to(DEV)
    idx = bra.route(q, k, w.S, w.topk)
    o = bra.attend(q, k, v, idx, w.heads, w.S)
    bad = idx.clone()
    bad[0, 5, 0] = w.R
    dq, dk, dv = bra.attend_backward(q, k, v, o, g, bad, w.heads, w.S)
    dq0, dk0, dv0 = bra.attend_backward(q, k, v, o, g, idx, w.heads, w.S)
    torch.cuda.synchronize()
    ys, xs = (torch.as_tensor(a) for a in O.region_token_coords(w.H, w.W, w.S, 5))
    dqf = dq.float().cpu()
    assert torch.isnan(dqf[0, ys, xs]).all()
    dqf[0, ys, xs] = 0
    assert not torch.isnan(dqf).any()
    assert not torch.isnan(dk).any() and not torch.isnan(dv).any()
    assert torch.equal(dq[1:], dq0[1:]) and torch.equal(dk[1:], dk0[1:]) and torch.equal(dv[1:], dv0[1:])
    ref = O.attend_backward(_f64(q.cpu()[:1]), _f64(k.cpu()[:1]), _f64(v.cpu()[:1]), idx.cpu().numpy()[:1],
                            _f64(g.cpu()[:1]) * _region_mask(w, 5), w.heads, w.S)
    for name, out, r in zip(("dK", "dV"), (dk, dv), ref[1:]):
        parity.assert_grad_close(_f64(out.cpu()[:1]), r, "bf16", name)
