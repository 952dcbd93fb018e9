"""GPU parity of the QKV projection with the fused region pooling, and of the
module from its input (projection, routing from the fused means, attention),
through the C ABI, against the fp64 oracle."""

import numpy as np
import pytest
import torch

import vision_transformer_dynamic_amd as bra
from vision_transformer_dynamic_amd import workloads as wl
from oracle import bra_oracle as O
from tests import parity
from tests.test_gpu_parity import EDGE, _sample_images

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _f64(t):
    return wl.to_f64(t)


def _supported(w):
    return w.C % 32 == 0 and w.C <= (256 if w.dtype == "bf16" else 128)


def _check_projection(w, bias=True, images=None):
    print(f"\n[qkv case] {w.name} bias={bias}", flush=True)
    x, wq, bq = wl.make_projection(w)
    bq = bq if bias else None
    xd, wd = x.to(DEV), wq.to(DEV)
    bd = bq.to(DEV) if bias else None
    q, k, v, qr, kr = bra.qkv_pool(xd, wd, bd, w.S)
    torch.cuda.synchronize()
    images = images if images is not None else _sample_images(w.B)
    ref = O.qkv_project(_f64(x[images]), _f64(wq), None if bq is None else _f64(bq))
    for name, out, r in zip("QKV", (q, k, v), ref):
        parity.assert_proj_close(_f64(out.cpu()[images]), r, w.dtype, f"{w.name} {name}")
    # the fused means are the means of the rounded Q and K
    for name, got, src in (("Q^r", qr, q), ("K^r", kr, k)):
        ref_m = O.region_mean(_f64(src.cpu()[images]), w.S)
        np.testing.assert_allclose(got.cpu().numpy()[images], ref_m, rtol=0, atol=2e-5, err_msg=name)
    return xd, wd, bd, (q, k, v)


@pytest.mark.parametrize("w", wl.WORKLOADS, ids=[w.name for w in wl.WORKLOADS])
def test_workload_projection_and_pool(w):
    _check_projection(w)


@pytest.mark.parametrize("w", [e for e in EDGE if _supported(e)], ids=[e.name for e in EDGE if _supported(e)])
def test_edge_shapes_projection(w):
    _check_projection(w, images=list(range(w.B)))


# region sizes and channel counts of both projection kernels: n = 2, 4, 8
# (runs inside a 16-token tile), 32 and 48 (regions over several tiles, a
# block's last tile empty), C = 96 and 128 (9 and 12 waves; two-unit prefetch)
PROJ_SHAPES = [
    wl.custom(2, 8, 4, 64, 2, 4, 3, "bf16", seed=95),     # n = 2
    wl.custom(2, 8, 8, 64, 2, 4, 3, "bf16", seed=96),     # n = 4
    wl.custom(1, 16, 8, 32, 1, 4, 2, "bf16", seed=97),    # n = 8
    wl.custom(2, 16, 16, 96, 3, 4, 2, "bf16", seed=98),   # C = 96, n = 16
    wl.custom(1, 24, 24, 128, 4, 3, 2, "bf16", seed=99),  # n = 64, C = 128
    wl.custom(2, 16, 8, 64, 2, 2, 2, "bf16", seed=100),   # n = 32: a region spans two 16-token tiles
    wl.custom(1, 16, 12, 64, 2, 2, 2, "bf16", seed=101),  # n = 48: one region per block, the last tile empty
    wl.custom(1, 16, 12, 128, 4, 2, 3, "bf16", seed=102), # n = 48, C = 128 (two-unit prefetch)
]


@pytest.mark.parametrize("w", PROJ_SHAPES, ids=[w.name for w in PROJ_SHAPES])
def test_projection_region_sizes(w):
    _check_projection(w, images=list(range(w.B)))


def test_projection_without_bias():
    _check_projection(wl.WORKLOADS[2], bias=False)


@pytest.mark.parametrize("w", wl.WORKLOADS, ids=[w.name for w in wl.WORKLOADS])
def test_forward_from_input(w):
    """bra_forward_qkv = projection + routing from the fused means + attention;
    with these draws (no near-ties) its routing is bra_route's and its output
    is bit-identical to bra_forward on the projected Q, K, V."""
    x, wq, bq = (t.to(DEV) for t in wl.make_projection(w))
    nbytes = bra.workspace_bytes(w.B, w.H, w.W, w.C, w.S, w.topk)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    o, q, k, v = bra.forward_qkv(x, wq, bq, w.heads, w.S, w.topk, workspace=ws)
    pooled = -(-4 * w.B * w.R * w.C // 256) * 256
    idx = ws[2 * pooled: 2 * pooled + 4 * w.B * w.R * w.topk].view(torch.int32).reshape(w.B, w.R, w.topk).clone()
    ref_o = bra.forward(q, k, v, w.heads, w.S, w.topk)
    ref_idx = bra.route(q, k, w.S, w.topk)
    torch.cuda.synchronize()
    assert torch.equal(idx, ref_idx)
    assert torch.equal(o, ref_o)
    images = _sample_images(w.B)
    q64, k64, v64 = (_f64(t.cpu()[images]) for t in (q, k, v))
    A = O.affinity(O.region_mean(q64, w.S), O.region_mean(k64, w.S))
    assert not parity.route_violations(A, idx.cpu().numpy()[images], w.topk)
    ref = O.attend(q64, k64, v64, idx.cpu().numpy()[images], w.heads, w.S)
    parity.assert_output_close(_f64(o.cpu()[images]), ref, w.dtype, w.name)


def test_projection_unsupported_channels():
    w = wl.custom(1, 14, 14, 256, 8, 7, 16, "f32", seed=91)
    x, wq, bq = (t.to(DEV) for t in wl.make_projection(w))
    with pytest.raises(NotImplementedError):
        bra.qkv_pool(x, wq, bq, w.S)
