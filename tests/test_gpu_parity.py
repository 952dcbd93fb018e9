"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Inputs are the seeded synthetic workloads; the oracle sees the exact values
the GPU sees (bf16 upcast exactly). Routing is checked with the tie-band rule,
outputs against ``oracle.attend`` run with the GPU's own routing table (so a
legitimate tie-band choice cannot show up as an output error). At the full
workload sizes the GPU runs the whole batch in the launch configuration the
benchmark uses and the oracle checks a sample of images.
"""

import numpy as np
import pytest
import torch

import vision_transformer_dynamic_amd as bra
from vision_transformer_dynamic_amd import workloads as wl
from oracle import bra_oracle as O
from tests import parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _gpu(*ts):
    return [t.to(DEV) for t in ts]


def _f64(t):
    return wl.to_f64(t)


def _sample_images(B, max_images=4):
    if B <= max_images:
        return list(range(B))
    return sorted({0, 1, B // 2, B - 1})


def _oracle_affinity(q64, k64, S):
    return O.affinity(O.region_mean(q64, S), O.region_mean(k64, S))


def _check_case(w, q, k, v, images=None, check_exact_routes=True):
    """Route + attend + forward on the GPU for one workload; compare sampled
    images with the oracle. Returns (route mismatches, max_abs, mean_rel)."""
    print(f"\n[case] {w.name}", flush=True)
    qd, kd, vd = _gpu(q, k, v)
    idx = bra.route(qd, kd, w.S, w.topk)
    out_attend = bra.attend(qd, kd, vd, idx, w.heads, w.S)
    out_fwd = bra.forward(qd, kd, vd, w.heads, w.S, w.topk)
    torch.cuda.synchronize()
    # forward is exactly route followed by attend
    assert torch.equal(out_fwd, out_attend)

    images = images if images is not None else _sample_images(w.B)
    q64, k64, v64 = _f64(q[images]), _f64(k[images]), _f64(v[images])
    idx_np = idx.cpu().numpy()[images]
    A = _oracle_affinity(q64, k64, w.S)
    bad = parity.route_violations(A, idx_np, w.topk)
    assert not bad, f"{w.name}: routing violations {bad[:5]}"
    mism = parity.exact_route_mismatches(O.topk_route(A, w.topk), idx_np)
    ref = O.attend(q64, k64, v64, idx_np, w.heads, w.S)
    out = _f64(out_fwd.cpu()[images])
    max_abs, mean_rel = parity.assert_output_close(out, ref, w.dtype, w.name)
    print(f"[case] {w.name}: route mismatches {mism}, max-abs {max_abs:.3e}, mean-rel {mean_rel:.3e}", flush=True)
    return mism, max_abs, mean_rel


@pytest.mark.parametrize("w", wl.WORKLOADS, ids=[w.name for w in wl.WORKLOADS])
def test_workload_parity(w):
    q, k, v = wl.make_inputs(w)
    mism, _, _ = _check_case(w, q, k, v)
    # iid / clustered content has no near-ties at these sizes: the canonical
    # table is reproduced exactly
    assert mism == 0


@pytest.mark.parametrize("w", wl.WORKLOADS[1:4], ids=[w.name for w in wl.WORKLOADS[1:4]])
def test_full_size_route_all_images(w):
    """Routing of every image of the full-size workloads against the oracle."""
    q, k, _ = wl.make_inputs(w)
    qd, kd = _gpu(q, k)
    idx = bra.route(qd, kd, w.S, w.topk).cpu().numpy()
    A = _oracle_affinity(_f64(q), _f64(k), w.S)
    bad = parity.route_violations(A, idx, w.topk)
    assert not bad, bad[:5]
    assert parity.exact_route_mismatches(O.topk_route(A, w.topk), idx) == 0


# bra_route takes any C that is a multiple of 8 (routing has no head split).
# Shapes whose C is not a multiple of 32 route with the vector kernel, as do
# those with more than 64 regions; the workloads above use the matrix-core one.
ROUTE_ANY_C = [
    wl.custom(2, 6, 6, 8, 1, 3, 3, "bf16", seed=50),      # 9 regions, C = 8
    wl.custom(2, 14, 14, 40, 1, 7, 4, "f32", seed=51),    # 49 regions, C = 40
    wl.custom(1, 16, 16, 24, 1, 8, 64, "bf16", seed=52),  # 64 regions, full routing
    wl.custom(1, 16, 16, 48, 1, 16, 9, "bf16", seed=53),  # 256 regions, C = 48
    wl.custom(3, 8, 8, 96, 3, 8, 1, "bf16", seed=54),     # 64 regions, k = 1, 3 x 32 channels
    wl.custom(2, 14, 14, 320, 10, 7, 4, "bf16", seed=55),  # 49 regions, C = 320: query rows not staged in LDS
    wl.custom(1, 16, 16, 288, 9, 16, 5, "f32", seed=56),   # 256 regions, C = 288: the same in the 256-candidate form
]


@pytest.mark.parametrize("w", ROUTE_ANY_C, ids=[w.name for w in ROUTE_ANY_C])
def test_route_any_channel_count(w):
    q, k, _ = wl.make_inputs(w)
    qd, kd = _gpu(q, k)
    idx = bra.route(qd, kd, w.S, w.topk).cpu().numpy()
    A = _oracle_affinity(_f64(q), _f64(k), w.S)
    bad = parity.route_violations(A, idx, w.topk)
    assert not bad, bad[:5]
    assert parity.exact_route_mismatches(O.topk_route(A, w.topk), idx) == 0


# Ragged and edge shapes: n not a multiple of 16, kv not a multiple of 64,
# more than 64 queries per region, a partial head group, H != W, many regions,
# full routing, one region, one token per region.
EDGE = [
    wl.custom(2, 6, 6, 32, 1, 2, 3, "bf16", seed=10),      # n=9, kv=27
    wl.custom(1, 20, 20, 64, 2, 2, 2, "bf16", seed=11),    # n=100: a partial query block, ragged chunks
    wl.custom(1, 8, 12, 192, 6, 4, 5, "bf16", seed=12),    # H!=W, 6 heads: partial head group
    wl.custom(2, 32, 32, 96, 3, 4, 1, "bf16", seed=19),    # 3 heads: a two-head group and a one-head group
    wl.custom(1, 26, 40, 64, 2, 2, 2, "bf16", seed=21),    # n=260, kv=520: three staged phases, two query blocks, ragged
    wl.custom(1, 16, 16, 32, 1, 16, 7, "bf16", seed=13),   # 256 regions, n=1
    wl.custom(1, 16, 16, 32, 1, 16, 256, "bf16", seed=14), # full routing over 256 regions
    wl.custom(2, 12, 12, 64, 2, 3, 9, "bf16", seed=15),    # k = S*S
    wl.custom(2, 9, 9, 64, 2, 1, 1, "bf16", seed=16),      # one region: global attention
    wl.custom(1, 14, 14, 256, 8, 7, 16, "f32", seed=17),   # fp32, stage-3 shape
    wl.custom(2, 24, 24, 64, 2, 3, 2, "f32", seed=18),     # fp32, n=64, two head group of 1
    wl.custom(1, 32, 32, 64, 2, 2, 2, "f32", seed=19),     # fp32, n=256: one 256-query block per head
    wl.custom(3, 10, 15, 96, 3, 5, 4, "bf16", seed=20, content="clustered"),
    # chunked kernel (more than 64 keys per query) launch shapes: 4 heads of
    # one 16-query tile each in 4 waves (each thread stages four 16-byte
    # vectors of a chunk), the same in fp32, and a full plus a partial
    # 128-query block
    wl.custom(2, 28, 28, 128, 4, 7, 6, "bf16", seed=21),   # n=16, kv=96
    wl.custom(1, 16, 16, 64, 2, 4, 6, "f32", seed=22),     # fp32, n=16, kv=96
    wl.custom(1, 20, 30, 64, 2, 2, 2, "bf16", seed=23),    # n=150: blocks of 128 and 22 queries
]


@pytest.mark.parametrize("w", EDGE, ids=[w.name for w in EDGE])
def test_edge_shapes(w):
    q, k, v = wl.make_inputs(w)
    _check_case(w, q, k, v, images=list(range(w.B)))


# Image-resident attention (bf16, at most 64 keys per query, n a multiple of
# 4, at least 128 (image, head) pairs): one workgroup stages a head's whole
# image in LDS. Region sizes 16, 4 (four regions per 16-query unit), 12 (two
# runs of 4 keys per block of 8), 8 (two regions per unit, also with an odd
# region count) and 64 (four query tiles per region), full and ragged key
# counts, H != W.
IMAGE_RESIDENT = [
    wl.custom(32, 28, 28, 128, 4, 7, 4, "bf16", seed=70),   # n=16, kv=64
    wl.custom(16, 14, 14, 256, 8, 7, 16, "bf16", seed=71),  # n=4, kv=64
    wl.custom(64, 14, 14, 64, 2, 7, 8, "bf16", seed=72),    # n=4, kv=32
    wl.custom(64, 21, 28, 64, 2, 7, 5, "bf16", seed=73),    # n=12 (3 x 4), kv=60
    wl.custom(128, 8, 16, 32, 1, 4, 3, "bf16", seed=74),    # n=8 (2 x 4), kv=24
    wl.custom(128, 8, 16, 32, 1, 4, 8, "bf16", seed=77),    # n=8, kv=64
    wl.custom(128, 6, 12, 32, 1, 3, 5, "bf16", seed=78),    # n=8, 9 regions: a unit with one region
    wl.custom(128, 24, 24, 32, 1, 3, 1, "bf16", seed=75),   # n=64: four query tiles per region
    wl.custom(128, 32, 32, 32, 1, 8, 4, "bf16", seed=79),   # 64 units (16 waves x 4), about 149 KB of LDS
]


@pytest.mark.parametrize("w", IMAGE_RESIDENT, ids=[w.name for w in IMAGE_RESIDENT])
def test_image_resident_shapes(w):
    q, k, v = wl.make_inputs(w)
    mism, _, _ = _check_case(w, q, k, v)
    assert mism == 0


def test_image_resident_out_of_range_entries_give_nan_rows_only():
    w = wl.custom(64, 14, 14, 64, 2, 7, 2, "bf16", seed=76)
    q, k, v = _gpu(*wl.make_inputs(w))
    idx = bra.route(q, k, w.S, w.topk)
    good = bra.attend(q, k, v, idx, w.heads, w.S).float().cpu()
    bad_idx = idx.clone()
    bad_idx[5, 3, 1] = 49
    bad_idx[63, 10, 0] = -1
    out = bra.attend(q, k, v, bad_idx, w.heads, w.S).float().cpu()
    o = out.reshape(64, 7, 2, 7, 2, 64).permute(0, 1, 3, 2, 4, 5).reshape(64, 49, 4, 64)
    gd = good.reshape(64, 7, 2, 7, 2, 64).permute(0, 1, 3, 2, 4, 5).reshape(64, 49, 4, 64)
    assert torch.isnan(o[5, 3]).all() and torch.isnan(o[63, 10]).all()
    o[5, 3] = 0
    o[63, 10] = 0
    gd[5, 3] = 0
    gd[63, 10] = 0
    assert torch.equal(o, gd)


# The (S, k) schedules of the explainer's Part 6.3 table over the four stage
# maps of a 224 x 224 input (56, 28, 14, 7; C = 64 * 2^stage, head dim 32):
# S = 7 with k = [1, 4, 16, 49], S = 7 with k = [1, 2, 8, 32], and
# S = [8, 4, 2, 1] with k = [2, 2, 2, 1]. Two images each.
_STAGE_MAPS = [(56, 64), (28, 128), (14, 256), (7, 512)]
_SCHEDULES = [((7, 7, 7, 7), (1, 4, 16, 49)), ((7, 7, 7, 7), (1, 2, 8, 32)), ((8, 4, 2, 1), (2, 2, 2, 1))]
PAGE_SCHEDULES = [
    wl.custom(2, hw, hw, c, c // 32, S[st], k[st], "bf16", seed=40 + 4 * row + st)
    for row, (S, k) in enumerate(_SCHEDULES)
    for st, (hw, c) in enumerate(_STAGE_MAPS)
]


@pytest.mark.parametrize("w", PAGE_SCHEDULES, ids=[w.name for w in PAGE_SCHEDULES])
def test_page_schedules(w):
    q, k, v = wl.make_inputs(w)
    mism, _, _ = _check_case(w, q, k, v, images=list(range(w.B)))
    assert mism == 0


def test_one_region_equals_global_attention():
    w = wl.custom(2, 8, 8, 64, 2, 1, 1, "f32", seed=21)
    q, k, v = wl.make_inputs(w)
    out = bra.forward(*_gpu(q, k, v), w.heads, w.S, w.topk).cpu()
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(t.double().reshape(2, 64, 2, 32).permute(0, 2, 1, 3) for t in (q, k, v)))
    ref = ref.permute(0, 2, 1, 3).reshape(2, 8, 8, 64).numpy()
    parity.assert_output_close(_f64(out), ref, "f32", "S=1 global attention")


def test_zero_keys_route_to_lowest_indices_and_average_values():
    w = wl.custom(2, 14, 14, 64, 2, 7, 5, "bf16", seed=22)
    q, _, v = wl.make_inputs(w)
    k = torch.zeros_like(q)
    qd, kd, vd = _gpu(q, k, v)
    idx = bra.route(qd, kd, w.S, w.topk).cpu()
    assert torch.equal(idx, torch.arange(5, dtype=torch.int32).expand(2, 49, 5))
    out = _f64(bra.forward(qd, kd, vd, w.heads, w.S, w.topk).cpu())
    ref = O.attend(_f64(q), _f64(k), _f64(v), idx.numpy(), w.heads, w.S)
    parity.assert_output_close(out, ref, "bf16", "K=0")


def test_unit_values_give_unit_output():
    w = wl.custom(2, 28, 28, 128, 4, 7, 4, "bf16", seed=23)
    q, k, _ = wl.make_inputs(w)
    v = torch.ones_like(q)
    out = bra.forward(*_gpu(q, k, v), w.heads, w.S, w.topk).float().cpu()
    assert torch.all(out == 1.0)


def test_planted_diagonal_routing_is_window_attention():
    B, H, W, C, heads, S = 2, 16, 16, 64, 2, 4
    R = S * S
    g = torch.Generator().manual_seed(24)
    means = torch.zeros(R, C)
    means[torch.arange(R), torch.arange(R)] = 4.0
    grid = means.reshape(S, S, C).repeat_interleave(H // S, 0).repeat_interleave(W // S, 1)
    q = (grid + 0.05 * torch.randn(B, H, W, C, generator=g)).to(torch.bfloat16)
    k = (grid + 0.05 * torch.randn(B, H, W, C, generator=g)).to(torch.bfloat16)
    v = torch.randn(B, H, W, C, generator=g).to(torch.bfloat16)
    qd, kd, vd = _gpu(q, k, v)
    idx = bra.route(qd, kd, S, 1).cpu()
    assert torch.equal(idx[..., 0], torch.arange(R, dtype=torch.int32).expand(B, R))
    out = _f64(bra.forward(qd, kd, vd, heads, S, 1).cpu())
    ref = O.attend(_f64(q), _f64(k), _f64(v), idx.numpy(), heads, S)
    parity.assert_output_close(out, ref, "bf16", "planted routing")


def test_route_order_does_not_change_output_beyond_rounding():
    w = wl.custom(2, 28, 28, 128, 4, 7, 4, "f32", seed=25)
    q, k, v = _gpu(*wl.make_inputs(w))
    idx = bra.route(q, k, w.S, w.topk)
    flipped = idx.flip(-1).contiguous()
    a = bra.attend(q, k, v, idx, w.heads, w.S)
    b = bra.attend(q, k, v, flipped, w.heads, w.S)
    assert (a - b).abs().max().item() <= 1e-5


def test_out_of_range_route_entries_give_nan_rows_only():
    w = wl.custom(1, 14, 14, 64, 2, 7, 2, "bf16", seed=26)
    q, k, v = _gpu(*wl.make_inputs(w))
    idx = bra.route(q, k, w.S, w.topk)
    good = bra.attend(q, k, v, idx, w.heads, w.S).float().cpu()
    bad_idx = idx.clone()
    bad_idx[0, 3, 1] = 49
    bad_idx[0, 10, 0] = -1
    out = bra.attend(q, k, v, bad_idx, w.heads, w.S).float().cpu()
    o = out.reshape(1, 7, 2, 7, 2, 64).permute(0, 1, 3, 2, 4, 5).reshape(1, 49, 4, 64)
    gd = good.reshape(1, 7, 2, 7, 2, 64).permute(0, 1, 3, 2, 4, 5).reshape(1, 49, 4, 64)
    assert torch.isnan(o[0, 3]).all() and torch.isnan(o[0, 10]).all()
    keep = [r for r in range(49) if r not in (3, 10)]
    assert torch.equal(o[0, keep], gd[0, keep])


def test_deterministic_and_stream_ordered():
    w = wl.WORKLOADS[2]
    q, k, v = _gpu(*wl.make_inputs(w))
    a = bra.forward(q, k, v, w.heads, w.S, w.topk)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        b = bra.forward(q, k, v, w.heads, w.S, w.topk)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("w", [wl.WORKLOADS[0], wl.WORKLOADS[1], wl.WORKLOADS[2], wl.WORKLOADS[3], wl.WORKLOADS[4],
                               wl.custom(1, 16, 16, 32, 1, 16, 7, "bf16", seed=27),
                               wl.custom(128, 24, 24, 32, 1, 3, 1, "bf16", seed=75)],
                         ids=lambda w: w.name)
def test_forward_routing_table_equals_bra_route(w):
    """bra_forward leaves its routing table in the workspace: it must equal the
    one bra_route computes, bit for bit."""
    q, k, v = _gpu(*wl.make_inputs(w))
    nbytes = bra.workspace_bytes(w.B, w.H, w.W, w.C, w.S, w.topk)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    bra.forward(q, k, v, w.heads, w.S, w.topk, workspace=ws)
    pooled = -(-4 * w.B * w.R * w.C // 256) * 256
    table = ws[2 * pooled: 2 * pooled + 4 * w.B * w.R * w.topk].view(torch.int32).reshape(w.B, w.R, w.topk)
    ref = bra.route(q, k, w.S, w.topk)
    torch.cuda.synchronize()
    assert torch.equal(table, ref)


def test_concurrent_calls_from_threads():
    """Calls from several host threads on their own streams, with shapes whose
    attention kernels need different amounts of LDS (the image-resident kernel
    at 28x28 and 14x14, the chunked kernel at a 256-token region in fp32),
    give the bits of the same calls made one after another."""
    import threading

    shapes = [wl.custom(32, 28, 28, 128, 4, 7, 4, "bf16", seed=90),
              wl.custom(16, 14, 14, 256, 8, 7, 16, "bf16", seed=91),
              wl.custom(1, 32, 32, 64, 2, 2, 2, "f32", seed=92)]
    inputs = [_gpu(*wl.make_inputs(w)) for w in shapes]
    ref = [bra.forward(*x, w.heads, w.S, w.topk) for w, x in zip(shapes, inputs)]
    torch.cuda.synchronize()
    got = [[None] * 8 for _ in shapes]
    errors = []

    def work(i):
        try:
            w, x = shapes[i], inputs[i]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for r in range(8):
                    got[i][r] = bra.forward(*x, w.heads, w.S, w.topk)
            s.synchronize()
        except Exception as e:  # reported below, on the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(shapes))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(len(shapes)):
        for r in range(8):
            assert torch.equal(got[i][r], ref[i]), (shapes[i].name, r)


@pytest.mark.parametrize("w", [wl.WORKLOADS[0], wl.WORKLOADS[2], wl.WORKLOADS[3], wl.WORKLOADS[4],
                               wl.custom(2, 16, 16, 48, 1, 16, 9, "bf16", seed=28)],
                         ids=lambda w: w.name)
def test_workspace_forms_are_bit_identical(w):
    """bra_route / bra_forward (stream-ordered scratch of their own) against
    bra_route_ws / bra_forward_ws (the caller's workspace): the same bits."""
    q, k, v = _gpu(*wl.make_inputs(w))
    nbytes = bra.workspace_bytes(w.B, w.H, w.W, w.C, w.S, w.topk)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    idx_a = bra.route(q, k, w.S, w.topk)
    idx_b = bra.route_ws(q, k, w.S, w.topk, ws)
    torch.cuda.synchronize()
    assert torch.equal(idx_a, idx_b)
    if w.C % w.heads == 0 and w.C // w.heads == 32:
        o_a = bra.forward(q, k, v, w.heads, w.S, w.topk)
        o_b = bra.forward_ws(q, k, v, w.heads, w.S, w.topk, ws)
        torch.cuda.synchronize()
        assert torch.equal(o_a, o_b)


@pytest.mark.parametrize("w", wl.WORKLOADS, ids=[w.name for w in wl.WORKLOADS])
def test_pooled_means_match_oracle(w):
    """The region means Q^r, K^r that the pool kernel leaves in the workspace
    (offsets 0 and align256(4 B S^2 C)) against the oracle's fp64 means of the
    exact inputs: the summary's region-average identity rests on them, and
    routing alone cannot see a common scale error of both. Bound: the fp32
    summation error of n terms, n 2^-24 mean|x|, plus 2e-6."""
    q, k, v = wl.make_inputs(w)
    qd, kd, vd = _gpu(q, k, v)
    nbytes = bra.workspace_bytes(w.B, w.H, w.W, w.C, w.S, w.topk)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    bra.forward_ws(qd, kd, vd, w.heads, w.S, w.topk, ws)
    torch.cuda.synchronize()
    pooled = -(-4 * w.B * w.R * w.C // 256) * 256
    for name, t, off in (("Q^r", q, 0), ("K^r", k, pooled)):
        got = ws[off: off + 4 * w.B * w.R * w.C].view(torch.float32).reshape(w.B, w.R, w.C).cpu().double().numpy()
        x = _f64(t)
        ref = O.region_mean(x, w.S)
        mabs = O.region_mean(np.abs(x), w.S)
        bound = 2e-6 + w.n * 2.0 ** -24 * mabs
        err = np.abs(got - ref)
        assert np.all(err <= bound), f"{w.name} {name}: worst excess {float((err - bound).max()):.3e}"
        print(f"[means] {w.name} {name}: max-abs {float(err.max()):.2e}", flush=True)


# Non-finite inputs are outside the method's definition, but the table must
# still be well formed: every slot written with a distinct region index, and
# the same bits on every call. The vector route form (C not a multiple of 32,
# or more than 64 regions) orders NaN affinities with the same keys as the
# matrix-core form.
NAN_ROUTE = [
    wl.custom(1, 16, 16, 48, 1, 16, 9, "bf16", seed=29),   # 256 regions
    wl.custom(2, 14, 14, 40, 1, 7, 4, "f32", seed=30),     # C = 40
    wl.custom(2, 14, 14, 64, 2, 7, 4, "bf16", seed=31),    # matrix-core form
]


@pytest.mark.parametrize("w", NAN_ROUTE, ids=[w.name for w in NAN_ROUTE])
def test_nan_token_still_writes_every_routing_slot(w):
    q, k, _ = wl.make_inputs(w)
    q[0, 1, 1, :] = float("nan")   # a token of region 0: Q^r[0, 0] is NaN, so is row 0
    k[0, 5, 3, :] = float("nan")   # every row has one NaN candidate
    qd, kd = _gpu(q, k)
    a = torch.full((w.B, w.R, w.topk), -7, dtype=torch.int32, device=DEV)
    b = torch.full((w.B, w.R, w.topk), -9, dtype=torch.int32, device=DEV)
    bra.route(qd, kd, w.S, w.topk, out=a)
    bra.route(qd, kd, w.S, w.topk, out=b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    t = a.cpu().numpy()
    assert t.min() >= 0 and t.max() < w.R
    for row in t.reshape(-1, w.topk):
        assert len(set(row.tolist())) == w.topk
    # image 1 has no NaN: it routes as the oracle does
    if w.B > 1:
        A = _oracle_affinity(_f64(q[1:]), _f64(k[1:]), w.S)
        assert parity.exact_route_mismatches(O.topk_route(A, w.topk), t[1:]) == 0


# Detection-shaped maps at S = 16 (256 regions; explainer Part 4.3, S = 16
# for object detection): the two measured detection workloads, and 96 x 96
# maps whose 36-token regions make every 64-key chunk ragged, k = 4 and 8.
DETECTION_SHAPES = wl.DETECTION + [
    wl.custom(2, 96, 96, 64, 2, 16, 4, "bf16", seed=96),
    wl.custom(2, 96, 96, 64, 2, 16, 8, "bf16", seed=97, content="clustered"),
    wl.custom(2, 64, 64, 64, 2, 16, 4, "bf16", seed=98),
]


@pytest.mark.parametrize("w", DETECTION_SHAPES, ids=[w.name for w in DETECTION_SHAPES])
def test_detection_shapes_s16(w):
    q, k, v = wl.make_inputs(w)
    mism, _, _ = _check_case(w, q, k, v, images=list(range(w.B)))
    assert mism == 0
