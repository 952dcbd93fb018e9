"""Pins of the fp64 CPU oracle against facts fixed by the pages and by mathematics.

No test here uses the HIP path. Each pin is chosen so that a plausible slip in
the oracle (a dropped term, a transposed operand, a wrong region or head
index, a wrong scale, a wrong tie rule) fails at least one of them.
"""

import os

import numpy as np
import pytest
import torch

from oracle import bra_oracle as O
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# --------------------------------------------------------------------------- #
# Pool + affinity: region-mean affinity equals the mean token-pair affinity
# (paper summary, Section 6 "Conclusion", regional representations).
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize(
    "B,H,W,C,S",
    [(2, 6, 6, 8, 3), (1, 6, 9, 5, 3), (1, 4, 8, 3, 2), (1, 8, 4, 4, 4), (2, 5, 5, 7, 1)],
)
def test_affinity_equals_mean_pairwise_token_affinity(B, H, W, C, S):
    Q = _rand((B, H, W, C), 1)
    K = _rand((B, H, W, C), 2)
    A = O.affinity(O.region_mean(Q, S), O.region_mean(K, S))
    A_ref = brute.pairwise_region_affinity(Q, K, S)
    np.testing.assert_allclose(A, A_ref, rtol=1e-12, atol=1e-12)
    if S > 1:
        # rows are query regions, columns key regions: not symmetric in general
        assert not np.allclose(A, np.swapaxes(A, -1, -2))


def test_region_mean_hand_example():
    # 4x4 map, S=2, one channel holding its flat index: region 0 is rows 0-1,
    # cols 0-1 -> values 0,1,4,5 -> mean 2.5; region 1 -> 2,3,6,7 -> 4.5;
    # region 2 -> 8,9,12,13 -> 10.5; region 3 -> 12.5.
    X = np.arange(16, dtype=np.float64).reshape(1, 4, 4, 1)
    np.testing.assert_array_equal(O.region_mean(X, 2)[0, :, 0], [2.5, 4.5, 10.5, 12.5])
    # 2x6 map, S=2: regions are 1x3; region 1 = row 0, cols 3-5 -> 3,4,5
    X = np.arange(12, dtype=np.float64).reshape(1, 2, 6, 1)
    np.testing.assert_array_equal(O.region_mean(X, 2)[0, :, 0], [1.0, 4.0, 7.0, 10.0])


# --------------------------------------------------------------------------- #
# Top-k routing
# --------------------------------------------------------------------------- #
def _brute_topk_row(row, k):
    order = sorted(range(len(row)), key=lambda j: (-row[j], j))
    return order[:k]


@pytest.mark.parametrize("R,k", [(16, 2), (49, 1), (49, 4), (49, 16), (64, 4), (49, 49), (9, 9), (1, 1)])
def test_topk_route_matches_full_sort(R, k):
    rng = np.random.default_rng(R * 100 + k)
    A = rng.standard_normal((3, R, R))
    # plant exact ties (rounded values) in one image
    A[1] = np.round(A[1], 1)
    I = O.topk_route(A, k)
    assert I.dtype == np.int32 and I.shape == (3, R, k)
    for b in range(3):
        for i in range(R):
            row = A[b, i]
            assert list(I[b, i]) == _brute_topk_row(list(row), k)
            sel = set(I[b, i].tolist())
            assert len(sel) == k and all(0 <= j < R for j in sel)
            unsel = [row[j] for j in range(R) if j not in sel]
            if unsel:
                assert min(row[list(sel)]) >= max(unsel)
    if k == R:
        assert np.array_equal(np.sort(I, axis=-1), np.broadcast_to(np.arange(R), I.shape))


def test_topk_ties_lower_index_first():
    A = np.array([[[1.0, 3.0, 3.0, 2.0, 3.0]]])
    assert O.topk_route(A, 3).tolist() == [[[1, 2, 4]]]
    assert O.topk_route(A, 4).tolist() == [[[1, 2, 4, 3]]]
    A = np.zeros((1, 1, 6))
    assert O.topk_route(A, 2).tolist() == [[[0, 1]]]


# --------------------------------------------------------------------------- #
# Attention: special cases that reduce to textbook routines
# --------------------------------------------------------------------------- #
def _sdpa(Q, K, V, heads, scale=None):
    B, H, W, C = Q.shape
    d = C // heads

    def split(X):
        return torch.from_numpy(X).reshape(B, H * W, heads, d).permute(0, 2, 1, 3).contiguous()

    o = torch.nn.functional.scaled_dot_product_attention(split(Q), split(K), split(V), scale=scale)
    return o.permute(0, 2, 1, 3).reshape(B, H, W, C).numpy()


@pytest.mark.parametrize(
    "B,H,W,C,heads,S",
    [(1, 8, 8, 8, 2, 2), (2, 6, 9, 6, 3, 3), (1, 4, 4, 4, 1, 4), (1, 6, 6, 12, 2, 1)],
)
def test_full_routing_equals_global_attention(B, H, W, C, heads, S):
    Q, K, V = (_rand((B, H, W, C), s) for s in (3, 4, 5))
    out, routes = O.bra(Q, K, V, heads, S, S * S)
    ref = brute.global_attention(Q, K, V, heads)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(out, _sdpa(Q, K, V, heads), rtol=1e-10, atol=1e-12)


def test_one_region_top1_equals_global_attention():
    Q, K, V = (_rand((2, 5, 7, 8), s) for s in (6, 7, 8))
    out, routes = O.bra(Q, K, V, heads=2, S=1, topk=1)
    assert routes.tolist() == [[[0]], [[0]]]
    np.testing.assert_allclose(out, _sdpa(Q, K, V, 2), rtol=1e-10, atol=1e-12)


def test_scale_is_a_parameter_and_defaults_to_inverse_sqrt_d():
    Q, K, V = (_rand((1, 4, 4, 8), s) for s in (9, 10, 11))
    out1, _ = O.bra(Q, K, V, heads=2, S=2, topk=4, scale=1.0)
    np.testing.assert_allclose(out1, _sdpa(Q, K, V, 2, scale=1.0), rtol=1e-10, atol=1e-12)
    out_d, _ = O.bra(Q, K, V, heads=2, S=2, topk=4)
    assert not np.allclose(out1, out_d)


def _planted(B, H, W, C, S, seed, partner=None, noise=0.05):
    """Q, K whose region means are scaled basis vectors: K region j has mean
    4*e_j; Q region i has mean 4*e_i (+ 2*e_partner(i) when given), so the
    region affinity is diagonally dominant (or has a known second choice)."""
    R = S * S
    assert C >= R
    rng = np.random.default_rng(seed)
    qm = np.zeros((R, C))
    km = np.zeros((R, C))
    for r in range(R):
        km[r, r] = 4.0
        qm[r, r] = 4.0
        if partner is not None:
            qm[r, partner[r]] += 2.0
    sh, sw = H // S, W // S

    def expand(m):
        g = m.reshape(S, S, C).repeat(sh, axis=0).repeat(sw, axis=1)
        return np.broadcast_to(g, (B, H, W, C))

    Q = expand(qm) + noise * rng.standard_normal((B, H, W, C))
    K = expand(km) + noise * rng.standard_normal((B, H, W, C))
    V = rng.standard_normal((B, H, W, C))
    return Q, K, V


@pytest.mark.parametrize("B,H,W,C,heads,S", [(2, 8, 8, 8, 2, 2), (1, 6, 9, 12, 3, 3), (1, 4, 8, 4, 1, 2)])
def test_planted_top1_routing_is_window_attention(B, H, W, C, heads, S):
    R = S * S
    Q, K, V = _planted(B, H, W, C, S, seed=12)
    out, routes = O.bra(Q, K, V, heads, S, 1)
    assert routes[..., 0].tolist() == [list(range(R))] * B
    ref = brute.window_attention_over(Q, K, V, heads, S, routes)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)
    # and it is not global attention
    assert not np.allclose(out, brute.global_attention(Q, K, V, heads))


def test_planted_top2_routing_gathers_the_partner_region():
    B, H, W, C, heads, S = 2, 6, 9, 12, 3, 3
    R = S * S
    partner = [(r * 4 + 5) % R for r in range(R)]
    partner = [p if p != r else (r + 1) % R for r, p in enumerate(partner)]
    Q, K, V = _planted(B, H, W, C, S, seed=13, partner=partner)
    out, routes = O.bra(Q, K, V, heads, S, 2)
    for b in range(B):
        assert routes[b].tolist() == [[r, partner[r]] for r in range(R)]
    ref = brute.window_attention_over(Q, K, V, heads, S, routes)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)


def test_zero_keys_give_mean_of_first_k_regions():
    B, H, W, C, heads, S, k = 2, 6, 6, 8, 2, 3, 3
    Q = _rand((B, H, W, C), 14)
    K = np.zeros((B, H, W, C))
    V = _rand((B, H, W, C), 15)
    out, routes = O.bra(Q, K, V, heads, S, k)
    assert (routes == np.arange(k)).all()  # all affinities tie -> lowest indices
    mean = brute.window_mean(V, S, range(k))
    np.testing.assert_allclose(out, np.broadcast_to(mean[:, None, None, :], out.shape), rtol=1e-12, atol=1e-13)


def test_unit_values_give_unit_output_and_convex_hull():
    B, H, W, C, heads, S, k = 1, 8, 8, 8, 2, 4, 3
    Q, K, V = (_rand((B, H, W, C), s) for s in (16, 17, 18))
    out, _ = O.bra(Q, K, np.ones_like(V), heads, S, k)
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-13)
    out, routes = O.bra(Q, K, V, heads, S, k)
    for i in range(S * S):
        gy, gx = O.gather_coords(H, W, S, routes[0, i])
        qy, qx = O.region_token_coords(H, W, S, i)
        lo = V[0, gy, gx, :].min(axis=0)
        hi = V[0, gy, gx, :].max(axis=0)
        o = out[0, qy, qx, :]
        assert (o >= lo - 1e-12).all() and (o <= hi + 1e-12).all()


def test_route_order_permutation_invariance():
    B, H, W, C, heads, S, k = 2, 8, 8, 8, 2, 4, 5
    Q, K, V = (_rand((B, H, W, C), s) for s in (19, 20, 21))
    routes = O.route(Q, K, S, k)
    rng = np.random.default_rng(22)
    shuffled = np.array([[rng.permutation(row) for row in img] for img in routes])
    a = O.attend(Q, K, V, routes, heads, S)
    b = O.attend(Q, K, V, shuffled, heads, S)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------- #
# Printed example: attended tokens per stage (explainer, Part 6.3 table)
# --------------------------------------------------------------------------- #
def test_attended_tokens_match_the_pages_table():
    rows = []
    with open(os.path.join(GOLDEN, "attended_tokens.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(x) for x in line.split()])
    assert len(rows) == 12
    for H, W, S, k, expect in rows:
        assert O.attended_tokens(H, W, S, k) == expect
        # the gather really concatenates that many tokens
        gy, gx = O.gather_coords(H, W, S, list(range(k)))
        assert len(gy) == expect and len(set(zip(gy.tolist(), gx.tolist()))) == expect


def test_check_config_rejects_undefined_shapes():
    O.check_config(1, 56, 56, 64, 2, 7, 1)
    with pytest.raises(ValueError):
        O.check_config(1, 56, 56, 64, 2, 5, 1)  # S does not divide H
    with pytest.raises(ValueError):
        O.check_config(1, 56, 56, 64, 3, 7, 1)  # heads does not divide C
    with pytest.raises(ValueError):
        O.check_config(1, 56, 56, 64, 2, 7, 0)
    with pytest.raises(ValueError):
        O.check_config(1, 56, 56, 64, 2, 7, 50)
    with pytest.raises(ValueError):
        O.check_config(0, 56, 56, 64, 2, 7, 1)


# --------------------------------------------------------------------------- #
# Local context term: 5 x 5 depthwise convolution of V (explainer Part 2.2
# step 4 and pseudocode step 7; paper summary Section 3)
# --------------------------------------------------------------------------- #
LCE_SHAPES = [(2, 7, 9, 8), (1, 3, 2, 4), (1, 1, 6, 3), (1, 12, 5, 16)]


@pytest.mark.parametrize("B,H,W,C", LCE_SHAPES)
def test_lce_equals_torch_depthwise_conv2d(B, H, W, C):
    V = _rand((B, H, W, C), 40)
    w = _rand((C, 5, 5), 41)
    b = _rand((C,), 42)
    ref = torch.nn.functional.conv2d(torch.from_numpy(V).permute(0, 3, 1, 2), torch.from_numpy(w)[:, None],
                                     torch.from_numpy(b), padding=2, groups=C)
    ref = ref.permute(0, 2, 3, 1).numpy()
    np.testing.assert_allclose(O.lce(V, w, b), ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O.lce(V, w), ref - b, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("B,H,W,C", LCE_SHAPES[:2])
def test_lce_equals_scipy_correlate(B, H, W, C):
    from scipy import ndimage

    V = _rand((B, H, W, C), 43)
    w = _rand((C, 5, 5), 44)
    out = O.lce(V, w)
    for bi in range(B):
        for c in range(C):
            ref = ndimage.correlate(V[bi, :, :, c], w[c], mode="constant", cval=0.0)
            np.testing.assert_allclose(out[bi, :, :, c], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("i,j", [(2, 2), (0, 0), (4, 1), (1, 3), (3, 4)])
def test_lce_single_tap_is_a_shift_with_zero_fill(i, j):
    B, H, W, C = 1, 5, 6, 2
    V = _rand((B, H, W, C), 45)
    w = np.zeros((C, 5, 5))
    w[:, i, j] = 1.0
    out = O.lce(V, w)
    for y in range(H):
        for x in range(W):
            yy, xx = y + i - 2, x + j - 2
            expect = V[0, yy, xx] if (0 <= yy < H and 0 <= xx < W) else np.zeros(C)
            np.testing.assert_array_equal(out[0, y, x], expect)


def test_lce_all_ones_counts_in_map_neighbours():
    B, H, W, C = 1, 7, 4, 3
    out = O.lce(np.ones((B, H, W, C)), np.ones((C, 5, 5)), np.full(C, 0.5))
    for y in range(H):
        for x in range(W):
            rows = min(y + 2, H - 1) - max(y - 2, 0) + 1
            cols = min(x + 2, W - 1) - max(x - 2, 0) + 1
            assert np.all(out[0, y, x] == rows * cols + 0.5)


def test_lce_is_added_to_the_attention_output():
    B, H, W, C, heads, S, k = 1, 8, 8, 8, 2, 4, 2
    Q, K, V = (_rand((B, H, W, C), s) for s in (46, 47, 48))
    w = _rand((C, 5, 5), 49)
    b = _rand((C,), 50)
    plain, routes = O.bra(Q, K, V, heads, S, k)
    full, routes2 = O.bra_lce(Q, K, V, heads, S, k, w, b)
    np.testing.assert_array_equal(routes, routes2)
    ref = torch.nn.functional.conv2d(torch.from_numpy(V).permute(0, 3, 1, 2), torch.from_numpy(w)[:, None],
                                     torch.from_numpy(b), padding=2, groups=C).permute(0, 2, 3, 1).numpy()
    np.testing.assert_allclose(full - plain, ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(O.attend_lce(Q, K, V, routes, heads, S, w, b), full, rtol=0, atol=0)
    with pytest.raises(ValueError):
        O.lce(V, w[:, :4])
    with pytest.raises(ValueError):
        O.lce(V, w, b[:3])


# --------------------------------------------------------------------------- #
# Backward with the routing held fixed
# --------------------------------------------------------------------------- #
def _fixed_route_loss_grads_fd(Q, K, V, routes, G, heads, S, h=1e-6):
    """Central finite differences of L = sum(attend(Q, K, V) * G) with the
    routing table fixed: uses only the forward oracle."""
    grads = []
    for which in range(3):
        X = [Q.copy(), K.copy(), V.copy()]
        g = np.zeros_like(X[which])
        for idx in np.ndindex(*X[which].shape):
            orig = X[which][idx]
            X[which][idx] = orig + h
            up = (O.attend(*X, routes, heads, S) * G).sum()
            X[which][idx] = orig - h
            dn = (O.attend(*X, routes, heads, S) * G).sum()
            X[which][idx] = orig
            g[idx] = (up - dn) / (2 * h)
        grads.append(g)
    return grads


@pytest.mark.parametrize("B,H,W,C,heads,S,k", [(1, 4, 4, 4, 2, 2, 2), (1, 4, 6, 2, 1, 2, 3)])
def test_backward_matches_finite_differences(B, H, W, C, heads, S, k):
    Q, K, V, G = (_rand((B, H, W, C), s) for s in (60, 61, 62, 63))
    routes = O.route(Q, K, S, k)
    fd = _fixed_route_loss_grads_fd(Q, K, V, routes, G, heads, S)
    an = O.attend_backward(Q, K, V, routes, G, heads, S)
    for name, a, f in zip("QKV", an, fd):
        np.testing.assert_allclose(a, f, rtol=1e-6, atol=1e-8, err_msg=f"d{name}")


def test_backward_full_routing_equals_sdpa_autograd():
    B, H, W, C, heads, S = 2, 4, 4, 8, 2, 2
    Q, K, V, G = (_rand((B, H, W, C), s) for s in (64, 65, 66, 67))
    routes = np.broadcast_to(np.arange(S * S, dtype=np.int32), (B, S * S, S * S)).copy()
    dQ, dK, dV = O.attend_backward(Q, K, V, routes, G, heads, S)
    ts = [torch.from_numpy(x).reshape(B, H * W, heads, C // heads).permute(0, 2, 1, 3).requires_grad_(True)
          for x in (Q, K, V)]
    out = torch.nn.functional.scaled_dot_product_attention(*ts)
    g = torch.from_numpy(G).reshape(B, H * W, heads, C // heads).permute(0, 2, 1, 3)
    (out * g).sum().backward()
    for a, t, name in zip((dQ, dK, dV), ts, "QKV"):
        ref = t.grad.permute(0, 2, 1, 3).reshape(B, H, W, C).numpy()
        np.testing.assert_allclose(a, ref, rtol=1e-10, atol=1e-12, err_msg=f"d{name}")


def test_backward_matches_autograd_through_a_torch_gather():
    """General routes (k < S^2, overlapping): torch autograd through
    advanced indexing + SDPA, per region, in fp64."""
    B, H, W, C, heads, S, k = 1, 6, 6, 4, 2, 3, 2
    Q, K, V, G = (_rand((B, H, W, C), s) for s in (68, 69, 70, 71))
    routes = O.route(Q, K, S, k)
    tq, tk, tv = (torch.from_numpy(x).clone().requires_grad_(True) for x in (Q, K, V))
    sh, sw = H // S, W // S
    loss = 0.0
    for i in range(S * S):
        ri, rj = divmod(i, S)
        qy, qx = np.meshgrid(np.arange(ri * sh, (ri + 1) * sh), np.arange(rj * sw, (rj + 1) * sw), indexing="ij")
        ys, xs = [], []
        for r in routes[0, i]:
            a, c = divmod(int(r), S)
            y, x = np.meshgrid(np.arange(a * sh, (a + 1) * sh), np.arange(c * sw, (c + 1) * sw), indexing="ij")
            ys.append(y.ravel())
            xs.append(x.ravel())
        gy, gx = torch.from_numpy(np.concatenate(ys)), torch.from_numpy(np.concatenate(xs))
        qy_t, qx_t = torch.from_numpy(qy.ravel()), torch.from_numpy(qx.ravel())
        d = C // heads
        q = tq[0, qy_t, qx_t].reshape(-1, heads, d).transpose(0, 1)
        kk = tk[0, gy, gx].reshape(-1, heads, d).transpose(0, 1)
        vv = tv[0, gy, gx].reshape(-1, heads, d).transpose(0, 1)
        o = torch.nn.functional.scaled_dot_product_attention(q, kk, vv).transpose(0, 1).reshape(-1, C)
        loss = loss + (o * torch.from_numpy(G[0, qy.ravel(), qx.ravel()])).sum()
    loss.backward()
    dQ, dK, dV = O.attend_backward(Q, K, V, routes, G, heads, S)
    for a, t, name in zip((dQ, dK, dV), (tq, tk, tv), "QKV"):
        np.testing.assert_allclose(a, t.grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=f"d{name}")


def test_backward_sum_rules():
    """Softmax rows sum to one: per image and head the key gradients sum to
    zero and the value gradients sum to the output gradients."""
    B, H, W, C, heads, S, k = 2, 8, 8, 8, 2, 4, 3
    Q, K, V, G = (_rand((B, H, W, C), s) for s in (72, 73, 74, 75))
    routes = O.route(Q, K, S, k)
    dQ, dK, dV = O.attend_backward(Q, K, V, routes, G, heads, S)
    np.testing.assert_allclose(dK.sum(axis=(1, 2)), 0.0, atol=1e-10)
    np.testing.assert_allclose(dV.sum(axis=(1, 2)), G.sum(axis=(1, 2)), rtol=1e-10, atol=1e-10)
    z = O.attend_backward(Q, K, V, routes, np.zeros_like(G), heads, S)
    assert all(np.all(x == 0) for x in z)


# --------------------------------------------------------------------------- #
# Linear projection (explainer Part 2.2 step 2, pseudocode step 2)
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("B,H,W,C", [(2, 4, 6, 8), (1, 3, 3, 16)])
def test_qkv_projection_equals_torch_linear(B, H, W, C):
    X = _rand((B, H, W, C), 90)
    Wq = _rand((3 * C, C), 91)
    bq = _rand((3 * C,), 92)
    ref = torch.nn.functional.linear(torch.from_numpy(X), torch.from_numpy(Wq), torch.from_numpy(bq)).numpy()
    Q, K, V = O.qkv_project(X, Wq, bq)
    np.testing.assert_allclose(np.concatenate([Q, K, V], axis=-1), ref, rtol=1e-12, atol=1e-12)


def test_qkv_identity_blocks_fix_the_chunk_order_and_bias():
    B, H, W, C = 1, 4, 4, 8
    X = _rand((B, H, W, C), 93)
    eye = np.eye(C)
    Q, K, V = O.qkv_project(X, np.concatenate([eye, 2 * eye, 3 * eye]))
    np.testing.assert_array_equal(Q, X)
    np.testing.assert_array_equal(K, 2 * X)
    np.testing.assert_array_equal(V, 3 * X)
    b = np.arange(3 * C, dtype=np.float64)
    Q, K, V = O.qkv_project(X, np.zeros((3 * C, C)), b)
    assert np.all(Q == b[:C]) and np.all(K == b[C:2 * C]) and np.all(V == b[2 * C:])
    with pytest.raises(ValueError):
        O.qkv_project(X, np.zeros((C, 3 * C)))


def test_bra_from_x_composes_projection_and_bra():
    B, H, W, C, heads, S, k = 1, 8, 8, 8, 2, 4, 2
    X = _rand((B, H, W, C), 94)
    Wq = _rand((3 * C, C), 95) / np.sqrt(C)
    out, routes, (Q, K, V) = O.bra_from_x(X, Wq, None, heads, S, k)
    ref, ref_routes = O.bra(X @ Wq[:C].T, X @ Wq[C:2 * C].T, X @ Wq[2 * C:].T, heads, S, k)
    np.testing.assert_array_equal(routes, ref_routes)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
