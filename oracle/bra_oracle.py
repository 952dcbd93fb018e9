"""fp64 CPU oracle of Bi-Level Routing Attention (BRA), forward pass.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, never by the product path.

Sources (web pages about BiFormer, CVPR 2023, arXiv 2303.08810). Citations
below use these tags:

  [EXP]  "BiFormer Reshapes Visual Attention with 'Bi-Level Routing'"
         (explainer article). Part 2.2 "The Overall BRA Flow" gives the four
         steps and the PyTorch-style pseudocode (steps 1-7); Part 3
         "Complexity Analysis"; Part 6.3 "A Counter-Intuitive Discovery"
         (table of S, k and attended tokens).
  [SUM]  "BiFormer: Vision Transformer with Bi-Level Routing Attention"
         (section-by-section summary of the paper). Section 3 "Our Approach:
         BiFormer" (region partition and routing; token-to-token attention);
         Section 6 "Conclusion" (regional representations by averaging);
         Appendix C "Choices of top-k and partition factor S".

What is computed (the method's definition, not an approximation of it):

  1. The H x W map is cut into S x S non-overlapping regions of
     (H/S)*(W/S) tokens each; S must divide H and W, no padding
     ([EXP] 2.2 step 1 and pseudocode step 1; [EXP] Part 3 list of
     engineering constraints; [SUM] Appendix C).
  2. Region-level query and key = mean of Q and of K over each region's
     tokens ([EXP] 2.2 step 3, pseudocode step 3; [SUM] Section 3 and 6).
  3. Region affinity A = Q^r (K^r)^T over all C channels ([EXP] pseudocode
     step 4).
  4. Routing index I_r = the k largest entries of each row of A
     ([EXP] pseudocode step 5; [SUM] Section 3, row i holds the k most
     relevant regions of region i).
  5. Gather the keys/values of the routed regions and run ordinary softmax
     attention from each query of region i over the union of its routed
     regions' tokens ([EXP] 2.2 step 4, pseudocode steps 6-7; [SUM]
     Section 3 "Token-to-token attention").

Readings where the pages leave a step open (each is also listed in the
design notes of the repository):

  * softmax scale 1/sqrt(d), d = C/heads (standard multi-head attention);
    ``scale`` is a parameter so an unscaled variant is one argument away;
  * routing is shared by all heads and uses all C channels (the pseudocode
    pools the full-channel query/key and has no head axis);
  * head m owns channels [m*d, (m+1)*d);
  * region r = (h // (H/S)) * S + (w // (W/S)) (row-major over the region
    grid); tokens inside a region in row-major order;
  * ties in top-k: larger affinity first, lower region index first on
    exact ties (a stable sort of -A);
  * the local context enhancement term (+ dwconv(V), [EXP] pseudocode
    step 7) is a separate function, ``lce``, added by ``bra_lce`` /
    ``attend_lce``: the operator without it takes no convolution weights.
    Its readings: a 5 x 5 depthwise convolution of V over the whole H x W
    map (not per region), stride 1, zero padding 2 (output the size of the
    map), PyTorch's convolution convention (cross-correlation: tap (i, j)
    of channel c multiplies V[y + i - 2, x + j - 2, c]), one filter per
    channel and an optional per-channel bias.

Pins (tests/test_oracle_pins.py, all ``-m "not gpu"``):
  region_mean + affinity : equal to the mean of all n*n token-pair dot
                           products (brute.pairwise_region_affinity), the
                           identity stated in [SUM] Section 6;
  topk_route             : full brute sort, invariants, k = S^2 gives all;
  attend / bra           : k = S^2 and (S = 1, k = 1) equal dense global
                           attention (brute + torch SDPA in fp64); planted
                           routing equals window attention built by
                           reshaping (brute); K = 0 gives the mean of the
                           gathered V; V = 1 gives 1; permutation
                           invariance in the route order;
  attended_tokens        : the [EXP] Part 6.3 table (tests/golden);
  attend_backward        : central finite differences of ``attend``
                           itself (no gradient formula involved), torch
                           autograd through SDPA in fp64 when every region
                           is routed, and the sum rules sum(dK) = 0 and
                           sum(dV) = sum(dO) per image and head;
  qkv_project            : torch.nn.functional.linear in fp64, identity
                           weight blocks (Q = X, K = 2X, V = 3X) that fix
                           the chunk order, a bias-only projection;
  lce                    : torch conv2d with groups = C and scipy.ndimage
                           correlate (two library routines), single-tap
                           filters = shifted maps with zero fill (brute
                           loops), all-ones filter on a map of ones = the
                           closed-form count of in-map neighbours.
"""

from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------- #
# Shapes and the region partition
# --------------------------------------------------------------------------- #
def check_config(B: int, H: int, W: int, C: int, heads: int, S: int, topk: int) -> None:
    """Raise ValueError for shapes the method does not define.

    S must divide H and W (no padding: [EXP] Part 3 engineering constraints,
    [SUM] Appendix C); heads must divide C; 1 <= topk <= S*S.
    """
    for name, v in (("B", B), ("H", H), ("W", W), ("C", C), ("heads", heads), ("S", S)):
        if int(v) <= 0:
            raise ValueError(f"{name} must be positive, got {v}")
    if H % S or W % S:
        raise ValueError(f"S={S} must divide H={H} and W={W}")
    if C % heads:
        raise ValueError(f"heads={heads} must divide C={C}")
    if not 1 <= topk <= S * S:
        raise ValueError(f"topk={topk} must be in [1, S*S={S * S}]")


def region_size(H: int, W: int, S: int) -> tuple[int, int]:
    """Rows and columns of one region: (H/S, W/S) ([EXP] 2.2 step 1)."""
    return H // S, W // S


def region_token_coords(H: int, W: int, S: int, r: int) -> tuple[np.ndarray, np.ndarray]:
    """(ys, xs) of the tokens of region r, row-major inside the region.

    Region r sits at region-grid row r // S and column r % S; it covers rows
    [ (r//S)*sh, (r//S+1)*sh ) and columns [ (r%S)*sw, (r%S+1)*sw ).
    """
    sh, sw = region_size(H, W, S)
    ri, rj = divmod(int(r), S)
    ys = []
    xs = []
    for y in range(ri * sh, (ri + 1) * sh):
        for x in range(rj * sw, (rj + 1) * sw):
            ys.append(y)
            xs.append(x)
    return np.asarray(ys, dtype=np.int64), np.asarray(xs, dtype=np.int64)


def attended_tokens(H: int, W: int, S: int, k: int) -> int:
    """Keys each query attends to: k routed regions of HW/S^2 tokens each."""
    sh, sw = region_size(H, W, S)
    return int(k) * sh * sw


# --------------------------------------------------------------------------- #
# Level 1: region routing
# --------------------------------------------------------------------------- #
def region_mean(X: np.ndarray, S: int) -> np.ndarray:
    """Region-level descriptor: mean of X over each region's tokens.

    X: [B, H, W, C] float64. Returns [B, S*S, C] float64.
    ([EXP] 2.2 step 3 and pseudocode step 3; [SUM] Section 6.)
    """
    X = np.asarray(X, dtype=np.float64)
    B, H, W, C = X.shape
    R = S * S
    out = np.empty((B, R, C), dtype=np.float64)
    for r in range(R):
        ys, xs = region_token_coords(H, W, S, r)
        out[:, r, :] = X[:, ys, xs, :].mean(axis=1)
    return out


def affinity(Qr: np.ndarray, Kr: np.ndarray) -> np.ndarray:
    """Region-to-region affinity A[b, i, j] = Qr[b, i, :] . Kr[b, j, :].

    Rows index the query region, columns the key region ([EXP] pseudocode
    step 4). Returns [B, R, R] float64.
    """
    Qr = np.asarray(Qr, dtype=np.float64)
    Kr = np.asarray(Kr, dtype=np.float64)
    return np.matmul(Qr, np.swapaxes(Kr, -1, -2))


def topk_route(A: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest entries of each row of A.

    Order: descending affinity, lower index first on exact ties (stable sort
    of -A). ([EXP] pseudocode step 5; [SUM] Section 3.) Returns int32
    [B, R, k].
    """
    A = np.asarray(A, dtype=np.float64)
    order = np.argsort(-A, axis=-1, kind="stable")
    return order[..., : int(k)].astype(np.int32)


def route(Q: np.ndarray, K: np.ndarray, S: int, topk: int) -> np.ndarray:
    """Region routing: pool, affinity, top-k. Q, K: [B, H, W, C] float64."""
    B, H, W, C = np.shape(Q)
    check_config(B, H, W, C, 1, S, topk)
    Qr = region_mean(Q, S)
    Kr = region_mean(K, S)
    return topk_route(affinity(Qr, Kr), topk)


# --------------------------------------------------------------------------- #
# Level 2: token-to-token attention over the routed regions
# --------------------------------------------------------------------------- #
def gather_coords(H: int, W: int, S: int, routed_regions) -> tuple[np.ndarray, np.ndarray]:
    """(ys, xs) of the union of the routed regions' tokens, region by region
    in route order ([EXP] pseudocode step 6)."""
    ys = []
    xs = []
    for r in routed_regions:
        y, x = region_token_coords(H, W, S, int(r))
        ys.append(y)
        xs.append(x)
    return np.concatenate(ys), np.concatenate(xs)


def softmax_attention(q: np.ndarray, kg: np.ndarray, vg: np.ndarray, scale: float) -> np.ndarray:
    """Naive softmax attention of queries q [n, d] over keys kg [m, d] and
    values vg [m, dv]: softmax(q kg^T * scale) vg, rows normalised
    explicitly; asserts every probability row sums to 1."""
    logits = (q @ kg.T) * scale
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = e / e.sum(axis=1, keepdims=True)
    assert np.all(np.abs(p.sum(axis=1) - 1.0) <= 1e-12), "softmax rows must sum to 1"
    return p @ vg


def attend(Q, K, V, routes, heads: int, S: int, scale: float | None = None) -> np.ndarray:
    """Token attention given a routing table.

    Q, K, V: [B, H, W, C] float64; routes: int [B, S*S, k]. For every image
    b, query region i and head m, the queries of region i attend, with
    ordinary softmax attention, to the tokens of the regions routes[b, i, :]
    ([EXP] 2.2 step 4 and pseudocode steps 6-7; [SUM] Section 3). Head m
    uses channels [m*d, (m+1)*d). Default scale 1/sqrt(d).
    Returns [B, H, W, C] float64.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    routes = np.asarray(routes)
    B, H, W, C = Q.shape
    R = S * S
    k = routes.shape[-1]
    check_config(B, H, W, C, heads, S, k)
    if routes.shape != (B, R, k):
        raise ValueError(f"routes must be [B, S*S, k] = {(B, R, k)}, got {routes.shape}")
    if routes.min() < 0 or routes.max() >= R:
        raise ValueError("route indices out of range")
    d = C // heads
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    O = np.zeros_like(Q)
    for b in range(B):
        for i in range(R):
            qy, qx = region_token_coords(H, W, S, i)
            gy, gx = gather_coords(H, W, S, routes[b, i])
            for m in range(heads):
                ch = slice(m * d, (m + 1) * d)
                q = Q[b, qy, qx, ch]
                kg = K[b, gy, gx, ch]
                vg = V[b, gy, gx, ch]
                O[b, qy, qx, ch] = softmax_attention(q, kg, vg, scale)
    return O


def bra(Q, K, V, heads: int, S: int, topk: int, scale: float | None = None):
    """Full BRA forward (without the local-context term): returns (O, routes)."""
    routes = route(Q, K, S, topk)
    return attend(Q, K, V, routes, heads, S, scale), routes


# --------------------------------------------------------------------------- #
# Local context enhancement: the "+ dwconv(value)" term
# --------------------------------------------------------------------------- #
LCE_SIZE = 5


def lce(V, weight, bias=None) -> np.ndarray:
    """Local context enhancement: a 5 x 5 depthwise convolution of V.

    [EXP] 2.2 step 4 (the local enhancement term, a 5 x 5 depthwise
    convolution) and pseudocode step 7 (``+ dwconv(value)``); [SUM] Section 3
    (token-to-token attention plus a depthwise-convolution local context
    term). Written out:

        out[b, y, x, c] = bias[c] + sum_{i, j in 0..4} weight[c, i, j]
                                    * V[b, y + i - 2, x + j - 2, c]

    where terms whose position falls outside the H x W map are omitted (zero
    padding). V: [B, H, W, C]; weight: [C, 5, 5]; bias: [C] or None.
    Returns [B, H, W, C] float64.
    """
    V = np.asarray(V, dtype=np.float64)
    weight = np.asarray(weight, dtype=np.float64)
    B, H, W, C = V.shape
    if weight.shape != (C, LCE_SIZE, LCE_SIZE):
        raise ValueError(f"weight must be [C, 5, 5] = {(C, LCE_SIZE, LCE_SIZE)}, got {weight.shape}")
    out = np.zeros_like(V)
    if bias is not None:
        bias = np.asarray(bias, dtype=np.float64)
        if bias.shape != (C,):
            raise ValueError(f"bias must be [C] = {(C,)}, got {bias.shape}")
        out += bias
    half = LCE_SIZE // 2
    for i in range(LCE_SIZE):
        dy = i - half
        y0, y1 = max(0, -dy), min(H, H - dy)  # rows y with 0 <= y + dy < H
        for j in range(LCE_SIZE):
            dx = j - half
            x0, x1 = max(0, -dx), min(W, W - dx)
            if y0 >= y1 or x0 >= x1:
                continue
            out[:, y0:y1, x0:x1, :] += weight[:, i, j] * V[:, y0 + dy:y1 + dy, x0 + dx:x1 + dx, :]
    return out


def attend_lce(Q, K, V, routes, heads: int, S: int, weight, bias=None, scale: float | None = None) -> np.ndarray:
    """Token attention over a given routing table plus the local context
    term: the module output of [EXP] pseudocode step 7."""
    return attend(Q, K, V, routes, heads, S, scale) + lce(V, weight, bias)


def bra_lce(Q, K, V, heads: int, S: int, topk: int, weight, bias=None, scale: float | None = None):
    """Full BRA forward with the local context term: returns (O, routes)."""
    O, routes = bra(Q, K, V, heads, S, topk, scale)
    return O + lce(V, weight, bias), routes


# --------------------------------------------------------------------------- #
# Backward of the token attention with the routing held fixed
# --------------------------------------------------------------------------- #
def softmax_attention_backward(q: np.ndarray, kg: np.ndarray, vg: np.ndarray, do: np.ndarray, scale: float):
    """Gradients of O = softmax(q kg^T * scale) vg for one (image, region,
    head), given dL/dO = do. Written out from the chain rule:

        P    = softmax(Z),  Z = scale * q kg^T          (rows normalised)
        dvg  = P^T do
        dP   = do vg^T
        dZ   = P * (dP - rowsum(P * dP))                (softmax Jacobian)
        dq   = scale * dZ kg
        dkg  = scale * dZ^T q

    Returns (dq [n, d], dkg [m, d], dvg [m, dv]).
    """
    z = (q @ kg.T) * scale
    e = np.exp(z - z.max(axis=1, keepdims=True))
    p = e / e.sum(axis=1, keepdims=True)
    dvg = p.T @ do
    dp = do @ vg.T
    dz = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = scale * (dz @ kg)
    dkg = scale * (dz.T @ q)
    return dq, dkg, dvg


def attend_backward(Q, K, V, routes, dO, heads: int, S: int, scale: float | None = None):
    """Gradients of ``attend`` with respect to Q, K and V, the routing table
    held fixed (top-k indices carry no gradient, so the region pooling gets
    none either). A key/value token routed to by several query regions
    accumulates the gradient of every one of them. Returns (dQ, dK, dV),
    each [B, H, W, C] float64."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    routes = np.asarray(routes)
    B, H, W, C = Q.shape
    R = S * S
    k = routes.shape[-1]
    check_config(B, H, W, C, heads, S, k)
    if routes.shape != (B, R, k):
        raise ValueError(f"routes must be [B, S*S, k] = {(B, R, k)}, got {routes.shape}")
    if routes.min() < 0 or routes.max() >= R:
        raise ValueError("route indices out of range")
    d = C // heads
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    for b in range(B):
        for i in range(R):
            qy, qx = region_token_coords(H, W, S, i)
            gy, gx = gather_coords(H, W, S, routes[b, i])
            for m in range(heads):
                ch = slice(m * d, (m + 1) * d)
                dq, dkg, dvg = softmax_attention_backward(Q[b, qy, qx, ch], K[b, gy, gx, ch], V[b, gy, gx, ch],
                                                          dO[b, qy, qx, ch], scale)
                dQ[b, qy, qx, ch] = dq
                # the routed regions are distinct, so (gy, gx) has no repeats
                # inside one row and += adds each token once
                dK[b, gy, gx, ch] += dkg
                dV[b, gy, gx, ch] += dvg
    return dQ, dK, dV


# --------------------------------------------------------------------------- #
# The linear projection in front of the routing
# --------------------------------------------------------------------------- #
def qkv_project(X, Wqkv, bqkv=None):
    """Q, K, V = linear_qkv(X).chunk(3, dim=-1).

    [EXP] 2.2 step 2 (Q, K, V from linear projections) and pseudocode step 2;
    [EXP] Part 3 counts it as the 3HWC^2 projection term. X: [B, H, W, C];
    Wqkv: [3C, C], rows are output features (a torch Linear weight), so the
    projection is X Wqkv^T; bqkv: [3C] or None. The output features are Q's
    C channels, then K's, then V's. Returns (Q, K, V), each [B, H, W, C]
    float64.
    """
    X = np.asarray(X, dtype=np.float64)
    Wqkv = np.asarray(Wqkv, dtype=np.float64)
    C = X.shape[-1]
    if Wqkv.shape != (3 * C, C):
        raise ValueError(f"Wqkv must be [3C, C] = {(3 * C, C)}, got {Wqkv.shape}")
    Y = np.matmul(X, Wqkv.T)
    if bqkv is not None:
        bqkv = np.asarray(bqkv, dtype=np.float64)
        if bqkv.shape != (3 * C,):
            raise ValueError(f"bqkv must be [3C] = {(3 * C,)}, got {bqkv.shape}")
        Y = Y + bqkv
    return Y[..., :C], Y[..., C:2 * C], Y[..., 2 * C:]


def bra_from_x(X, Wqkv, bqkv, heads: int, S: int, topk: int, scale: float | None = None):
    """Projection, routing and attention from the block input X: returns
    (O, routes, (Q, K, V))."""
    Q, K, V = qkv_project(X, Wqkv, bqkv)
    O, routes = bra(Q, K, V, heads, S, topk, scale)
    return O, routes, (Q, K, V)
