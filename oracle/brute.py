"""Brute-force formulations that pin ``bra_oracle`` (test infrastructure only).

Each function here computes a quantity that the method must reproduce in a
special case, written differently from ``bra_oracle`` (reshapes instead of
coordinate lists, pairwise sums instead of means) so that one misreading is
unlikely to sit in both. Small inputs only.

  pairwise_region_affinity : the mean over all token pairs (a in region i,
      b in region j) of q_a . k_b. By bilinearity this equals the dot
      product of the region means, the identity the BiFormer paper summary
      ("BiFormer: Vision Transformer with Bi-Level Routing Attention",
      Section 6 "Conclusion", regional representations) states.
  global_attention : dense multi-head softmax attention over all H*W tokens,
      what BRA reduces to when every region is routed (k = S^2) or when the
      whole map is one region (S = 1, k = 1).
  window_attention_over : attention where region i's queries see exactly a
      given list of regions, with the regions cut out by reshaping the map
      into [S, H/S, S, W/S]; with each region routed to itself only this is
      non-overlapping window attention.
"""

from __future__ import annotations

import numpy as np


def _windows(X: np.ndarray, S: int) -> np.ndarray:
    """[B, H, W, C] -> [B, S*S, (H/S)*(W/S), C], regions row-major over the
    region grid, tokens row-major inside a region, by reshape/transpose."""
    B, H, W, C = X.shape
    sh, sw = H // S, W // S
    t = X.reshape(B, S, sh, S, sw, C).transpose(0, 1, 3, 2, 4, 5)
    return t.reshape(B, S * S, sh * sw, C)


def _unwindows(Xw: np.ndarray, H: int, W: int, S: int) -> np.ndarray:
    B, R, n, C = Xw.shape
    sh, sw = H // S, W // S
    t = Xw.reshape(B, S, S, sh, sw, C).transpose(0, 1, 3, 2, 4, 5)
    return t.reshape(B, H, W, C)


def pairwise_region_affinity(Q: np.ndarray, K: np.ndarray, S: int) -> np.ndarray:
    """A[b, i, j] = (1/n^2) * sum over token pairs (a in i, c in j) of q_a . k_c,
    summed pair by pair with explicit loops over regions (tiny inputs)."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    Qw = _windows(Q, S)
    Kw = _windows(K, S)
    B, R, n, C = Qw.shape
    A = np.zeros((B, R, R))
    for b in range(B):
        for i in range(R):
            for j in range(R):
                total = 0.0
                for a in range(n):
                    for c in range(n):
                        total += float(np.dot(Qw[b, i, a], Kw[b, j, c]))
                A[b, i, j] = total / (n * n)
    return A


def global_attention(Q, K, V, heads: int, scale: float | None = None) -> np.ndarray:
    """Dense multi-head attention over all tokens of each image, fp64."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, H, W, C = Q.shape
    d = C // heads
    if scale is None:
        scale = d ** -0.5
    q = Q.reshape(B, H * W, heads, d).transpose(0, 2, 1, 3)
    k = K.reshape(B, H * W, heads, d).transpose(0, 2, 1, 3)
    v = V.reshape(B, H * W, heads, d).transpose(0, 2, 1, 3)
    s = np.einsum("bhqd,bhkd->bhqk", q, k) * scale
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    o = np.einsum("bhqk,bhkd->bhqd", p, v)
    return o.transpose(0, 2, 1, 3).reshape(B, H, W, C)


def window_attention_over(Q, K, V, heads: int, S: int, routes, scale: float | None = None) -> np.ndarray:
    """Region i's queries attend to the concatenated windows routes[b, i, :],
    with windows cut by reshaping. routes: [B, S*S, k] int."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, H, W, C = Q.shape
    d = C // heads
    if scale is None:
        scale = d ** -0.5
    Qw, Kw, Vw = _windows(Q, S), _windows(K, S), _windows(V, S)
    R, n = Qw.shape[1], Qw.shape[2]
    out = np.zeros_like(Qw)
    for b in range(B):
        for i in range(R):
            kk = np.concatenate([Kw[b, r] for r in routes[b][i]], axis=0)
            vv = np.concatenate([Vw[b, r] for r in routes[b][i]], axis=0)
            for m in range(heads):
                c0, c1 = m * d, (m + 1) * d
                s = Qw[b, i, :, c0:c1] @ kk[:, c0:c1].T * scale
                w = np.exp(s - s.max(axis=1, keepdims=True))
                w /= w.sum(axis=1, keepdims=True)
                out[b, i, :, c0:c1] = w @ vv[:, c0:c1]
    return _unwindows(out, H, W, S)


def window_mean(V, S: int, regions) -> np.ndarray:
    """Mean of V over the tokens of the listed regions, per image: [B, C]."""
    Vw = _windows(np.asarray(V, dtype=np.float64), S)
    return Vw[:, list(regions)].reshape(Vw.shape[0], -1, Vw.shape[-1]).mean(axis=1)
