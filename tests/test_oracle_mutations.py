"""Plant plausible mistakes in the oracle (on the CPU) and check the pins catch them.

Each mutation replaces one oracle function with a subtly wrong variant; at
least one pin in ``test_oracle_pins`` must then fail. This guards the pins
themselves: a pin set that a transposed operand or a wrong index slips
through is not a pin.
"""

import inspect

import numpy as np
import pytest

from oracle import bra_oracle as O
import tests.test_oracle_pins as pins

_orig_affinity = O.affinity
_orig_softmax = O.softmax_attention
_orig_mean = O.region_mean
_orig_attend = O.attend
_orig_lce = O.lce
_orig_sab = O.softmax_attention_backward
_orig_qkv = O.qkv_project


def _transposed_affinity(Qr, Kr):
    return _orig_affinity(Kr, Qr)


def _ties_higher_index_first(A, k):
    return np.argsort(A, axis=-1, kind="stable")[..., ::-1][..., : int(k)].astype(np.int32)


def _column_major_regions(H, W, S, r):
    sh, sw = H // S, W // S
    rj, ri = divmod(int(r), S)
    ys, xs = np.meshgrid(np.arange(ri * sh, (ri + 1) * sh), np.arange(rj * sw, (rj + 1) * sw), indexing="ij")
    return ys.reshape(-1), xs.reshape(-1)


def _swapped_region_extent(H, W, S, r):
    sw, sh = H // S, W // S  # rows/cols of a region swapped
    ri, rj = divmod(int(r), S)
    ys, xs = np.meshgrid(np.arange(ri * sh, (ri + 1) * sh), np.arange(rj * sw, (rj + 1) * sw), indexing="ij")
    ys, xs = ys.reshape(-1), xs.reshape(-1)
    return np.minimum(ys, H - 1), np.minimum(xs, W - 1)


def _no_scale(q, kg, vg, scale):
    return _orig_softmax(q, kg, vg, 1.0)


def _softmax_over_queries(q, kg, vg, scale):
    s = (q @ kg.T) * scale
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return (e / e.sum(axis=0, keepdims=True)) @ vg


def _dropped_max_term_key(q, kg, vg, scale):
    # drops the last gathered key (an off-by-one in the gather length)
    return _orig_softmax(q, kg[:-1], vg[:-1], scale)


def _sum_not_mean(X, S):
    B, H, W, C = np.shape(X)
    return _orig_mean(X, S) * ((H // S) * (W // S))


def _interleaved_heads(Q, K, V, routes, heads, S, scale=None):
    Q = np.asarray(Q)
    C = Q.shape[-1]
    d = C // heads
    perm = np.arange(C).reshape(d, heads).T.reshape(-1)
    inv = np.argsort(perm)
    return _orig_attend(Q[..., perm], np.asarray(K)[..., perm], np.asarray(V)[..., perm], routes, heads, S, scale)[..., inv]


def _convolution_not_correlation(V, weight, bias=None):
    return _orig_lce(V, np.asarray(weight)[:, ::-1, ::-1], bias)


def _transposed_filter(V, weight, bias=None):
    return _orig_lce(V, np.swapaxes(np.asarray(weight), 1, 2), bias)


def _circular_padding(V, weight, bias=None):
    V = np.asarray(V, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    out = np.zeros_like(V) + (0.0 if bias is None else np.asarray(bias, dtype=np.float64))
    for i in range(5):
        for j in range(5):
            out += w[:, i, j] * np.roll(V, (2 - i, 2 - j), axis=(1, 2))
    return out


def _dropped_bias(V, weight, bias=None):
    return _orig_lce(V, weight, None)


def _off_by_one_padding(V, weight, bias=None):
    V = np.asarray(V, dtype=np.float64)
    Vp = np.pad(V, ((0, 0), (1, 3), (1, 3), (0, 0)))  # pads 1 before instead of 2
    w = np.asarray(weight, dtype=np.float64)
    B, H, W, C = V.shape
    out = np.zeros_like(V) + (0.0 if bias is None else np.asarray(bias, dtype=np.float64))
    for i in range(5):
        for j in range(5):
            out += w[:, i, j] * Vp[:, i:i + H, j:j + W, :]
    return out


def _bwd_no_rowsum_term(q, kg, vg, do, scale):
    z = (q @ kg.T) * scale
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    dz = p * (do @ vg.T)
    return scale * (dz @ kg), scale * (dz.T @ q), p.T @ do


def _bwd_unscaled_dq(q, kg, vg, do, scale):
    dq, dk, dv = _orig_sab(q, kg, vg, do, scale)
    return dq / scale, dk, dv


def _bwd_value_grad_from_logits(q, kg, vg, do, scale):
    dq, dk, dv = _orig_sab(q, kg, vg, do, scale)
    z = (q @ kg.T) * scale
    return dq, dk, np.exp(z - z.max()).T @ do  # unnormalised probabilities


def _bwd_scatter_overwrites(Q, K, V, routes, dO, heads, S, scale=None):
    # last query region wins instead of accumulating
    Q = np.asarray(Q, dtype=np.float64)
    B, H, W, C = Q.shape
    d = C // heads
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    dQ, dK, dV = (np.zeros_like(Q) for _ in range(3))
    for b in range(B):
        for i in range(S * S):
            qy, qx = O.region_token_coords(H, W, S, i)
            gy, gx = O.gather_coords(H, W, S, routes[b, i])
            for m in range(heads):
                ch = slice(m * d, (m + 1) * d)
                dq, dk, dv = _orig_sab(Q[b, qy, qx, ch], np.asarray(K)[b, gy, gx, ch], np.asarray(V)[b, gy, gx, ch],
                                       np.asarray(dO)[b, qy, qx, ch], scale)
                dQ[b, qy, qx, ch] = dq
                dK[b, gy, gx, ch] = dk
                dV[b, gy, gx, ch] = dv
    return dQ, dK, dV


def _qkv_chunk_order_kqv(X, Wqkv, bqkv=None):
    q, k, v = _orig_qkv(X, Wqkv, bqkv)
    return k, q, v


def _qkv_weight_read_column_major(X, Wqkv, bqkv=None):
    W = np.asarray(Wqkv)
    return _orig_qkv(X, W.reshape(W.shape[1], W.shape[0]).T, bqkv)


def _qkv_dropped_bias(X, Wqkv, bqkv=None):
    return _orig_qkv(X, Wqkv, None)


MUTATIONS = {
    "qkv_chunk_order": ("qkv_project", _qkv_chunk_order_kqv),
    "qkv_weight_column_major": ("qkv_project", _qkv_weight_read_column_major),
    "qkv_dropped_bias": ("qkv_project", _qkv_dropped_bias),
    "bwd_no_rowsum_term": ("softmax_attention_backward", _bwd_no_rowsum_term),
    "bwd_unscaled_dq": ("softmax_attention_backward", _bwd_unscaled_dq),
    "bwd_value_grad_unnormalised": ("softmax_attention_backward", _bwd_value_grad_from_logits),
    "bwd_scatter_overwrites": ("attend_backward", _bwd_scatter_overwrites),
    "lce_convolution_not_correlation": ("lce", _convolution_not_correlation),
    "lce_transposed_filter": ("lce", _transposed_filter),
    "lce_circular_padding": ("lce", _circular_padding),
    "lce_dropped_bias": ("lce", _dropped_bias),
    "lce_off_by_one_padding": ("lce", _off_by_one_padding),
    "transposed_affinity": ("affinity", _transposed_affinity),
    "ties_higher_index_first": ("topk_route", _ties_higher_index_first),
    "column_major_regions": ("region_token_coords", _column_major_regions),
    "swapped_region_extent": ("region_token_coords", _swapped_region_extent),
    "no_softmax_scale": ("softmax_attention", _no_scale),
    "softmax_over_queries": ("softmax_attention", _softmax_over_queries),
    "dropped_gathered_key": ("softmax_attention", _dropped_max_term_key),
    "pool_sum_not_mean": ("region_mean", _sum_not_mean),
    "interleaved_head_channels": ("attend", _interleaved_heads),
}


def _pin_cases():
    """Every pin test with one representative parameter set."""
    cases = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if not params:
            cases.append((fn, {}))
            continue
        argnames, values = params[0].args[0], params[0].args[1]
        names = [a.strip() for a in argnames.split(",")]
        for v in values:
            v = v if isinstance(v, tuple) else (v,)
            cases.append((fn, dict(zip(names, v))))
    return cases


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(mutation, monkeypatch):
    attr, fn = MUTATIONS[mutation]
    monkeypatch.setattr(O, attr, fn)
    failures = 0
    for case, kwargs in _pin_cases():
        try:
            case(**kwargs)
        except (AssertionError, ValueError, IndexError):
            failures += 1
    assert failures > 0, f"no pin caught mutation {mutation}"
