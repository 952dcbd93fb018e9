"""Comparison helpers for the GPU parity tests (acceptance criteria in code).

Routing: the GPU table must match the oracle's exactly, except where the
k-th and (k+1)-th affinities of a row differ by less than 1e-5 relative. With
tau the oracle's k-th largest affinity of the row and
eps_j = 1e-5 * max(|a_j|, |tau|), every routed j must have a_j >= tau - eps_j,
every other j must have a_j <= tau + eps_j, the k entries must be distinct
and in range, and consecutive entries must not increase by more than eps.

Outputs: fp32 max-abs <= 1e-4; bf16 max-abs <= 2e-2 and
mean-rel = sum|O - O_ref| / sum|O_ref| <= 5e-3, against the fp64 oracle run
on the exact (upcast) inputs and the GPU's own routing table.

With the local context term the output is no longer bounded by the values'
range, so the bf16 elementwise bound adds the output roundings: at most two
(the unfused path rounds the attention output, then the sum), each within
2^-8 of the value: |O - O_ref| <= 2e-2 + 2 * 2^-8 * |O_ref|. The mean-rel
bound and the fp32 bound stay as above.
"""

from __future__ import annotations

import numpy as np

TIE_REL = 1e-5
F32_MAX_ABS = 1e-4
BF16_MAX_ABS = 2e-2
BF16_MEAN_REL = 5e-3


def route_violations(A: np.ndarray, idx: np.ndarray, k: int):
    """List of (b, i, reason) where the GPU table idx [B, R, k] breaks the
    tie-band rule against the oracle affinity A [B, R, R] (float64)."""
    bad = []
    B, R, _ = A.shape
    srt = -np.sort(-A, axis=-1)
    for b in range(B):
        for i in range(R):
            row = A[b, i]
            sel = idx[b, i].astype(np.int64)
            if sel.min() < 0 or sel.max() >= R:
                bad.append((b, i, "index out of range"))
                continue
            if len(set(sel.tolist())) != k:
                bad.append((b, i, "duplicate index"))
                continue
            tau = srt[b, i, k - 1]
            eps = TIE_REL * np.maximum(np.abs(row), abs(tau))
            mask = np.zeros(R, dtype=bool)
            mask[sel] = True
            if np.any(row[mask] < tau - eps[mask]):
                bad.append((b, i, "routed region below the k-th affinity"))
            if np.any(row[~mask] > tau + eps[~mask]):
                bad.append((b, i, "unrouted region above the k-th affinity"))
            vals = row[sel]
            if np.any(vals[1:] > vals[:-1] + TIE_REL * np.maximum(np.abs(vals[1:]), np.abs(vals[:-1]))):
                bad.append((b, i, "not in descending affinity order"))
    return bad


def exact_route_mismatches(oracle_idx: np.ndarray, idx: np.ndarray) -> int:
    """Rows whose index list differs from the oracle's canonical one."""
    return int(np.any(oracle_idx != idx, axis=-1).sum())


def output_errors(out: np.ndarray, ref: np.ndarray):
    diff = np.abs(out - ref)
    max_abs = float(diff.max()) if diff.size else 0.0
    denom = float(np.abs(ref).sum())
    mean_rel = float(diff.sum() / denom) if denom > 0 else 0.0
    return max_abs, mean_rel


def assert_output_close(out: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    assert np.all(np.isfinite(out)), f"{what}: non-finite outputs"
    max_abs, mean_rel = output_errors(out, ref)
    if dtype == "f32":
        assert max_abs <= F32_MAX_ABS, f"{what}: fp32 max-abs {max_abs:.3e} > {F32_MAX_ABS}"
    else:
        assert max_abs <= BF16_MAX_ABS, f"{what}: bf16 max-abs {max_abs:.3e} > {BF16_MAX_ABS}"
        assert mean_rel <= BF16_MEAN_REL, f"{what}: bf16 mean-rel {mean_rel:.3e} > {BF16_MEAN_REL}"
    return max_abs, mean_rel


BF16_UNIT_ROUNDOFF = 2.0 ** -8


def assert_lce_output_close(out: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    """Parity bound for outputs that include the local context term."""
    assert np.all(np.isfinite(out)), f"{what}: non-finite outputs"
    max_abs, mean_rel = output_errors(out, ref)
    if dtype == "f32":
        assert max_abs <= F32_MAX_ABS, f"{what}: fp32 max-abs {max_abs:.3e} > {F32_MAX_ABS}"
    else:
        bound = BF16_MAX_ABS + 2 * BF16_UNIT_ROUNDOFF * np.abs(ref)
        excess = np.abs(out - ref) - bound
        worst = float(excess.max()) if excess.size else 0.0
        assert worst <= 0, f"{what}: bf16 error exceeds 2e-2 + 2^-7 |ref| by {worst:.3e} (max-abs {max_abs:.3e})"
        assert mean_rel <= BF16_MEAN_REL, f"{what}: bf16 mean-rel {mean_rel:.3e} > {BF16_MEAN_REL}"
    return max_abs, mean_rel


GRAD_F32_REL = 1e-4
GRAD_BF16_REL = 2e-2
GRAD_BF16_MEAN_REL = 5e-3


def assert_grad_close(out: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    """Parity bound for gradients. Their size depends on the data, so the
    elementwise bound scales with the tensor's largest reference value: fp32
    1e-4 * max(1, max|ref|); bf16 2e-2 * max(1, max|ref|) (bf16 rounding of
    the probabilities and of dZ inside the products, 2^-8 relative each, and
    of the stored gradient) plus mean-rel <= 5e-3, the forward's bar (the
    measured bf16 mean-rel is 2.1e-3 to 3.4e-3 over every tested shape)."""
    assert np.all(np.isfinite(out)), f"{what}: non-finite gradients"
    max_abs, mean_rel = output_errors(out, ref)
    scale = max(1.0, float(np.abs(ref).max()) if ref.size else 1.0)
    if dtype == "f32":
        assert max_abs <= GRAD_F32_REL * scale, f"{what}: fp32 max-abs {max_abs:.3e} > {GRAD_F32_REL} * {scale:.2f}"
    else:
        assert max_abs <= GRAD_BF16_REL * scale, f"{what}: bf16 max-abs {max_abs:.3e} > {GRAD_BF16_REL} * {scale:.2f}"
        assert mean_rel <= GRAD_BF16_MEAN_REL, f"{what}: bf16 mean-rel {mean_rel:.3e} > {GRAD_BF16_MEAN_REL}"
    return max_abs, mean_rel


PROJ_F32_REL = 1e-4
PROJ_BF16_ABS = 1e-3


def assert_proj_close(out: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    """Parity bound for the projection outputs: one rounding of an fp32 sum of
    exact products. fp32: max-abs <= 1e-4 * max(1, max|ref|); bf16:
    |out - ref| <= 2^-8 |ref| + 1e-3 elementwise (the rounding, plus room for
    the fp32 accumulation)."""
    assert np.all(np.isfinite(out)), f"{what}: non-finite outputs"
    max_abs, mean_rel = output_errors(out, ref)
    if dtype == "f32":
        scale = max(1.0, float(np.abs(ref).max()) if ref.size else 1.0)
        assert max_abs <= PROJ_F32_REL * scale, f"{what}: fp32 max-abs {max_abs:.3e}"
    else:
        excess = np.abs(out - ref) - (BF16_UNIT_ROUNDOFF * np.abs(ref) + PROJ_BF16_ABS)
        assert float(excess.max()) <= 0, f"{what}: bf16 error exceeds 2^-8 |ref| + 1e-3 by {float(excess.max()):.3e}"
    return max_abs, mean_rel
