"""Shared checks of GPU results against the CPU oracle.

Parity rules:
  C1  ids are bit-exact against the oracle's selection run on the GPU's own fp32
      scores (same precision on both sides), including order and -1 padding;
  C2  every valid score is within rtol * A of the float64 score, A = sum |q c|
      (the dot-product rounding-error scale); masked scores are exactly -inf;
  C3  against the oracle's float64 scores, the selected sets may differ only on
      ids whose score lies within the tolerance band of the K-th score.
rtol is 1e-5 for fp32 inputs and 2e-3 for bf16 inputs (fp32 accumulation).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

RTOL = {"f32": 1e-5, "bf16": 2e-3}
NEG_INF_BITS = np.uint32(0xFF800000)


def to_dev(a: np.ndarray, dev="cuda:0"):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def check_scores(s_gpu: np.ndarray, S: np.ndarray, A: np.ndarray, rtol: float):
    valid = S != -np.inf
    bits = s_gpu.view(np.uint32)
    assert np.all(bits[~valid] == NEG_INF_BITS), "masked scores must be exactly -inf"
    assert np.isfinite(s_gpu[valid]).all()
    err = np.abs(s_gpu[valid].astype(np.float64) - S[valid])
    tol = rtol * A[valid]
    bad = np.nonzero(err > tol)[0]
    assert bad.size == 0, f"{bad.size} scores out of tolerance; worst err/A = {(err / np.maximum(A[valid], 1e-300)).max():.3e}"
    return float((err / np.maximum(A[valid], 1e-300)).max()) if err.size else 0.0


def check_ids_exact(ids_gpu, counts_gpu, scores_gpu, nv, K, sorted_out):
    ids_ref, counts_ref = oracle.select(scores_gpu, nv, K, sorted_out)
    if counts_gpu is not None:
        np.testing.assert_array_equal(counts_gpu, counts_ref)
    for b in range(ids_ref.shape[0]):
        if not np.array_equal(ids_gpu[b], ids_ref[b]):
            d = np.nonzero(ids_gpu[b] != ids_ref[b])[0]
            raise AssertionError(f"row {b}: {d.size} id slots differ, first at {d[0]}: "
                                 f"gpu {ids_gpu[b, d[0]]} oracle {ids_ref[b, d[0]]}")


def check_ids_band(ids_gpu, S, A, nv, K, rtol):
    """C3: selection from float64 scores may differ only inside the K-th score's band."""
    ids_ref, counts_ref = oracle.select(S, nv, K, False)
    for b in range(S.shape[0]):
        m = counts_ref[b]
        g = set(int(i) for i in ids_gpu[b] if i >= 0)
        r = set(int(i) for i in ids_ref[b, :m])
        assert len(g) == m
        diff = g ^ r
        if not diff:
            continue
        kstar = int(ids_ref[b, :m][np.argmin(S[b, ids_ref[b, :m]])])
        for i in diff:
            assert abs(S[b, i] - S[b, kstar]) <= rtol * (A[b, i] + A[b, kstar]), (b, i, kstar)


def check_assign(a, best, xb, cb, rows=None, rtol=RTOL["bf16"]):
    """k-means assignment on the given rows: the GPU's winning value is half the
    score of the centroid it chose (C2), and a winner other than the oracle's is
    allowed only inside the tolerance band of the best score (C3). Returns the
    number of rows whose winner differs."""
    rows = np.arange(xb.shape[0]) if rows is None else rows
    a_ref, S, A = oracle.assign(xb[rows], cb)
    ag = a[rows]
    i = np.arange(rows.size)
    if best is not None:
        np.testing.assert_array_less(np.abs(2.0 * best[rows] - S[i, ag]),
                                     rtol * A[i, ag] + 1e-30)
    off = np.nonzero(ag != a_ref)[0]
    for k in off:
        assert S[k, a_ref[k]] - S[k, ag[k]] <= rtol * (A[k, a_ref[k]] + A[k, ag[k]]), k
    return off.size
