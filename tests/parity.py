"""Tolerances and comparisons shared by the GPU parity tests.

Score tolerance: |s_gpu - s_oracle| <= 2e-2 * max(1, |s_oracle|) (bf16 path
against the float64 oracle); GPU MIS against GPU independent scoring:
<= 1e-3 * max(1, |s|).  Top-10 order: a pair of candidates ordered differently
by the GPU and the oracle is a failure only when their oracle scores differ
by more than twice the request's largest measured score error (a closer pair
cannot be told apart at the measured precision); strict swaps are reported.
"""
import numpy as np

SCORE_TOL = 2e-2
MIS_VS_IND_TOL = 1e-3


def score_err(gpu, ref):
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    return float(np.max(np.abs(gpu - ref) / np.maximum(1.0, np.abs(ref))))


def top10_check(gpu, ref, k=10):
    """Returns (ok, n_strict_swaps)."""
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    k = min(k, gpu.shape[0])
    dmax = float(np.max(np.abs(gpu - ref)))
    cand = np.union1d(np.argsort(-gpu, kind="stable")[:k], np.argsort(-ref, kind="stable")[:k])
    strict = 0
    ok = True
    for i in cand:
        for j in cand:
            if i < j and (gpu[i] - gpu[j]) * (ref[i] - ref[j]) < 0:
                strict += 1
                if abs(ref[i] - ref[j]) > 2 * dmax:
                    ok = False
    same = np.array_equal(np.argsort(-gpu, kind="stable")[:k], np.argsort(-ref, kind="stable")[:k])
    return ok, (0 if same else max(strict, 1))
