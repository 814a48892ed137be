"""Acceptance rule for GPU outputs against the fp64 oracle.

For each checked point i, with the oracle's best score b_i, runner-up r_i and
threshold t_i = 1e-3 * (|b_i| + 1):

* strict point (r_i - b_i >= t_i, or the gap is not a finite number): the
  GPU label must equal the oracle label exactly;
* near-tie point (gap < t_i): several labels are correct.  The GPU label
  must be in the near-tie set {k : s_ik - b_i < t_i} and must be the lowest
  index among bitwise-identical centroid rows (identical rows give identical
  fp32 scores, so the lower one must win);
* min_dist must be within 2e-3 * (|d| + 1) of the oracle's squared distance
  d to the GPU's chosen centroid; non-finite d must match in class (NaN with
  NaN, +inf with +inf).
"""

from __future__ import annotations

import numpy as np

import oracle

GAP_REL = 1e-3
DIST_REL = 2e-3


def lowest_identical_row(C: np.ndarray) -> np.ndarray:
    """For each row of C, the lowest index of a bitwise-identical row."""
    C = np.ascontiguousarray(C)
    rows = C.view(np.dtype((np.void, C.dtype.itemsize * C.shape[1]))).ravel()
    _, first, inverse = np.unique(rows, return_index=True, return_inverse=True)
    return first[inverse.ravel()]


def check(X, C, labels, min_dist, idx=None, ref=None, lowest=None):
    """Check GPU ``labels``/``min_dist`` (numpy, all N points) on points ``idx``.

    Returns a dict of counts; raises AssertionError listing the first bad
    points.  ``ref`` may hold a precomputed ``oracle.assign`` of ``X[idx]``.
    """
    labels = np.asarray(labels)
    min_dist = np.asarray(min_dist)
    if idx is None:
        idx = np.arange(X.shape[0])
    idx = np.asarray(idx)
    Xs = np.ascontiguousarray(X[idx])
    gl = labels[idx].astype(np.int32)
    gd = min_dist[idx].astype(np.float64)
    K = C.shape[0]
    assert np.all((gl >= 0) & (gl < K)), "label out of range"
    if ref is None:
        ref = oracle.assign(Xs, C)
    ol, best, second = ref["labels"], ref["best"], ref["second"]
    if lowest is None:
        lowest = lowest_identical_row(C)

    with np.errstate(invalid="ignore"):
        thr = GAP_REL * (np.abs(best) + 1.0)
        near = (second - best) < thr             # NaN gap -> strict
    strict = ~near
    bad_strict = strict & (gl != ol)

    differ = gl != ol
    s_g = np.where(differ, oracle.score_for(Xs, C, gl), best)
    with np.errstate(invalid="ignore"):
        in_set = (s_g - best) < thr
    bad_near = near & differ & (~in_set | (lowest[gl] != gl))

    d_ref = np.where(differ, oracle.sqdist_for(Xs, C, gl), ref["dist"])
    fin = np.isfinite(d_ref)
    with np.errstate(invalid="ignore"):
        bad_dist = fin & ~(np.abs(gd - d_ref) <= DIST_REL * (np.abs(d_ref) + 1.0))
    same_class = (np.isnan(d_ref) & np.isnan(gd)) | (np.isinf(d_ref) & (gd == d_ref))
    bad_class = ~fin & ~same_class

    bad = bad_strict | bad_near | bad_dist | bad_class
    stats = dict(points=len(idx), strict=int(strict.sum()), near=int(near.sum()),
                 near_label_differs=int((near & differ).sum()),
                 bad_strict=int(bad_strict.sum()), bad_near=int(bad_near.sum()),
                 bad_dist=int(bad_dist.sum()), bad_class=int(bad_class.sum()))
    if bad.any():
        lines = []
        for j in np.flatnonzero(bad)[:10]:
            lines.append(f"point {idx[j]}: gpu=({gl[j]}, {gd[j]!r}) oracle=({ol[j]}, "
                         f"{ref['dist'][j]!r}) best={best[j]!r} second={second[j]!r} "
                         f"s_gpu={s_g[j]!r} d_ref={d_ref[j]!r}")
        raise AssertionError(f"parity failure {stats}\n" + "\n".join(lines))
    return stats


def sample_indices(N: int, seed: int = 0, head: int = 2048, rand: int = 2048, tail: int = 64):
    """First ``head`` points, ``rand`` random ones and the last ``tail``."""
    rng = np.random.default_rng(seed)
    parts = [np.arange(min(head, N)), rng.integers(0, N, size=min(rand, N)),
             np.arange(max(0, N - tail), N)]
    return np.unique(np.concatenate(parts))
