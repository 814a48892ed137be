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
    stats, report = evaluate(X, C, labels, min_dist, idx, ref, lowest)
    if report:
        raise AssertionError(f"parity failure {stats}\n" + report)
    return stats


def evaluate(X, C, labels, min_dist, idx=None, ref=None, lowest=None):
    """The rule of ``check`` without raising: (counts, report of the first
    bad points, empty when every checked point passes)."""
    labels = np.asarray(labels)
    min_dist = np.asarray(min_dist)
    if idx is None:
        idx = np.arange(X.shape[0])
    idx = np.asarray(idx)
    Xs = np.ascontiguousarray(X[idx])
    gl = labels[idx].astype(np.int32)
    gd = min_dist[idx].astype(np.float64)
    K = C.shape[0]
    if not np.all((gl >= 0) & (gl < K)):
        j = int(np.flatnonzero((gl < 0) | (gl >= K))[0])
        return (dict(points=len(idx), bad=int(((gl < 0) | (gl >= K)).sum()),
                     label_out_of_range=True),
                f"point {idx[j]}: label {gl[j]} out of range [0, {K})")
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
    lines = []
    for j in np.flatnonzero(bad)[:10]:
        lines.append(f"point {idx[j]}: gpu=({gl[j]}, {gd[j]!r}) oracle=({ol[j]}, "
                     f"{ref['dist'][j]!r}) best={best[j]!r} second={second[j]!r} "
                     f"s_gpu={s_g[j]!r} d_ref={d_ref[j]!r}")
    stats["bad"] = int(bad.sum())
    return stats, "\n".join(lines)


def sample_indices(N: int, seed: int = 0, head: int = 2048, rand: int = 2048, tail: int = 64):
    """First ``head`` points, ``rand`` random ones and the last ``tail``."""
    rng = np.random.default_rng(seed)
    parts = [np.arange(min(head, N)), rng.integers(0, N, size=min(rand, N)),
             np.arange(max(0, N - tail), N)]
    return np.unique(np.concatenate(parts))


# ---------------------------------------------------------------------------
# Centroid update
# ---------------------------------------------------------------------------
#
# For a cluster of n points with exact mean m (the oracle's fp64 mean: bf16
# sums of this size are exact in fp64) and S = sum of |x_ij| over its
# points, any fp32 summation order is within (n - 1) u S of the exact sum
# (u = 2^-24; the bound of recursive and of any tree summation), and the
# division adds u |m|.  So a GPU mean must satisfy
#
#     |mean_gpu - m| <= tol = 1.01 u ((n - 1) S / n + |m|) + 2^-149,
#
# and its bf16 row, the rounding of some value within tol of m, must lie
# between rne(m - tol) and rne(m + tol) (rounding is monotone).  Counts are
# exact; an empty cluster's row is the old row bit for bit; non-finite means
# match in class.

U32 = 2.0 ** -24


def _members_abs_sum(X, labels, K):
    """Per cluster and coordinate, the sum of |x_ij| over its points (fp32
    accumulation: this only sizes the tolerance)."""
    S = np.zeros((K, X.shape[1]))
    idx = np.flatnonzero((labels >= 0) & (labels < K))
    if len(idx) == 0:
        return S
    idx = idx[np.argsort(labels[idx], kind="stable")]
    lab = labels[idx]
    Xa = np.abs((X[idx].astype(np.uint32) << 16).view(np.float32))
    first, starts = np.unique(lab, return_index=True)
    S[first] = np.add.reduceat(Xa, starts, axis=0)
    return S


def _widen(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_update(X, labels, C_old, C_new, norms, counts, means=None, ref=None):
    """Check a GPU centroid update (numpy arrays) against the oracle."""
    labels = np.asarray(labels, dtype=np.int32)
    C_new = np.asarray(C_new, dtype=np.uint16)
    K, D = C_old.shape
    if ref is None:
        ref = oracle.update(X, labels, C_old)
    problems = []
    if not np.array_equal(np.asarray(counts, dtype=np.int64), ref["counts"]):
        bad = np.flatnonzero(np.asarray(counts) != ref["counts"])[:5]
        problems.append(f"counts differ at {bad}: gpu={np.asarray(counts)[bad]} "
                        f"oracle={ref['counts'][bad]}")
    empty = ref["counts"] == 0
    if not np.array_equal(C_new[empty], C_old[empty]):
        problems.append("an empty cluster's row changed")
    m = ref["means"]
    n = np.maximum(ref["counts"], 1).astype(np.float64)[:, None]
    S = _members_abs_sum(X, labels, K)
    with np.errstate(invalid="ignore", over="ignore"):
        tol = 1.01 * U32 * ((n - 1.0) / n * S + np.abs(m)) + 2.0 ** -149
        lo = _widen(oracle.bf16_from_double(m - tol))
        hi = _widen(oracle.bf16_from_double(m + tol))
    got = _widen(C_new)
    fin = np.isfinite(m) & ~empty[:, None]
    with np.errstate(invalid="ignore"):
        bad_row = fin & ~((got >= lo) & (got <= hi))
    nonfin = ~np.isfinite(m) & ~empty[:, None]
    bad_cls = nonfin & ~((np.isnan(m) & np.isnan(got)) | (np.isinf(m) & (got == m)))
    if bad_row.any():
        k, j = np.argwhere(bad_row)[0]
        problems.append(f"{int(bad_row.sum())} bf16 elements out of bounds, first [{k},{j}]: "
                        f"gpu={got[k, j]!r} oracle mean={m[k, j]!r} tol={tol[k, j]!r}")
    if bad_cls.any():
        k, j = np.argwhere(bad_cls)[0]
        problems.append(f"non-finite class mismatch at [{k},{j}]: gpu={got[k, j]!r} "
                        f"oracle={m[k, j]!r}")
    if means is not None:
        mg = np.asarray(means, dtype=np.float32).astype(np.float64)
        with np.errstate(invalid="ignore"):
            bad_m = fin & ~(np.abs(mg - m) <= tol)
        if not np.array_equal(mg[empty], _widen(C_old[empty])):
            problems.append("an empty cluster's fp32 mean is not its old row")
        if bad_m.any():
            k, j = np.argwhere(bad_m)[0]
            problems.append(f"{int(bad_m.sum())} fp32 means out of bounds, first [{k},{j}]: "
                            f"gpu={mg[k, j]!r} oracle={m[k, j]!r} tol={tol[k, j]!r}")
        # the bf16 row is the rounding of the fp32 mean the GPU computed
        if not np.array_equal(oracle.bf16_from_double(mg)[~empty], C_new[~empty]):
            problems.append("bf16 row is not the rounding of the fp32 mean")
    # norms: a property of whatever rows came out
    cn = _widen(C_new)
    with np.errstate(invalid="ignore", over="ignore"):
        nn = (cn * cn).sum(1)
        g = np.asarray(norms, dtype=np.float64)
        okn = np.isfinite(nn)
        bad_n = okn & ~(np.abs(g - nn) <= 2e-6 * nn + 1e-30)
    if bad_n.any():
        k = np.flatnonzero(bad_n)[0]
        problems.append(f"norm of row {k}: gpu={g[k]!r} sum of squares={nn[k]!r}")
    if problems:
        raise AssertionError("update parity failure:\n" + "\n".join(problems))
    return dict(clusters=K, empty=int(empty.sum()),
                exact=int((got[fin] == _widen(oracle.bf16_from_double(m))[fin]).sum()),
                elements=int(fin.sum()))
