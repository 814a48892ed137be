"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` takes a loaded oracle library (the real one, or a copy built
from a deliberately broken source in ``test_oracle_pins.py``) and raises
``AssertionError`` when the oracle disagrees with what the mathematics fixes:
exact rational brute force on tiny inputs (using the distance form
``sum (x-c)^2``, not the oracle's expanded form), invariants, closed forms,
and reductions to textbook routines.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

import oracle
from means_nearest_centroid_amd import workloads as W


def _exact(bits_row):
    return [Fraction(float(v)) for v in W.bf16_bits_to_f32(bits_row)]


def brute_force(X, C):
    """Exact squared distances with rationals; lowest-index argmin."""
    Xe = [_exact(r) for r in X]
    Ce = [_exact(r) for r in C]
    labels, dmin, d2nd, xx = [], [], [], []
    for x in Xe:
        d = [sum((a - b) * (a - b) for a, b in zip(x, c)) for c in Ce]
        m = min(d)
        lab = d.index(m)
        labels.append(lab)
        dmin.append(m)
        rest = d[:lab] + d[lab + 1:]
        d2nd.append(min(rest) if rest else None)
        xx.append(sum(a * a for a in x))
    return np.array(labels), dmin, d2nd, xx


def _rel_close(a, b, rel=1e-12):
    a = float(a)
    b = float(b)
    return abs(a - b) <= rel * (abs(b) + 1.0)


# ----------------------------------------------------------------------------
# Tiny inputs
# ----------------------------------------------------------------------------

def tiny_cases():
    """Small random and adversarial inputs for the brute-force pin."""
    cases = []
    for seed, (N, D, K) in enumerate([(24, 16, 9), (16, 64, 40), (20, 16, 33)]):
        cases.append(W.gaussian_mixture(N, D, K, 100 + seed)[:2])
    # wide-spread values (many binades) and exact duplicates
    rng = np.random.default_rng(7)
    X = W.f32_to_bf16_bits(rng.standard_normal((12, 16)).astype(np.float32)
                           * np.float32(2.0) ** rng.integers(-6, 7, (12, 16)).astype(np.float32))
    C = W.f32_to_bf16_bits(rng.standard_normal((10, 16)).astype(np.float32))
    C[7] = C[2]
    C[9] = C[2]
    X[3] = C[2]
    X[4] = C[9]
    cases.append((X, C))
    # small-integer grid: many exact ties
    Xg = W.dyadic_to_bf16_bits(rng.integers(-2, 3, (30, 16)), 0)
    Cg = W.dyadic_to_bf16_bits(rng.integers(-2, 3, (12, 16)), 0)
    cases.append((Xg, Cg))
    return cases


def pin_bruteforce(lib):
    """Labels equal the exact argmin; scores and distances equal exact ones."""
    for X, C in tiny_cases():
        ref = oracle.assign(X, C, lib=lib)
        lab, dmin, d2nd, xx = brute_force(X, C)
        assert np.array_equal(ref["labels"], lab), "labels differ from exact argmin"
        for i in range(len(lab)):
            assert _rel_close(ref["dist"][i], dmin[i]), "dist differs from exact"
            # s_best + ||x||^2 is the exact minimal squared distance
            assert _rel_close(ref["best"][i] + float(xx[i]), dmin[i]), "best score wrong"
            if d2nd[i] is not None:
                assert _rel_close(ref["second"][i] + float(xx[i]), d2nd[i]), "runner-up wrong"


def pin_score_and_sqdist_for(lib):
    """The checker helpers: ``score_for`` and ``sqdist_for`` for EVERY
    (point, centroid) pair of the tiny cases against exact rationals, with
    the score taken from the distance form (s_ik = ||x - c_k||^2 - ||x||^2,
    an identity, not the oracle's expanded formula), plus one random label
    per point so a helper that reads the wrong point's label fails; and the
    IEEE classes of non-finite cases, derived by hand."""
    rng = np.random.default_rng(8)
    for X, C in tiny_cases():
        N, K = X.shape[0], C.shape[0]
        Xe = [_exact(r) for r in X]
        Ce = [_exact(r) for r in C]
        dist = [[sum((a - b) * (a - b) for a, b in zip(x, c)) for c in Ce] for x in Xe]
        xx = [sum(a * a for a in x) for x in Xe]
        label_sets = [np.full(N, k, np.int32) for k in range(K)]
        label_sets.append(rng.integers(0, K, N).astype(np.int32))
        for lab in label_sets:
            s = oracle.score_for(X, C, lab, lib=lib)
            d = oracle.sqdist_for(X, C, lab, lib=lib)
            for i in range(N):
                k = int(lab[i])
                assert _rel_close(d[i], dist[i][k]), "sqdist_for differs from exact"
                assert _rel_close(s[i], dist[i][k] - xx[i]), "score_for differs from exact"
    # Non-finite: +inf at j against c_kj > 0 scores -inf (distance +inf); a
    # NaN coordinate makes both NaN; -0.0 coordinates change nothing.
    X, C, _ = W.gaussian_mixture(4, 16, 6, 19)
    Cf = W.bf16_bits_to_f32(C).astype(np.float64)
    k_pos = int(np.flatnonzero(Cf[:, 3] > 0)[0])
    k_neg = int(np.flatnonzero(Cf[:, 3] < 0)[0])
    Xn = X.copy()
    Xn[0, 3] = W.BF16_PINF
    Xn[1, 3] = W.BF16_PINF
    Xn[2, 5] = W.BF16_QNAN
    Xn[3, ::2] = W.BF16_NZERO
    lab = np.array([k_pos, k_neg, 0, 2], np.int32)
    s = oracle.score_for(Xn, C, lab, lib=lib)
    d = oracle.sqdist_for(Xn, C, lab, lib=lib)
    assert s[0] == -np.inf and d[0] == np.inf, "+inf against a positive coordinate"
    assert s[1] == np.inf and d[1] == np.inf, "+inf against a negative coordinate"
    assert np.isnan(s[2]) and np.isnan(d[2]), "NaN coordinate"
    Xp = Xn[3:4].copy()
    Xp[0, ::2] = W.BF16_PZERO
    assert s[3] == oracle.score_for(Xp, C, lab[3:], lib=lib)[0], "signed zero score"
    assert d[3] == oracle.sqdist_for(Xp, C, lab[3:], lib=lib)[0], "signed zero distance"


def pin_centroid_norms(lib):
    """n_k equals the exact rational sum of squares."""
    for _, C in tiny_cases():
        n = oracle.centroid_norms(C, lib=lib)
        for k in range(C.shape[0]):
            assert _rel_close(n[k], sum(v * v for v in _exact(C[k]))), "norm wrong"


def pin_permutation(lib):
    """Permuting centroids permutes labels (points with a clear winner)."""
    X, C, _ = W.gaussian_mixture(300, 32, 50, 11)
    ref = oracle.assign(X, C, lib=lib)
    perm = np.random.default_rng(3).permutation(C.shape[0])
    ref_p = oracle.assign(X, C[perm], lib=lib)
    inv = np.argsort(perm)
    assert np.array_equal(inv[ref["labels"]], ref_p["labels"]), "centroid permutation"
    assert np.array_equal(ref["dist"], ref_p["dist"]), "centroid permutation dist"
    pp = np.random.default_rng(4).permutation(X.shape[0])
    ref_q = oracle.assign(X[pp], C, lib=lib)
    assert np.array_equal(ref["labels"][pp], ref_q["labels"]), "point permutation"


def pin_duplicates_and_equal(lib):
    """Identical centroid rows resolve to the lowest index; all-equal -> 0."""
    X, C, _ = W.gaussian_mixture(200, 32, 40, 12)
    ref = oracle.assign(X, C, lib=lib)
    C2 = np.concatenate([C, C[::-1]])            # every row duplicated later
    ref2 = oracle.assign(X, C2, lib=lib)
    assert np.array_equal(ref["labels"], ref2["labels"]), "duplicate rows"
    Ceq = np.repeat(C[5:6], 17, axis=0)
    ref3 = oracle.assign(X, Ceq, lib=lib)
    assert np.all(ref3["labels"] == 0), "all-equal centroids"
    C4 = C.copy()
    C4[30] = C4[3]
    lab4 = oracle.assign(X, C4, lib=lib)["labels"]
    assert not np.any(lab4 == 30), "a later duplicate won a tie"


def pin_scaling(lib):
    """x, c -> 2^a x, 2^a c: labels unchanged, dist scaled by exactly 4^a."""
    X, C, _ = W.gaussian_mixture(200, 32, 40, 13)
    ref = oracle.assign(X, C, lib=lib)
    for a in (-3, 2, 5):
        f = np.float32(2.0 ** a)
        Xs = W.f32_to_bf16_bits(W.bf16_bits_to_f32(X) * f)
        Cs = W.f32_to_bf16_bits(W.bf16_bits_to_f32(C) * f)
        r = oracle.assign(Xs, Cs, lib=lib)
        assert np.array_equal(r["labels"], ref["labels"]), "scaling changed labels"
        assert np.array_equal(r["dist"], ref["dist"] * 4.0 ** a), "scaling dist"


def pin_exact_member(lib):
    """x equal to a centroid row: that row wins with distance 0."""
    X, C, _ = W.gaussian_mixture(60, 32, 45, 14)
    picks = np.random.default_rng(5).integers(0, C.shape[0], 60)
    Xc = C[picks]
    r = oracle.assign(Xc, C, lib=lib)
    assert np.array_equal(r["labels"], picks), "x == c_j must pick j"
    assert np.all(r["dist"] == 0.0), "x == c_j must have distance 0"


def pin_zero_point(lib):
    """x = 0: the score is the norm, so the label is argmin of the norms."""
    _, C, _ = W.gaussian_mixture(1, 48, 70, 15)
    X = np.zeros((3, 48), dtype=np.uint16)
    X[1, ::2] = W.BF16_NZERO                      # -0.0 coordinates
    Cf = W.bf16_bits_to_f32(C).astype(np.float64)
    norms = np.einsum("kd,kd->k", Cf, Cf)
    r = oracle.assign(X, C, lib=lib)
    assert np.all(r["labels"] == int(np.argmin(norms))), "x = 0 must pick argmin norm"
    assert np.allclose(r["dist"], norms.min(), rtol=1e-15, atol=0), "x = 0 distance"


def pin_one_dimensional(lib):
    """One live coordinate: nearest centre on a line, by sorted search."""
    D = 16
    rng = np.random.default_rng(16)
    cvals = W.f32_to_bf16_bits(rng.standard_normal(50).astype(np.float32))
    cvals[10] = cvals[3]                           # a duplicate value
    xvals = W.f32_to_bf16_bits(rng.standard_normal(400).astype(np.float32) * 1.3)
    C = np.zeros((50, D), np.uint16)
    C[:, 5] = cvals
    X = np.zeros((400, D), np.uint16)
    X[:, 5] = xvals
    r = oracle.assign(X, C, lib=lib)
    cv = W.bf16_bits_to_f32(cvals).astype(np.float64)
    xv = W.bf16_bits_to_f32(xvals).astype(np.float64)
    uniq = np.unique(cv)                          # sorted distinct values
    first_idx = np.array([np.flatnonzero(cv == u)[0] for u in uniq])
    pos = np.searchsorted(uniq, xv)
    lo = np.clip(pos - 1, 0, len(uniq) - 1)
    hi = np.clip(pos, 0, len(uniq) - 1)
    dlo, dhi = np.abs(xv - uniq[lo]), np.abs(xv - uniq[hi])
    # nearest value; on an exact tie the lower original index wins
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (first_idx[hi] < first_idx[lo]))
    expect = np.where(pick_hi, first_idx[hi], first_idx[lo])
    assert np.array_equal(r["labels"], expect), "1-D nearest centre"


def pin_dyadic_ties(lib):
    """Exactly equidistant pair on a dyadic grid: lower index, 1/64 + eta^2."""
    X, C, meta = W.adversarial(64, 32, 256, 21, n_dyadic_pairs=8, n_equal=4,
                               nan_slice=False)
    r = oracle.assign(X, C, lib=lib)
    idx = meta["dyadic_points"]
    assert np.array_equal(r["labels"][idx], meta["dyadic_labels"]), "dyadic tie label"
    assert np.array_equal(r["dist"][idx], meta["dyadic_sqdist"]), "dyadic distance"
    assert np.all(r["second"][idx] == r["best"][idx]), "dyadic tie must be exact"


def pin_nonfinite(lib):
    """Rule for NaN / +-inf / signed zero, derived by hand per case."""
    X, C, _ = W.gaussian_mixture(8, 32, 60, 17)
    Cf = W.bf16_bits_to_f32(C).astype(np.float64)
    assert np.all(Cf != 0)
    base = oracle.assign(X, C, lib=lib)
    Xn = X.copy()
    Xn[0, 4] = W.BF16_QNAN                       # NaN: every score NaN -> 0
    Xn[1, 7] = W.BF16_PINF                       # +inf: s = -inf where c_kj > 0
    Xn[2, 9] = W.BF16_NINF                       # -inf: s = -inf where c_kj < 0
    Xn[3, 1] = W.BF16_PINF                       # +inf, -inf together
    Xn[3, 2] = W.BF16_NINF
    Xn[4, ::3] = W.BF16_NZERO                    # -0.0 vs +0.0 below
    Xn[5, :] = W.BF16_NZERO                       # all -0.0 -> argmin norm
    Xn[6, 3] = W.BF16_QNAN
    Xn[6, 4] = W.BF16_PINF
    r = oracle.assign(Xn, C, lib=lib)
    lab, dist = r["labels"], r["dist"]
    assert lab[0] == 0 and np.isnan(dist[0]), "NaN coordinate"
    assert lab[1] == np.flatnonzero(Cf[:, 7] > 0)[0] and dist[1] == np.inf, "+inf"
    assert lab[2] == np.flatnonzero(Cf[:, 9] < 0)[0] and dist[2] == np.inf, "-inf"
    both = np.flatnonzero((Cf[:, 1] > 0) & (Cf[:, 2] < 0))
    assert lab[3] == both[0] and dist[3] == np.inf, "+inf and -inf"
    Xp = Xn[4:5].copy()
    Xp[0, ::3] = W.BF16_PZERO
    rp = oracle.assign(Xp, C, lib=lib)
    assert lab[4] == rp["labels"][0] and dist[4] == rp["dist"][0], "signed zero"
    norms = (Cf * Cf).sum(1)
    assert lab[5] == int(np.argmin(norms)), "all -0.0 row"
    assert lab[6] == 0 and np.isnan(dist[6]), "NaN with +inf"
    assert np.array_equal(lab[7], base["labels"][7]), "untouched point"

    # Non-finite centroid rows: never win against finite rows.
    C2 = C.copy()
    C2[0, 3] = W.BF16_QNAN
    C2[1, 5] = W.BF16_PINF
    C2[2, 6] = W.BF16_NINF
    r2 = oracle.assign(X, C2, lib=lib)
    assert not np.any(np.isin(r2["labels"], (0, 1, 2))), "non-finite centroid won"
    # Every score +inf (x_j < 0 against c_kj = +inf, x_j > 0 against -inf):
    # the lowest +inf index wins, i.e. 0; with one NaN row first, index 1.
    x = np.zeros((1, 32), np.uint16)
    x[0, 0] = W.dyadic_to_bf16_bits(np.array([-1]), 0)[0]
    Cinf = np.zeros((5, 32), np.uint16)
    Cinf[:, 0] = W.BF16_PINF
    r3 = oracle.assign(x, Cinf, lib=lib)
    assert r3["labels"][0] == 0 and r3["best"][0] == np.inf, "all +inf scores"
    Cinf[0, 1] = W.BF16_QNAN
    r4 = oracle.assign(x, Cinf, lib=lib)
    assert r4["labels"][0] == 1, "NaN ranks after +inf"


def pin_single_centroid(lib):
    X, C, _ = W.gaussian_mixture(50, 16, 1, 18)
    r = oracle.assign(X, C, lib=lib)
    assert np.all(r["labels"] == 0) and np.all(np.isnan(r["second"]))


# ----------------------------------------------------------------------------
# Centroid update
# ----------------------------------------------------------------------------

def exact_bf16_bits(q) -> int:
    """Round a rational to bf16 (nearest, ties to even), from the format's
    definition: 8 significant bits, binary32 exponent range, spacing 2^-133
    below 2^-126, overflow past the largest finite value to infinity."""
    if q == 0:
        return 0
    sign = 0x8000 if q < 0 else 0
    a = abs(Fraction(q))
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    scaled = a * Fraction(2) ** (7 - e)
    r = scaled.numerator // scaled.denominator
    rem = scaled - r
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and r % 2 == 1):
        r += 1
    value = Fraction(r) * Fraction(2) ** (e - 7)
    if value > 255 * Fraction(2) ** 120:
        return sign | 0x7F80
    f32 = np.array([float(value)], dtype=np.float32)     # exact: 8 bits
    return sign | int(f32.view(np.uint32)[0] >> 16)


def pin_bf16_rounding(lib):
    """fp64 -> bf16 rounding against exact rational rounding, and against the
    integer-bit rounding of fp32 values in the input generator."""
    rng = np.random.default_rng(40)
    f = (rng.standard_normal(4000) * 2.0 ** rng.integers(-140, 125, 4000)).astype(np.float32)
    f = f[np.isfinite(f)]
    got = oracle.bf16_from_double(f.astype(np.float64), lib=lib)
    assert np.array_equal(got, W.f32_to_bf16_bits(f)), "fp32-representable values"
    # Values an fp32 intermediate would round twice: just above / below a tie.
    vals = []
    for e in (-130, -127, -20, 0, 5, 100, 127):
        for m in (1, 2, 3, 77, 127):
            base = Fraction(128 + m) * Fraction(2) ** (e - 7)
            half = Fraction(1) * Fraction(2) ** (e - 8)
            for off in (0, Fraction(1) * Fraction(2) ** (e - 40), -Fraction(1) * Fraction(2) ** (e - 40)):
                vals.append(base + half + off)
                vals.append(-(base + half + off))
    vals += [Fraction(2) ** -133, Fraction(3) * Fraction(2) ** -135,
             Fraction(2) ** -134, Fraction(2) ** -134 + Fraction(2) ** -160,
             Fraction(255) * Fraction(2) ** 120 + Fraction(2) ** 118,    # rounds down
             Fraction(511) * Fraction(2) ** 119]                          # tie -> inf
    d = np.array([float(v) for v in vals])
    exact = [Fraction(float(v)) for v in vals]     # the fp64 value itself
    got = oracle.bf16_from_double(d, lib=lib)
    want = np.array([exact_bf16_bits(v) for v in exact], dtype=np.uint16)
    assert np.array_equal(got, want), "rational rounding"
    sp = oracle.bf16_from_double(np.array([np.nan, -np.nan, np.inf, -np.inf, 0.0, -0.0]), lib=lib)
    assert list(sp) == [0x7FC0, 0xFFC0, 0x7F80, 0xFF80, 0x0000, 0x8000], "special values"


def update_cases():
    rng = np.random.default_rng(41)
    cases = []
    for seed, (N, D, K) in enumerate([(40, 16, 6), (25, 32, 9), (60, 16, 3)]):
        X, C, a = W.gaussian_mixture(N, D, K, 200 + seed)
        lab = a.astype(np.int32)
        lab[:: 7] = rng.integers(0, K, len(lab[:: 7]))
        cases.append((X, C, lab))
    # many binades, a cluster left empty, labels outside [0, K)
    X = W.f32_to_bf16_bits((rng.standard_normal((30, 16))
                            * 2.0 ** rng.integers(-12, 12, (30, 16))).astype(np.float32))
    C = W.f32_to_bf16_bits(rng.standard_normal((5, 16)).astype(np.float32))
    lab = rng.integers(0, 4, 30).astype(np.int32)      # cluster 4 empty
    lab[3], lab[11], lab[12] = -1, 5, 1 << 30
    cases.append((X, C, lab))
    return cases


def pin_update_bruteforce(lib):
    """Counts, means and bf16 centroids equal the exact rational result."""
    for X, C, lab in update_cases():
        r = oracle.update(X, lab, C, lib=lib)
        K, D = C.shape
        Xe = [_exact(row) for row in X]
        for k in range(K):
            members = [i for i in range(len(lab)) if lab[i] == k]
            assert r["counts"][k] == len(members), "count"
            if not members:
                assert np.array_equal(r["C_new"][k], C[k]), "empty cluster must keep its row"
                continue
            for j in range(D):
                m = sum(Xe[i][j] for i in members) / len(members)
                assert _rel_close(r["means"][k, j], m, 1e-15), "mean"
                assert r["C_new"][k, j] == exact_bf16_bits(m), "bf16 mean"


def pin_update_closed_forms(lib):
    """Identical members give that row back bit for bit; a mean of dyadic
    rows is exact; permuting points changes nothing; scaling by 2^a scales
    the means exactly; labels from an assignment of C's own rows return C."""
    X, C, a = W.gaussian_mixture(300, 32, 20, 42)
    lab = a.astype(np.int32)
    r = oracle.update(X, lab, C, lib=lib)
    Xs = C[lab]                                   # every point on its centroid
    rs = oracle.update(Xs, lab, C, lib=lib)
    present = np.unique(lab)
    assert np.array_equal(rs["C_new"][present], C[present]), "identical members"
    # dyadic rows: the mean of +-1/8 grid points has few bits, so it is exact
    G = W.dyadic_to_bf16_bits(np.random.default_rng(43).integers(-9, 10, (64, 32)), 3)
    lg = np.repeat(np.arange(16, dtype=np.int32), 4)
    rg = oracle.update(G, lg, C[:16], lib=lib)
    Gf = W.bf16_bits_to_f32(G).astype(np.float64).reshape(16, 4, 32)
    assert np.array_equal(rg["means"], Gf.mean(1)), "dyadic means"
    assert np.array_equal(W.bf16_bits_to_f32(rg["C_new"]).astype(np.float64),
                          Gf.mean(1)), "dyadic bf16"
    perm = np.random.default_rng(44).permutation(len(lab))
    rp = oracle.update(X[perm], lab[perm], C, lib=lib)
    assert np.array_equal(rp["counts"], r["counts"]), "permutation counts"
    assert np.allclose(rp["means"], r["means"], rtol=1e-15, atol=0), "permutation means"
    for e in (-4, 3):
        f = np.float32(2.0 ** e)
        Xe = W.f32_to_bf16_bits(W.bf16_bits_to_f32(X) * f)
        Ce = W.f32_to_bf16_bits(W.bf16_bits_to_f32(C) * f)
        re = oracle.update(Xe, lab, Ce, lib=lib)
        assert np.array_equal(re["means"], r["means"] * 2.0 ** e), "scaling means"
        assert np.array_equal(re["C_new"], W.f32_to_bf16_bits(
            W.bf16_bits_to_f32(r["C_new"]) * f)), "scaling bf16"
    # Lloyd fixed point: the points are the centroids and assign to themselves.
    own = oracle.assign(C, C, lib=lib)["labels"]
    assert np.array_equal(own, np.arange(C.shape[0])), "distinct rows"
    rf = oracle.update(C, own, C, lib=lib)
    assert np.array_equal(rf["C_new"], C) and np.all(rf["counts"] == 1), "fixed point"
    # No points at all: every cluster empty.
    r0 = oracle.update(X[:0], lab[:0], C, lib=lib)
    assert np.array_equal(r0["C_new"], C) and not r0["counts"].any(), "no points"


ALL_PINS = (pin_bruteforce, pin_score_and_sqdist_for, pin_centroid_norms, pin_permutation,
            pin_duplicates_and_equal, pin_scaling, pin_exact_member,
            pin_zero_point, pin_one_dimensional, pin_dyadic_ties,
            pin_nonfinite, pin_single_centroid, pin_bf16_rounding,
            pin_update_bruteforce, pin_update_closed_forms)
