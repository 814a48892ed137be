"""Seeded synthetic inputs for the k-means assignment step.

This module only *makes inputs*: Gaussian-mixture point and centroid sets in
bf16, plus the adversarial structures (duplicate rows, equal rows, exactly
equidistant points, non-finite coordinates).  It computes nothing that the
assignment itself computes (no scores, norms, distances or argmins), so both
the HIP path and the CPU oracle can be fed from it without sharing arithmetic.

Workload shape follows the benchmark description on flashlib PR #22
("Optimize Blackwell k-means assignment reduction", nightly-comparison
section, "Benchmark methodology"): three independently seeded bf16
input/centroid sets with seeds 17, 29 and 43, rotated between calls.

Recipe (all draws are float32 from numpy's PCG64 ``default_rng(seed)``, then
rounded to bf16 with round-to-nearest-even):

1. ``mu[n_centers][D] ~ N(0, 1)``            true centres
2. ``a[N] ~ Uniform{0 .. n_centers-1}``      generating centre of each point
3. ``x_i = mu[a_i] + 0.1 * N(0, 1)``         points
4. ``c_k = mu[k] + 0.05 * N(0, 1)``          centroids (n_centers == K)

bf16 values are carried as ``uint16`` bit patterns everywhere.
"""

from __future__ import annotations

import numpy as np

SEEDS = (17, 29, 43)

#: The five workloads: tiny, large-K/small-D, headline, large-N/large-D,
#: adversarial.  Index 0 is unused so that workload i is ``CONFIGS[i]``.
CONFIGS = {
    1: dict(N=4096, D=64, K=256, adversarial=False,
            name="tiny N=4096 D=64 K=256"),
    2: dict(N=65536, D=64, K=4096, adversarial=False,
            name="large-K small-D N=65536 D=64 K=4096"),
    3: dict(N=262144, D=128, K=4096, adversarial=False,
            name="headline N=262144 D=128 K=4096"),
    4: dict(N=1048576, D=256, K=4096, adversarial=False,
            name="large-N large-D N=1048576 D=256 K=4096"),
    5: dict(N=262144, D=128, K=16384, adversarial=True,
            name="adversarial N=262144 D=128 K=16384"),
}

BF16_QNAN = np.uint16(0x7FC0)
BF16_PINF = np.uint16(0x7F80)
BF16_NINF = np.uint16(0xFF80)
BF16_PZERO = np.uint16(0x0000)
BF16_NZERO = np.uint16(0x8000)


# --------------------------------------------------------------------------
# bf16 encoding
# --------------------------------------------------------------------------

def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    NaN maps to a quiet NaN with the input's sign; +-inf stay +-inf; values
    that round past the largest finite bf16 become inf, as IEEE rounding does.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        sign = ((u >> np.uint32(16)) & np.uint32(0x8000)).astype(np.uint16)
        r = np.where(nan, sign | BF16_QNAN, r).astype(np.uint16)
    return r


def bf16_bits_to_f32(b) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact: a 16-bit shift)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def dyadic_to_bf16_bits(num: np.ndarray, shift: int) -> np.ndarray:
    """Encode the exact values ``num / 2**shift`` (small integers) as bf16.

    Used to build inputs whose products and sums are exact in fp32.  Raises
    if a value would not be representable exactly.
    """
    v = np.asarray(num, dtype=np.float64) / float(2 ** shift)
    f = v.astype(np.float32)
    bits = f32_to_bf16_bits(f)
    if not np.array_equal(bf16_bits_to_f32(bits).astype(np.float64), v):
        raise ValueError("value not exactly representable in bf16")
    return bits


# --------------------------------------------------------------------------
# Gaussian mixture
# --------------------------------------------------------------------------

def gaussian_mixture(N: int, D: int, K: int, seed: int,
                     point_sigma: float = 0.1, centroid_sigma: float = 0.05,
                     return_parts: bool = False):
    """Draw one seeded Gaussian-mixture set; returns ``(X, C, a)``.

    ``X`` is ``uint16[N, D]`` (bf16 bits), ``C`` is ``uint16[K, D]``, ``a``
    is the generating-centre index of each point (``int64[N]``).
    With ``return_parts`` the float32 centres and noise arrays are returned
    too (used by the adversarial builder).
    """
    rng = np.random.default_rng(seed)
    mu = rng.standard_normal((K, D), dtype=np.float32)
    a = rng.integers(0, K, size=N, dtype=np.int64) if K > 0 else np.zeros(N, np.int64)
    xn = rng.standard_normal((N, D), dtype=np.float32)
    cn = rng.standard_normal((K, D), dtype=np.float32)
    X32 = mu[a] if N > 0 else np.zeros((0, D), np.float32)
    X32 = X32 + np.float32(point_sigma) * xn
    C32 = mu + np.float32(centroid_sigma) * cn
    X = f32_to_bf16_bits(X32)
    C = f32_to_bf16_bits(C32)
    if return_parts:
        return X, C, a, dict(mu=mu, xn=xn, cn=cn)
    return X, C, a


# --------------------------------------------------------------------------
# Adversarial structure
# --------------------------------------------------------------------------

NAN_SLICE_POINTS = 4096
NAN_CATEGORIES = (
    "plain",          # 0: untouched
    "nan",            # 1: one NaN coordinate
    "pinf",           # 2: one +inf coordinate
    "ninf",           # 3: one -inf coordinate
    "pinf_ninf",      # 4: +inf and -inf at two coordinates
    "signed_zeros",   # 5: about half the coordinates set to +0.0 / -0.0
    "all_zero",       # 6: every coordinate +-0.0
    "nan_pinf",       # 7: NaN and +inf together
)


def _pick_block_pair(rng, K, block, used, tries=10000):
    """Pick s < t in different ``block``-sized index blocks, both unused."""
    nb = (K + block - 1) // block
    for _ in range(tries):
        bs, bt = sorted(rng.choice(nb, size=2, replace=False))
        s = int(bs * block + rng.integers(0, min(block, K - bs * block)))
        t = int(bt * block + rng.integers(0, min(block, K - bt * block)))
        if s != t and s not in used and t not in used:
            return s, t
    raise RuntimeError("could not place an index pair")


def adversarial(N: int, D: int, K: int, seed: int, n_dyadic_pairs: int = 1024,
                points_per_pair: int = 4, n_equal: int = 64,
                dup_fraction: float = 0.01, nan_slice: bool = True):
    """Gaussian mixture plus adversarial structure; returns ``(X, C, meta)``.

    Structure (index sets (i)-(iii) are disjoint; all choices are seeded):

    (i)   ``round(dup_fraction*K)`` duplicate rows ``C[t] = C[s]`` with
          ``s < t`` in different 512-row blocks (K/4-row blocks when
          K < 2048), starting with the boundary pairs ``s = 512m-1, t = 512m``.  Points generated from centre ``t``
          are re-drawn around centre ``s``.
    (ii)  ``n_equal`` equal rows at indices ``e0 + 256m`` (spread over all of
          K); points generated from any of them are re-drawn around ``e0``.
    (iii) ``n_dyadic_pairs`` pairs ``(a, b)``, ``a < b`` in different 512-row
          blocks, with ``C[a] = g + e_j/8`` and ``C[b] = g - e_j/8`` for a
          grid vector ``g`` in ``(1/8)Z^D``; ``points_per_pair`` points per
          pair, ``x = g + eta*e_m`` (``m != j``), overwrite the tail of X.
          Every product and partial sum of these rows is exact in fp32, so
          ``a`` and ``b`` tie exactly and the squared distance is
          ``1/64 + eta^2`` exactly.
    (iv)  The first ``NAN_SLICE_POINTS`` points carry non-finite and signed
          zero coordinates, category ``i % 8`` (see ``NAN_CATEGORIES``).
    """
    X, C, a, parts = gaussian_mixture(N, D, K, seed, return_parts=True)
    mu, xn = parts["mu"], parts["xn"]
    rng = np.random.default_rng([seed, 0xAD5E])
    used: set[int] = set()
    block = 512 if K >= 2048 else max(1, K // 4)

    # (ii) equal rows, stride 256 over K
    stride = max(1, K // max(1, n_equal))
    e0 = int(rng.integers(0, stride))
    equal_rows = [e0 + stride * m for m in range(n_equal) if e0 + stride * m < K]
    used.update(equal_rows)
    for r in equal_rows[1:]:
        C[r] = C[e0]

    # (i) duplicates, boundary pairs first
    n_dup = int(round(dup_fraction * K))
    dup_pairs: list[tuple[int, int]] = []
    m = 1
    while len(dup_pairs) < min(n_dup, 16) and block * m < K:
        s, t = block * m - 1, block * m
        if s not in used and t not in used:
            dup_pairs.append((s, t))
            used.update((s, t))
        m += 1
    while len(dup_pairs) < n_dup:
        s, t = _pick_block_pair(rng, K, block, used)
        dup_pairs.append((s, t))
        used.update((s, t))
    for s, t in dup_pairs:
        C[t] = C[s]

    # (iii) dyadic exactly-equidistant pairs
    n_pairs = min(n_dyadic_pairs, max(0, (N // max(1, points_per_pair)) // 4))
    dyadic_pairs = []
    dyadic_points = []  # (point index, expected label, expected squared distance)
    etas = (0, 1, -1, 2)  # eta in units of 1/8
    tail = N - n_pairs * points_per_pair
    for p in range(n_pairs):
        ia, ib = _pick_block_pair(rng, K, block, used)
        used.update((ia, ib))
        g = rng.integers(-14, 15, size=D)          # grid vector, units of 1/8
        j = int(rng.integers(0, D))
        ca = g.copy(); ca[j] += 1
        cb = g.copy(); cb[j] -= 1
        C[ia] = dyadic_to_bf16_bits(ca, 3)
        C[ib] = dyadic_to_bf16_bits(cb, 3)
        dyadic_pairs.append((ia, ib, j))
        for q in range(points_per_pair):
            eta = etas[q % len(etas)]
            mm = (j + 1 + int(rng.integers(0, D - 1))) % D if D > 1 else j
            x = g.copy()
            if mm != j:
                x[mm] += eta
            i = tail + p * points_per_pair + q
            X[i] = dyadic_to_bf16_bits(x, 3)
            d2 = (1 + (eta * eta if mm != j else 0)) / 64.0
            dyadic_points.append((i, ia, d2))

    # Re-draw points whose generating centre was consumed by (i)-(iii).
    special = np.zeros(K, dtype=bool)
    special[list(used)] = True
    remap = np.arange(K)
    for s, t in dup_pairs:
        remap[t] = s
    for r in equal_rows:
        remap[r] = e0
    free = np.flatnonzero(~special)
    for ia, ib, _ in dyadic_pairs:
        remap[ia] = free[int(rng.integers(0, len(free)))]
        remap[ib] = free[int(rng.integers(0, len(free)))]
    body = np.arange(N) < tail
    moved = body & (remap[a] != a)
    if moved.any():
        idx = np.flatnonzero(moved)
        a = a.copy()
        a[idx] = remap[a[idx]]
        X[idx] = f32_to_bf16_bits(mu[a[idx]] + np.float32(0.1) * xn[idx])

    # (iv) non-finite / signed-zero slice
    nan_cat = np.zeros(0, dtype=np.int64)
    if nan_slice:
        ns = min(NAN_SLICE_POINTS, tail)
        nan_cat = np.arange(ns) % len(NAN_CATEGORIES)
        for i in range(ns):
            cat = NAN_CATEGORIES[nan_cat[i]]
            j1, j2 = (int(v) for v in rng.choice(D, size=2, replace=False)) if D > 1 else (0, 0)
            if cat == "nan":
                X[i, j1] = BF16_QNAN
            elif cat == "pinf":
                X[i, j1] = BF16_PINF
            elif cat == "ninf":
                X[i, j1] = BF16_NINF
            elif cat == "pinf_ninf":
                X[i, j1] = BF16_PINF
                X[i, j2] = BF16_NINF
            elif cat == "signed_zeros":
                sel = rng.random(D) < 0.5
                sgn = rng.random(D) < 0.5
                X[i, sel] = np.where(sgn[sel], BF16_NZERO, BF16_PZERO)
            elif cat == "all_zero":
                sgn = rng.random(D) < 0.5
                X[i] = np.where(sgn, BF16_NZERO, BF16_PZERO)
            elif cat == "nan_pinf":
                X[i, j1] = BF16_QNAN
                X[i, j2] = BF16_PINF

    meta = dict(
        dup_pairs=np.array(dup_pairs, dtype=np.int64).reshape(-1, 2),
        equal_rows=np.array(equal_rows, dtype=np.int64),
        dyadic_pairs=np.array(dyadic_pairs, dtype=np.int64).reshape(-1, 3),
        dyadic_points=np.array([p[0] for p in dyadic_points], dtype=np.int64),
        dyadic_labels=np.array([p[1] for p in dyadic_points], dtype=np.int64),
        dyadic_sqdist=np.array([p[2] for p in dyadic_points], dtype=np.float64),
        nan_slice=np.arange(len(nan_cat), dtype=np.int64),
        nan_category=nan_cat,
        generating_centre=a,
    )
    return X, C, meta


#: The 13 (N, D, K) shapes of the pages' benchmark (flashlib PR #22,
#: "Performance" table; the same rows in the nightly comparison's "Benchmark
#: results"), bf16 Gaussian mixtures with K true centres, seeds ``SEEDS``.
SWEEP_SHAPES = (
    (65536, 64, 512), (65536, 64, 4096), (65536, 64, 16384),
    (65536, 128, 512), (65536, 128, 4096),
    (262144, 128, 4096), (262144, 128, 16384), (1048576, 128, 4096),
    (65536, 256, 512), (65536, 256, 4096),
    (262144, 256, 4096), (262144, 256, 16384), (1048576, 256, 4096),
)


def make_config(i: int, seed: int):
    """Inputs of workload ``i`` (1..5) for ``seed``: ``(X, C, meta)``."""
    cfg = CONFIGS[i]
    if cfg["adversarial"]:
        return adversarial(cfg["N"], cfg["D"], cfg["K"], seed)
    X, C, a = gaussian_mixture(cfg["N"], cfg["D"], cfg["K"], seed)
    return X, C, dict(generating_centre=a)
