"""HIP path against the fp64 oracle, through the C ABI, on an MI355X.

Small shapes (ragged in N, K and D, spanning several tiles) and the five
workloads, at their full sizes with the production dispatch, are checked on
every point; the 13 benchmark shapes on samples.  Acceptance rule:
``parity.py``.
"""

import os

import numpy as np
import pytest

import oracle
import parity
from means_nearest_centroid_amd import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
km = pytest.importorskip("means_nearest_centroid_amd")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    km.load_library()           # raises if the HIP library is missing
    return torch.device("cuda:0")


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def run(X, C, path=km.PATH_AUTO, count=0):
    Xd, Cd = dev(X), dev(C)
    n = km.kmeans_centroid_norms(Cd)
    lab, md = km.kmeans_assign_path(Xd, Cd, n, path, count)
    torch.cuda.synchronize()
    return lab.cpu().numpy(), md.cpu().numpy()


def test_native_library_is_loaded():
    with open("/proc/self/maps") as f:
        maps = f.read()
    assert os.path.realpath(km.LIBRARY) in maps, "HIP library not mapped"
    hip = {ln.split()[-1] for ln in maps.splitlines() if "libamdhip64" in ln}
    assert len(hip) == 1, f"more than one HIP runtime mapped: {hip}"


@pytest.mark.parametrize("K,D", [(1, 16), (37, 64), (300, 128), (129, 256), (70, 512),
                                 (5000, 80), (33, 192)])
def test_norms(K, D):
    _, C, _ = W.gaussian_mixture(1, D, K, 5)
    got = km.kmeans_centroid_norms(dev(C)).cpu().numpy().astype(np.float64)
    ref = oracle.centroid_norms(C)
    assert np.allclose(got, ref, rtol=2e-6, atol=1e-6)
    C2 = C.copy()
    C2[-1] = C2[0]
    g2 = km.kmeans_centroid_norms(dev(C2)).cpu().numpy()
    assert g2[-1].tobytes() == g2[0].tobytes(), "identical rows, different norms"


SMALL = [  # (N, D, K): ragged tails in every dimension, several tiles
    (4133, 64, 275), (1000, 16, 37), (777, 128, 300), (2050, 256, 129),
    (513, 512, 70), (300, 80, 45), (64, 32, 1), (1, 16, 5), (257, 48, 1000),
    (3000, 128, 2049),
]


@pytest.mark.parametrize("path,count", [(km.PATH_AUTO, 0), (km.PATH_DIRECT, 0),
                                        (km.PATH_DIRECT, 1), (km.PATH_SPLIT, 0),
                                        (km.PATH_SPLIT, 3)],
                         ids=["auto", "wide", "narrow", "split", "split3"])
@pytest.mark.parametrize("N,D,K", SMALL)
def test_small_shapes(N, D, K, path, count):
    X, C, _ = W.gaussian_mixture(N, D, K, 1000 + N + K)
    lab, md = run(X, C, path, count)
    parity.check(X, C, lab, md)


@pytest.mark.parametrize("seed", W.SEEDS)
def test_workload1_full(seed):
    X, C, _ = W.make_config(1, seed)
    lab, md = run(X, C)
    st = parity.check(X, C, lab, md)
    assert st["bad_strict"] == 0


@pytest.mark.parametrize("seed", W.SEEDS)
def test_workload2_full(seed):
    X, C, _ = W.make_config(2, seed)
    lab, md = run(X, C)
    parity.check(X, C, lab, md)


@pytest.mark.parametrize("seed", W.SEEDS)
def test_workload3_full(seed):
    X, C, _ = W.make_config(3, seed)
    lab, md = run(X, C)
    parity.check(X, C, lab, md)


def test_workload4_full():
    X, C, _ = W.make_config(4, 17)
    lab, md = run(X, C)
    parity.check(X, C, lab, md)


# The pages' 13 benchmark shapes.  The pages checked the first 2048
# assignments of every seeded set; here those plus random and tail samples
# (all three seeds up to N = 262144, seed 17 at N = 1048576).
SWEEP_CASES = [(n, d, k, seed) for (n, d, k) in W.SWEEP_SHAPES
               for seed in (W.SEEDS if n <= 262144 else W.SEEDS[:1])]


@pytest.mark.parametrize("N,D,K,seed", SWEEP_CASES,
                         ids=[f"{n}x{d}x{k}-s{s}" for n, d, k, s in SWEEP_CASES])
def test_sweep_shape_sampled(N, D, K, seed):
    X, C, _ = W.gaussian_mixture(N, D, K, seed)
    lab, md = run(X, C)
    parity.check(X, C, lab, md, idx=parity.sample_indices(N, seed, 2048, 512, 64))


# Every point of the sweep shapes whose dispatch no workload covers: the
# K-split path with four ranges (65536 x 64 x 16384, every seed) and the
# wide direct path at N = 1M, D = 128 (seed 17).
FULL_SWEEP_CASES = [(65536, 64, 16384, s) for s in W.SEEDS] + [(1048576, 128, 4096, 17)]


@pytest.mark.parametrize("N,D,K,seed", FULL_SWEEP_CASES,
                         ids=[f"{n}x{d}x{k}-s{s}" for n, d, k, s in FULL_SWEEP_CASES])
def test_sweep_shape_every_point(N, D, K, seed):
    X, C, _ = W.gaussian_mixture(N, D, K, seed)
    plan = km.kmeans_plan(N, D, K, torch.cuda.get_device_properties(0).multi_processor_count)
    if N == 65536:
        assert plan["path"] == km.PATH_SPLIT and plan["splits"] == 4, plan
    lab, md = run(X, C)
    parity.check(X, C, lab, md)


@pytest.fixture(scope="module", params=W.SEEDS, ids=[f"s{s}" for s in W.SEEDS])
def workload5(request):
    """The adversarial workload at each of the three seeds (generated and
    assigned once per seed; the tests below run per seed)."""
    X, C, meta = W.make_config(5, request.param)
    lab, md = run(X, C)
    return X, C, meta, lab, md


def test_workload5_full(workload5):
    X, C, meta, lab, md = workload5
    parity.check(X, C, lab, md)


def test_workload5_nan_slice(workload5):
    X, C, meta, lab, md = workload5
    parity.check(X, C, lab, md, idx=meta["nan_slice"])


def test_workload5_dyadic_ties_bit_exact(workload5):
    X, C, meta, lab, md = workload5
    idx = meta["dyadic_points"]
    assert np.array_equal(lab[idx], meta["dyadic_labels"])
    assert np.array_equal(md[idx].astype(np.float64), meta["dyadic_sqdist"])


def test_workload5_persistent_and_split_bitwise(workload5):
    """The adversarial set (non-finite slice, duplicates, equal rows, dyadic
    ties) through the persistent and a K-split path: bitwise the direct
    path's outputs."""
    X, C, meta, lab, md = workload5
    for path, count in ((km.PATH_PERSISTENT, 0), (km.PATH_PERSISTENT, 37), (km.PATH_SPLIT, 3)):
        lp, mp = run(X, C, path, count)
        assert np.array_equal(lab, lp), (path, count)
        assert md.tobytes() == mp.tobytes(), (path, count)


def test_workload5_duplicates_and_equal_rows(workload5):
    X, C, meta, lab, md = workload5
    for s, t in meta["dup_pairs"]:
        assert not np.any(lab == t), f"duplicate row {t} beat its copy {s}"
    eq = meta["equal_rows"]
    assert not np.any(np.isin(lab, eq[1:])), "a non-lowest equal row won"
    near_eq = np.flatnonzero(np.isin(meta["generating_centre"], eq))
    near_eq = near_eq[near_eq >= W.NAN_SLICE_POINTS]
    assert len(near_eq) > 0
    parity.check(X, C, lab, md, idx=near_eq)
    srcs = meta["dup_pairs"][:, 0]
    near_dup = np.flatnonzero(np.isin(meta["generating_centre"], srcs))
    near_dup = near_dup[near_dup >= W.NAN_SLICE_POINTS][:2048]
    assert len(near_dup) > 0
    parity.check(X, C, lab, md, idx=near_dup)


# Every pair of rows inside one 32-row tile, and a few triples, made
# bitwise identical; the points sit next to the copied row, so the copies are
# each point's nearest centroids with exactly equal scores and the lowest
# index must win.  Covers the in-lane slot search (which rows a lane holds
# depends on the MFMA layout: D = 64 and 512 use one, 128 and 256 the other)
# and the merge across the lanes of a point.
def _tile_ties(D, seed):
    rng = np.random.default_rng(seed)
    groups = [(i, j) for i in range(32) for j in range(i + 1, 32)]
    groups += [(0, 16, 17), (3, 19, 31), (4, 8, 12), (0, 1, 2), (28, 29, 30)]
    per = 4                                        # points per tile
    K = 32 * len(groups)
    C = rng.standard_normal((K, D), dtype=np.float32)
    X = np.empty((per * len(groups), D), dtype=np.float32)
    want = np.empty(per * len(groups), dtype=np.int64)
    for t, g in enumerate(groups):
        base = 32 * t
        for r in g[1:]:
            C[base + r] = C[base + g[0]]
        X[per * t:per * (t + 1)] = C[base + g[0]] + 0.01 * rng.standard_normal((per, D), dtype=np.float32)
        want[per * t:per * (t + 1)] = base + g[0]
    return W.f32_to_bf16_bits(X), W.f32_to_bf16_bits(C), want


@pytest.mark.parametrize("D", [64, 128, 256, 512])
def test_ties_inside_a_tile_every_row_pair(D):
    X, C, want = _tile_ties(D, 1000 + D)
    ref = oracle.assign(X, C)
    assert np.array_equal(ref["labels"], want)     # the construction does what it says
    # narrow tiles save the improving tile's scores and search them after the
    # loop; wide tiles search on the spot: both must find the lowest row
    for path, count in ((km.PATH_AUTO, 0), (km.PATH_DIRECT, 1), (km.PATH_DIRECT, 0),
                        (km.PATH_SPLIT, 3)):
        lab, md = run(X, C, path, count)
        bad = np.flatnonzero(lab != want)
        assert bad.size == 0, (D, path, [(int(b), int(lab[b]), int(want[b])) for b in bad[:5]])
        parity.check(X, C, lab, md)


def test_nonfinite_centroids():
    X, C, _ = W.gaussian_mixture(700, 64, 300, 77)
    C[3, 5] = W.BF16_QNAN
    C[40, 7] = W.BF16_PINF
    C[41, 9] = W.BF16_NINF
    C[299, 0] = W.BF16_PINF
    X[10, 3] = W.BF16_PINF
    X[11, 4] = W.BF16_NINF
    X[12, 5] = W.BF16_QNAN
    for path, count in ((km.PATH_DIRECT, 0), (km.PATH_DIRECT, 1), (km.PATH_SPLIT, 0),
                        (km.PATH_SPLIT, 3), (km.PATH_PERSISTENT, 0)):
        lab, md = run(X, C, path, count)
        parity.check(X, C, lab, md)


def test_all_scores_infinite_or_nan():
    """Every score +inf or NaN: lowest +inf index wins, else 0 (cold path)."""
    D = 32
    x = np.zeros((3, D), np.uint16)
    x[:, 0] = W.dyadic_to_bf16_bits(np.array([-1]), 0)[0]
    x[2, 1] = W.BF16_QNAN
    C = np.zeros((70, D), np.uint16)
    C[:, 0] = W.BF16_PINF             # x_0 = -1: score +inf for every row
    C[0, 2] = W.BF16_QNAN             # row 0: NaN score
    C[1, 1] = W.BF16_NINF             # row 1 with x_1 = 0: inf*0 -> NaN
    lab, md = run(x, C, km.PATH_DIRECT)
    lab2, md2 = run(x, C, km.PATH_SPLIT, 2)
    lab3, md3 = run(x, C, km.PATH_PERSISTENT, 0)
    assert lab[0] == 2 and lab[1] == 2 and lab[2] == 0
    assert np.isinf(md[0]) and np.isnan(md[2])
    assert np.array_equal(lab, lab2) and np.array_equal(lab, lab3)
    assert md.tobytes() == md3.tobytes()
    parity.check(x, C, lab, md)


def test_zero_and_signed_zero_points():
    X, C, _ = W.gaussian_mixture(200, 64, 100, 78)
    X[0] = W.BF16_PZERO
    X[1] = W.BF16_NZERO
    X[2, ::2] = W.BF16_NZERO
    lab, md = run(X, C)
    parity.check(X, C, lab, md)
    assert lab[0] == lab[1]


def test_denormal_inputs():
    """bf16 denormals in points and centroids (exponent bits zero): products
    of them underflow in fp32, so scores tie or nearly tie; the outputs must
    still satisfy the acceptance rule and be finite."""
    rng = np.random.default_rng(83)
    X, C, _ = W.gaussian_mixture(500, 64, 90, 83)
    X = X.copy()
    C = C.copy()
    den_x = rng.integers(1, 0x80, size=X.shape).astype(np.uint16) | (
        rng.integers(0, 2, size=X.shape).astype(np.uint16) << 15)
    den_c = rng.integers(1, 0x80, size=C.shape).astype(np.uint16)
    X[:100] = den_x[:100]                       # all-denormal points
    X[100:200, ::3] = den_x[100:200, ::3]       # some denormal coordinates
    C[:30] = den_c[:30]                         # all-denormal centroids
    C[30:60, ::2] = den_c[30:60, ::2]
    lab, md = run(X, C)
    assert np.all(np.isfinite(md))
    parity.check(X, C, lab, md)


def test_single_centroid():
    X, C, _ = W.gaussian_mixture(1000, 128, 1, 79)
    lab, md = run(X, C)
    assert np.all(lab == 0)
    parity.check(X, C, lab, md)


def test_empty_input():
    C = dev(W.gaussian_mixture(1, 64, 10, 80)[1])
    X = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    n = km.kmeans_centroid_norms(C)
    lab, md = km.kmeans_assign(X, C, n)
    torch.cuda.synchronize()
    assert lab.numel() == 0 and md.numel() == 0


def test_maximum_d_and_large_k():
    X, C, _ = W.gaussian_mixture(600, 512, 3000, 81)
    lab, md = run(X, C)
    parity.check(X, C, lab, md)


def test_centroids_over_2gib():
    """70M centroid rows of D=16 (2.24 GB) at a large N: one buffer resource
    would exceed its 32-bit range, so the plan splits K.  Every row is a far
    constant except 256 near rows at the start and 256 past the 2 GiB mark,
    so the oracle needs only the distinct rows."""
    N, D, K = 262144, 16, 70_000_000
    plan = km.kmeans_plan(N, D, K)
    assert plan["path"] == km.PATH_SPLIT and plan["splits"] >= 2
    X, near, _ = W.gaussian_mixture(N, D, 512, 140)
    far = W.f32_to_bf16_bits(np.full(D, 40.0, np.float32))
    C = np.empty((K, D), np.uint16)
    C[:] = far
    C[:256] = near[:256]
    C[K - 256:] = near[256:]
    lab, md = run(X, C)
    del C
    mapped = np.where(lab < 256, lab + 1, np.where(lab >= K - 256, lab - (K - 256) + 257, 0))
    C_eff = np.vstack([far[None, :], near])
    parity.check(X, C_eff, mapped, md, idx=parity.sample_indices(N, 141, 1024, 2048, 64))
    assert np.count_nonzero(lab >= K - 256) > N // 4     # the far end of C was read


def test_large_k_small_n():
    X, C, _ = W.gaussian_mixture(300, 64, 70000, 82)
    lab, md = run(X, C)
    parity.check(X, C, lab, md)


# ---------------------------------------------------------------- metamorphic

@pytest.mark.parametrize("N,D,K", [(32768, 128, 4096), (16384, 32, 4096), (98304, 128, 1100),
                                   (24576, 128, 4000)])
def test_underfilled_shapes_take_their_plan_and_match(N, D, K):
    """Shapes where wide tiles leave CUs idle: the automatic plan (a K split,
    or direct wide tiles rather than a two-round split) against the oracle on
    a sample, and bitwise against narrow tiles."""
    X, C, _ = W.gaussian_mixture(N, D, K, 150 + D)
    lab, md = run(X, C)
    parity.check(X, C, lab, md, idx=parity.sample_indices(N, 151, 1024, 1024, 64))
    ln, mn = run(X, C, km.PATH_DIRECT, 1)
    assert np.array_equal(lab, ln) and md.tobytes() == mn.tobytes()


@pytest.mark.parametrize("N,D,K", [(5000, 64, 4096), (20000, 128, 1000), (3000, 256, 777)])
def test_split_equals_direct_bitwise(N, D, K):
    X, C, _ = W.gaussian_mixture(N, D, K, 90 + D)
    ld, md_d = run(X, C, km.PATH_DIRECT)
    for splits in (0, 2, 3, 7):
        ls, md_s = run(X, C, km.PATH_SPLIT, splits)
        assert np.array_equal(ld, ls)
        assert md_d.tobytes() == md_s.tobytes()


@pytest.mark.parametrize("N,D,K", [(5000, 64, 4096), (3000, 128, 700), (2500, 16, 1000),
                                   (700, 48, 300), (1100, 256, 129), (70000, 64, 600)])
def test_narrow_tiles_equal_wide_bitwise(N, D, K):
    """Narrow point tiles only regroup points over workgroups: every score,
    and so every output, is bitwise that of the wide tiles."""
    X, C, _ = W.gaussian_mixture(N, D, K, 120 + D)
    lw, mw = run(X, C, km.PATH_DIRECT, 0)
    ln, mn = run(X, C, km.PATH_DIRECT, 1)
    assert np.array_equal(lw, ln)
    assert mw.tobytes() == mn.tobytes()


@pytest.mark.parametrize("N,D,K", [(300000, 128, 520), (262244, 128, 300), (270000, 64, 700)])
def test_wave_tail_launch_equals_wide_bitwise(N, D, K):
    """A partial last round of wide tiles runs as a second launch of narrow
    tiles on offset pointers; outputs must be bitwise those of one wide
    launch, and correct around the boundary between the two launches."""
    plan = km.kmeans_plan(N, D, K)
    wide = 512 if D == 128 else 1024                # points of a wide workgroup
    head = (N // wide // 256) * 256 * wide          # whole rounds: one per CU, 256 CUs
    assert plan["workgroups"] > head // wide        # a tail launch is planned
    X, C, _ = W.gaussian_mixture(N, D, K, 130 + D)
    la, ma = run(X, C)
    lw, mw = run(X, C, km.PATH_DIRECT, 0)
    assert np.array_equal(la, lw)
    assert ma.tobytes() == mw.tobytes()
    idx = np.unique(np.concatenate([np.arange(head - 64, min(N, head + 64)),
                                    parity.sample_indices(N, 131, 256, 512, 64)]))
    parity.check(X, C, la, ma, idx=idx)


@pytest.mark.parametrize("N,D,K,count", [
    (5000, 64, 4096, 0),        # fewer tiles than CUs: one workgroup per tile
    (300000, 128, 520, 0),      # 586 tiles over one workgroup per CU
    (300000, 128, 520, 7),      # seven workgroups draw ~580 tickets
    (100000, 16, 300, 3), (40000, 32, 257, 5), (70000, 256, 700, 0), (20000, 512, 300, 2),
    (9000, 48, 129, 4), (1000, 80, 4000, 1),
])
def test_persistent_equals_direct_bitwise(N, D, K, count):
    """The persistent path runs the same tiles as the direct path, in an order
    set by a queue: every output must be bitwise the direct path's, on a first
    and a second call (the queue must be back at zero after a launch)."""
    X, C, _ = W.gaussian_mixture(N, D, K, 140 + D)
    ld, md = run(X, C, km.PATH_DIRECT, 0)
    for _ in range(2):
        lp, mp = run(X, C, km.PATH_PERSISTENT, count)
        assert np.array_equal(ld, lp)
        assert md.tobytes() == mp.tobytes()
    parity.check(X, C, lp, mp, idx=parity.sample_indices(N, 141, 256, 512, 64))


def test_persistent_queue_per_stream_and_after_release():
    """Each stream has its own queue; a released queue is made again, zeroed,
    on the stream's next call."""
    X, C, _ = W.gaussian_mixture(200000, 128, 300, 142)
    ld, md = run(X, C, km.PATH_DIRECT, 0)
    Xd, Cd = dev(X), dev(C)
    n = km.kmeans_centroid_norms(Cd)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for rnd in range(3):
        for s in streams:
            with torch.cuda.stream(s):
                outs.append(km.kmeans_assign_path(Xd, Cd, n, km.PATH_PERSISTENT, 5))
        if rnd == 1:
            for s in streams:
                with torch.cuda.stream(s):
                    km.kmeans_release_workspace()
    torch.cuda.synchronize()
    for lab, mdist in outs:
        assert np.array_equal(ld, lab.cpu().numpy())
        assert md.tobytes() == mdist.cpu().numpy().tobytes()


def test_deterministic_repeat():
    X, C, _ = W.make_config(2, 29)
    a = run(X, C)
    b = run(X, C)
    assert np.array_equal(a[0], b[0]) and a[1].tobytes() == b[1].tobytes()


def test_point_permutation_bitwise():
    X, C, _ = W.gaussian_mixture(9000, 128, 700, 91)
    lab, md = run(X, C)
    perm = np.random.default_rng(1).permutation(X.shape[0])
    lp, mp = run(X[perm], C)
    assert np.array_equal(lab[perm], lp) and md[perm].tobytes() == mp.tobytes()


def test_centroid_permutation():
    X, C, _ = W.gaussian_mixture(9000, 64, 700, 92)
    lab, md = run(X, C)
    perm = np.random.default_rng(2).permutation(C.shape[0])
    lp, mp = run(X, C[perm])
    ref = oracle.assign(X, C)
    with np.errstate(invalid="ignore"):
        strict = (ref["second"] - ref["best"]) >= 1e-3 * (np.abs(ref["best"]) + 1)
    # label j under C[perm] is original row perm[j]
    assert np.array_equal(perm[lp][strict], lab[strict])
    assert md[strict].tobytes() == mp[strict].tobytes()


@pytest.mark.parametrize("a", [-4, 3])
def test_power_of_two_scaling_bitwise(a):
    X, C, _ = W.gaussian_mixture(4000, 128, 500, 93)
    lab, md = run(X, C)
    f = np.float32(2.0 ** a)
    Xs = W.f32_to_bf16_bits(W.bf16_bits_to_f32(X) * f)
    Cs = W.f32_to_bf16_bits(W.bf16_bits_to_f32(C) * f)
    ls, ms = run(Xs, Cs)
    assert np.array_equal(lab, ls)
    assert np.array_equal(md.astype(np.float64) * 4.0 ** a, ms.astype(np.float64))


def test_non_default_stream():
    X, C, _ = W.gaussian_mixture(3000, 64, 500, 94)
    Xd, Cd = dev(X), dev(C)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        n = km.kmeans_centroid_norms(Cd)
        lab, md = km.kmeans_assign(Xd, Cd, n)
    s.synchronize()
    parity.check(X, C, lab.cpu().numpy(), md.cpu().numpy())


def test_api_errors_on_device_tensors():
    C = dev(W.gaussian_mixture(1, 64, 10, 95)[1])
    X = dev(W.gaussian_mixture(33, 64, 10, 95)[0])
    n = km.kmeans_centroid_norms(C)
    bad = X.view(-1)[1:1 + 32 * 64].view(32, 64)   # 2-byte offset
    with pytest.raises(km.KmeansError) as e:
        km.kmeans_assign(bad, C, n)
    assert e.value.status == km.KMEANS_ERR_ALIGNMENT
    Xw = dev(W.gaussian_mixture(8, 40, 10, 95)[0])
    Cw = dev(W.gaussian_mixture(1, 40, 10, 95)[1])
    with pytest.raises(km.KmeansError) as e:
        km.kmeans_centroid_norms(Cw)
    assert e.value.status == km.KMEANS_ERR_UNSUPPORTED


def test_output_tensors_are_validated_before_any_launch():
    """The C ABI sees only pointers, so the binding checks every caller-given
    output (and the norms) before the call: a wrong dtype, a short tensor, a
    strided view or another device raises ValueError and nothing is written."""
    X = dev(W.gaussian_mixture(100, 64, 10, 96)[0])
    C = dev(W.gaussian_mixture(1, 64, 10, 96)[1])
    n = km.kmeans_centroid_norms(C)
    N = X.shape[0]
    good_lab = torch.full((N,), -7, dtype=torch.int32, device="cuda")
    good_md = torch.full((N,), -7.0, dtype=torch.float32, device="cuda")
    bad_outputs = [
        dict(labels=torch.full((N,), -7, dtype=torch.int64, device="cuda")),
        dict(labels=torch.full((N - 1,), -7, dtype=torch.int32, device="cuda")),
        dict(labels=torch.full((2 * N,), -7, dtype=torch.int32, device="cuda")[::2]),
        dict(labels=torch.full((N,), -7, dtype=torch.int32)),
        dict(min_dist=torch.full((N,), -7.0, dtype=torch.float64, device="cuda")),
        dict(min_dist=torch.full((N - 3,), -7.0, dtype=torch.float32, device="cuda")),
    ]
    for bad in bad_outputs:
        kw = dict(labels=good_lab, min_dist=good_md)
        kw.update(bad)
        with pytest.raises(ValueError):
            km.kmeans_assign(X, C, n, **kw)
        with pytest.raises(ValueError):
            km.kmeans_assign_path(X, C, n, km.PATH_SPLIT, 2, **kw)
        torch.cuda.synchronize()
        for t in bad.values():
            assert bool((t == -7).all()), "an output was written before the check"
    assert bool((good_lab == -7).all()) and bool((good_md == -7.0).all())
    for bad_n in (n[:-1], n.double(), torch.cat([n, n])[::2], n.cpu()):
        with pytest.raises(ValueError):
            km.kmeans_assign(X, C, bad_n)
    short = torch.full((9,), -7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        km.kmeans_centroid_norms(C, norms=short)
    torch.cuda.synchronize()
    assert bool((short == -7.0).all())


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("offset", [1.5, 2.5, 10.0, 30.0, 200.0])
def test_data_far_from_origin(offset, D):
    """Half of the coordinates shifted by `offset`: ||x||^2 is then tens to
    millions of times the distance to the nearest centroid, so a distance
    formed as ||x||^2 + score loses accuracy as the shift grows; the kernel
    sums (x - c)^2 directly past a ratio that depends on D, and min_dist must
    meet the acceptance rule on both sides of that switch (the small shifts
    sit just below and just above it).  Split and persistent must equal the
    direct path bit for bit."""
    rng = np.random.default_rng(int(offset * 10) + D)
    N, K = 6000, 300
    mu = rng.standard_normal((K, D), dtype=np.float32)
    shift = np.zeros(D, np.float32)
    shift[::2] = offset
    a = rng.integers(0, K, N)
    X = W.f32_to_bf16_bits(mu[a] + shift + 0.1 * rng.standard_normal((N, D), dtype=np.float32))
    C = W.f32_to_bf16_bits(mu + shift + 0.05 * rng.standard_normal((K, D), dtype=np.float32))
    lab, md = run(X, C)
    st = parity.check(X, C, lab, md)
    assert st["bad_dist"] == 0
    for path, count in ((km.PATH_SPLIT, 3), (km.PATH_PERSISTENT, 2)):
        ls, ms = run(X, C, path, count)
        assert np.array_equal(lab, ls) and md.tobytes() == ms.tobytes(), (path, count)
