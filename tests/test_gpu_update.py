"""Centroid update (HIP, through the C ABI) against the fp64 oracle on an MI355X.

Labels are inputs here: the generator's generating centres with some points
relabelled at random and some stray labels outside [0, K) -- never labels
computed by the HIP path.  Acceptance rule: ``parity.check_update``.
"""

import functools

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
    km.load_library()
    return torch.device("cuda:0")


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


# Both update paths (the radix sort and the buckets) on every case that
# fits the bucket path; the automatic choice runs in the Lloyd test.
PATHS = pytest.mark.parametrize("path", [1, 2], ids=["sort", "buckets"])


def run_update(X, lab, C, with_means=True, inplace=False, path=0):
    Xd, Cd = dev(X), dev(C)
    ld = torch.from_numpy(np.ascontiguousarray(lab, dtype=np.int32)).cuda()
    Cn, n, cnt, m = km.kmeans_update(Xd, ld, Cd, C_new=Cd if inplace else None,
                                     with_means=with_means, path=path)
    ref_norms = km.kmeans_centroid_norms(Cn)
    torch.cuda.synchronize()
    out = dict(C_new=host_bits(Cn), norms=n.cpu().numpy(), counts=cnt.cpu().numpy(),
               means=m.cpu().numpy() if m is not None else None)
    assert out["norms"].tobytes() == ref_norms.cpu().numpy().tobytes(), \
        "update norms differ from kmeans_centroid_norms of the new rows"
    return out


def check(X, lab, C, out):
    return parity.check_update(X, lab, C, out["C_new"], out["norms"], out["counts"],
                               out["means"])


def noisy_labels(a, K, seed, relabel=0.05, stray=0.01):
    rng = np.random.default_rng(seed)
    lab = np.asarray(a, dtype=np.int32).copy()
    n = len(lab)
    r = rng.random(n) < relabel
    lab[r] = rng.integers(0, K, int(r.sum()))
    s = rng.random(n) < stray
    lab[s] = rng.choice(np.array([-1, K, K + 7, -(1 << 30), (1 << 31) - 1], dtype=np.int64),
                        int(s.sum())).astype(np.int32)
    return lab


SMALL = [  # (N, D, K): ragged everywhere, K > N, 1, 2 and 3 radix passes,
    # buckets of 1 to 4 clusters (the last one partly past K)
    (4133, 64, 275), (1000, 16, 37), (777, 128, 300), (2050, 256, 129), (513, 512, 70),
    (300, 80, 45), (64, 32, 1), (1, 16, 5), (257, 48, 1000), (3000, 128, 2049),
    (5000, 192, 70000), (20000, 96, 255), (20000, 112, 256),
    (9000, 64, 5000), (7000, 256, 9000), (6000, 512, 16384), (30000, 128, 12289),
    (9000, 64, 4095), (7000, 256, 3073),
    # buckets of 8 and 16 clusters (sorted by cluster in LDS) at odd D
    (5000, 80, 8000), (3000, 48, 16384), (4000, 192, 6000), (6000, 112, 12000),
]


@PATHS
@pytest.mark.parametrize("N,D,K", SMALL)
def test_small_shapes(N, D, K, path):
    if path == 2 and K > 16384:
        pytest.skip("K over the bucket path's limit (covered by the sort path)")
    X, C, a = W.gaussian_mixture(N, D, K, 300 + N + K)
    lab = noisy_labels(a, K, N)
    st = check(X, lab, C, run_update(X, lab, C, path=path))
    assert st["clusters"] == K


@PATHS
def test_more_than_two_million_points(path):
    """N over 2^21: the sort path's radix passes run their scan kernel (more
    than 128 sort tiles) and the bucket path's bin waves take their points in
    several batches (tiles of 8192 points)."""
    N, D, K = 3_000_000, 16, 300
    X, C, a = W.gaussian_mixture(N, D, K, 81)
    lab = noisy_labels(a, K, 81)
    st = check(X, lab, C, run_update(X, lab, C, path=path))
    assert st["clusters"] == K


@PATHS
def test_buckets_around_the_lds_slot_list(path):
    """About 2000 points per bucket of one cluster: most buckets keep all
    their slot words in LDS (four chunks of sums), those above 2048 take the
    chunk-by-chunk resolution, in the same call; each bucket workgroup
    thread owns ~8 points of two tiles, so some take a second round of
    slot-word loads."""
    N, D, K = 520_000, 16, 256
    X, C, a = W.gaussian_mixture(N, D, K, 82)
    lab = noisy_labels(a, K, 82)
    sizes = np.bincount(lab[(lab >= 0) & (lab < K)], minlength=K)
    assert sizes.max() > 2048 and (sizes <= 2048).sum() > K // 2
    st = check(X, lab, C, run_update(X, lab, C, path=path))
    assert st["clusters"] == K


@functools.lru_cache(maxsize=1)
def _largest_bucket_path_set():
    N, D, K = 1 << 24, 16, 4096
    X, C, a = W.gaussian_mixture(N, D, K, 83)
    return X, C, noisy_labels(a, K, 83)


@PATHS
def test_largest_bucket_path_shape(path):
    """N = 2^24, the bucket path's limit, with buckets of four clusters: the
    last point indices fill all 24 index bits of a sorted slot word next to
    its two cluster bits, and the bin tiles hold 32768 points each."""
    X, C, lab = _largest_bucket_path_set()
    K = C.shape[0]
    st = check(X, lab, C, run_update(X, lab, C, path=path))
    assert st["clusters"] == K


@PATHS
def test_skewed_and_chunk_aligned_clusters(path):
    """One cluster holding most points (its rows span hundreds of reduce
    chunks), and cluster sizes that put boundaries exactly on chunk edges."""
    N, D, K = 40000, 128, 64
    X, C, _ = W.gaussian_mixture(N, D, K, 71)
    sizes = [128, 128, 256, 1, 127, 129, 255, 257, 0, 384]
    lab = np.full(N, 5, dtype=np.int32)                 # the big cluster
    pos = 0
    for k, s in enumerate(sizes):
        if k == 5:
            continue
        lab[pos:pos + s] = k
        pos += s
    rng = np.random.default_rng(72)
    big = np.flatnonzero(lab == 5)
    lab[rng.choice(big, 500, replace=False)] = rng.integers(10, K, 500)
    lab = lab[rng.permutation(N)]
    out = run_update(X, lab, C, path=path)
    check(X, lab, C, out)
    assert out["counts"][8] == 0 and out["counts"][5] > 30000


@PATHS
def test_large_bucket_of_sixteen_clusters(path):
    """K = 16384 (buckets of 16 clusters) with bucket 0 holding over 2048
    points (three large clusters): it is sorted and summed 512 slots at a
    time and its clusters' runs cross chunk edges and wave quarters; the
    other buckets fit LDS whole."""
    N, D, K = 40000, 64, 16384
    X, C, a = W.gaussian_mixture(N, D, K, 79)
    lab = noisy_labels(a, K, 79)
    rng = np.random.default_rng(80)
    idx = rng.permutation(N)
    lab[idx[:5000]] = 5                                  # bucket 0: clusters 0..15
    lab[idx[5000:5000 + 512 - 1]] = 6
    lab[idx[5511:5511 + 300]] = 15
    assert (lab[(lab >= 0) & (lab < 16)].size) > 2048
    out = run_update(X, lab, C, path=path)
    st = check(X, lab, C, out)
    assert st["clusters"] == K and out["counts"][5] >= 5000


@PATHS
def test_all_points_one_cluster_and_all_stray(path):
    X, C, _ = W.gaussian_mixture(9000, 64, 20, 73)
    lab = np.full(9000, 13, dtype=np.int32)
    check(X, lab, C, run_update(X, lab, C, path=path))
    lab = np.full(9000, -5, dtype=np.int32)
    out = run_update(X, lab, C, path=path)
    check(X, lab, C, out)
    assert np.array_equal(out["C_new"], C) and not out["counts"].any()


@PATHS
def test_no_points(path):
    _, C, _ = W.gaussian_mixture(1, 128, 300, 74)
    X = np.zeros((0, 128), np.uint16)
    out = run_update(X, np.zeros(0, np.int32), C, path=path)
    assert np.array_equal(out["C_new"], C) and not out["counts"].any()
    assert np.array_equal(out["means"], parity._widen(C).astype(np.float32))


@PATHS
def test_single_cluster(path):
    X, C, _ = W.gaussian_mixture(5000, 256, 1, 75)
    lab = np.zeros(5000, np.int32)
    lab[::97] = 3
    out = run_update(X, lab, C, path=path)
    check(X, lab, C, out)
    assert out["counts"][0] == 5000 - len(lab[::97])


@PATHS
def test_in_place_and_without_means_match(path):
    X, C, a = W.gaussian_mixture(6000, 128, 500, 76)
    lab = noisy_labels(a, 500, 76, relabel=0.3)
    lab[lab == 17] = 18                                  # an empty cluster
    out = run_update(X, lab, C, path=path)
    check(X, lab, C, out)
    out2 = run_update(X, lab, C, with_means=False, inplace=True, path=path)
    assert np.array_equal(out["C_new"], out2["C_new"])
    assert out["norms"].tobytes() == out2["norms"].tobytes()
    assert np.array_equal(out["counts"], out2["counts"])


@PATHS
def test_repeat_calls_are_bitwise_identical(path):
    X, C, a = W.gaussian_mixture(65536, 64, 4096, 77)
    lab = noisy_labels(a, 4096, 77)
    outs = [run_update(X, lab, C, path=path) for _ in range(3)]
    for o in outs[1:]:
        for key in ("C_new", "norms", "counts", "means"):
            assert outs[0][key].tobytes() == o[key].tobytes(), key
    check(X, lab, C, outs[0])


@PATHS
def test_nonfinite_points(path):
    X, C, a = W.gaussian_mixture(3000, 64, 40, 78)
    lab = a.astype(np.int32)
    X[10, 3] = W.BF16_QNAN
    X[11, 4] = W.BF16_PINF
    X[12, 5] = W.BF16_NINF
    X[13, 6] = W.BF16_PINF
    X[14, 6] = W.BF16_NINF
    lab[13] = lab[14]                                    # +inf and -inf: NaN mean
    X[15] = W.BF16_NZERO
    out = run_update(X, lab, C, path=path)
    check(X, lab, C, out)
    m = out["means"]
    assert np.isnan(m[lab[10], 3]) and np.isnan(m[lab[13], 6])
    assert m[lab[11], 4] == np.inf and m[lab[12], 5] == -np.inf


@PATHS
@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_workload_full(cfg, path):
    X, C, meta = W.make_config(cfg, 17)
    K = C.shape[0]
    if path == 2 and K > 16384:
        pytest.skip("K over the bucket path's limit (covered by the sort path)")
    lab = noisy_labels(meta["generating_centre"], K, cfg)
    st = check(X, lab, C, run_update(X, lab, C, path=path))
    assert st["elements"] > 0


def test_lloyd_iterations_on_gpu():
    """assign -> update -> assign ...: the update's norms are what the
    norms pre-pass gives for the new rows, the counts cover every point, and
    the mean squared distance does not grow by more than the bf16 rounding
    of the centroids allows (Lloyd's monotone descent)."""
    X, C, _ = W.gaussian_mixture(65536, 128, 1024, 79)
    Xd, Cd = dev(X), dev(C)
    norms = km.kmeans_centroid_norms(Cd)
    prev = None
    for _ in range(4):
        labels, md = km.kmeans_assign(Xd, Cd, norms)
        cur = float(md.double().mean())
        if prev is not None:
            assert cur <= prev * (1 + 1e-3), (cur, prev)
        prev = cur
        Cd, norms, counts, _ = km.kmeans_update(Xd, labels, Cd)
        torch.cuda.synchronize()
        assert int(counts.sum()) == X.shape[0]
        assert torch.equal(norms, km.kmeans_centroid_norms(Cd))
