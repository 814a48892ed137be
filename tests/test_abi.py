"""C ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects bad arguments on the host before any HIP call."""

import ctypes
import os
import re

import pytest

import means_nearest_centroid_amd as km
from means_nearest_centroid_amd import build as kbuild


@pytest.fixture(scope="module")
def lib():
    srcs = kbuild.SOURCES + [os.path.join(kbuild.CSRC, "kmeans_internal.h"), km.HEADER]
    if not os.path.exists(km.LIBRARY) or any(
            os.path.getmtime(s) > os.path.getmtime(km.LIBRARY) for s in srcs):
        kbuild.build()
    return km.load_library()


def declared_functions():
    text = open(km.HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kmeans_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for f in ("kmeans_centroid_norms", "kmeans_assign", "kmeans_assign_static",
              "kmeans_assign_path",
              "kmeans_plan", "kmeans_update", "kmeans_update_path", "kmeans_release_workspace",
              "kmeans_last_error",
              "kmeans_abi_version"):
        assert f in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in the header but not exported"


def test_probe_library_exports_its_header():
    from means_nearest_centroid_amd import build as kbuild
    if not os.path.exists(kbuild.PROBE_LIBRARY):
        kbuild.build()
    probe = ctypes.CDLL(kbuild.PROBE_LIBRARY)
    header = os.path.join(os.path.dirname(km.HEADER), "kmeans_mfma_stream.h")
    text = re.sub(r"/\*.*?\*/", "", open(header).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(kmeans_[a-z_0-9]+)\s*\(", text)))
    assert names == ["kmeans_clock_sampler", "kmeans_mfma_stream", "kmeans_mfma_stream_threads"]
    for name in names:
        assert hasattr(probe, name)
    assert probe.kmeans_mfma_stream_threads() == 256
    f = probe.kmeans_mfma_stream
    f.argtypes = [ctypes.c_void_p] * 2 + [ctypes.c_int32] * 3 + [ctypes.c_void_p] * 2
    # invalid arguments are refused before any HIP call
    assert f(None, FAKE, 64, 10, 1, FAKE, NUL) == 1
    assert f(FAKE, FAKE, 0, 10, 1, FAKE, NUL) == 1
    assert f(FAKE, FAKE, 64, 10, 70000, FAKE, NUL) == 1
    assert f(FAKE_ODD, FAKE, 64, 10, 1, FAKE, NUL) == 1
    g = probe.kmeans_clock_sampler
    g.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    assert g(None, 8, 100, NUL) == 1
    assert g(FAKE, 0, 100, NUL) == 1
    assert g(FAKE, 2000, 100, NUL) == 1
    assert g(FAKE, 8, 0, NUL) == 1
    assert g(FAKE_ODD, 8, 100, NUL) == 1


def test_abi_version(lib):
    m = re.search(r"#define\s+KMEANS_ABI_VERSION\s+(\d+)", open(km.HEADER).read())
    assert lib.kmeans_abi_version() == int(m.group(1))


FAKE = ctypes.c_void_p(0x10000)        # never dereferenced: validation fails first
FAKE_ODD = ctypes.c_void_p(0x10002)    # 2-byte aligned only
NUL = ctypes.c_void_p(0)


def assign_status(lib, X=FAKE, C=FAKE, n=FAKE, N=10, D=64, K=5, lab=FAKE, md=FAKE):
    return lib.kmeans_assign(X, C, n, N, D, K, lab, md, NUL)


@pytest.mark.parametrize("kw,status", [
    (dict(N=-1), km.KMEANS_ERR_INVALID_ARG),
    (dict(K=0), km.KMEANS_ERR_INVALID_ARG),
    (dict(K=-3), km.KMEANS_ERR_INVALID_ARG),
    (dict(D=40), km.KMEANS_ERR_UNSUPPORTED),
    (dict(D=8), km.KMEANS_ERR_UNSUPPORTED),
    (dict(D=528), km.KMEANS_ERR_UNSUPPORTED),
    (dict(D=0), km.KMEANS_ERR_UNSUPPORTED),
    (dict(N=1 << 31), km.KMEANS_ERR_UNSUPPORTED),
    (dict(K=1 << 31), km.KMEANS_ERR_UNSUPPORTED),
    (dict(X=NUL), km.KMEANS_ERR_INVALID_ARG),
    (dict(C=NUL), km.KMEANS_ERR_INVALID_ARG),
    (dict(n=NUL), km.KMEANS_ERR_INVALID_ARG),
    (dict(lab=NUL), km.KMEANS_ERR_INVALID_ARG),
    (dict(md=NUL), km.KMEANS_ERR_INVALID_ARG),
    (dict(X=FAKE_ODD), km.KMEANS_ERR_ALIGNMENT),
    (dict(C=FAKE_ODD), km.KMEANS_ERR_ALIGNMENT),
    (dict(n=FAKE_ODD), km.KMEANS_ERR_ALIGNMENT),
    (dict(md=FAKE_ODD), km.KMEANS_ERR_ALIGNMENT),
])
def test_assign_rejects_bad_arguments(lib, kw, status):
    assert assign_status(lib, **kw) == status
    assert lib.kmeans_last_error().decode()


def test_assign_empty_is_noop(lib):
    # N == 0 returns before touching any pointer or the HIP runtime.
    assert assign_status(lib, X=NUL, C=NUL, n=NUL, lab=NUL, md=NUL, N=0) == km.KMEANS_OK
    assert lib.kmeans_last_error().decode() == ""


def test_assign_path_rejects_bad_plan(lib):
    st = lib.kmeans_assign_path(FAKE, FAKE, FAKE, 10, 64, 5, FAKE, FAKE, 7, 0, NUL)
    assert st == km.KMEANS_ERR_INVALID_ARG
    st = lib.kmeans_assign_path(FAKE, FAKE, FAKE, 10, 64, 5, FAKE, FAKE, 4, 0, NUL)
    assert st == km.KMEANS_ERR_INVALID_ARG
    st = lib.kmeans_assign_path(FAKE, FAKE, FAKE, 10, 64, 5, FAKE, FAKE, 2, -1, NUL)
    assert st == km.KMEANS_ERR_INVALID_ARG
    st = lib.kmeans_assign_path(FAKE, FAKE, FAKE, 10, 64, 5, FAKE, FAKE, 3, -1, NUL)
    assert st == km.KMEANS_ERR_INVALID_ARG


def test_norms_rejects_bad_arguments(lib):
    f = lib.kmeans_centroid_norms
    assert f(FAKE, -1, 64, FAKE, NUL) == km.KMEANS_ERR_INVALID_ARG
    assert f(FAKE, 5, 24, FAKE, NUL) == km.KMEANS_ERR_UNSUPPORTED
    assert f(NUL, 5, 64, FAKE, NUL) == km.KMEANS_ERR_INVALID_ARG
    assert f(FAKE, 5, 64, NUL, NUL) == km.KMEANS_ERR_INVALID_ARG
    assert f(FAKE_ODD, 5, 64, FAKE, NUL) == km.KMEANS_ERR_ALIGNMENT
    assert f(NUL, 0, 64, NUL, NUL) == km.KMEANS_OK


def test_plan_for_the_workloads(lib):
    from means_nearest_centroid_amd.workloads import CONFIGS
    plans = {i: km.kmeans_plan(c["N"], c["D"], c["K"]) for i, c in CONFIGS.items()}
    for i in (3, 4, 5):
        assert plans[i]["path"] == km.PATH_DIRECT and plans[i]["splits"] == 1
    assert plans[3]["points_per_wg"] == 512 and plans[4]["points_per_wg"] == 256
    for i in (1, 2):       # small N: narrow tiles (one 32-point block per wave)
        assert plans[i]["path"] == km.PATH_DIRECT and plans[i]["points_per_wg"] == 256
    for i, c in CONFIGS.items():
        p = plans[i]
        assert p["padded_d"] >= c["D"] and p["padded_d"] % 16 == 0
        assert p["workgroups"] * p["points_per_wg"] >= c["N"]
        assert p["splits"] * p["k_block"] >= 1


# Dispatch on the pages' 13 shapes for a 256-CU GPU, as (path, K-ranges,
# points per workgroup): narrow tiles where N alone cannot fill the GPU and K
# is at most 16 centroid blocks, the K-split above that, wide tiles at large N.
SWEEP_PLANS = {
    (65536, 64, 512): (1, 1, 256), (65536, 64, 4096): (1, 1, 256),
    (65536, 64, 16384): (2, 4, 1024), (65536, 128, 512): (1, 1, 256),
    (65536, 128, 4096): (1, 1, 256), (262144, 128, 4096): (1, 1, 512),
    (262144, 128, 16384): (1, 1, 512), (1048576, 128, 4096): (1, 1, 512),
    (65536, 256, 512): (1, 1, 256), (65536, 256, 4096): (1, 1, 256),
    (262144, 256, 4096): (1, 1, 256), (262144, 256, 16384): (1, 1, 256),
    (1048576, 256, 4096): (1, 1, 256),
}


def test_plan_for_the_sweep_shapes(lib):
    from means_nearest_centroid_amd.workloads import SWEEP_SHAPES
    assert set(SWEEP_SHAPES) == set(SWEEP_PLANS)
    for shape, want in SWEEP_PLANS.items():
        p = km.kmeans_plan(*shape, 256)
        assert (p["path"], p["splits"], p["points_per_wg"]) == want, shape
        assert km.kmeans_plan(*shape) == p      # 0 CUs: the MI355X default


@pytest.mark.parametrize("N,D,K,path,splits,wgs", [
    (32768, 128, 4096, km.PATH_SPLIT, 4, 64),      # narrow tiles would fill half the CUs
    (16384, 128, 4096, km.PATH_SPLIT, 8, 32),
    (16384, 32, 4096, km.PATH_SPLIT, 8, 16),
    (49152, 128, 16384, km.PATH_SPLIT, 2, 96),     # split count rounded down: one round
    (98304, 128, 4096, km.PATH_DIRECT, 1, 192),    # not a two-round split
    (40960, 64, 4096, km.PATH_DIRECT, 1, 160),     # narrow: the split has < 2x its workgroups
    (49152, 128, 4096, km.PATH_DIRECT, 1, 192),
])
def test_plan_when_wide_tiles_underfill(lib, N, D, K, path, splits, wgs):
    p = km.kmeans_plan(N, D, K, 256)
    assert (p["path"], p["splits"], p["workgroups"]) == (path, splits, wgs), p


def test_plan_follows_the_compute_unit_count(lib):
    assert km.kmeans_plan(65536, 128, 16384, 256)["splits"] == 2
    assert km.kmeans_plan(65536, 128, 16384, 128)["path"] == km.PATH_DIRECT
    assert km.kmeans_plan(65536, 128, 16384, 1024)["splits"] == 8   # one full round
    # narrow tiles only when they fit in one round
    assert km.kmeans_plan(65536, 64, 4096, 256)["points_per_wg"] == 256
    assert km.kmeans_plan(65536, 64, 4096, 64)["points_per_wg"] == 1024


@pytest.mark.parametrize("N,D,K", [(1, 16, 1), (100, 80, 7), (5000, 192, 3000),
                                   (70000, 512, 100000), (1 << 20, 64, 64)])
def test_plan_covers_every_point_and_centroid(lib, N, D, K):
    p = km.kmeans_plan(N, D, K)
    assert p["workgroups"] * p["points_per_wg"] >= N
    assert p["padded_d"] >= D and (p["padded_d"] & (p["padded_d"] - 1)) == 0
    assert 1 <= p["splits"] <= 64
    assert p["path"] in (km.PATH_DIRECT, km.PATH_SPLIT)
    if p["path"] == km.PATH_DIRECT:
        assert p["splits"] == 1


def test_centroids_over_2gib_are_split_or_refused(lib):
    # 2,100,000 rows of 1 KiB exceed one 2 GiB K-range: split, never direct.
    p = km.kmeans_plan(64, 512, 2100000)
    assert p["path"] == km.PATH_SPLIT and p["splits"] >= 2
    assert km.kmeans_plan(64, 512, 2000000)["path"] == km.PATH_SPLIT   # small N anyway
    for path in (km.PATH_DIRECT, km.PATH_PERSISTENT):
        st = lib.kmeans_assign_path(FAKE, FAKE, FAKE, 10, 512, 2100000, FAKE, FAKE, path, 0, NUL)
        assert st == km.KMEANS_ERR_UNSUPPORTED
    # Over 64 ranges of 2 GiB: unsupported on every path.
    with pytest.raises(km.KmeansError):
        km.kmeans_plan(64, 512, 200000000)
    st = lib.kmeans_assign(FAKE, FAKE, FAKE, 10, 512, 200000000, FAKE, FAKE, NUL)
    assert st == km.KMEANS_ERR_UNSUPPORTED


def test_plan_rejects_bad_shapes(lib):
    with pytest.raises(km.KmeansError):
        km.kmeans_plan(10, 72, 5)
    with pytest.raises(km.KmeansError):
        km.kmeans_plan(10, 64, 0)


def update_status(lib, X=FAKE, lab=FAKE, C=FAKE, N=10, D=64, K=5, Cn=FAKE, n=FAKE, cnt=FAKE,
                  m=NUL):
    return lib.kmeans_update(X, lab, C, N, D, K, Cn, n, cnt, m, NUL)


@pytest.mark.parametrize("kw,status", [
    (dict(N=-1), km.KMEANS_ERR_INVALID_ARG),
    (dict(K=0), km.KMEANS_ERR_INVALID_ARG),
    (dict(D=40), km.KMEANS_ERR_UNSUPPORTED),
    (dict(D=1024), km.KMEANS_ERR_UNSUPPORTED),
    (dict(N=1 << 31), km.KMEANS_ERR_UNSUPPORTED),
    (dict(K=1 << 31), km.KMEANS_ERR_UNSUPPORTED),
    (dict(X=NUL), km.KMEANS_ERR_INVALID_ARG),
    (dict(lab=NUL), km.KMEANS_ERR_INVALID_ARG),
    (dict(C=NUL), km.KMEANS_ERR_INVALID_ARG),
    (dict(Cn=NUL), km.KMEANS_ERR_INVALID_ARG),
    (dict(n=NUL), km.KMEANS_ERR_INVALID_ARG),
    (dict(cnt=NUL), km.KMEANS_ERR_INVALID_ARG),
    (dict(N=0, C=NUL), km.KMEANS_ERR_INVALID_ARG),    # outputs are written even at N = 0
    (dict(X=FAKE_ODD), km.KMEANS_ERR_ALIGNMENT),
    (dict(C=FAKE_ODD), km.KMEANS_ERR_ALIGNMENT),
    (dict(Cn=FAKE_ODD), km.KMEANS_ERR_ALIGNMENT),
    (dict(lab=ctypes.c_void_p(0x10001)), km.KMEANS_ERR_ALIGNMENT),
    (dict(m=ctypes.c_void_p(0x10001)), km.KMEANS_ERR_ALIGNMENT),
])
def test_update_rejects_bad_arguments(lib, kw, status):
    assert update_status(lib, **kw) == status
    assert lib.kmeans_last_error().decode()


@pytest.mark.parametrize("kw,path,status", [
    (dict(), -1, km.KMEANS_ERR_INVALID_ARG),
    (dict(), 3, km.KMEANS_ERR_INVALID_ARG),
    (dict(N=(1 << 24) + 1), km.UPDATE_BUCKETS, km.KMEANS_ERR_UNSUPPORTED),
    (dict(K=16385), km.UPDATE_BUCKETS, km.KMEANS_ERR_UNSUPPORTED),
    (dict(X=NUL), km.UPDATE_BUCKETS, km.KMEANS_ERR_INVALID_ARG),
])
def test_update_path_rejects_bad_arguments(lib, kw, path, status):
    a = dict(X=FAKE, lab=FAKE, C=FAKE, N=10, D=64, K=5, Cn=FAKE, n=FAKE, cnt=FAKE, m=NUL)
    a.update(kw)
    st = lib.kmeans_update_path(a["X"], a["lab"], a["C"], a["N"], a["D"], a["K"], a["Cn"],
                                a["n"], a["cnt"], a["m"], path, NUL)
    assert st == status
    assert lib.kmeans_last_error().decode()
