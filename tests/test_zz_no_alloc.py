"""kmeans_assign_static (no allocation inside the call) against kmeans_assign,
through the C ABI, on an MI355X: two calls in a row on the K-split path, the
second with a smaller input, each bitwise equal to kmeans_assign's outputs
and within the acceptance rule against the oracle; a split plan too large
for the fixed buffer is refused before any launch."""

import ctypes

import numpy as np
import pytest

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


def test_static_scratch_matches_workspace_path_twice():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    lib = km.load_library()
    stream = torch.cuda.current_stream()
    for N, D, K, seed in ((65536, 64, 16384, 17), (20000, 64, 8192, 29)):
        plan = km.kmeans_plan(N, D, K, cus)
        assert plan["path"] == km.PATH_SPLIT, plan          # the path that uses scratch
        X, C, _ = W.gaussian_mixture(N, D, K, seed)
        Xd, Cd = dev(X), dev(C)
        n = km.kmeans_centroid_norms(Cd)
        lab_s = torch.full((N,), -1, dtype=torch.int32, device="cuda")
        md_s = torch.full((N,), -1.0, dtype=torch.float32, device="cuda")
        st = lib.kmeans_assign_static(Xd.data_ptr(), Cd.data_ptr(), n.data_ptr(), N, D, K,
                                      lab_s.data_ptr(), md_s.data_ptr(),
                                      ctypes.c_void_p(stream.cuda_stream))
        assert st == km.KMEANS_OK, lib.kmeans_last_error()
        lab_w, md_w = km.kmeans_assign(Xd, Cd, n)
        torch.cuda.synchronize()
        assert torch.equal(lab_s, lab_w), (N, D, K)
        assert md_s.cpu().numpy().tobytes() == md_w.cpu().numpy().tobytes(), (N, D, K)
        lab, md = lab_s.cpu().numpy(), md_s.cpu().numpy()
        parity.check(X, C, lab, md, idx=parity.sample_indices(N, seed, 2048, 1024, 64))
    # through the Python binding as well (same entry point)
    lab_b, md_b = km.kmeans_assign_static(Xd, Cd, n)
    torch.cuda.synchronize()
    assert torch.equal(lab_b, lab_w) and torch.equal(md_b, md_w)


def test_static_scratch_refuses_a_plan_larger_than_the_buffer():
    """Centroids over 2 GiB force two K-ranges; at N = 2^20 their scratch
    (20 MiB) exceeds the 16 MiB buffer: refused on the host, so the
    (never dereferenced) pointers below are never used."""
    lib = km.load_library()
    N, D, K = 1 << 20, 512, (1 << 21) + 64
    fake = ctypes.c_void_p(1 << 20)
    st = lib.kmeans_assign_static(fake, fake, fake, N, D, K, fake, fake, ctypes.c_void_p(0))
    assert st == km.KMEANS_ERR_UNSUPPORTED
    assert b"static buffer" in lib.kmeans_last_error()
