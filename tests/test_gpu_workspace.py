"""The per-stream workspace (HIP, through the C ABI) on an MI355X.

kmeans_assign's K-split path and kmeans_update keep their scratch in one
device buffer per (device, stream) between calls; it grows in stream order
and is never shared between streams.  Calls here are queued back to back,
growing and shrinking the buffer with earlier calls still in flight, on
several streams and from several host threads, and every output is checked
against a result that never touched a workspace: the direct path for the
assignment (split and direct compute the same scores, so outputs agree
bitwise) and the fp64 oracle's acceptance rule for the update.
"""

import threading

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


def inputs(N, D, K, seed):
    X, C, a = W.gaussian_mixture(N, D, K, seed)
    Xd, Cd = dev(X), dev(C)
    n = km.kmeans_centroid_norms(Cd)
    return X, C, a, Xd, Cd, n


def direct(Xd, Cd, n):
    lab, md = km.kmeans_assign_path(Xd, Cd, n, km.PATH_DIRECT, 0)
    torch.cuda.synchronize()
    return lab.cpu().numpy(), md.cpu().numpy()


def same(got, want):
    assert np.array_equal(got[0].cpu().numpy(), want[0])
    assert got[1].cpu().numpy().tobytes() == want[1].tobytes()


def update_check(X, lab, C, out):
    Cn, nr, cnt, m = out
    st = parity.check_update(X, lab, C, Cn.view(torch.int16).cpu().numpy().view(np.uint16),
                             nr.cpu().numpy(), cnt.cpu().numpy(), m.cpu().numpy())
    assert st["clusters"] == C.shape[0]


# Sizes that grow and shrink the buffer: split-path scratch is 8 bytes per
# point per K-range plus 4 per point; the update's about 16 per point.
SHAPES = [(2000, 64, 1000, 3), (30000, 128, 4096, 4), (1500, 64, 777, 2), (9000, 256, 600, 5)]


def test_split_path_while_the_buffer_grows_and_shrinks():
    sets = [inputs(N, D, K, 500 + i) for i, (N, D, K, _) in enumerate(SHAPES)]
    want = [direct(s[3], s[4], s[5]) for s in sets]
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        got = [km.kmeans_assign_path(x[3], x[4], x[5], km.PATH_SPLIT, sh[3], stream=s)
               for x, sh in zip(sets + sets, SHAPES + SHAPES)]
    s.synchronize()
    for g, w in zip(got, want + want):
        same(g, w)
    km.kmeans_release_workspace(s)
    s.synchronize()


def test_update_and_split_path_share_a_stream():
    N, D, K = 40000, 128, 1500
    X, C, a, Xd, Cd, n = inputs(N, D, K, 610)
    lab = np.asarray(a, dtype=np.int32)
    ld = torch.from_numpy(lab).cuda()
    small = inputs(1200, 64, 900, 611)
    want_small = direct(small[3], small[4], small[5])
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        u1 = km.kmeans_update(Xd, ld, Cd, with_means=True, stream=s)
        a1 = km.kmeans_assign_path(small[3], small[4], small[5], km.PATH_SPLIT, 3, stream=s)
        u2 = km.kmeans_update(Xd[:3000].contiguous(), ld[:3000].contiguous(), Cd,
                              with_means=True, stream=s)
        a2 = km.kmeans_assign_path(small[3], small[4], small[5], km.PATH_SPLIT, 5, stream=s)
    s.synchronize()
    update_check(X, lab, C, u1)
    update_check(X[:3000], lab[:3000], C, u2)
    same(a1, want_small)
    same(a2, want_small)
    km.kmeans_release_workspace(s)
    s.synchronize()


def test_streams_keep_separate_buffers():
    sets = [inputs(N, D, K, 700 + i) for i, (N, D, K, _) in enumerate(SHAPES[:3])]
    want = [direct(s[3], s[4], s[5]) for s in sets]
    streams = [torch.cuda.Stream() for _ in range(3)]
    torch.cuda.synchronize()
    got = []
    for rep in range(4):   # interleaved, nothing synchronised in between
        for i, s in enumerate(streams):
            x, sh = sets[(i + rep) % 3], SHAPES[(i + rep) % 3]
            with torch.cuda.stream(s):
                got.append(((i + rep) % 3,
                            km.kmeans_assign_path(x[3], x[4], x[5], km.PATH_SPLIT, sh[3],
                                                  stream=s)))
    for s in streams:
        s.synchronize()
    for j, g in got:
        same(g, want[j])
    for s in streams:
        km.kmeans_release_workspace(s)
        s.synchronize()


def test_host_threads_on_their_own_streams():
    sets = [inputs(N, D, K, 800 + i) for i, (N, D, K, _) in enumerate(SHAPES[:2])]
    want = [direct(s[3], s[4], s[5]) for s in sets]
    torch.cuda.synchronize()
    results, errors = {}, []

    def work(t):
        try:
            s = torch.cuda.Stream()
            outs = []
            with torch.cuda.stream(s):
                for rep in range(6):
                    j = (t + rep) % 2
                    x = sets[j]
                    outs.append((j, km.kmeans_assign_path(x[3], x[4], x[5], km.PATH_SPLIT,
                                                          SHAPES[j][3], stream=s)))
            s.synchronize()
            results[t] = [(j, o[0].cpu().numpy(), o[1].cpu().numpy()) for j, o in outs]
            km.kmeans_release_workspace(s)
            s.synchronize()
        except Exception as e:   # reported below, in the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=100)
    assert not errors, errors
    assert sorted(results) == [0, 1, 2, 3]
    for outs in results.values():
        for j, lab, md in outs:
            assert np.array_equal(lab, want[j][0])
            assert md.tobytes() == want[j][1].tobytes()


def test_release_is_a_no_op_without_a_buffer_and_calls_work_after_it():
    s = torch.cuda.Stream()
    km.kmeans_release_workspace(s)            # nothing kept yet
    km.kmeans_release_workspace(None)         # the current stream
    x = inputs(3000, 128, 700, 900)
    want = direct(x[3], x[4], x[5])
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        g1 = km.kmeans_assign_path(x[3], x[4], x[5], km.PATH_SPLIT, 3, stream=s)
        km.kmeans_release_workspace(s)        # behind g1, in stream order
        g2 = km.kmeans_assign_path(x[3], x[4], x[5], km.PATH_SPLIT, 3, stream=s)
    s.synchronize()
    same(g1, want)
    same(g2, want)
    km.kmeans_release_workspace(s)
    km.kmeans_release_workspace(s)            # twice: the second finds nothing
    s.synchronize()


def test_per_thread_default_stream_gets_a_buffer_per_thread():
    """hipStreamPerThread is one handle naming a different stream in every
    thread: each thread must get its own buffer, or concurrent calls from
    two threads would share one."""
    import ctypes
    lib = km.load_library()
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipStreamSynchronize.argtypes = [ctypes.c_void_p]
    per_thread = ctypes.c_void_p(2)          # hipStreamPerThread
    sets = [inputs(N, D, K, 950 + i) for i, (N, D, K, _) in enumerate(SHAPES[:2])]
    want = [direct(s[3], s[4], s[5]) for s in sets]
    torch.cuda.synchronize()
    results, errors = {}, []

    def work(t):
        try:
            outs = []
            for rep in range(6):
                j = (t + rep) % 2
                x = sets[j]
                N, D, K = x[3].shape[0], x[3].shape[1], x[4].shape[0]
                lab = torch.empty(N, dtype=torch.int32, device="cuda")
                md = torch.empty(N, dtype=torch.float32, device="cuda")
                torch.cuda.current_stream().synchronize()   # outputs allocated
                st = lib.kmeans_assign_path(
                    ctypes.c_void_p(x[3].data_ptr()), ctypes.c_void_p(x[4].data_ptr()),
                    ctypes.c_void_p(x[5].data_ptr()), N, D, K, ctypes.c_void_p(lab.data_ptr()),
                    ctypes.c_void_p(md.data_ptr()), km.PATH_SPLIT, SHAPES[j][3], per_thread)
                assert st == 0, lib.kmeans_last_error()
                outs.append((j, lab, md))
            assert hip.hipStreamSynchronize(per_thread) == 0
            results[t] = [(j, lab.cpu().numpy(), md.cpu().numpy()) for j, lab, md in outs]
            assert lib.kmeans_release_workspace(per_thread) == 0
            assert hip.hipStreamSynchronize(per_thread) == 0
        except Exception as e:   # reported below, in the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=100)
    assert not errors, errors
    assert sorted(results) == [0, 1, 2, 3]
    for outs in results.values():
        for j, lab, md in outs:
            assert np.array_equal(lab, want[j][0])
            assert md.tobytes() == want[j][1].tobytes()
