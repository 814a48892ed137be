"""kmeans_assign_static inside a captured HIP graph (through torch.cuda.CUDAGraph),
on the direct path and on the K-split path whose scratch is the library's
fixed device buffer: every replay, with eager work and synchronisation between
replays, must give the eager call's outputs bit for bit.  The inputs are
changed in place between replays, so a replay that reused stale results would
be caught."""

import numpy as np
import pytest

from means_nearest_centroid_amd import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
km = pytest.importorskip("means_nearest_centroid_amd")


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("N,D,K,path", [(65536, 128, 1000, km.PATH_DIRECT),
                                        (16384, 128, 4096, km.PATH_SPLIT)])
def test_static_assign_replays_in_a_graph(N, D, K, path):
    assert km.kmeans_plan(N, D, K, torch.cuda.get_device_properties(0).multi_processor_count)["path"] == path
    sets = [W.gaussian_mixture(N, D, K, seed)[:2] for seed in (161, 162, 163)]
    Xg, Cg = dev(sets[0][0]), dev(sets[0][1])
    ng = km.kmeans_centroid_norms(Cg)
    lab = torch.empty(N, dtype=torch.int32, device="cuda")
    md = torch.empty(N, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                      # warm-up: resolves the fixed buffer
        km.kmeans_assign_static(Xg, Cg, ng, lab, md)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        km.kmeans_centroid_norms(Cg, ng)
        km.kmeans_assign_static(Xg, Cg, ng, lab, md)
    for rep in range(6):
        X, C = sets[rep % 3]
        Xg.copy_(dev(X))
        Cg.copy_(dev(C))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_l, got_m = lab.clone(), md.clone()
        Xe, Ce = dev(X), dev(C)
        le, me = km.kmeans_assign(Xe, Ce, km.kmeans_centroid_norms(Ce))
        torch.cuda.synchronize()
        assert torch.equal(got_l, le), rep
        assert got_m.cpu().numpy().tobytes() == me.cpu().numpy().tobytes(), rep
