"""The MFMA-stream probe that bench.py reads the assign kernel against: it
runs on the GPU, refuses bad arguments, and computes what it claims (its
sink values are finite and deterministic; zero operands give exactly the
C-tile sums)."""

import ctypes

import numpy as np
import pytest
import torch

from means_nearest_centroid_amd import build as kbuild

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def probe():
    lib = ctypes.CDLL(kbuild.PROBE_LIBRARY)
    lib.kmeans_mfma_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p]
    lib.kmeans_mfma_stream.restype = ctypes.c_int32
    return lib


def run(probe, a, b, rows, tiles, wgs):
    threads = probe.kmeans_mfma_stream_threads()
    sink = torch.full((wgs * threads,), float("nan"), dtype=torch.float32, device="cuda")
    st = probe.kmeans_mfma_stream(a.data_ptr(), b.data_ptr(), rows, tiles, wgs, sink.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return st, sink.cpu().numpy()


def test_probe_runs_and_is_deterministic(probe):
    g = torch.Generator().manual_seed(5)
    a = torch.randn(256, 128, generator=g).to(torch.bfloat16).cuda()
    b = torch.randn(256, 128, generator=g).to(torch.bfloat16).cuda()
    st, s1 = run(probe, a, b, 256, 7, 3)
    assert st == 0 and np.all(np.isfinite(s1))
    st, s2 = run(probe, a, b, 256, 7, 3)
    assert st == 0 and s1.tobytes() == s2.tobytes()


def test_probe_zero_operands_give_the_c_tile_sums(probe):
    # With A = B = 0 every MFMA result is its C tile, whose element r in lane
    # quarter q (lane // 16) is r + 4q (element 0, never read, changes per
    # tile).  Per pair of tiles the probe reads elements 1 + j % 3 of the
    # eight chains of one set and 1 + (j + 1) % 3 of the other, and at the
    # end 1 + (j + 2) % 3: each lane's sink value is floor(tiles / 2) *
    # (32 + 64q) + 16 + 32q, exactly.
    z = torch.zeros((64, 128), dtype=torch.bfloat16, device="cuda")
    for tiles in (1, 2, 5):
        st, s = run(probe, z, z, 64, tiles, 2)
        assert st == 0
        q = (np.arange(s.size) % 64) // 16
        exp = (tiles // 2) * (32.0 + 64.0 * q) + 16.0 + 32.0 * q
        assert np.array_equal(s, exp.astype(np.float32)), tiles


def test_probe_rejects_bad_arguments(probe):
    z = torch.zeros((64, 128), dtype=torch.bfloat16, device="cuda")
    st, _ = run(probe, z, z, 0, 1, 1)
    assert st == 1
    st, _ = run(probe, z, z, 64, 0, 1)
    assert st == 1


def test_clock_sampler_reads_a_plausible_clock(probe):
    lib = ctypes.CDLL(kbuild.PROBE_LIBRARY)
    lib.kmeans_clock_sampler.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_void_p]
    lib.kmeans_clock_sampler.restype = ctypes.c_int32
    out = torch.zeros(4 * 8, dtype=torch.int64, device="cuda")
    st = lib.kmeans_clock_sampler(out.data_ptr(), 8, 2000,
                                  torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    o = out.view(8, 4).cpu().numpy()
    assert np.all(o[:, 0] >= 2000 * 100)            # at least the requested 100 MHz ticks
    assert np.all(o[:, 0] < 2000 * 100 * 10)        # and the loop ended
    mhz = 100.0 * o[:, 1] / o[:, 0]
    assert np.all((mhz > 100) & (mhz < 4000)), mhz
    assert np.all(o[:, 3] == 0)
