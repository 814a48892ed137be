"""Hand-derived worked examples (tests/golden/hand_examples.json): the oracle
on the CPU and the HIP path on the GPU must reproduce them exactly."""

import json
import os

import numpy as np
import pytest

import oracle
from means_nearest_centroid_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "hand_examples.json")


def _value(v):
    return {"inf": np.inf, "-inf": -np.inf, "nan": np.nan, "-0": -0.0}.get(v, v) \
        if isinstance(v, str) else float(v)


def _matrix(rows, D):
    m = np.zeros((len(rows), D), np.float32)
    for i, r in enumerate(rows):
        m[i, :len(r)] = [_value(v) for v in r]
    bits = W.f32_to_bf16_bits(m)
    assert np.array_equal(W.bf16_bits_to_f32(bits), m, equal_nan=True)   # exact in bf16
    return bits


def examples():
    g = json.load(open(GOLDEN))
    for e in g["examples"]:
        yield (e["name"], _matrix(e["X"], g["D"]), _matrix(e["C"], g["D"]),
               np.array(e["labels"]), np.array([_value(v) for v in e["min_dist"]]))


CASES = list(examples())


def same(a, b):
    return np.array_equal(np.asarray(a, np.float64), np.asarray(b, np.float64), equal_nan=True)


@pytest.mark.parametrize("name,X,C,labels,dist", CASES, ids=[c[0] for c in CASES])
def test_oracle_reproduces_hand_example(name, X, C, labels, dist, oracle_lib):
    r = oracle.assign(X, C)
    assert np.array_equal(r["labels"], labels)
    assert same(r["dist"], dist)


@pytest.mark.gpu
@pytest.mark.parametrize("name,X,C,labels,dist", CASES, ids=[c[0] for c in CASES])
def test_gpu_reproduces_hand_example(name, X, C, labels, dist):
    import torch
    import means_nearest_centroid_amd as km

    def dev(b):
        return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).cuda()

    Cd = dev(C)
    lab, md = km.kmeans_assign(dev(X), Cd, km.kmeans_centroid_norms(Cd))
    torch.cuda.synchronize()
    assert np.array_equal(lab.cpu().numpy(), labels)
    assert same(md.cpu().numpy(), dist)
