"""The acceptance rule itself (CPU): outputs the oracle produces pass, and
each kind of wrong output is caught."""

import numpy as np
import pytest

import oracle
from means_nearest_centroid_amd import workloads as W
import parity


@pytest.fixture(scope="module")
def case():
    X, C, _ = W.gaussian_mixture(200, 32, 60, 7)
    C = C.copy()
    C[41] = C[3]                      # bitwise duplicate of row 3 (higher index)
    X = X.copy()
    X[0] = C[3]                       # point 0 sits on the duplicated row
    X[1] = C[10]                      # point 1 sits on row 10 (strict)
    # Row 12 = row 11 with one coordinate moved by one bf16 ulp: a near tie
    # for a point on row 11, not a bitwise duplicate.
    C[12] = C[11]
    C[12, 5] = C[11, 5] + 1
    X[2] = C[11]
    X[3, :] = C[20]
    X[3, 0] = W.BF16_QNAN            # NaN coordinate: every score NaN
    ref = oracle.assign(X, C)
    return X, C, ref


def outputs(ref):
    return ref["labels"].astype(np.int32).copy(), ref["dist"].astype(np.float32).copy()


def test_oracle_outputs_pass(case):
    X, C, ref = case
    lab, md = outputs(ref)
    st = parity.check(X, C, lab, md, ref=ref)
    assert st["bad_strict"] == st["bad_near"] == st["bad_dist"] == st["bad_class"] == 0


def test_wrong_strict_label_fails(case):
    X, C, ref = case
    lab, md = outputs(ref)
    assert lab[1] == 10
    lab[1] = 11
    with pytest.raises(AssertionError, match="bad_strict"):
        parity.check(X, C, lab, md, ref=ref)


def test_higher_duplicate_fails_and_near_tie_passes(case):
    X, C, ref = case
    lab, md = outputs(ref)
    assert lab[0] == 3
    lab[0] = 41                       # same scores, but not the lowest index
    with pytest.raises(AssertionError):
        parity.check(X, C, lab, md, ref=ref)
    lab, md = outputs(ref)
    assert lab[2] in (11, 12)
    lab[2] = 23 - lab[2]              # the other member of the near tie
    md[2] = oracle.sqdist_for(X[2:3], C, lab[2:3])[0]
    parity.check(X, C, lab, md, ref=ref)


def test_min_dist_tolerance(case):
    X, C, ref = case
    lab, md = outputs(ref)
    j = 5
    md[j] = np.float32(ref["dist"][j] + 1e-4 * (abs(ref["dist"][j]) + 1))
    parity.check(X, C, lab, md, ref=ref)
    md[j] = np.float32(ref["dist"][j] + 1e-2 * (abs(ref["dist"][j]) + 1))
    with pytest.raises(AssertionError, match="bad_dist"):
        parity.check(X, C, lab, md, ref=ref)


def test_nonfinite_class_must_match(case):
    X, C, ref = case
    lab, md = outputs(ref)
    assert np.isnan(ref["dist"][3]) and lab[3] == 0
    md[3] = 1.0
    with pytest.raises(AssertionError, match="bad_class"):
        parity.check(X, C, lab, md, ref=ref)


def test_out_of_range_label_fails(case):
    X, C, ref = case
    lab, md = outputs(ref)
    lab[7] = C.shape[0]
    with pytest.raises(AssertionError, match="out of range"):
        parity.check(X, C, lab, md, ref=ref)


# ---- centroid update rule -------------------------------------------------

@pytest.fixture(scope="module")
def upd_case():
    X, C, a = W.gaussian_mixture(4000, 64, 200, 61)
    lab = a.astype(np.int32)
    lab[:40] = -1
    lab[lab == 9] = 10                     # cluster 9 empty
    ref = oracle.update(X, lab, C)
    return X, C, lab, ref


def upd_outputs(C, ref):
    """The oracle's result written as a GPU would return it."""
    m32 = ref["means"].astype(np.float32)
    Cn = oracle.bf16_from_double(m32.astype(np.float64))
    empty = ref["counts"] == 0
    Cn[empty] = C[empty]
    nn = (parity._widen(Cn) ** 2).sum(1).astype(np.float32)
    return Cn, nn, ref["counts"].astype(np.int32), m32


def test_update_oracle_outputs_pass(upd_case):
    X, C, lab, ref = upd_case
    st = parity.check_update(X, lab, C, *upd_outputs(C, ref), ref=ref)
    assert st["empty"] == 1 and st["exact"] > 0.99 * st["elements"]


def test_update_wrong_count_fails(upd_case):
    X, C, lab, ref = upd_case
    Cn, nn, cnt, m = upd_outputs(C, ref)
    cnt[3] += 1
    with pytest.raises(AssertionError, match="counts differ"):
        parity.check_update(X, lab, C, Cn, nn, cnt, m, ref=ref)


def test_update_empty_row_must_be_kept(upd_case):
    X, C, lab, ref = upd_case
    Cn, nn, cnt, m = upd_outputs(C, ref)
    Cn[9, 0] ^= 1
    with pytest.raises(AssertionError, match="empty cluster's row"):
        parity.check_update(X, lab, C, Cn, nn, cnt, ref=ref)


def test_update_dropped_point_fails(upd_case):
    X, C, lab, ref = upd_case
    Cn, nn, cnt, m = upd_outputs(C, ref)
    k = int(lab[100])
    members = np.flatnonzero(lab == k)
    xs = parity._widen(X[members[1:]])                 # one point left out
    m[k] = (xs.sum(0) / len(members)).astype(np.float32)
    with pytest.raises(AssertionError, match="fp32 means out of bounds"):
        parity.check_update(X, lab, C, Cn, nn, cnt, m, ref=ref)


def test_update_bf16_off_by_one_ulp_fails(upd_case):
    X, C, lab, ref = upd_case
    Cn, nn, cnt, m = upd_outputs(C, ref)
    Cn[5, 7] += 1                                      # next bf16 up
    with pytest.raises(AssertionError, match="bf16 elements out of bounds"):
        parity.check_update(X, lab, C, Cn, nn, cnt, ref=ref)


def test_update_row_must_round_its_mean(upd_case):
    X, C, lab, ref = upd_case
    Cn, nn, cnt, m = upd_outputs(C, ref)
    m[5, 7] = np.nextafter(m[5, 7], np.float32(np.inf))   # within tol, row unchanged
    parity.check_update(X, lab, C, Cn, nn, cnt, m, ref=ref)
    k, j = 6, 3
    Cn[k, j] = Cn[k, j] + 1 if parity._widen(Cn[k, j]) > 0 else Cn[k, j] - 1
    with pytest.raises(AssertionError, match="bf16"):
        parity.check_update(X, lab, C, Cn, nn, cnt, m, ref=ref)


def test_update_wrong_norm_fails(upd_case):
    X, C, lab, ref = upd_case
    Cn, nn, cnt, m = upd_outputs(C, ref)
    nn[4] *= np.float32(1.001)
    with pytest.raises(AssertionError, match="norm of row 4"):
        parity.check_update(X, lab, C, Cn, nn, cnt, m, ref=ref)
