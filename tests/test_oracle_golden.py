"""Pin the oracle to the hand-derived example in tests/golden/hand_example_n8.{json,md}."""
import json
import math
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def ex():
    with open(os.path.join(HERE, "golden", "hand_example_n8.json")) as f:
        e = json.load(f)
    N, d = e["N"], e["d"]
    q = np.tile(np.array(e["q_row"], dtype=np.float64), (1, N, 1))
    k = np.zeros((1, N, d))
    k[0, :, 0] = [math.log(x) for x in e["k_first_exp"]]
    k[0, :, 1:] = np.array(e["k_rest"])
    v = np.zeros((1, N, d))
    for j in range(N):
        v[0, j] = [j, 1.0, -j, 0.0]
    e["arrays"] = (q, k, v)
    return e


def _check_rows(e, count, idx, prob, part):
    exp = e[part]
    assert count[0].tolist() == exp["count"]
    for I, row in enumerate(exp["rows"]):
        o = oracle.tri_offset(I)
        assert idx[0, o:o + len(row)].tolist() == row
        want = np.array(exp["prob_num"][I], dtype=np.float64) / exp["prob_den"][I]
        np.testing.assert_allclose(prob[0, o:o + I + 1], want, rtol=1e-13, atol=0)


def _check_out(e, out, lse, exp):
    for i, (num, den) in enumerate(exp["out_first"]):
        f = num / den
        np.testing.assert_allclose(out[0, i], [f, 1.0, -f, 0.0], rtol=1e-13, atol=1e-13)
        assert abs(lse[0, i] - math.log(exp["lse_exp"][i])) <= 1e-13


def test_importance_and_permutation(ex):
    q, k, v = ex["arrays"]
    imp = oracle.key_importance(q, k, ex["B"], scale=ex["scale"])
    want = np.array(ex["importance_num"], dtype=np.float64) / ex["importance_den"]
    np.testing.assert_allclose(imp[0], want, rtol=1e-13, atol=0)
    perm = oracle.segment_permutation(imp, ex["S"])
    assert perm[0].tolist() == ex["perm"]


def test_default_scale_is_inverse_sqrt_d(ex):
    q, k, v = ex["arrays"]
    assert oracle.default_scale(ex["d"]) == ex["scale"]
    imp = oracle.key_importance(q, k, ex["B"])
    want = np.array(ex["importance_num"], dtype=np.float64) / ex["importance_den"]
    np.testing.assert_allclose(imp[0], want, rtol=1e-13, atol=0)


@pytest.mark.parametrize("part", ["perm_on", "perm_off"])
def test_mask_and_attention(ex, part):
    q, k, v = ex["arrays"]
    perm = np.array([ex["perm"]]) if part == "perm_on" else None
    count, idx, prob = oracle.block_mask(q, k, perm, ex["B"], ex["S"], ex["tau"],
                                         ex["force_diag"], ex["force_first"], scale=ex["scale"])
    _check_rows(ex, count, idx, prob, part)
    out, lse, kept, _ = oracle.block_sparse_attention(q, k, v, perm, count, idx, ex["B"], ex["S"],
                                                      scale=ex["scale"])
    _check_out(ex, out, lse, ex[part])


def test_tile_max_and_calibration(ex):
    q, k, v = ex["arrays"]
    tm = oracle.tile_max(q, k, ex["B"], scale=ex["scale"])
    np.testing.assert_allclose(tm[0], [math.log(x) for x in ex["tile_max_exp"]], rtol=0, atol=1e-13)
    theta = oracle.calibrate_thresholds(tm, 4, ex["calib_keep"])
    for I, t in enumerate(ex["theta_exp"]):
        if t is None:
            assert theta[0, I] == -np.inf
        else:
            assert abs(theta[0, I] - math.log(t)) <= 1e-13


def test_early_stop(ex):
    q, k, v = ex["arrays"]
    perm = np.array([ex["perm"]])
    count, idx, _ = oracle.block_mask(q, k, perm, ex["B"], ex["S"], ex["tau"], True, True,
                                      scale=ex["scale"])
    es = ex["early_stop"]
    theta = np.array([[(-np.inf if t is None else math.log(t)) for t in es["theta_exp"]]])
    out, lse, kept, _ = oracle.block_sparse_attention(q, k, v, perm, count, idx, ex["B"], ex["S"],
                                                      scale=ex["scale"], theta=theta)
    assert [kept[(0, I)] for I in range(4)] == es["kept_rows"]
    _check_out(ex, out, lse, es)
