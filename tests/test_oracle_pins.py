"""Pins of the fp64 oracle: invariants, closed forms and special cases fixed by the pages.

The four required self-checks: (1) a full mask reproduces dense causal attention, (2) moving K/V
physically or jointly permuting them leaves outputs unchanged, (3) softmax rows sum to one,
(4) tiny cases match the brute force (test_oracle_brute.py).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from conftest import small_inputs

SHAPES = [
    # N, Hq, Hkv, d, B, S  (100 and 72 leave a ragged last block and a ragged last segment)
    (96, 4, 2, 8, 8, 32),
    (100, 2, 1, 8, 8, 32),
    (72, 2, 2, 4, 8, 16),
]


def _pipeline(q, k, v, B, S, tau, perm_on=True, diag=True, first=True):
    imp = oracle.key_importance(q, k, B)
    perm = oracle.segment_permutation(imp, S) if perm_on else None
    count, idx, prob = oracle.block_mask(q, k, perm, B, S, tau, diag, first)
    return imp, perm, count, idx, prob


def _sdpa(q, k, v):
    G = q.shape[0] // k.shape[0]
    kt = torch.from_numpy(np.repeat(k, G, axis=0))
    vt = torch.from_numpy(np.repeat(v, G, axis=0))
    o = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q), kt, vt, is_causal=True)
    return o.numpy()


# ---------------------------------------------------------------- check 1: full mask == dense causal

@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("perm_on", [True, False])
def test_full_mask_is_dense_causal(shape, perm_on):
    N, Hq, Hkv, d, B, S = shape
    q, k, v = small_inputs(N, Hq, Hkv, d, n_stripes=4, band=16, seed=11)
    _, perm, count, idx, _ = _pipeline(q, k, v, B, S, 1.0, perm_on)
    NB = oracle.num_blocks(N, B)
    assert (count == np.arange(1, NB + 1)[None, :]).all()
    out, lse, _, _ = oracle.block_sparse_attention(q, k, v, perm, count, idx, B, S)
    ref, ref_lse = oracle.dense_attention(q, k, v)
    assert np.abs(out - ref).max() <= 1e-12
    assert np.abs(lse - ref_lse).max() <= 1e-12
    assert np.abs(out - _sdpa(q, k, v)).max() <= 1e-12


def test_dense_attention_matches_library_sdpa():
    q, k, v = small_inputs(64, 2, 1, 16, n_stripes=2, seed=3)
    ref, _ = oracle.dense_attention(q, k, v)
    assert np.abs(ref - _sdpa(q, k, v)).max() <= 1e-12


# ---------------------------------------------------------------- check 2: permutation semantics

@pytest.mark.parametrize("shape", SHAPES)
def test_index_list_equals_physical_gather(shape):
    """Reading past segments through perm == physically moving those rows first (S2O §1)."""
    N, Hq, Hkv, d, B, S = shape
    q, k, v = small_inputs(N, Hq, Hkv, d, n_stripes=4, band=16, seed=5)
    _, perm, count, idx, prob = _pipeline(q, k, v, B, S, 0.6)
    out, lse, _, _ = oracle.block_sparse_attention(q, k, v, perm, count, idx, B, S)
    NB = oracle.num_blocks(N, B)
    for sigma in range(1, -(-N // S)):
        kp, vp = k.copy(), v.copy()
        kp[:, :sigma * S] = np.take_along_axis(k, perm[:, :sigma * S, None], axis=1)
        vp[:, :sigma * S] = np.take_along_axis(v, perm[:, :sigma * S, None], axis=1)
        rows_I = [I for I in range(NB) if oracle.segment_of_block(I, B, S) == sigma]
        c2, i2, p2 = oracle.block_mask(q, kp, None, B, S, 0.6)
        for I in rows_I:
            o = oracle.tri_offset(I)
            assert (c2[:, I] == count[:, I]).all()
            assert (i2[:, o:o + I + 1] == idx[:, o:o + I + 1]).all()
            assert np.abs(p2[:, o:o + I + 1] - prob[:, o:o + I + 1]).max() <= 1e-13
        rows = [(h, I) for h in range(Hq) for I in rows_I]
        o2, l2, _, _ = oracle.block_sparse_attention(q, kp, vp, None, count, idx, B, S, rows=rows)
        t0 = rows_I[0] * B
        assert np.array_equal(o2[:, t0:min(N, (rows_I[-1] + 1) * B)], out[:, t0:min(N, (rows_I[-1] + 1) * B)])


def test_joint_kv_permutation_invariance_and_query_equivariance():
    """Non-causal attention ignores the order of (k, v) pairs; permuting queries permutes the output
    (Sparser Block-Sparse Attention via Token Permutation, §1)."""
    q, k, v = small_inputs(80, 2, 1, 8, n_stripes=3, seed=9)
    rng = np.random.default_rng(0)
    P = rng.permutation(80)
    ref, _ = oracle.dense_attention(q, k, v, causal=False)
    o1, _ = oracle.dense_attention(q, k[:, P], v[:, P], causal=False)
    assert np.abs(o1 - ref).max() <= 1e-12
    o2, _ = oracle.dense_attention(q[:, P], k, v, causal=False)
    assert np.abs(o2 - ref[:, P]).max() <= 1e-12
    inv = np.argsort(P)
    o3, _ = oracle.dense_attention(q[:, P], k[:, P], v[:, P], causal=False)
    assert np.abs(o3[:, inv] - ref).max() <= 1e-12


@pytest.mark.parametrize("shape", SHAPES)
def test_past_segment_permutation_leaves_later_queries_unchanged(shape):
    """Jointly permuting K, V inside a strictly earlier segment does not change causal outputs of
    later queries (segment causality, Sparser Block-Sparse Attention via Token Permutation, §2)."""
    N, Hq, Hkv, d, B, S = shape
    q, k, v = small_inputs(N, Hq, Hkv, d, n_stripes=4, seed=21)
    rng = np.random.default_rng(1)
    P = np.arange(N)
    P[:S] = rng.permutation(S)
    out, lse, _, _ = oracle.block_sparse_attention(q, k, v, None, None, None, B, S)
    o2, l2, _, _ = oracle.block_sparse_attention(q, k[:, P], v[:, P], None, None, None, B, S)
    assert np.abs(o2[:, S:] - out[:, S:]).max() <= 1e-12
    assert np.abs(l2[:, S:] - lse[:, S:]).max() <= 1e-12
    # the importance proxy moves with the keys, so the permutation lists the same keys
    imp = oracle.key_importance(q, k, B)
    imp2 = oracle.key_importance(q, k[:, P], B)
    assert np.abs(imp2 - imp[:, P]).max() <= 1e-15 + 1e-12 * np.abs(imp).max()


# ---------------------------------------------------------------- check 3: normalisation

@pytest.mark.parametrize("shape", SHAPES)
def test_softmax_rows_sum_to_one(shape):
    N, Hq, Hkv, d, B, S = shape
    q, k, v = small_inputs(N, Hq, Hkv, d, n_stripes=4, band=16, seed=13)
    imp, perm, count, idx, prob = _pipeline(q, k, v, B, S, 0.7)
    assert np.abs(imp.sum(axis=1) - 1.0).max() <= 1e-12
    NB = oracle.num_blocks(N, B)
    for I in range(NB):
        o = oracle.tri_offset(I)
        assert np.abs(prob[:, o:o + I + 1].sum(axis=1) - 1.0).max() <= 1e-12
    _, _, _, w = oracle.block_sparse_attention(q, k, v, perm, count, idx, B, S, return_weights=True)
    assert len(w) == Hq * N
    for (h, i), (keys, p) in w.items():
        assert abs(p.sum() - 1.0) <= 1e-12
        assert (keys <= i).all() or (p[keys > i] == 0).all()


# ---------------------------------------------------------------- closed forms: mask

@pytest.mark.parametrize("perm_on", [True, False])
def test_zero_queries_give_uniform_mass(perm_on):
    """Q = 0 makes every pooled logit 0: p is uniform, ties go to lower J, so a row keeps blocks
    0 .. ceil(tau (I+1)) - 1 plus the forced diagonal."""
    N, Hq, Hkv, d, B, S = 96, 2, 1, 8, 8, 32
    q, k, v = small_inputs(N, Hq, Hkv, d, n_stripes=4, seed=4)
    q[:] = 0.0
    tau = 0.61
    _, perm, count, idx, prob = _pipeline(q, k, v, B, S, tau, perm_on, diag=True, first=False)
    NB = oracle.num_blocks(N, B)
    for I in range(NB):
        want = sorted(set(range(math.ceil(tau * (I + 1)))) | {I})
        o = oracle.tri_offset(I)
        for h in range(Hq):
            assert idx[h, o:o + count[h, I]].tolist() == want
            assert np.allclose(prob[h, o:o + I + 1], 1.0 / (I + 1), rtol=1e-15, atol=0)


def test_mass_boundary_is_inclusive():
    """Cumulative mass exactly equal to tau stops the prefix (C_k >= tau): with 4 or 8 equal
    blocks and tau = 0.5 the sums 0.25+0.25 and 4 * 0.125 are exact."""
    N, B, S = 64, 8, 64
    q, k, v = small_inputs(N, 1, 1, 4, seed=2)
    q[:] = 0.0
    count, idx, _ = oracle.block_mask(q, k, None, B, S, 0.5, force_diag=False, force_first=False)
    assert idx[0, oracle.tri_offset(3):oracle.tri_offset(3) + count[0, 3]].tolist() == [0, 1]
    assert idx[0, oracle.tri_offset(7):oracle.tri_offset(7) + count[0, 7]].tolist() == [0, 1, 2, 3]


@pytest.mark.parametrize("tau", [1.0, 1.5])
def test_tau_at_least_one_selects_all(tau):
    q, k, v = small_inputs(100, 2, 1, 8, n_stripes=4, seed=8)
    _, _, count, idx, _ = _pipeline(q, k, v, 8, 32, tau, diag=False, first=False)
    NB = oracle.num_blocks(100, 8)
    for I in range(NB):
        o = oracle.tri_offset(I)
        assert idx[:, o:o + I + 1].tolist() == [list(range(I + 1))] * 2


def test_one_block_segments_make_permutation_irrelevant_to_mask():
    """S = B: a permuted block holds the same keys as the natural block, so the mask is the same."""
    q, k, v = small_inputs(96, 4, 2, 8, n_stripes=4, band=16, seed=6)
    _, _, c1, i1, p1 = _pipeline(q, k, v, 8, 8, 0.8, perm_on=True)
    _, _, c2, i2, p2 = _pipeline(q, k, v, 8, 8, 0.8, perm_on=False)
    assert np.array_equal(c1, c2) and np.array_equal(i1, i2)
    assert np.abs(np.nan_to_num(p1) - np.nan_to_num(p2)).max() <= 1e-15


def test_forced_blocks_are_kept():
    q, k, v = small_inputs(100, 2, 1, 8, n_stripes=4, seed=12)
    _, _, count, idx, _ = _pipeline(q, k, v, 8, 32, 0.05, diag=True, first=True)
    for I in range(oracle.num_blocks(100, 8)):
        o = oracle.tri_offset(I)
        for h in range(2):
            row = idx[h, o:o + count[h, I]].tolist()
            assert row == sorted(row) and 0 in row and I in row and len(row) <= 3


# ---------------------------------------------------------------- closed forms: permutation

def test_zero_keys_give_identity_permutation():
    q, k, v = small_inputs(96, 2, 1, 8, seed=1)
    k[:] = 0.0
    imp = oracle.key_importance(q, k, 8)
    perm = oracle.segment_permutation(imp, 32)
    assert np.array_equal(perm, np.tile(np.arange(96), (1, 1)))
    # uniform causal weights: key j gets (1/R) sum_{i >= max(j, N-B)} 1/(i+1)
    rows = np.arange(88, 96)
    want = np.array([sum(1.0 / (i + 1) for i in rows if i >= j) for j in range(96)]) / (2 * len(rows)) * 2
    assert np.abs(imp[0] - want).max() <= 1e-15


def test_queries_outside_last_block_do_not_change_permutation():
    q, k, v = small_inputs(96, 4, 2, 8, n_stripes=4, band=16, seed=7)
    imp = oracle.key_importance(q, k, 8)
    q2 = q.copy()
    q2[:, :88] = np.random.default_rng(3).standard_normal(q2[:, :88].shape)
    imp2 = oracle.key_importance(q2, k, 8)
    assert np.array_equal(imp, imp2)
    assert np.array_equal(oracle.segment_permutation(imp, 32), oracle.segment_permutation(imp2, 32))


def test_permutation_maps_each_segment_onto_itself():
    q, k, v = small_inputs(100, 4, 2, 8, n_stripes=6, band=16, seed=17)
    imp = oracle.key_importance(q, k, 8)
    perm = oracle.segment_permutation(imp, 32)
    for g in range(2):
        for a in range(0, 100, 32):
            seg = perm[g, a:min(a + 32, 100)]
            assert sorted(seg.tolist()) == list(range(a, min(a + 32, 100)))
            assert (np.diff(imp[g, seg]) <= 0).all()


# ---------------------------------------------------------------- closed forms: attention / early stop

def test_constant_values_give_constant_output():
    q, k, v = small_inputs(100, 4, 2, 8, n_stripes=4, band=16, seed=10)
    v[:] = np.array([0.5, -1.25, 3.0, 0.0, 1.0, -2.0, 0.75, 4.0])
    _, perm, count, idx, _ = _pipeline(q, k, v, 8, 32, 0.5)
    theta = np.random.default_rng(0).normal(0.0, 1.0, (4, oracle.num_blocks(100, 8)))
    out, _, _, _ = oracle.block_sparse_attention(q, k, v, perm, count, idx, 8, 32, theta=theta)
    assert np.abs(out - v[0, 0]).max() <= 1e-12


def test_threshold_limits():
    N, B, S = 100, 8, 32
    q, k, v = small_inputs(N, 2, 1, 8, n_stripes=4, band=16, seed=14)
    NB = oracle.num_blocks(N, B)
    ref, ref_lse = oracle.dense_attention(q, k, v)
    lo = np.full((2, NB), -np.inf)
    out, lse, kept, _ = oracle.block_sparse_attention(q, k, v, None, None, None, B, S, theta=lo)
    assert np.abs(out - ref).max() <= 1e-12
    hi = np.full((2, NB), np.inf)
    out, lse, kept, _ = oracle.block_sparse_attention(q, k, v, None, None, None, B, S, theta=hi)
    assert all(lst == [I] for (h, I), lst in kept.items())
    blk = np.arange(N) // B
    diag_only, _ = oracle.dense_attention(q, k, v, allowed=blk[:, None] == blk[None, :])
    assert np.abs(out - diag_only).max() <= 1e-12


def test_calibration_on_same_inputs_keeps_exactly_k():
    N, B, keep = 160, 8, 6
    q, k, v = small_inputs(N, 2, 1, 8, n_stripes=4, band=16, seed=15)
    NB = oracle.num_blocks(N, B)
    tm = oracle.tile_max(q, k, B)
    theta = oracle.calibrate_thresholds(tm, NB, keep)
    _, _, kept, _ = oracle.block_sparse_attention(q, k, v, None, None, None, B, None, theta=theta)
    for (h, I), lst in kept.items():
        if I + 1 <= keep:
            assert lst == list(range(I + 1))
        else:
            row = tm[h, oracle.tri_offset(I):oracle.tri_offset(I) + I + 1]
            top = set(np.argsort(-row)[:keep].tolist())
            assert set(lst) == top | {I}
            assert len(lst) == (keep if I in top else keep + 1)


def test_tile_max_matches_dense_logits():
    N, B = 72, 8
    q, k, v = small_inputs(N, 2, 1, 8, n_stripes=3, seed=16)
    tm = oracle.tile_max(q, k, B)
    c = 1.0 / math.sqrt(8)
    for h in range(2):
        s = c * q[h] @ k[0].T
        for I in range(9):
            for J in range(I + 1):
                blockvals = [s[i, j] for i in range(I * B, (I + 1) * B) for j in range(J * B, (J + 1) * B) if j <= i]
                assert abs(tm[h, oracle.tri_offset(I) + J] - max(blockvals)) <= 1e-13 * max(1.0, abs(max(blockvals)))



# ---------------------------------------------------------------- marginal-gain early stop (S2O)

@pytest.mark.parametrize("shape", SHAPES)
def test_ranked_order_is_own_segment_then_history_by_pooled_probability(shape):
    N, Hq, Hkv, d, B, S = shape
    q, k, v = small_inputs(N, Hq, Hkv, d, n_stripes=4, band=16, seed=21)
    perm = oracle.segment_permutation(oracle.key_importance(q, k, B), S)
    count, idx, n_intra = oracle.ranked_blocks(q, k, perm, B, S)
    _, _, prob = oracle.block_mask(q, k, perm, B, S, 1.0, False, False)
    NB = oracle.num_blocks(N, B)
    for h in range(Hq):
        for I in range(NB):
            o = oracle.tri_offset(I)
            row = idx[h, o:o + count[h, I]].tolist()
            assert count[h, I] == I + 1 and sorted(row) == list(range(I + 1))
            ni = int(n_intra[h, I])
            sI = oracle.segment_of_block(I, B, S)
            assert row[:ni] == [J for J in range(I + 1) if oracle.segment_of_block(J, B, S) == sI]
            p = prob[h, o:o + I + 1]
            hist = row[ni:]
            assert all(oracle.segment_of_block(J, B, S) < sI for J in hist)
            # softmax of the pooled logits is non-increasing along the history order
            assert all(p[a] >= p[b] for a, b in zip(hist, hist[1:]))


@pytest.mark.parametrize("shape", SHAPES)
def test_marginal_gain_zero_threshold_is_dense_causal(shape):
    N, Hq, Hkv, d, B, S = shape
    q, k, v = small_inputs(N, Hq, Hkv, d, n_stripes=4, band=16, seed=22)
    perm = oracle.segment_permutation(oracle.key_importance(q, k, B), S)
    count, idx, _ = oracle.ranked_blocks(q, k, perm, B, S)
    out, lse, done = oracle.s2o_attention(q, k, v, perm, count, idx, B, S, 0.0)
    assert all(len(lst) == I + 1 for (h, I), lst in done.items())
    ref, ref_lse = oracle.dense_attention(q, k, v)
    assert np.abs(out - ref).max() <= 1e-12
    assert np.abs(lse - ref_lse).max() <= 1e-12


@pytest.mark.parametrize("shape", SHAPES)
def test_marginal_gain_threshold_one_stops_after_one_history_block(shape):
    # a block's share of a denominator that also holds the own-segment keys is always below 1
    N, Hq, Hkv, d, B, S = shape
    q, k, v = small_inputs(N, Hq, Hkv, d, n_stripes=4, band=16, seed=23)
    perm = oracle.segment_permutation(oracle.key_importance(q, k, B), S)
    count, idx, n_intra = oracle.ranked_blocks(q, k, perm, B, S)
    _, _, done = oracle.s2o_attention(q, k, v, perm, count, idx, B, S, 1.0)
    for (h, I), lst in done.items():
        o = oracle.tri_offset(I)
        ni = int(n_intra[h, I])
        want = idx[h, o:o + min(ni + 1, I + 1)].tolist()
        assert lst == want, (h, I)


def test_marginal_gain_stop_is_monotone_in_threshold():
    N, Hq, Hkv, d, B, S = 96, 2, 1, 8, 8, 32
    q, k, v = small_inputs(N, Hq, Hkv, d, n_stripes=4, band=16, seed=24)
    perm = oracle.segment_permutation(oracle.key_importance(q, k, B), S)
    count, idx, _ = oracle.ranked_blocks(q, k, perm, B, S)
    prev = None
    for tau in (0.0, 1e-4, 1e-3, 1e-2, 0.1, 1.0):
        _, _, done = oracle.s2o_attention(q, k, v, perm, count, idx, B, S, tau)
        n = {key: len(val) for key, val in done.items()}
        if prev is not None:
            assert all(n[key] <= prev[key] for key in n)
        prev = n


# ----------------------------------------------------------------------------- S2O prefix ranking

def test_prefix_ranking_orders_each_prefix_by_the_segment_mean_query():
    """Segment rows u + w and u - w (every head of the group) have mean u; keys k_j = a_j u with
    known a_j, so the order by r . k_j is the order of a_j: descending, ties by position."""
    N, Hq, Hkv, d, S = 48, 4, 2, 6, 16
    rng = np.random.default_rng(5)
    q = np.zeros((Hq, N, d))
    k = np.zeros((Hkv, N, d))
    a = {}
    for g in range(Hkv):
        u = rng.standard_normal(d)
        w = rng.standard_normal(d) * 3.0
        for h in range(g * 2, g * 2 + 2):
            for i in range(N):
                q[h, i] = u + (w if i % 2 == 0 else -w)
        a[g] = rng.permutation(N).astype(np.float64) - 20.0
        a[g][7] = a[g][3]                      # one tie: position 3 before 7
        k[g] = a[g][:, None] * u[None, :]
    pi, score = oracle.prefix_kv_ranking(q, k, S)
    assert pi.shape == (Hkv, oracle.prefix_ranking_length(N, S)) == (Hkv, S + 2 * S)
    for g in range(Hkv):
        for sigma in (1, 2):
            o = oracle.prefix_offset(sigma, S)
            got = pi[g, o:o + sigma * S].tolist()
            want = sorted(range(sigma * S), key=lambda j: (-a[g][j], j))
            assert got == want, (g, sigma)
            assert got.index(3) < got.index(7)
            assert np.all(np.diff(score[g, o:o + sigma * S]) <= 0)


def test_prefix_ranking_ignores_the_order_of_queries_inside_a_segment():
    N, Hq, Hkv, d, B, S = 96, 4, 2, 8, 8, 32
    q, k, _ = small_inputs(N, Hq, Hkv, d, n_stripes=4, band=16, seed=31)
    pi, _ = oracle.prefix_kv_ranking(q, k, S)
    q2 = q.copy()
    rng = np.random.default_rng(1)
    for sigma in range(N // S):
        rows = np.arange(sigma * S, (sigma + 1) * S)
        q2[:, rows] = q[:, rng.permutation(rows)]
    q2[[0, 1]] = q2[[1, 0]]                    # swap the two heads of KV group 0
    pi2, _ = oracle.prefix_kv_ranking(q2, k, S)
    assert np.array_equal(pi, pi2)
    # and it does depend on the queries of the segment: negate segment 2's rows of group 0
    q3 = q.copy()
    q3[0:2, 2 * S:3 * S] *= -1.0
    pi3, _ = oracle.prefix_kv_ranking(q3, k, S)
    o = oracle.prefix_offset(2, S)
    assert not np.array_equal(pi3[0, o:o + 2 * S], pi[0, o:o + 2 * S])
    assert np.array_equal(pi3[0, :o], pi[0, :o]) and np.array_equal(pi3[0, o + 2 * S:], pi[0, o + 2 * S:])
    assert np.array_equal(pi3[1], pi[1])


@pytest.mark.parametrize("shape", SHAPES)
def test_two_pass_zero_threshold_is_dense_causal(shape):
    N, Hq, Hkv, d, B, S = shape
    q, k, v = small_inputs(N, Hq, Hkv, d, n_stripes=4, band=16, seed=32)
    pi, _ = oracle.prefix_kv_ranking(q, k, S)
    out, lse, done = oracle.s2o_prefix_attention(q, k, v, pi, B, S, 0.0)
    assert all(sorted(lst) == list(range(I + 1)) for (h, I), lst in done.items())
    ref, ref_lse = oracle.dense_attention(q, k, v)
    assert np.abs(out - ref).max() <= 1e-12
    assert np.abs(lse - ref_lse).max() <= 1e-12


@pytest.mark.parametrize("shape", SHAPES)
def test_two_pass_threshold_one_stops_after_the_first_history_block(shape):
    N, Hq, Hkv, d, B, S = shape
    q, k, v = small_inputs(N, Hq, Hkv, d, n_stripes=4, band=16, seed=33)
    pi, _ = oracle.prefix_kv_ranking(q, k, S)
    _, _, done = oracle.s2o_prefix_attention(q, k, v, pi, B, S, 1.0)
    for (h, I), lst in done.items():
        J0 = ((I * B) // S) * S // B
        assert lst == list(range(J0, I + 1)) + ([0] if J0 > 0 else []), (h, I, lst)


def test_two_pass_stop_is_monotone_and_history_blocks_hold_the_top_keys():
    N, Hq, Hkv, d, B, S = 96, 2, 1, 8, 8, 32
    q, k, v = small_inputs(N, Hq, Hkv, d, n_stripes=4, band=16, seed=34)
    pi, score = oracle.prefix_kv_ranking(q, k, S)
    prev = None
    for tau in (0.0, 1e-4, 1e-3, 1e-2, 0.1, 1.0):
        _, _, done = oracle.s2o_prefix_attention(q, k, v, pi, B, S, tau)
        n = {key: len(val) for key, val in done.items()}
        if prev is not None:
            assert all(n[key] <= prev[key] for key in n)
        prev = n
    # history block 0 of segment 2 holds the B prefix keys of largest score
    r = oracle.segment_representatives(q, Hkv, S)
    z = k[0, :2 * S] @ r[0, 2]
    o = oracle.prefix_offset(2, S)
    assert set(pi[0, o:o + B].tolist()) == set(np.argsort(-z, kind="stable")[:B].tolist())


def test_two_pass_attention_on_a_given_processed_set():
    N, Hq, Hkv, d, B, S = 96, 4, 2, 8, 8, 32
    q, k, v = small_inputs(N, Hq, Hkv, d, n_stripes=4, band=16, seed=35)
    pi, _ = oracle.prefix_kv_ranking(q, k, S)
    out, lse, done = oracle.s2o_prefix_attention(q, k, v, pi, B, S, 0.05)
    out2, lse2 = oracle.two_pass_attention_on(q, k, v, pi, done, B, S)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    full = {(h, I): list(range(I + 1)) for h in range(Hq) for I in range(N // B)}
    out3, lse3 = oracle.two_pass_attention_on(q, k, v, pi, full, B, S)
    ref, ref_lse = oracle.dense_attention(q, k, v)
    assert np.abs(out3 - ref).max() <= 1e-12 and np.abs(lse3 - ref_lse).max() <= 1e-12


# ----------------------------------------------------------------------------- S2O query permutation

def test_query_permutation_orders_each_segment_by_the_guide_score():
    """Keys all equal u (guide = u); query rows a_i w in every head: score a_i (w . u), so each
    segment lists its positions by a_i descending (ascending when w . u < 0), ties by position."""
    N, Hq, Hkv, d, S = 40, 4, 2, 5, 16
    rng = np.random.default_rng(8)
    q = np.zeros((Hq, N, d))
    k = np.zeros((Hkv, N, d))
    a = rng.permutation(N).astype(np.float64)
    a[9] = a[4]                                   # a tie inside segment 0
    for g in range(Hkv):
        u = rng.standard_normal(d)
        w = u if g == 0 else -u                   # group 1 scores are -a_i |u|^2
        k[g] = u
        for h in range(2 * g, 2 * g + 2):
            q[h] = a[:, None] * w[None, :]
    qperm = oracle.query_permutation(q, k, S)
    for g in range(Hkv):
        sgn = 1.0 if g == 0 else -1.0
        for s0 in range(0, N, S):
            pos = list(range(s0, min(s0 + S, N)))
            assert qperm[g, s0:s0 + len(pos)].tolist() == sorted(pos, key=lambda i: (-sgn * a[i], i))
    assert qperm[0, :16].tolist().index(4) < qperm[0, :16].tolist().index(9)


@pytest.mark.parametrize("shape", SHAPES)
def test_query_permuted_two_pass_zero_threshold_is_dense_causal(shape):
    N, Hq, Hkv, d, B, S = shape
    q, k, v = small_inputs(N, Hq, Hkv, d, n_stripes=4, band=16, seed=36)
    pi, _ = oracle.prefix_kv_ranking(q, k, S)
    qperm = oracle.query_permutation(q, k, S)
    assert not np.array_equal(qperm, np.broadcast_to(np.arange(N), qperm.shape))
    out, lse, done = oracle.s2o_prefix_attention(q, k, v, pi, B, S, 0.0, qperm=qperm)
    ref, ref_lse = oracle.dense_attention(q, k, v)
    assert np.abs(out - ref).max() <= 1e-12 and np.abs(lse - ref_lse).max() <= 1e-12


def test_identity_query_permutation_changes_nothing_but_the_listed_own_blocks():
    N, Hq, Hkv, d, B, S = 96, 4, 2, 8, 8, 32
    q, k, v = small_inputs(N, Hq, Hkv, d, n_stripes=4, band=16, seed=37)
    pi, _ = oracle.prefix_kv_ranking(q, k, S)
    ident = np.broadcast_to(np.arange(N), (Hkv, N)).copy()
    for tau in (0.0, 0.05, 1.0):
        out, lse, done = oracle.s2o_prefix_attention(q, k, v, pi, B, S, tau)
        out2, lse2, done2 = oracle.s2o_prefix_attention(q, k, v, pi, B, S, tau, qperm=ident)
        assert np.abs(out - out2).max() <= 1e-13 and np.abs(lse - lse2).max() <= 1e-13
        for key in done:
            assert [J for J in done2[key] if J <= key[1]] == done[key]


def test_query_permutation_moves_rows_not_results():
    """Permuting the queries of a segment only moves which block a query sits in: with tau = 0 the
    result is the same dense attention; with tau > 0 the stop sees other blocks, yet every row is
    written at its own position (no row is left NaN)."""
    N, Hq, Hkv, d, B, S = 96, 2, 1, 8, 8, 32
    q, k, v = small_inputs(N, Hq, Hkv, d, n_stripes=4, band=16, seed=38)
    pi, _ = oracle.prefix_kv_ranking(q, k, S)
    qperm = oracle.query_permutation(q, k, S)
    out, lse, _ = oracle.s2o_prefix_attention(q, k, v, pi, B, S, 0.1, qperm=qperm)
    assert not np.isnan(out).any() and not np.isnan(lse).any()


# ----------------------------------------------------------------------------- SampleAttention

def test_trunk_rows_closed_form():
    assert oracle.trunk_rows(100, 4, 5).tolist() == (list(range(20, 25)) + list(range(45, 50))
                                                     + list(range(70, 75)) + list(range(95, 100)))
    assert oracle.trunk_rows(10, 3, 2).tolist() == [2, 3, 6, 7, 8, 9]   # chunks of 4, 4, 2
    with pytest.raises(ValueError):
        oracle.trunk_rows(10, 3, 3)                                   # the last trunk has 2 positions


def test_sampled_masses_of_uniform_attention():
    """Q = 0: every sampled row i spreads 1/(i+1) over keys 0..i, so col[j] = mean_i [j <= i]/(i+1)
    and slash[delta] = mean_i [delta <= i]/(i+1)."""
    N, Hq, Hkv, d = 64, 2, 1, 4
    q = np.zeros((Hq, N, d))
    k = np.random.default_rng(2).standard_normal((Hkv, N, d))
    rows = oracle.trunk_rows(N, 4, 3)
    col, slash = oracle.sampled_masses(q, k, 4, 3)
    want = np.array([np.mean([(1.0 / (i + 1)) if x <= i else 0.0 for i in rows]) for x in range(N)])
    np.testing.assert_allclose(col[0], want, rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(slash[1], want, rtol=1e-13, atol=1e-16)   # the same formula in delta


@pytest.mark.parametrize("shape", SHAPES)
def test_sampled_masses_are_distributions(shape):
    N, Hq, Hkv, d, B, S = shape
    q, k, _ = small_inputs(N, Hq, Hkv, d, n_stripes=4, band=16, seed=40)
    col, slash = oracle.sampled_masses(q, k, 4, 2)
    assert np.all(col >= 0) and np.all(slash >= 0)
    np.testing.assert_allclose(col.sum(axis=1), 1.0, rtol=1e-12)
    np.testing.assert_allclose(slash.sum(axis=1), 1.0, rtol=1e-12)
    last = oracle.trunk_rows(N, 4, 2).max()
    assert np.all(col[:, last + 1:] == 0) and np.all(slash[:, last + 1:] == 0)


def test_sample_attention_finds_a_planted_column_and_a_planted_slash():
    N, Hq, Hkv, d, B = 128, 2, 1, 16, 16
    rng = np.random.default_rng(4)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q = rng.standard_normal((Hq, N, d)) * 0.1
    k = rng.standard_normal((Hkv, N, d)) * 0.1
    # head 0: a strong column at key 37 (every query aligned with u)
    q[0] += 4.0 * u
    k[0, 37] += 4.0 * u
    # head 1 shares the keys; give its queries a strong diagonal 5 back: q_i ~ k_{i-5}
    q[1] = 0.1 * rng.standard_normal((N, d))
    q[1, 5:] += 6.0 * k[0, :N - 5] / np.linalg.norm(k[0, :N - 5], axis=1, keepdims=True)
    count, idx, ck, sk, col, slash = oracle.sample_attention_mask(q, k, B, 0.5, 4, 4)
    assert np.argmax(col[0]) == 37 and ck[0, 37]
    assert np.argmax(slash[1]) == 5 and sk[1, 5]
    for I in range(N // B):
        row = idx[0, oracle.tri_offset(I):oracle.tri_offset(I) + count[0, I]].tolist()
        if I >= 37 // B:
            assert 37 // B in row
    # tile (3, 2) holds pairs i - j = 5 (i = 48, j = 43), tile (5, 2) does not (smallest i - j is 49)
    row3 = idx[1, oracle.tri_offset(3):oracle.tri_offset(3) + count[1, 3]].tolist()
    assert 2 in row3


def test_sample_attention_full_target_keeps_every_tile():
    N, Hq, Hkv, d, B = 96, 2, 1, 8, 8
    q, k, _ = small_inputs(N, Hq, Hkv, d, n_stripes=4, band=16, seed=41)
    count, _, ck, sk, _, _ = oracle.sample_attention_mask(q, k, B, 1.0, 3, 4)
    assert ck.all() and sk.all()
    assert (count == np.arange(1, N // B + 1)[None, :]).all()


def test_pooled_block_logits_are_the_mask_scores():
    """softmax of each row of pooled_block_logits is block_mask's p; with every query u and keys
    a_j u the logit of (I, J) is c |u|^2 times the mean a over block J."""
    N, Hq, Hkv, d, B, S = 96, 4, 2, 8, 8, 32
    q, k, _ = small_inputs(N, Hq, Hkv, d, n_stripes=4, band=16, seed=42)
    perm = oracle.segment_permutation(oracle.key_importance(q, k, B), S)
    z = oracle.pooled_block_logits(q, k, perm, B, S)
    _, _, prob = oracle.block_mask(q, k, perm, B, S, 0.9)
    for h in range(Hq):
        for I in range(N // B):
            o = oracle.tri_offset(I)
            e = np.exp(z[h, o:o + I + 1] - z[h, o:o + I + 1].max())
            np.testing.assert_allclose(e / e.sum(), prob[h, o:o + I + 1], rtol=1e-12, atol=1e-300)
    u = np.random.default_rng(3).standard_normal(d)
    a = np.arange(N, dtype=np.float64) / N
    q2 = np.broadcast_to(u, (Hq, N, d)).copy()
    k2 = np.broadcast_to(a[:, None] * u[None, :], (Hkv, N, d)).copy()
    z2 = oracle.pooled_block_logits(q2, k2, None, B, S)
    c = 1.0 / np.sqrt(d)
    for I in (0, 5, N // B - 1):
        o = oracle.tri_offset(I)
        want = [c * (u @ u) * a[J * B:(J + 1) * B].mean() for J in range(I + 1)]
        np.testing.assert_allclose(z2[0, o:o + I + 1], want, rtol=1e-12)


def test_mass_cut_hand_example_and_characterisation():
    """mass_cut keeps the heaviest members (ties by lower index) until their mass reaches tau: a
    hand-worked vector, then the properties that fix the answer on random vectors — the kept set
    reaches tau, dropping its lightest member falls below tau, and no unkept member outranks a
    kept one."""
    m = np.array([0.1, 0.4, 0.3, 0.2])
    assert oracle.mass_cut(m, 0.65).tolist() == [False, True, True, False]
    assert oracle.mass_cut(m, 0.4).tolist() == [False, True, False, False]   # reaching tau exactly is enough
    assert oracle.mass_cut(m, 0.75).tolist() == [False, True, True, True]
    assert oracle.mass_cut(m, 1.0).all() and oracle.mass_cut(m, 2.0).all()
    assert oracle.mass_cut(np.array([0.25, 0.25, 0.25, 0.25]), 0.5).tolist() == [True, True, False, False]
    rng = np.random.default_rng(11)
    for _ in range(200):
        n = int(rng.integers(1, 12))
        w = rng.random(n) ** 3
        w[rng.random(n) < 0.3] = w[0]          # planted ties
        w = w / w.sum() if w.sum() > 0 else np.full(n, 1.0 / n)
        tau = float(rng.choice([0.2, 0.5, 0.9, 0.99]))
        keep = oracle.mass_cut(w, tau)
        kept, rest = np.nonzero(keep)[0], np.nonzero(~keep)[0]
        total = w[keep].sum()
        if total < tau:                          # only when even every member falls short
            assert keep.all()
            continue
        lightest = max(kept, key=lambda i: (-w[i], i))      # last in the (heavy first, index) order
        assert total - w[lightest] < tau
        for i in rest:
            for j in kept:
                assert (w[j], -j) > (w[i], -i)


def test_kept_bitmap_hand_example():
    """Bit tri_offset(I) + J of head h's row: for NB = 3 the tiles (0,0), (2,0), (2,2) are bits 0, 3
    and 5 (rows start at bits 0, 1, 3); a second head and a tile past bit 31 land in their own
    words."""
    bm = oracle.kept_bitmap({(0, 0): [0], (0, 2): [0, 2]}, 1, 3)
    assert bm.dtype == np.uint32 and bm.shape == (1, 1) and int(bm[0, 0]) == 0b101001
    bm = oracle.kept_bitmap({(1, 7): [4]}, 2, 8)       # tri_offset(7) + 4 = 28 + 4 = 32
    assert bm.shape == (2, 2) and bm[0].tolist() == [0, 0] and bm[1].tolist() == [0, 1]
