"""check 4: the NumPy oracle agrees with the pure-Python brute force on tiny shapes."""
import math

import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from oracle import brute
from conftest import small_inputs


@st.composite
def tiny_case(draw):
    B = draw(st.sampled_from([2, 4, 8]))
    S = B * draw(st.sampled_from([1, 2, 4]))
    nb = draw(st.integers(1, 10))
    N = draw(st.integers(max(1, (nb - 1) * B + 1), nb * B))      # ragged last block allowed
    Hkv = draw(st.sampled_from([1, 2]))
    G = draw(st.sampled_from([1, 2]))
    d = draw(st.integers(1, 8))
    tau = draw(st.sampled_from([0.3, 0.5, 0.8, 0.95, 1.0]))
    diag = draw(st.booleans())
    first = draw(st.booleans())
    perm_on = draw(st.booleans())
    seed = draw(st.integers(0, 2 ** 20))
    stripes = draw(st.integers(0, 3))
    return dict(B=B, S=S, N=N, Hkv=Hkv, Hq=Hkv * G, d=d, tau=tau, diag=diag, first=first,
                perm_on=perm_on, seed=seed, stripes=stripes)


@settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(tiny_case())
def test_oracle_matches_brute_force(c):
    N, Hq, Hkv, d, B, S = c["N"], c["Hq"], c["Hkv"], c["d"], c["B"], c["S"]
    q, k, v = small_inputs(N, Hq, Hkv, d, n_stripes=c["stripes"], band=0, seed=c["seed"])
    scale = 1.0 / math.sqrt(d)

    imp = oracle.key_importance(q, k, B)
    imp_b = brute.importance(q, k, B, scale)
    np.testing.assert_allclose(imp, np.array(imp_b), rtol=1e-12, atol=1e-300)

    perm = oracle.segment_permutation(imp, S)
    brute.check_permutation(perm, imp_b, S)
    use_perm = perm if c["perm_on"] else None

    count, idx, prob = oracle.block_mask(q, k, use_perm, B, S, c["tau"], c["diag"], c["first"])
    sel_b, prob_b = brute.mask(q, k, use_perm, B, S, c["tau"], c["diag"], c["first"], scale)
    NB = oracle.num_blocks(N, B)
    for h in range(Hq):
        for I in range(NB):
            o = oracle.tri_offset(I)
            np.testing.assert_allclose(prob[h, o:o + I + 1], prob_b[(h, I)], rtol=1e-12, atol=1e-300)
            assert idx[h, o:o + count[h, I]].tolist() == sel_b[(h, I)], (h, I)

    out, lse, _, _ = oracle.block_sparse_attention(q, k, v, use_perm, count, idx, B, S)
    out_b, lse_b, _ = brute.attention(q, k, v, use_perm, sel_b, B, S, scale)
    np.testing.assert_allclose(out, np.array(out_b, dtype=np.float64), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(lse_b, dtype=np.float64), rtol=1e-12, atol=1e-12)

    # early stop with a threshold between the row's tile maxima, so some tiles drop
    rng = np.random.default_rng(c["seed"])
    tm = oracle.tile_max(q, k, B)
    theta = np.empty((Hq, NB))
    for h in range(Hq):
        for I in range(NB):
            row = tm[h, oracle.tri_offset(I):oracle.tri_offset(I) + I + 1]
            theta[h, I] = rng.uniform(row.min() - 0.1, row.max() + 0.1)
    out, lse, kept, _ = oracle.block_sparse_attention(q, k, v, use_perm, count, idx, B, S, theta=theta)
    out_b, lse_b, kept_b = brute.attention(q, k, v, use_perm, sel_b, B, S, scale, theta=theta)
    assert kept == kept_b
    np.testing.assert_allclose(out, np.array(out_b, dtype=np.float64), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(lse_b, dtype=np.float64), rtol=1e-12, atol=1e-12)


@settings(max_examples=30, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(tiny_case(), st.sampled_from([0.0, 1e-3, 1e-2, 5e-2, 0.2, 1.0]))
def test_marginal_gain_stop_matches_brute_force(c, gain_tau):
    N, Hq, Hkv, d, B, S = c["N"], c["Hq"], c["Hkv"], c["d"], c["B"], c["S"]
    q, k, v = small_inputs(N, Hq, Hkv, d, n_stripes=c["stripes"], band=0, seed=c["seed"])
    scale = 1.0 / math.sqrt(d)
    perm = oracle.segment_permutation(oracle.key_importance(q, k, B), S) if c["perm_on"] else None
    count, idx, n_intra = oracle.ranked_blocks(q, k, perm, B, S)
    out, lse, done = oracle.s2o_attention(q, k, v, perm, count, idx, B, S, gain_tau)
    done_b = brute.s2o_processed(q, k, perm, B, S, gain_tau, scale)
    assert done == done_b
    out_b, lse_b, _ = brute.attention(q, k, v, perm, {key: sorted(val) for key, val in done_b.items()}, B, S, scale)
    np.testing.assert_allclose(out, np.array(out_b, dtype=np.float64), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(lse_b, dtype=np.float64), rtol=1e-12, atol=1e-12)


@settings(max_examples=15, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(tiny_case())
def test_marginal_gain_ratios_place_the_brute_force_stop(c):
    # at each position whose ratio is a new low among the earlier-segment positions, a threshold
    # just above it makes the brute force stop exactly there, and one just below lets it go on
    N, Hq, Hkv, d, B, S = c["N"], c["Hq"], c["Hkv"], c["d"], c["B"], c["S"]
    q, k, _ = small_inputs(N, Hq, Hkv, d, n_stripes=c["stripes"], band=0, seed=c["seed"])
    scale = 1.0 / math.sqrt(d)
    perm = oracle.segment_permutation(oracle.key_importance(q, k, B), S) if c["perm_on"] else None
    count, idx, _ = oracle.ranked_blocks(q, k, perm, B, S)
    ratios = oracle.s2o_gain_ratios(q, k, perm, count, idx, B, S)
    checks = []
    for (h, I), r in ratios.items():
        assert np.all(np.isnan(r) | ((r > 0) & (r <= 1 + 1e-12))), (h, I, r)
        low = math.inf
        for p, x in enumerate(r):
            if not np.isnan(x) and x < low * (1 - 1e-6):
                checks.append((h, I, p, float(x), low))
                low = x
    for h, I, p, x, low in checks[:6]:
        above = brute.s2o_processed(q, k, perm, B, S, x * (1 + 1e-9), scale)[(h, I)]
        assert len(above) == p + 1, (h, I, p, x, above)
        below = brute.s2o_processed(q, k, perm, B, S, x * (1 - 1e-9), scale)[(h, I)]
        assert len(below) > p + 1 or len(below) == int(count[h, I]), (h, I, p, x, below)


def _same_ranking(got, want, score_of, tol=1e-12):
    """Equal lists up to swaps of keys whose scores agree within tol (relative)."""
    assert sorted(got) == sorted(want)
    for a, b in zip(got, want):
        if a != b:
            za, zb = score_of(a), score_of(b)
            assert abs(za - zb) <= tol * max(abs(za), abs(zb), 1e-300), (a, b, za, zb)


@settings(max_examples=25, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(tiny_case(), st.sampled_from([0.0, 1e-2, 5e-2, 0.2, 1.0]))
def test_prefix_ranking_and_two_pass_stop_match_brute_force(c, gain_tau):
    N, Hq, Hkv, d, B, S = c["N"], c["Hq"], c["Hkv"], c["d"], c["B"], c["S"]
    q, k, v = small_inputs(N, Hq, Hkv, d, n_stripes=c["stripes"], band=0, seed=c["seed"])
    scale = 1.0 / math.sqrt(d)
    pi, score = oracle.prefix_kv_ranking(q, k, S)
    rank_b = brute.prefix_ranking(q, k, S)
    r = oracle.segment_representatives(q, Hkv, S)
    for (g, sigma), order in rank_b.items():
        o = oracle.prefix_offset(sigma, S)
        got = pi[g, o:o + sigma * S].tolist()
        _same_ranking(got, order, lambda j: float(k[g, j] @ r[g, sigma]))
        np.testing.assert_allclose(score[g, o:o + sigma * S], k[g, got] @ r[g, sigma], rtol=0, atol=0)
    # the stop and the output, both on the oracle's ranking
    ranking = {(g, sigma): pi[g, oracle.prefix_offset(sigma, S):oracle.prefix_offset(sigma, S) + sigma * S].tolist()
               for g in range(Hkv) for sigma in range(1, oracle.num_segments(N, S))}
    out, lse, done = oracle.s2o_prefix_attention(q, k, v, pi, B, S, gain_tau)
    done_b = brute.s2o_prefix_processed(q, k, ranking, B, S, gain_tau, scale)
    assert done == done_b
    keysets = {}
    for (h, I), lst in done_b.items():
        sigma = (I * B) // S
        J0 = sigma * S // B
        rank = ranking.get((h // (Hq // Hkv), sigma), [])
        keysets[(h, I)] = [j for J in lst for j in (range(J * B, min((J + 1) * B, N)) if J >= J0 else rank[J * B:(J + 1) * B])]
    out_b, lse_b = brute.attention_over_keys(q, k, v, keysets, B, scale)
    np.testing.assert_allclose(out, np.array(out_b, dtype=np.float64), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(lse_b, dtype=np.float64), rtol=1e-12, atol=1e-12)


@settings(max_examples=20, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(tiny_case(), st.sampled_from([0.0, 1e-2, 0.2, 1.0]))
def test_query_permutation_and_its_two_pass_stop_match_brute_force(c, gain_tau):
    N, Hq, Hkv, d, B, S = c["N"], c["Hq"], c["Hkv"], c["d"], c["B"], c["S"]
    q, k, v = small_inputs(N, Hq, Hkv, d, n_stripes=c["stripes"], band=0, seed=c["seed"])
    scale = 1.0 / math.sqrt(d)
    qperm = oracle.query_permutation(q, k, S)
    qorder_b = brute.query_order(q, k, S)
    z = oracle.query_guide_scores(q, k)
    for g in range(Hkv):
        _same_ranking(qperm[g].tolist(), qorder_b[g], lambda i: float(z[g, i]))
    qorder = [qperm[g].tolist() for g in range(Hkv)]  # both sides on the oracle's order from here
    pi, _ = oracle.prefix_kv_ranking(q, k, S)
    ranking = {(g, sigma): pi[g, oracle.prefix_offset(sigma, S):oracle.prefix_offset(sigma, S) + sigma * S].tolist()
               for g in range(Hkv) for sigma in range(1, oracle.num_segments(N, S))}
    out, lse, done = oracle.s2o_prefix_attention(q, k, v, pi, B, S, gain_tau, qperm=qperm)
    done_b = brute.s2o_prefix_processed(q, k, ranking, B, S, gain_tau, scale, qorder=qorder)
    assert done == done_b
    keysets = {}
    for (h, I), lst in done_b.items():
        sigma = (I * B) // S
        J0 = sigma * S // B
        rank = ranking.get((h // (Hq // Hkv), sigma), [])
        keysets[(h, I)] = [j for J in lst for j in (range(J * B, min((J + 1) * B, N)) if J >= J0 else rank[J * B:(J + 1) * B])]
    out_b, lse_b = brute.attention_over_keys(q, k, v, keysets, B, scale, qorder=qorder)
    np.testing.assert_allclose(out, np.array(out_b, dtype=np.float64), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(lse_b, dtype=np.float64), rtol=1e-12, atol=1e-12)


@settings(max_examples=25, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(tiny_case(), st.sampled_from([(1, 1), (2, 2), (3, 1), (4, 2)]), st.sampled_from([0.3, 0.6, 0.9, 1.0]))
def test_sample_attention_mask_matches_brute_force(c, trunks, tau):
    N, Hq, Hkv, d, B = c["N"], c["Hq"], c["Hkv"], c["d"], c["B"]
    nt, rpt = trunks
    C = -(-N // nt)
    if (nt - 1) * C + rpt > N:
        return  # the sampling needs rpt positions in every trunk
    q, k, _ = small_inputs(N, Hq, Hkv, d, n_stripes=c["stripes"], band=0, seed=c["seed"])
    scale = 1.0 / math.sqrt(d)
    count, idx, ck, sk, col, sl = oracle.sample_attention_mask(q, k, B, tau, nt, rpt, c["diag"], c["first"])
    masks_b, cols_b, sl_b, colm_b, slm_b = brute.sample_mask(q, k, B, tau, nt, rpt, c["diag"], c["first"], scale)
    np.testing.assert_allclose(col, np.array(colm_b), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(sl, np.array(slm_b), rtol=1e-12, atol=1e-15)
    for h in range(Hq):
        assert set(np.nonzero(ck[h])[0].tolist()) == cols_b[h], h
        assert set(np.nonzero(sk[h])[0].tolist()) == sl_b[h], h
        for I in range(oracle.num_blocks(N, B)):
            o = oracle.tri_offset(I)
            assert idx[h, o:o + int(count[h, I])].tolist() == masks_b[(h, I)], (h, I)


@settings(max_examples=15, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(tiny_case(), st.booleans())
def test_two_pass_ratios_place_the_brute_force_stop(c, with_qperm):
    # the two-pass counterpart of test_marginal_gain_ratios_place_the_brute_force_stop: at each
    # history position whose ratio is a new low, a threshold just above it stops the brute force
    # there and one just below lets it go on (with and without the query permutation)
    N, Hq, Hkv, d, B, S = c["N"], c["Hq"], c["Hkv"], c["d"], c["B"], c["S"]
    q, k, _ = small_inputs(N, Hq, Hkv, d, n_stripes=c["stripes"], band=0, seed=c["seed"])
    scale = 1.0 / math.sqrt(d)
    pi, _ = oracle.prefix_kv_ranking(q, k, S)
    qperm = oracle.query_permutation(q, k, S) if with_qperm else None
    qorder = None if qperm is None else [qperm[g].tolist() for g in range(Hkv)]
    ranking = {(g, sigma): pi[g, oracle.prefix_offset(sigma, S):oracle.prefix_offset(sigma, S) + sigma * S].tolist()
               for g in range(Hkv) for sigma in range(1, oracle.num_segments(N, S))}
    ratios = oracle.s2o_prefix_gain_ratios(q, k, pi, B, S, qperm=qperm)
    checks = []
    for (h, I), r in ratios.items():
        assert np.all(np.isnan(r) | ((r > 0) & (r <= 1 + 1e-12))), (h, I, r)
        low = math.inf
        for p, x in enumerate(r):
            if not np.isnan(x) and x < low * (1 - 1e-6):
                checks.append((h, I, p, float(x), len(r)))
                low = x
    for h, I, p, x, full in checks[:6]:
        above = brute.s2o_prefix_processed(q, k, ranking, B, S, x * (1 + 1e-9), scale, qorder=qorder)[(h, I)]
        assert len(above) == p + 1, (h, I, p, x, above)
        below = brute.s2o_prefix_processed(q, k, ranking, B, S, x * (1 - 1e-9), scale, qorder=qorder)[(h, I)]
        assert len(below) > p + 1 or len(below) == full, (h, I, p, x, below)
