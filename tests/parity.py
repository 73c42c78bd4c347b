"""Comparison helpers for GPU-vs-oracle parity (imported by the gpu tests, smoke and bench).

Importance values: the GPU forms each logit c q.k from fixed-point digits of the bf16 rows (six
7-bit digits of a 42-bit integer at the row's largest exponent E, digit products of weight at
least 2^-42 of the leading one summed exactly in int32), so a logit is off by at most
  delta = c (u_q sum|k| + u_k sum|q| + d u_q u_k (1 + IMP_DROP)),  u = 2^(E - 168),
(the truncated elements and the dropped digit products; E of a key is the largest over its 64-key
chunk, never above the largest over all keys, so imp_logit_error takes the largest u over the rows
and keys of each KV group: a few 1e-10 on the workloads); every exponential, sum and
log-sum-exp after that is fp64, and only the chunk-normalised exponentials e (in (0, 1]) are kept
rounded to fp32 between launches.  A term exp(s - lse) of the (positive) mean then moves by at
most exp(2 delta) - 1 from the logit error and 2^-24 from the storage, so imp_gpu must lie within
imp_rtol = 2^-24 + 2.001 delta + 1e-12 relative (the 1e-12 for the fp64 steps) plus
IMP_ATOL = 2^-149 of the oracle's (compare_importance).

Tie rules, used wherever a floating-point comparison decides an integer result:
  * permutation: a rank where GPU and oracle list different keys is a recorded tie iff the two
    keys' oracle importances differ by at most 1e-6 relative (above twice imp_rtol);
  * block mask: a differing row is a recorded tie iff every differing block has
    |p_J - p_(k*)| <= 1e-6, or is the cut block or the next one in the oracle's order while the
    oracle's running mass C_{k*-1} or C_{k*} is within 1e-6 of tau; at most 1% of rows may tie;
  * early stop: the kernel decides  fl32(fl32(max S) * c32) >= theta  on scores S that the matrix
    cores sum in fp32 from exact bf16 x bf16 products.  Each score is then within
    gamma_d * sum_t |q_t k_t| of the exact dot product (gamma_n = n u / (1 - n u), u = 2^-24, the
    bound of any order of n fp32 additions), the max of a tile within the largest such bound over
    its valid entries, and the scaled value within that times c plus 4 u |m| more (the rounding of
    c to fp32 and of the product).  gate_error_bound gives this E per tile.  A decision must equal
    the fp64 oracle's  m >= theta  wherever |m - theta| > E; those inside the band are counted and
    reported (compare_gate).  The GPU gate must also equal the decision on the GPU's own reported
    tile maxima (the same fp32 values the kernel compares);
  * ranked order (marginal-gain stop): a position where GPU and oracle list different blocks is a
    recorded tie iff the two blocks' oracle pooled logits differ by at most 1e-6 relative;
  * historical ranking (S2O prefix order): the GPU ranks fp32-rounded scores; a rank where GPU and
    oracle list different keys is a recorded tie iff the two keys' oracle scores differ by at most
    1e-6 relative;
  * SampleAttention mask: the GPU's column / slash masses (fp64 sums of exponentials stored in
    fp32, as for the importance) must match the oracle's within imp_rtol relative (+ IMP_ATOL); a kept column or slash set may differ from the one the oracle's masses give only by
    members whose mass is within 1e-6 of the cut mass, or when the cumulative mass at the cut is
    within 1e-6 of the target; the GPU's mask must equal the tiles of the sets its own masses give;
  * marginal-gain stop: the kernel forms dl_i / l_i from bf16-rounded probabilities (each off by
    at most 2^-9 relative, so the ratio by under 0.4%); a stop or a go-on must agree with the
    oracle's exact ratio wherever that ratio is more than S2O_BAND (relative) from gain_tau.
"""
from __future__ import annotations

import numpy as np

import oracle

TIE = 1e-6
O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
S2O_BAND = 1e-2
F32_U = 2.0 ** -24
IMP_ATOL = 2.0 ** -149


# Weight of the digit products the logits leave out, per element and in units of u_q u_k: levels
# a + b = 6..10 of two six-digit numbers (11 - L pairs at level L, |digit products| <= 2^14).
IMP_DROP = 2 ** 14 * (5 * 2 ** 28 + 4 * 2 ** 21 + 3 * 2 ** 14 + 2 * 2 ** 7 + 1)


def _row_unit(x: np.ndarray) -> np.ndarray:
    """2^(E - 168) per row of bf16 values held in fp64, E the row's largest exponent field (at
    least 1): the unit of the row's 42-bit fixed-point form."""
    amax = np.abs(x).max(axis=-1)
    _, ex = np.frexp(amax)  # amax = f 2^ex, f in [0.5, 1): exponent field ex + 126 for a normal
    e = np.where(amax > 0, ex + 126, 0)
    return np.ldexp(1.0, np.maximum(e, 1) - 168)


def imp_logit_error(q: np.ndarray, k: np.ndarray, scale: float | None = None) -> float:
    """Upper bound of |GPU logit - c q.k| over every query row of each KV group's heads and every
    key of that group (the rule in the module docstring; sums of maxima bound the max of sums)."""
    Hq, _, d = q.shape
    Hkv = k.shape[0]
    G = Hq // Hkv
    c = 1.0 / np.sqrt(d) if scale is None else scale
    worst = 0.0
    for g in range(Hkv):
        qg = q[g * G:(g + 1) * G].reshape(-1, d)
        uq, sq = _row_unit(qg).max(), np.abs(qg).sum(axis=-1).max()
        uk, sk = _row_unit(k[g]).max(), np.abs(k[g]).sum(axis=-1).max()
        worst = max(worst, c * (uq * sk + uk * sq + d * uq * uk * (1 + IMP_DROP)))
    return float(worst)


def imp_rtol(q: np.ndarray, k: np.ndarray, scale: float | None = None) -> float:
    """Relative tolerance of GPU importances (and SampleAttention masses) for these inputs."""
    return F32_U + 2.001 * imp_logit_error(q, k, scale) + 1e-12


def compare_importance(imp_g: np.ndarray, imp_o: np.ndarray, rtol: float) -> float:
    """Assert the GPU importance is within rtol relative (+ IMP_ATOL) of the oracle's; return the
    largest relative error seen."""
    err = np.abs(imp_g - imp_o)
    lim = rtol * np.abs(imp_o) + IMP_ATOL
    bad = np.argwhere(err > lim)
    assert bad.size == 0, f"importance off at {bad[:5].tolist()}: gpu {imp_g[tuple(bad[0])]!r} oracle {imp_o[tuple(bad[0])]!r}"
    nz = imp_o != 0
    return float((err[nz] / np.abs(imp_o[nz])).max()) if nz.any() else 0.0


def fp32_sum_gamma(n: int) -> float:
    """gamma_n = n u / (1 - n u): relative bound of summing n terms in fp32 in any order."""
    return n * F32_U / (1.0 - n * F32_U)


def gate_error_bound(q, k, perm, B, S, rows, scale=None):
    """{(h, I): array over J <= I} of the fp32 error bound E of the GPU's scaled tile max, without
    the 4 u |m| term (added by compare_gate): c * gamma_d * max over the tile's valid (i, j), j <= i,
    of sum_t |q_it k_jt|.  perm: [Hkv][N] or None; rows are read as the gate reads them."""
    Hq, N, d = q.shape
    G = Hq // k.shape[0]
    c = 1.0 / np.sqrt(d) if scale is None else scale
    gam = fp32_sum_gamma(d)
    aq, ak = np.abs(q), np.abs(k)
    out = {}
    for h, I in rows:
        qi = oracle.block_range(I, B, N)
        pg = None if perm is None else perm[h // G]
        e = np.empty(I + 1)
        for J in range(I + 1):
            kj = oracle.key_rows_of_block(J, I, pg, B, S, N)
            sabs = aq[h, qi] @ ak[h // G, kj].T
            e[J] = np.where(kj[None, :] <= qi[:, None], sabs, -np.inf).max()
        out[(h, I)] = c * gam * e
    return out


def compare_gate(kept, sel, tm_exact, bound, theta):
    """Assert every early-stop decision of the rows in `bound` ({(h, I): E over J}) equals the
    exact decision m >= theta wherever |m - theta| > E + 4 u |m|, and that the diagonal is kept.
    kept: {(h, I): kept J}; sel: {(h, I): the J the gate looked at}; tm_exact: {(h, I): m over J}.
    Returns (decisions, decisions inside the band)."""
    n = band = 0
    for (h, I), e in bound.items():
        got = set(kept[(h, I)])
        assert got <= set(sel[(h, I)]), f"gate row ({h},{I}) kept a tile it was not given"
        th = float(theta[h, I])
        for J in sel[(h, I)]:
            if J == I:
                assert J in got, f"gate row ({h},{I}): diagonal dropped"
                continue
            m = float(tm_exact[(h, I)][J])
            n += 1
            if abs(m - th) <= e[J] + 4 * F32_U * abs(m):
                band += 1
                continue
            assert (J in got) == (m >= th), \
                f"gate ({h},{I},{J}): kept {J in got}, exact max {m!r}, theta {th!r}, bound {e[J]:.3e}"
    return n, band


def compare_perm(perm_gpu: np.ndarray, perm_o: np.ndarray, imp_o: np.ndarray, S: int) -> int:
    """Assert the GPU permutation equals the oracle's up to recorded ties; return the tie count."""
    Hkv, N = perm_o.shape
    for g in range(Hkv):
        for a in range(0, N, S):
            seg = perm_gpu[g, a:min(a + S, N)]
            assert sorted(seg.tolist()) == list(range(a, min(a + S, N))), f"perm head {g} segment {a // S} not a bijection"
    ties = 0
    for g, p in np.argwhere(perm_gpu != perm_o):
        x, y = int(perm_gpu[g, p]), int(perm_o[g, p])
        ix, iy = imp_o[g, x], imp_o[g, y]
        rel = abs(ix - iy) / max(abs(ix), abs(iy), 1e-300)
        assert rel <= TIE, f"perm head {g} rank {p}: gpu key {x} ({ix!r}) vs oracle key {y} ({iy!r})"
        ties += 1
    return ties


def _row(idx, count, h, I):
    o = oracle.tri_offset(I)
    return [int(x) for x in idx[h, o:o + int(count[h, I])]]


def compare_mask(count_g, idx_g, count_o, idx_o, prob_o, tau: float, max_tie_frac: float = 0.01) -> int:
    """Assert the GPU mask equals the oracle's up to recorded ties; return the number of tie rows.

    A row may differ only by blocks whose p is within TIE of the cut block's p (the sort order among
    near-equal probabilities), or -- when the oracle's cumulative mass just before or at the cut is
    within TIE of tau -- by the cut block order[k*-1] (left out) or the next one order[k*] (taken
    too).  At most max_tie_frac of the rows (and at least 2) may be tie rows."""
    Hq, NB = count_o.shape
    ties = 0
    for h in range(Hq):
        for I in range(NB):
            rg, ro = _row(idx_g, count_g, h, I), _row(idx_o, count_o, h, I)
            assert rg == sorted(set(rg)) and all(0 <= J <= I for J in rg), f"row ({h},{I}) malformed {rg}"
            if rg == ro:
                continue
            o = oracle.tri_offset(I)
            p = prob_o[h, o:o + I + 1]
            order = np.lexsort((np.arange(I + 1), -p))
            csum = np.cumsum(p[order])
            hit = np.nonzero(csum >= tau)[0]
            kstar = int(hit[0]) + 1 if (tau < 1.0 and hit.size) else I + 1
            pk = p[order[kstar - 1]]
            diff = set(rg) ^ set(ro)
            allowed = {J for J in range(I + 1) if abs(p[J] - pk) <= TIE}
            near_c = abs(csum[kstar - 1] - tau) <= TIE or (kstar >= 2 and abs(csum[kstar - 2] - tau) <= TIE)
            if near_c:
                allowed.add(int(order[kstar - 1]))
                if kstar < I + 1:
                    allowed.add(int(order[kstar]))
            assert diff <= allowed, f"mask row ({h},{I}): gpu {rg} vs oracle {ro} differ by {sorted(diff - allowed)}"
            ties += 1
    assert ties <= max(2, int(max_tie_frac * Hq * NB)), f"{ties} tie rows of {Hq * NB}"
    return ties


def compare_ranked(count_g, idx_g, count_o, idx_o, z_o) -> int:
    """Assert the GPU ranked lists equal the oracle's up to recorded ties; return the tie count."""
    Hq, NB = count_o.shape
    assert np.array_equal(count_g, count_o), "ranked counts differ"
    ties = 0
    for h in range(Hq):
        for I in range(NB):
            rg, ro = _row(idx_g, count_g, h, I), _row(idx_o, count_o, h, I)
            assert sorted(rg) == list(range(I + 1)), f"ranked row ({h},{I}) is not a permutation of 0..I"
            o = oracle.tri_offset(I)
            for p, (a, b) in enumerate(zip(rg, ro)):
                if a != b:
                    za, zb = z_o[h, o + a], z_o[h, o + b]
                    assert abs(za - zb) <= TIE * max(abs(za), abs(zb), 1.0), \
                        f"ranked row ({h},{I}) position {p}: gpu {a} (z {za!r}) vs oracle {b} (z {zb!r})"
                    ties += 1
    return ties


def compare_s2o_stops(kept, count_g, idx_g, ratios, gain_tau: float, band: float = S2O_BAND, row_stride=None):
    """Assert each row's processed blocks (kept: {(h, I): ascending J}) are a prefix of the GPU's
    ranked list whose end the oracle's gain ratios allow; return (rows, rows decided in the band).
    row_stride: entries per row when the lists are not packed as a triangle."""
    near = 0
    for (h, I), r in ratios.items():
        if row_stride is None:
            lst = _row(idx_g, count_g, h, I)
        else:
            lst = [int(x) for x in idx_g[h, I * row_stride:I * row_stride + int(count_g[h, I])]]
        got = kept[(h, I)]
        n = len(got)
        assert n >= 1 and sorted(lst[:n]) == got, f"s2o row ({h},{I}): processed {got} is not a prefix of {lst}"
        hist = ~np.isnan(r)
        for p in range(n - 1):
            assert not hist[p] or r[p] >= gain_tau * (1 - band), \
                f"s2o row ({h},{I}): went on past position {p} with ratio {r[p]!r} < {gain_tau}"
        if n < len(lst):
            assert hist[n - 1] and r[n - 1] < gain_tau * (1 + band), \
                f"s2o row ({h},{I}): stopped at position {n - 1} (ratio {r[n - 1]!r}, threshold {gain_tau})"
        stop = np.nonzero(hist & (r < gain_tau))[0]
        exact_n = int(stop[0]) + 1 if stop.size else len(lst)
        near += exact_n != n
    return len(ratios), near


def compare_prefix_rank(pi_g, pi_o, score_o, S: int) -> int:
    """Assert every (g, sigma) list of the GPU's historical ranking is a permutation of its prefix and
    equals the oracle's up to recorded ties; return the tie count."""
    Hkv, L = pi_o.shape
    assert pi_g.shape == pi_o.shape, (pi_g.shape, pi_o.shape)
    ties = 0
    sigma = 1
    while oracle.prefix_offset(sigma, S) < L:
        o, n = oracle.prefix_offset(sigma, S), sigma * S
        for g in range(Hkv):
            a, b = pi_g[g, o:o + n], pi_o[g, o:o + n]
            assert np.array_equal(np.sort(a), np.arange(n)), f"ranking ({g},{sigma}) is not a permutation of its prefix"
            diff = np.nonzero(a != b)[0]
            if diff.size:
                z = np.empty(n)
                z[b] = score_o[g, o:o + n]
                za, zb = z[a[diff]], z[b[diff]]
                tol = TIE * np.maximum(np.maximum(np.abs(za), np.abs(zb)), 1e-30)
                bad = np.nonzero(np.abs(za - zb) > tol)[0]
                assert bad.size == 0, (f"ranking ({g},{sigma}) rank {diff[bad[0]]}: gpu key {a[diff[bad[0]]]} "
                                       f"(score {za[bad[0]]!r}) vs oracle key {b[diff[bad[0]]]} ({zb[bad[0]]!r})")
                ties += diff.size
        sigma += 1
    return ties


def two_pass_lists(Hq: int, N: int, B: int, S: int, permuted_queries: bool = False):
    """count/idx of S2O's two-pass lists: the own segment's blocks ascending (up to I, or to the
    segment's last block with permuted queries), then prefix blocks 0 .. J0-1.  Rows are laid out
    as the packed triangle, or NB entries per row with permuted queries."""
    NB = -(-N // B)
    count = np.zeros((Hq, NB), dtype=np.int64)
    idx = np.full((Hq, NB * NB if permuted_queries else NB * (NB + 1) // 2), -1, dtype=np.int64)
    for I in range(NB):
        sigma = (I * B) // S
        J0 = sigma * S // B
        Jend = -(-min((sigma + 1) * S, N) // B) - 1 if permuted_queries else I
        o = I * NB if permuted_queries else oracle.tri_offset(I)
        lst = list(range(J0, Jend + 1)) + list(range(J0))
        count[:, I] = len(lst)
        idx[:, o:o + len(lst)] = lst
    return count, idx


def bitmap_to_kept_square(bm: np.ndarray, NB: int):
    """{(h, I): [J ...]} from a [Hq][words] bitmap with NB bits per row (bit I*NB + J)."""
    bm = bm.astype(np.uint32)
    kept = {}
    for h in range(bm.shape[0]):
        for I in range(NB):
            kept[(h, I)] = [J for J in range(NB) if (bm[h, (I * NB + J) // 32] >> np.uint32((I * NB + J) % 32)) & 1]
    return kept


def _cut_is_near_tie(m: np.ndarray, tau: float, a: np.ndarray, b: np.ndarray) -> bool:
    """Whether two kept sets of the mass cut over m may differ by rounding: every differing member
    has a mass within TIE of the cut mass, or the running sum at the cut is within TIE of tau."""
    n = len(m)
    order = np.lexsort((np.arange(n), -m))
    cs = np.cumsum(m[order])
    hit = np.nonzero(cs >= tau)[0]
    kstar = int(hit[0]) + 1 if (tau < 1.0 and hit.size) else n
    cut_mass = m[order[kstar - 1]]
    diff = np.nonzero(a != b)[0]
    near_m = np.all(np.abs(m[diff] - cut_mass) <= TIE)
    near_c = abs(cs[kstar - 1] - tau) <= TIE or (kstar >= 2 and abs(cs[kstar - 2] - tau) <= TIE)
    return bool(near_m or near_c)


def compare_sample_mask(count_g, idx_g, col_g, slash_g, col_o, slash_o, tau: float, B: int, force_diag: bool,
                        force_first: bool, rtol: float) -> int:
    """Assert the GPU SampleAttention mask against the oracle (rules above; rtol = imp_rtol of the
    inputs); return the tie count."""
    compare_importance(col_g, col_o, rtol)
    compare_importance(slash_g, slash_o, rtol)
    Hq = col_o.shape[0]
    ck_g = np.stack([oracle.mass_cut(col_g[h], tau) for h in range(Hq)])
    sk_g = np.stack([oracle.mass_cut(slash_g[h], tau) for h in range(Hq)])
    ties = 0
    for h in range(Hq):
        for keep_g, m in ((ck_g[h], col_o[h]), (sk_g[h], slash_o[h])):
            keep_o = oracle.mass_cut(m, tau)
            if not np.array_equal(keep_g, keep_o):
                assert _cut_is_near_tie(m, tau, keep_g, keep_o), f"head {h}: kept pattern set differs beyond ties"
                ties += 1
    count_w, idx_w = oracle.mask_from_patterns(ck_g, sk_g, B, force_diag, force_first)
    assert np.array_equal(count_g, count_w), "mask counts differ from the GPU masses' patterns"
    for h in range(Hq):
        for I in range(count_w.shape[1]):
            assert _row(idx_g, count_g, h, I) == _row(idx_w, count_w, h, I), f"mask row ({h},{I})"
    return ties


def compare_out(out_g: np.ndarray, out_o: np.ndarray, what: str = "out"):
    """Max and mean abs error over the rows the oracle computed (non-NaN)."""
    ok = ~np.isnan(out_o)
    err = np.abs(out_g[ok] - out_o[ok])
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= O_MAX_ABS and mean <= O_MEAN_ABS, f"{what}: max abs {mx:.3e}, mean abs {mean:.3e}"
    return mx, mean


def compare_lse(lse_g: np.ndarray, lse_o: np.ndarray):
    ok = ~np.isnan(lse_o)
    a, b = lse_g[ok], lse_o[ok]
    inf = np.isinf(b)
    assert np.array_equal(np.isinf(a), inf), "lse: -inf pattern differs"
    err = np.abs(a[~inf] - b[~inf])
    assert err.size == 0 or err.max() <= O_MAX_ABS, f"lse: max abs {err.max():.3e}"


def bitmap_to_kept(bm: np.ndarray, NB: int):
    """{(h, I): [J ...]} from a [Hq][words] kept-tile bitmap."""
    bm = bm.astype(np.uint32)
    kept = {}
    for h in range(bm.shape[0]):
        for I in range(NB):
            o = oracle.tri_offset(I)
            kept[(h, I)] = [J for J in range(I + 1) if (bm[h, (o + J) // 32] >> np.uint32((o + J) % 32)) & 1]
    return kept


def kept_to_mask(kept, Hq: int, NB: int):
    count = np.zeros((Hq, NB), dtype=np.int64)
    idx = np.full((Hq, NB * (NB + 1) // 2), -1, dtype=np.int64)
    for (h, I), lst in kept.items():
        o = oracle.tri_offset(I)
        count[h, I] = len(lst)
        idx[h, o:o + len(lst)] = lst
    return count, idx
