"""Pure-Python brute force of every stage, for tiny shapes (test infrastructure only).

Written independently of ``pbsa_oracle``: per-(h, i, j) predicates, explicit loops, ``math.fsum``
for every sum, and an exhaustive search over block subsets for the mask instead of a sort.  It is
the check that pins the NumPy oracle on shapes with N <= 64, d <= 8 and at most 13 blocks.
"""
from __future__ import annotations

import itertools
import math
from typing import Dict, List, Optional, Tuple


def _dot(a, b) -> float:
    return math.fsum(float(x) * float(y) for x, y in zip(a, b))


def _seg(pos_block_start: int, S: Optional[int]) -> int:
    return 0 if S is None else pos_block_start // S


def importance(q, k, B: int, scale: float) -> List[List[float]]:
    """imp[g][j] = (1 / (G * R)) * sum over the last-block rows of the causal softmax weight of j."""
    Hq, N = len(q), len(q[0])
    Hkv = len(k)
    G = Hq // Hkv
    rows = list(range(max(0, N - B), N))
    imp = []
    for g in range(Hkv):
        parts: List[List[float]] = [[] for _ in range(N)]
        for h in range(g * G, (g + 1) * G):
            for i in rows:
                s = [scale * _dot(q[h][i], k[g][j]) for j in range(i + 1)]
                m = max(s)
                z = math.fsum(math.exp(x - m) for x in s)
                lse = m + math.log(z)
                for j in range(i + 1):
                    parts[j].append(math.exp(s[j] - lse))
        imp.append([math.fsum(parts[j]) / (G * len(rows)) for j in range(N)])
    return imp


def check_permutation(perm, imp, S: int, tol: float = 1e-12) -> None:
    """perm must map each segment onto itself and list it by importance desc, position asc."""
    Hkv, N = len(perm), len(perm[0])
    for g in range(Hkv):
        for a in range(0, N, S):
            b = min(a + S, N)
            seg = [int(x) for x in perm[g][a:b]]
            assert sorted(seg) == list(range(a, b)), "not a bijection on its segment"
            for r in range(len(seg) - 1):
                x, y = seg[r], seg[r + 1]
                ix, iy = imp[g][x], imp[g][y]
                if abs(ix - iy) <= tol * max(abs(ix), abs(iy), 1e-300):
                    assert x < y, "equal importance not in position order"
                else:
                    assert ix > iy, "importance not descending"


def _key_rows(J: int, I: int, perm_g, B: int, S: Optional[int], N: int) -> List[int]:
    out = []
    for t in range(B):
        p = J * B + t
        if p >= N:
            break
        if perm_g is not None and _seg(J * B, S) < _seg(I * B, S):
            out.append(int(perm_g[p]))
        else:
            out.append(p)
    return out


def mask(q, k, perm, B: int, S: Optional[int], tau: float, force_diag: bool, force_first: bool,
         scale: float) -> Tuple[Dict[Tuple[int, int], List[int]], Dict[Tuple[int, int], List[float]]]:
    """Selected blocks per (h, I) by exhaustive subset search (I <= 12).

    Among all subsets of {0..I} whose pooled probability mass reaches tau, take the smallest
    cardinality, then the largest mass, then the lexicographically smallest index tuple.
    """
    Hq, N, d = len(q), len(q[0]), len(q[0][0])
    Hkv = len(k)
    G = Hq // Hkv
    NB = -(-N // B)
    sel, probs = {}, {}
    for h in range(Hq):
        g = h // G
        pg = None if perm is None else perm[g]
        for I in range(NB):
            qrows = list(range(I * B, min((I + 1) * B, N)))
            qbar = [math.fsum(float(q[h][i][t]) for i in qrows) / len(qrows) for t in range(d)]
            z = []
            for J in range(I + 1):
                kr = _key_rows(J, I, pg, B, S, N)
                kbar = [math.fsum(float(k[g][j][t]) for j in kr) / len(kr) for t in range(d)]
                z.append(scale * _dot(qbar, kbar))
            m = max(z)
            tot = math.fsum(math.exp(x - m) for x in z)
            p = [math.exp(x - m) / tot for x in z]
            probs[(h, I)] = p
            best = None
            if tau >= 1.0:
                best = tuple(range(I + 1))
            else:
                for size in range(1, I + 2):
                    cands = []
                    for sub in itertools.combinations(range(I + 1), size):
                        mass = math.fsum(p[J] for J in sub)
                        if mass >= tau:
                            cands.append((-mass, sub))
                    if cands:
                        best = min(cands)[1]
                        break
                if best is None:
                    best = tuple(range(I + 1))
            chosen = set(best)
            if force_diag:
                chosen.add(I)
            if force_first:
                chosen.add(0)
            sel[(h, I)] = sorted(chosen)
    return sel, probs


def attention(q, k, v, perm, sel: Dict[Tuple[int, int], List[int]], B: int, S: Optional[int],
              scale: float, theta=None):
    """o[h][i] and lse[h][i] over the union of (kept) selected blocks, per-element predicates."""
    Hq, N, d = len(q), len(q[0]), len(q[0][0])
    Hkv = len(k)
    G = Hq // Hkv
    NB = -(-N // B)
    out = [[None] * N for _ in range(Hq)]
    lse = [[None] * N for _ in range(Hq)]
    kept = {}
    for h in range(Hq):
        g = h // G
        pg = None if perm is None else perm[g]
        for I in range(NB):
            qrows = list(range(I * B, min((I + 1) * B, N)))
            blocks = []
            for J in sel[(h, I)]:
                kr = _key_rows(J, I, pg, B, S, N)
                if theta is not None and J != I:
                    mx = max(scale * _dot(q[h][i], k[g][j]) for i in qrows for j in kr if j <= i)
                    if mx < theta[h][I]:
                        continue
                blocks.append((J, kr))
            kept[(h, I)] = [J for J, _ in blocks]
            for i in qrows:
                keys = [j for _, kr in blocks for j in kr if j <= i]
                if not keys:
                    out[h][i] = [0.0] * d
                    lse[h][i] = -math.inf
                    continue
                s = [scale * _dot(q[h][i], k[g][j]) for j in keys]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                z = math.fsum(w)
                out[h][i] = [math.fsum(w[n] * float(v[g][j][t]) for n, j in enumerate(keys)) / z
                             for t in range(d)]
                lse[h][i] = m + math.log(z)
    return out, lse, kept


def s2o_processed(q, k, perm, B: int, S: int, gain_tau: float, scale: float) -> Dict[Tuple[int, int], List[int]]:
    """Blocks the marginal-gain early stop processes per (h, I), from its definition.

    Order: the blocks of I's own segment ascending, then the earlier-segment blocks picked one by
    one as the remaining block with the largest pooled logit (the smallest J among equals).  The
    stop is the first earlier-segment block b of that order after which, for every query i of
    block I, the exact share of b in the softmax denominator over all processed keys (each sum an
    fsum of exp(s - M_i) with M_i the max over every key <= i of the row) is below gain_tau.
    """
    Hq, N, d = len(q), len(q[0]), len(q[0][0])
    Hkv = len(k)
    G = Hq // Hkv
    NB = -(-N // B)
    out = {}
    for h in range(Hq):
        g = h // G
        pg = None if perm is None else perm[g]
        for I in range(NB):
            qrows = list(range(I * B, min((I + 1) * B, N)))
            qbar = [math.fsum(float(q[h][i][t]) for i in qrows) / len(qrows) for t in range(d)]
            z = {}
            for J in range(I + 1):
                kr = _key_rows(J, I, pg, B, S, N)
                kbar = [math.fsum(float(k[g][j][t]) for j in kr) / len(kr) for t in range(d)]
                z[J] = scale * _dot(qbar, kbar)
            own = [J for J in range(I + 1) if _seg(J * B, S) == _seg(I * B, S)]
            rest = [J for J in range(I + 1) if _seg(J * B, S) < _seg(I * B, S)]
            order = list(own)
            while rest:
                best = max(rest, key=lambda J: (z[J], -J))
                order.append(best)
                rest.remove(best)
            logit = {(i, j): scale * _dot(q[h][i], k[g][j]) for i in qrows
                     for J in order for j in _key_rows(J, I, pg, B, S, N) if j <= i}
            ref = {i: max(v for (ii, _), v in logit.items() if ii == i) for i in qrows}
            done = []
            for t, J in enumerate(order):
                done.append(J)
                if _seg(J * B, S) == _seg(I * B, S):
                    continue
                stop = True
                for i in qrows:
                    keys_all = [j for JJ in done for j in _key_rows(JJ, I, pg, B, S, N) if j <= i]
                    keys_b = [j for j in _key_rows(J, I, pg, B, S, N) if j <= i]
                    ell = math.fsum(math.exp(logit[(i, j)] - ref[i]) for j in keys_all)
                    dl = math.fsum(math.exp(logit[(i, j)] - ref[i]) for j in keys_b)
                    if not dl < gain_tau * ell:
                        stop = False
                        break
                if stop:
                    break
            out[(h, I)] = done
    return out


def prefix_ranking(q, k, S: int) -> Dict[Tuple[int, int], List[int]]:
    """{(g, sigma): keys of the prefix [0, sigma*S) in ranked order} for sigma >= 1, from the
    definition: the representative is the fsum mean of the segment's query rows over the G heads of
    KV head g; keys are picked one by one as the remaining key with the largest r . k_j (the
    smallest j among equals)."""
    Hq, N, d = len(q), len(q[0]), len(q[0][0])
    Hkv = len(k)
    G = Hq // Hkv
    nseg = -(-N // S)
    res = {}
    for g in range(Hkv):
        for sigma in range(1, nseg):
            qrows = [q[h][i] for h in range(g * G, (g + 1) * G) for i in range(sigma * S, min((sigma + 1) * S, N))]
            r = [math.fsum(float(x[t]) for x in qrows) / len(qrows) for t in range(d)]
            z = {j: _dot(r, k[g][j]) for j in range(sigma * S)}
            rest = list(range(sigma * S))
            order = []
            while rest:
                best = max(rest, key=lambda j: (z[j], -j))
                order.append(best)
                rest.remove(best)
            res[(g, sigma)] = order
    return res


def query_order(q, k, S: int) -> List[List[int]]:
    """qperm[g] from the definition: guide u = fsum mean of KV head g's keys; score of position i =
    fsum mean over the G heads of q_{h,i} . u; inside each segment positions picked one by one as
    the remaining one of largest score (smallest position among equals)."""
    Hq, N, d = len(q), len(q[0]), len(q[0][0])
    Hkv = len(k)
    G = Hq // Hkv
    res = []
    for g in range(Hkv):
        u = [math.fsum(float(k[g][j][t]) for j in range(N)) / N for t in range(d)]
        z = [math.fsum(_dot(q[h][i], u) for h in range(g * G, (g + 1) * G)) / G for i in range(N)]
        order = []
        for a in range(0, N, S):
            rest = list(range(a, min(a + S, N)))
            while rest:
                best = max(rest, key=lambda i: (z[i], -i))
                order.append(best)
                rest.remove(best)
        res.append(order)
    return res


def s2o_prefix_processed(q, k, ranking: Dict[Tuple[int, int], List[int]], B: int, S: int, gain_tau: float,
                         scale: float, qorder: Optional[List[List[int]]] = None) -> Dict[Tuple[int, int], List[int]]:
    """Entries the two-pass marginal-gain stop processes per (h, I), from its definition: the
    blocks of I's own segment in natural order (J0 .. I, J0 its first block), then history blocks
    J = 0, 1, ... holding ranked keys J*B .. J*B+B-1 of the segment's order; stop after the first
    history block whose exact share (fsum of exp(s - M_i), M_i the max over every listed key <= i)
    of every query's denominator over the processed keys is below gain_tau.  With qorder, query
    block I holds positions qorder[g][I*B ...] and pass 1 spans every block of the own segment."""
    Hq, N = len(q), len(q[0])
    Hkv = len(k)
    G = Hq // Hkv
    NB = -(-N // B)
    out = {}
    for h in range(Hq):
        g = h // G
        for I in range(NB):
            sigma = (I * B) // S
            J0 = sigma * S // B
            rank = ranking.get((g, sigma), [])

            def rows_of(J):
                if J >= J0:
                    return list(range(J * B, min((J + 1) * B, N)))
                return rank[J * B:(J + 1) * B]
            if qorder is None:
                order = list(range(J0, I + 1)) + list(range(J0))
                qrows = list(range(I * B, min((I + 1) * B, N)))
            else:
                last = -(-min((sigma + 1) * S, N) // B) - 1
                order = list(range(J0, last + 1)) + list(range(J0))
                qrows = qorder[g][I * B:min((I + 1) * B, N)]
            logit = {(i, j): scale * _dot(q[h][i], k[g][j]) for i in qrows for J in order for j in rows_of(J) if j <= i}
            ref = {i: max(v for (ii, _), v in logit.items() if ii == i) for i in qrows}
            done = []
            for J in order:
                done.append(J)
                if J >= J0:
                    continue
                stop = True
                for i in qrows:
                    keys_all = [j for JJ in done for j in rows_of(JJ) if j <= i]
                    keys_b = [j for j in rows_of(J) if j <= i]
                    ell = math.fsum(math.exp(logit[(i, j)] - ref[i]) for j in keys_all)
                    dl = math.fsum(math.exp(logit[(i, j)] - ref[i]) for j in keys_b)
                    if not dl < gain_tau * ell:
                        stop = False
                        break
                if stop:
                    break
            out[(h, I)] = done
    return out


def attention_over_keys(q, k, v, keysets: Dict[Tuple[int, int], List[int]], B: int, scale: float,
                        qorder: Optional[List[List[int]]] = None):
    """out[h][i], lse[h][i] for the rows of the given (h, I): softmax over keysets[(h, I)] restricted
    to j <= i, each sum an fsum (rows not listed stay None).  Row (h, I) holds query positions
    I*B ... or, with qorder, qorder[g][I*B ...]."""
    Hq, N, d = len(q), len(q[0]), len(q[0][0])
    G = Hq // len(k)
    out = [[None] * N for _ in range(Hq)]
    lse = [[None] * N for _ in range(Hq)]
    for (h, I), keys in keysets.items():
        g = h // G
        qrows = range(I * B, min((I + 1) * B, N)) if qorder is None else qorder[g][I * B:min((I + 1) * B, N)]
        for i in qrows:
            ks = [j for j in keys if j <= i]
            s = [scale * _dot(q[h][i], k[g][j]) for j in ks]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = math.fsum(w)
            out[h][i] = [math.fsum(w[a] * float(v[g][ks[a]][t]) for a in range(len(ks))) / z for t in range(d)]
            lse[h][i] = m + math.log(z)
    return out, lse


def sample_mask(q, k, B: int, tau: float, n_trunks: int, rows_per_trunk: int, force_diag: bool, force_first: bool,
                scale: float):
    """SampleAttention's mask from its definition: sampled rows (last rows of equal chunks), exact
    causal softmax rows (fsum), per-column and per-diagonal mean mass (fsum), each family cut by
    repeated selection of its heaviest member (smallest index among equals) until the fsum of the
    chosen reaches tau (all members when tau >= 1 or never reached), and tile (I, J) kept when some
    pair i in I, j in J, j <= i has j a chosen column or i - j a chosen diagonal, or when forced.
    Returns ({(h, I): [J ...]}, [col set per head], [slash set per head], col, slash)."""
    Hq, N = len(q), len(q[0])
    G = Hq // len(k)
    C = -(-N // n_trunks)
    rows = [i for t in range(n_trunks) for i in range(min((t + 1) * C, N) - rows_per_trunk, min((t + 1) * C, N))]
    NB = -(-N // B)
    masks, cols, slashes, colm, slm = {}, [], [], [], []
    for h in range(Hq):
        g = h // G
        pc = [[] for _ in range(N)]
        ps = [[] for _ in range(N)]
        for i in rows:
            s = [scale * _dot(q[h][i], k[g][j]) for j in range(i + 1)]
            m = max(s)
            z = math.fsum(math.exp(x - m) for x in s)
            for j in range(i + 1):
                p = math.exp(s[j] - m) / z
                pc[j].append(p)
                ps[i - j].append(p)
        col = [math.fsum(x) / len(rows) for x in pc]
        sl = [math.fsum(x) / len(rows) for x in ps]

        def cut(mv):
            if tau >= 1.0:
                return set(range(N))
            rest, chosen = list(range(N)), []
            while rest and math.fsum(mv[x] for x in chosen) < tau:
                best = max(rest, key=lambda x: (mv[x], -x))
                chosen.append(best)
                rest.remove(best)
            return set(chosen)
        cs, ss = cut(col), cut(sl)
        for I in range(NB):
            lst = []
            for J in range(I + 1):
                keep = (force_diag and J == I) or (force_first and J == 0)
                for i in range(I * B, min((I + 1) * B, N)):
                    for j in range(J * B, min((J + 1) * B, N)):
                        if j <= i and (j in cs or (i - j) in ss):
                            keep = True
                if keep:
                    lst.append(J)
            masks[(h, I)] = lst
        cols.append(cs)
        slashes.append(ss)
        colm.append(col)
        slm.append(sl)
    return masks, cols, slashes, colm, slm
