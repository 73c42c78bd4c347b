"""fp64 NumPy oracle for permuted block-sparse attention prefill (test infrastructure only).

Notation (batch 1): N tokens, Hq query heads, Hkv KV heads, G = Hq / Hkv, g(h) = h // G,
head dim d, block size B (query block = key block), segment size S (a multiple of B),
NB = ceil(N / B) blocks, block J = tokens [J*B, min((J+1)*B, N)), segment of block J
sigma(J) = (J*B) // S, logit scale c = 1/sqrt(d) unless given.

Inputs are fp64 arrays laid out [heads][tokens][d]; the GPU path receives the same values as
bf16, so callers pass the bf16-rounded values widened to fp64.

Readings taken where the pages leave a step open (each is listed with its reason in the
design notes of the repository):
  * importance rows are the last B query positions [max(0, N-B), N) of every query head of the
    KV group; masked (j > i) entries count as zero; the mean divides by G * (number of rows);
  * one permutation per KV head, sorting by importance descending, ties by position ascending;
  * a query block reads its own segment in natural order; only strictly earlier segments are
    read through the permutation;
  * pooled block score = c * (mean query of the block) . (mean key of the key block), softmax
    over J <= I, no intra-block causal mask on the diagonal block's score;
  * the mask keeps the shortest prefix of the (p desc, J asc) order whose cumulative mass
    reaches tau (>=), plus the forced blocks; tau >= 1 keeps every J <= I;
  * the early-stop gate is decided per whole tile on the exact max of the scaled causal
    logits; a skipped tile contributes nothing to the softmax state;
  * the marginal-gain early stop visits the query block's own segment first (ascending), then the
    earlier-segment blocks by pooled logit descending (ties by J), and stops a tile row after the
    first earlier-segment block whose share of every query's softmax denominator (that block
    included) is below the threshold; that block stays processed;
  * S2O's historical ranking uses one representative query per (KV head, segment): the mean of the
    segment's query rows over the G query heads; it orders every key of the causal prefix (the
    earlier segments) by its dot product with that query, descending, ties by position;
  * S2O's query permutation scores each query against one guide vector per KV head, the mean key,
    averaged over the G query heads, and sorts each segment's positions by it (descending, ties by
    position); a permuted query block then needs the whole own segment in pass 1 under the
    per-token causal mask, and its output rows go back to their natural positions;
  * SampleAttention's estimator samples the last rows of n_trunks equal chunks, takes the exact
    causal softmax of those rows, averages it per key column and per diagonal offset, keeps for
    each family separately the heaviest members up to the CIA mass target (the block_mask rule),
    and keeps every tile that holds a kept column or that a kept diagonal crosses.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np


# ----------------------------------------------------------------------------- geometry

def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def num_blocks(n: int, b: int) -> int:
    return -(-n // b)


def block_range(J: int, B: int, N: int) -> np.ndarray:
    """Token positions of natural block J."""
    return np.arange(J * B, min((J + 1) * B, N))


def segment_of_block(J: int, B: int, S: Optional[int]) -> int:
    """Segment index of block J (Sparser Block-Sparse Attention via Token Permutation, §2)."""
    if S is None:
        return 0
    return (J * B) // S


def tri_offset(I: int) -> int:
    """Start of row I in the row-major packed lower triangle of an NB x NB block matrix."""
    return I * (I + 1) // 2


def key_rows_of_block(J: int, I: int, perm_g: Optional[np.ndarray], B: int, S: Optional[int],
                      N: int) -> np.ndarray:
    """Physical key positions that block J stands for when read by query block I.

    S2O (§1, "Online Permutation via Index-Driven Loading"): tensors keep their HBM layout and an
    index array says which tokens a tile loads.  Permutation stays inside segments and never
    crosses segment causality (Sparser Block-Sparse Attention via Token Permutation, §2), so a
    block in a segment strictly before I's segment is read through the permutation, and a block
    in I's own segment is read in natural order.
    """
    if perm_g is not None and segment_of_block(J, B, S) < segment_of_block(I, B, S):
        return np.asarray(perm_g[J * B:min((J + 1) * B, N)], dtype=np.int64)
    return block_range(J, B, N)


# ----------------------------------------------------------------------------- stage 1: permutation

def key_importance(q: np.ndarray, k: np.ndarray, block_size: int,
                   scale: Optional[float] = None) -> np.ndarray:
    """Global key-importance vector imp [Hkv][N] from the last block of queries.

    Sparser Block-Sparse Attention via Token Permutation, §3 ("Proxy Scoring"): the importance of
    every key is the mean, over the last block of queries, of the attention probability that key
    receives.  For KV head g the rows are (h, i) with g(h) = g and i in [max(0, N-B), N); each
    row's probabilities are the causal softmax over keys j <= i.
    """
    Hq, N, d = q.shape
    Hkv = k.shape[0]
    G = Hq // Hkv
    c = default_scale(d) if scale is None else scale
    rows = np.arange(max(0, N - block_size), N)
    keys = np.arange(N)
    allowed = keys[None, :] <= rows[:, None]
    imp = np.zeros((Hkv, N))
    for g in range(Hkv):
        acc = np.zeros(N)
        for h in range(g * G, (g + 1) * G):
            s = c * (q[h, rows] @ k[g].T)                      # [rows][N]
            s = np.where(allowed, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            lse = m + np.log(np.exp(s - m).sum(axis=1, keepdims=True))
            acc += np.exp(s - lse).sum(axis=0)                 # masked entries are exp(-inf) = 0
        imp[g] = acc / (G * len(rows))
    return imp


def segment_permutation(imp: np.ndarray, segment_size: int) -> np.ndarray:
    """Per-KV-head index list perm [Hkv][N]: each segment's positions by importance, descending.

    Sparser Block-Sparse Attention via Token Permutation, §2 (segments of S tokens, permutation
    only inside a segment) and §3 ("Sorting": keys of a segment in descending order of global
    importance).  Equal importance keeps the original order (stable).  perm[g, a + r] is the
    position of the r-th most important key of segment [a, a + S).
    """
    Hkv, N = imp.shape
    perm = np.empty((Hkv, N), dtype=np.int64)
    for g in range(Hkv):
        for a in range(0, N, segment_size):
            b = min(a + segment_size, N)
            pos = np.arange(a, b)
            order = np.lexsort((pos, -imp[g, a:b]))            # primary: -imp asc; then pos asc
            perm[g, a:b] = pos[order]
    return perm


# ----------------------------------------------------------------------------- stage 2: block mask

def pool_blocks(x: np.ndarray, block_size: int) -> np.ndarray:
    """Mean of each natural block's rows: [H][N][d] -> [H][NB][d]."""
    H, N, d = x.shape
    NB = num_blocks(N, block_size)
    out = np.empty((H, NB, d))
    for J in range(NB):
        out[:, J] = x[:, J * block_size:min((J + 1) * block_size, N)].mean(axis=1)
    return out


def pool_permuted_blocks(k: np.ndarray, perm: np.ndarray, block_size: int) -> np.ndarray:
    """Mean key of each block of the permuted order: rows perm[g, J*B ...]."""
    Hkv, N, d = k.shape
    NB = num_blocks(N, block_size)
    out = np.empty((Hkv, NB, d))
    for g in range(Hkv):
        for J in range(NB):
            out[g, J] = k[g, perm[g, J * block_size:min((J + 1) * block_size, N)]].mean(axis=0)
    return out


class _PooledLogits:
    """z_IJ = c * Qbar_{h,I} . Kbar_J for J <= I (Sparser Block-Sparse Attention via Token
    Permutation, §4: mean pooling, on the permuted keys for blocks of earlier segments)."""

    def __init__(self, q, k, perm, block_size, segment_size, scale):
        Hq, N, d = q.shape
        self.G = Hq // k.shape[0]
        self.B, self.S = block_size, segment_size
        self.c = default_scale(d) if scale is None else scale
        self.qbar = pool_blocks(q, block_size)
        self.knat = pool_blocks(k, block_size)
        self.kperm = pool_permuted_blocks(k, perm, block_size) if perm is not None else self.knat

    def row(self, h: int, I: int) -> np.ndarray:
        g = h // self.G
        sI = segment_of_block(I, self.B, self.S)
        kbar = np.stack([self.kperm[g, J] if segment_of_block(J, self.B, self.S) < sI else self.knat[g, J]
                         for J in range(I + 1)])
        return self.c * (kbar @ self.qbar[h, I])


def pooled_block_logits(q: np.ndarray, k: np.ndarray, perm: Optional[np.ndarray], block_size: int,
                        segment_size: Optional[int], scale: Optional[float] = None) -> np.ndarray:
    """z of every row, fp64 [Hq][NB(NB+1)/2], row (h, I) at I(I+1)/2: the logits whose softmax is
    block_mask's prob and whose order ranked_blocks follows."""
    Hq, N, _ = q.shape
    NB = num_blocks(N, block_size)
    logits = _PooledLogits(q, k, perm, block_size, segment_size, scale)
    z = np.full((Hq, NB * (NB + 1) // 2), np.nan)
    for h in range(Hq):
        for I in range(NB):
            z[h, tri_offset(I):tri_offset(I) + I + 1] = logits.row(h, I)
    return z


def block_mask(q: np.ndarray, k: np.ndarray, perm: Optional[np.ndarray], block_size: int,
               segment_size: Optional[int], mass_tau: float, force_diag: bool = True,
               force_first: bool = True, scale: Optional[float] = None):
    """Per (query head, query block) list of selected key blocks.

    Sparser Block-Sparse Attention via Token Permutation, §4 ("Block Selection"): block
    importance is estimated by mean pooling, on the permuted keys.  The keep rule is a
    cumulative-mass target: SampleAttention (Technical Deep Dive) controls sparsity by the
    attention mass that must be preserved per query.

    Row (h, I): z_J = c * Qbar_{h,I} . Kbar_J for J <= I, with Kbar_J pooled over the rows block J
    stands for when read by I (``key_rows_of_block``); p = softmax(z); order J by (p desc, J asc);
    keep the shortest prefix whose running sum reaches mass_tau (all J <= I when mass_tau >= 1 or
    when rounding keeps the sum below it); add I (force_diag) and 0 (force_first).

    Returns (count [Hq][NB] int64, idx [Hq][NB(NB+1)/2] int64 ascending per row, -1 padded,
    prob [Hq][NB(NB+1)/2] fp64 = p per row).
    """
    Hq, N, d = q.shape
    B = block_size
    NB = num_blocks(N, B)
    logits = _PooledLogits(q, k, perm, block_size, segment_size, scale)
    ntri = NB * (NB + 1) // 2
    count = np.zeros((Hq, NB), dtype=np.int64)
    idx = np.full((Hq, ntri), -1, dtype=np.int64)
    prob = np.full((Hq, ntri), np.nan)
    for h in range(Hq):
        for I in range(NB):
            z = logits.row(h, I)
            e = np.exp(z - z.max())
            p = e / e.sum()
            order = np.lexsort((np.arange(I + 1), -p))
            kstar = I + 1
            if mass_tau < 1.0:
                hit = np.nonzero(np.cumsum(p[order]) >= mass_tau)[0]
                if hit.size:
                    kstar = int(hit[0]) + 1
            chosen = set(int(J) for J in order[:kstar])
            if force_diag:
                chosen.add(I)
            if force_first:
                chosen.add(0)
            lst = sorted(chosen)
            o = tri_offset(I)
            count[h, I] = len(lst)
            idx[h, o:o + len(lst)] = lst
            prob[h, o:o + I + 1] = p
    return count, idx, prob


def ranked_blocks(q: np.ndarray, k: np.ndarray, perm: Optional[np.ndarray], block_size: int,
                  segment_size: int, scale: Optional[float] = None):
    """Order in which the marginal-gain early stop visits the key blocks of each query block.

    S2O, "Early-Stopping Rule": candidate blocks are processed in descending order of estimated
    importance; "Kernel Implementation": pass 1 computes the dense causal window inside the query's
    own segment, pass 2 walks the historical prefix in the permuted order.  Reading: row (h, I)
    lists every J <= I; first the blocks of I's own segment, ascending (pass 1), then the blocks of
    earlier segments (pass 2) by the pooled block logit z of stage 2 (the estimate of Sparser
    Block-Sparse Attention via Token Permutation, §4; softmax is monotone in z, so this is also the
    order by p), descending, ties by J ascending.

    Returns (count [Hq][NB] = I + 1, idx [Hq][NB(NB+1)/2] int64, n_intra [Hq][NB]).
    """
    Hq, N, d = q.shape
    B, S = block_size, segment_size
    NB = num_blocks(N, B)
    logits = _PooledLogits(q, k, perm, block_size, segment_size, scale)
    count = np.zeros((Hq, NB), dtype=np.int64)
    idx = np.full((Hq, NB * (NB + 1) // 2), -1, dtype=np.int64)
    n_intra = np.zeros((Hq, NB), dtype=np.int64)
    for h in range(Hq):
        for I in range(NB):
            sI = segment_of_block(I, B, S)
            intra = [J for J in range(I + 1) if segment_of_block(J, B, S) == sI]
            hist = [J for J in range(I + 1) if segment_of_block(J, B, S) < sI]
            z = logits.row(h, I)
            hist.sort(key=lambda J: (-z[J], J))
            o = tri_offset(I)
            idx[h, o:o + I + 1] = intra + hist
            count[h, I] = I + 1
            n_intra[h, I] = len(intra)
    return count, idx, n_intra


def _s2o_row_gains(q, k, perm_g, h, g, I, lst, B, S, N, c, rows_of=None, qi=None):
    """For row (h, I) and its list in order: (dl, ell), each [len(lst)][rows of block I], where dl[p]
    is what block lst[p] adds to each query's softmax denominator and ell[p] the denominator over
    lst[0..p].  One reference per query (the max over every listed key) scales both; it cancels in
    the ratio dl / ell.  rows_of(J) gives a list entry's key positions (default: key_rows_of_block
    through perm_g); qi: the query positions of the row (default: natural block I)."""
    if qi is None:
        qi = block_range(I, B, N)
    if rows_of is None:
        rows_of = lambda J: key_rows_of_block(J, I, perm_g, B, S, N)  # noqa: E731
    blk = []
    for J in lst:
        kj = rows_of(J)
        st = c * (q[h, qi] @ k[g, kj].T)
        blk.append(np.where(kj[None, :] <= qi[:, None], st, -np.inf))
    ref = np.max(np.concatenate(blk, axis=1), axis=1)
    dl = np.stack([np.exp(st - ref[:, None]).sum(axis=1) for st in blk])
    return dl, np.cumsum(dl, axis=0)


def s2o_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, perm: Optional[np.ndarray],
                  count: np.ndarray, idx: np.ndarray, block_size: int, segment_size: int,
                  gain_tau: float, scale: Optional[float] = None,
                  rows: Optional[Iterable[Tuple[int, int]]] = None):
    """Attention with the marginal-gain early stop over a ranked block list.

    S2O, "Early-Stopping Rule": the attention mass each processed block adds (delta l) is tracked,
    and once it falls below a threshold relative to the accumulated score the rest of the list is
    skipped.  Reading: row (h, I) takes the list in order; the blocks of I's own segment are always
    processed; after each earlier-segment block b, with l_i the softmax denominator of query i over
    every key processed so far (b included) and dl_i the part b contributed, the row stops when
    dl_i < gain_tau * l_i for every query i of the block; b itself stays processed.  The output is
    exact softmax attention over the processed blocks (block_sparse_attention on that set).

    Returns (out [Hq][N][d], lse [Hq][N], processed {(h, I): [J in processing order]}).
    """
    Hq, N, d = q.shape
    G = Hq // k.shape[0]
    B, S = block_size, segment_size
    NB = num_blocks(N, B)
    c = default_scale(d) if scale is None else scale
    todo = [(h, I) for h in range(Hq) for I in range(NB)] if rows is None else list(rows)
    processed: Dict[Tuple[int, int], List[int]] = {}
    for h, I in todo:
        g = h // G
        o = tri_offset(I)
        lst = [int(J) for J in idx[h, o:o + int(count[h, I])]]
        sI = segment_of_block(I, B, S)
        dl, ell = _s2o_row_gains(q, k, None if perm is None else perm[g], h, g, I, lst, B, S, N, c)
        done: List[int] = []
        for p, J in enumerate(lst):
            done.append(J)
            if segment_of_block(J, B, S) < sI and np.all(dl[p] < gain_tau * ell[p]):
                break
        processed[(h, I)] = done
    kc, ki = _lists_to_mask(processed, Hq, NB)
    rows_done = list(processed.keys())
    out, lse, _, _ = block_sparse_attention(q, k, v, perm, kc, ki, B, S, scale=scale, rows=rows_done)
    return out, lse, processed


def s2o_gain_ratios(q: np.ndarray, k: np.ndarray, perm: Optional[np.ndarray], count: np.ndarray,
                    idx: np.ndarray, block_size: int, segment_size: int, scale: Optional[float] = None,
                    rows: Optional[Iterable[Tuple[int, int]]] = None) -> Dict[Tuple[int, int], np.ndarray]:
    """The statistic the marginal-gain stop compares with its threshold, at every list position.

    For row (h, I), position p of the list (the whole list, no stop applied): max over the queries
    i of block I of dl_i / l_i as defined in s2o_attention; NaN at positions of I's own segment,
    where the rule does not apply.  s2o_attention stops at the first position whose value is below
    gain_tau (up to the rounding of the division), so the value at the stop position is how close
    that decision was.
    """
    Hq, N, d = q.shape
    G = Hq // k.shape[0]
    B, S = block_size, segment_size
    NB = num_blocks(N, B)
    c = default_scale(d) if scale is None else scale
    todo = [(h, I) for h in range(Hq) for I in range(NB)] if rows is None else list(rows)
    out: Dict[Tuple[int, int], np.ndarray] = {}
    for h, I in todo:
        g = h // G
        o = tri_offset(I)
        lst = [int(J) for J in idx[h, o:o + int(count[h, I])]]
        sI = segment_of_block(I, B, S)
        dl, ell = _s2o_row_gains(q, k, None if perm is None else perm[g], h, g, I, lst, B, S, N, c)
        r = (dl / ell).max(axis=1)
        r[[segment_of_block(J, B, S) >= sI for J in lst]] = np.nan
        out[(h, I)] = r
    return out


# ----------------------------------------------------------------------------- SampleAttention estimator

def trunk_rows(n: int, n_trunks: int, rows_per_trunk: int) -> np.ndarray:
    """Query positions sampled by SampleAttention's trunk sampling (Technical Deep Dive, Stage 1:
    queries are sampled from chunks spread over the whole sequence, not from one place).

    Reading: the sequence is cut into n_trunks chunks of C = ceil(n / n_trunks) positions and the
    last rows_per_trunk positions of every chunk are sampled (the rows of a chunk that see its whole
    causal prefix).  Every chunk must hold at least rows_per_trunk positions."""
    C = -(-n // n_trunks)
    rows = []
    for t in range(n_trunks):
        end = min((t + 1) * C, n)
        if end - rows_per_trunk < t * C:
            raise ValueError("a trunk holds fewer positions than rows_per_trunk")
        rows.extend(range(end - rows_per_trunk, end))
    return np.asarray(rows, dtype=np.int64)


def sampled_masses(q: np.ndarray, k: np.ndarray, n_trunks: int, rows_per_trunk: int,
                   scale: Optional[float] = None):
    """(col [Hq][N], slash [Hq][N]) from the exact causal softmax rows of the sampled queries.

    SampleAttention, Technical Deep Dive: stage 1 estimates the attention scores from the sampled
    rows; stage 2 looks for key columns and slashes (diagonals) that hold the attention mass.
    col[h][j] is the mean over the sampled rows i of head h of p_ij; slash[h][delta] the mean of
    p_{i, i-delta} (zero where delta > i).  Each sums to 1 over its index."""
    Hq, N, d = q.shape
    G = Hq // k.shape[0]
    c = default_scale(d) if scale is None else scale
    rows = trunk_rows(N, n_trunks, rows_per_trunk)
    R = len(rows)
    col = np.zeros((Hq, N))
    slash = np.zeros((Hq, N))
    j = np.arange(N)
    for h in range(Hq):
        s = c * (q[h, rows] @ k[h // G].T)
        s = np.where(j[None, :] <= rows[:, None], s, -np.inf)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        col[h] = p.sum(axis=0) / R
        for r, i in enumerate(rows):
            slash[h, :i + 1] += p[r, i::-1]            # delta = i - j for j = i, i-1, ..., 0
        slash[h] /= R
    return col, slash


def mass_cut(m: np.ndarray, tau: float) -> np.ndarray:
    """Shortest prefix of the order (m descending, index ascending) whose running sum reaches tau,
    as a boolean mask; every index when tau >= 1 or the sum stays below tau (the mass rule of
    block_mask, applied to key columns or diagonals)."""
    n = len(m)
    if tau >= 1.0:
        return np.ones(n, dtype=bool)
    order = np.lexsort((np.arange(n), -m))
    hit = np.nonzero(np.cumsum(m[order]) >= tau)[0]
    keep = np.zeros(n, dtype=bool)
    keep[order[:int(hit[0]) + 1] if hit.size else order] = True
    return keep


def sample_attention_mask(q: np.ndarray, k: np.ndarray, block_size: int, cia_tau: float, n_trunks: int,
                          rows_per_trunk: int, force_diag: bool = True, force_first: bool = False,
                          scale: Optional[float] = None):
    """Block mask of SampleAttention's two stages (Technical Deep Dive).

    Stage 1: sampled_masses.  Stage 2, decoupled filtering: the key columns and the slashes are
    filtered separately, each family keeping the shortest set of its heaviest members whose mass
    reaches the CIA target cia_tau (the mass every query should keep).  The block-level mask keeps
    tile (I, J), J <= I, when it holds a kept column, when a kept slash crosses it (some i in I,
    j in J, j <= i with i - j = delta), or when forced (J = I with force_diag, J = 0 with
    force_first).

    Returns (count [Hq][NB], idx [Hq][NB(NB+1)/2] ascending per row, col_keep [Hq][N],
    slash_keep [Hq][N], col, slash)."""
    Hq, N, d = q.shape
    B = block_size
    NB = num_blocks(N, B)
    col, slash = sampled_masses(q, k, n_trunks, rows_per_trunk, scale)
    col_keep = np.stack([mass_cut(col[h], cia_tau) for h in range(Hq)])
    slash_keep = np.stack([mass_cut(slash[h], cia_tau) for h in range(Hq)])
    count, idx = mask_from_patterns(col_keep, slash_keep, B, force_diag, force_first)
    return count, idx, col_keep, slash_keep, col, slash


def mask_from_patterns(col_keep: np.ndarray, slash_keep: np.ndarray, block_size: int, force_diag: bool = True,
                       force_first: bool = False):
    """Block mask of kept key columns and slashes ([Hq][N] booleans): tile (I, J), J <= I, kept when
    block J holds a kept column, when a kept offset lies in the tile's range of i - j, or when
    forced.  Returns (count, idx) as block_mask does."""
    Hq, N = col_keep.shape
    B = block_size
    NB = num_blocks(N, B)
    count = np.zeros((Hq, NB), dtype=np.int64)
    idx = np.full((Hq, NB * (NB + 1) // 2), -1, dtype=np.int64)
    for h in range(Hq):
        for I in range(NB):
            qi = block_range(I, B, N)
            lst = []
            for J in range(I + 1):
                kj = block_range(J, B, N)
                keep = (force_diag and J == I) or (force_first and J == 0) or bool(col_keep[h, kj].any())
                if not keep:
                    lo = max(0, int(qi[0]) - int(kj[-1]))
                    hi = int(qi[-1]) - int(kj[0])
                    keep = bool(slash_keep[h, lo:hi + 1].any())
                if keep:
                    lst.append(J)
            o = tri_offset(I)
            count[h, I] = len(lst)
            idx[h, o:o + len(lst)] = lst
    return count, idx


# ----------------------------------------------------------------------------- S2O prefix ranking

def num_segments(n: int, segment_size: int) -> int:
    return -(-n // segment_size)


def prefix_offset(sigma: int, segment_size: int) -> int:
    """Start of segment sigma's prefix order in a [Hkv][...] prefix ranking: the orders of segments
    1 .. sigma-1 come first, of lengths S, 2S, ..."""
    return segment_size * sigma * (sigma - 1) // 2


def prefix_ranking_length(n: int, segment_size: int) -> int:
    nseg = num_segments(n, segment_size)
    return prefix_offset(nseg, segment_size)


def segment_representatives(q: np.ndarray, num_kv_heads: int, segment_size: int) -> np.ndarray:
    """r[g][sigma] = mean of the query rows of segment sigma over the G query heads of KV head g.

    S2O, Methodology §1, Historical KV Permutation: the keys before a segment are scored against a
    representative query of the segment.  Reading: that query is the mean of the segment's query
    rows, taken over every query head that shares the KV head (one order per KV head, as K and V
    are stored per KV head)."""
    Hq, N, d = q.shape
    G = Hq // num_kv_heads
    S = segment_size
    nseg = num_segments(N, S)
    r = np.empty((num_kv_heads, nseg, d))
    for g in range(num_kv_heads):
        for sigma in range(nseg):
            rows = q[g * G:(g + 1) * G, sigma * S:min((sigma + 1) * S, N)].reshape(-1, d)
            r[g, sigma] = rows.mean(axis=0)
    return r


def prefix_kv_ranking(q: np.ndarray, k: np.ndarray, segment_size: int):
    """Per KV head g and segment sigma >= 1: every key j < sigma*S (the causal prefix of the
    segment) ordered by the score r_{g,sigma} . k_j, descending, ties by j ascending.

    S2O, Methodology §1, Historical KV Permutation (scores against a representative query, only
    prefix tokens, one global order over the prefix).  Returns (pi, score), both [Hkv][L] with
    L = prefix_ranking_length(N, S): segment sigma's order at prefix_offset(sigma, S), int64 key
    positions and their fp64 scores."""
    Hkv, N, d = k.shape
    S = segment_size
    nseg = num_segments(N, S)
    L = prefix_ranking_length(N, S)
    r = segment_representatives(q, Hkv, S)
    pi = np.zeros((Hkv, L), dtype=np.int64)
    score = np.zeros((Hkv, L))
    for g in range(Hkv):
        for sigma in range(1, nseg):
            n = sigma * S
            z = k[g, :n] @ r[g, sigma]
            order = np.lexsort((np.arange(n), -z))
            o = prefix_offset(sigma, S)
            pi[g, o:o + n] = order
            score[g, o:o + n] = z[order]
    return pi, score


def query_guide_scores(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """score[g][i] = (1/G) * sum over the G query heads of g of q_{h,i} . u_g, with the guide vector
    u_g the mean key of KV head g over the sequence.

    S2O, Methodology §1, Query Permutation: queries are reordered inside a segment by a coarse
    importance score against one shared guide vector.  Reading: the guide is the mean key, so the
    score is a query's mean logit over the keys (up to the scale), large for the queries that form
    bright horizontal stripes."""
    Hq, N, d = q.shape
    Hkv = k.shape[0]
    G = Hq // Hkv
    score = np.zeros((Hkv, N))
    for g in range(Hkv):
        u = k[g].mean(axis=0)
        score[g] = np.mean([q[h] @ u for h in range(g * G, (g + 1) * G)], axis=0)
    return score


def query_permutation(q: np.ndarray, k: np.ndarray, segment_size: int) -> np.ndarray:
    """qperm[g][N]: inside each segment, the query positions by guide score descending, ties by
    position (one order per KV head, shared by its G query heads).  Query block I of the permuted
    order holds positions qperm[g][I*B ...]; segments keep their place (PBS-Attn §2: permutations
    stay inside segments)."""
    Hkv = k.shape[0]
    N = q.shape[1]
    S = segment_size
    score = query_guide_scores(q, k)
    qperm = np.zeros((Hkv, N), dtype=np.int64)
    for g in range(Hkv):
        for a in range(0, N, S):
            b = min(a + S, N)
            pos = np.arange(a, b)
            qperm[g, a:b] = pos[np.lexsort((pos, -score[g, a:b]))]
    return qperm


def _prefix_rows_of(pi, g, I, B, S, N):
    """Key positions of list entry J for query block I: natural block J in I's own segment
    (J >= J0, the first block of the segment), else block J of the segment's prefix order."""
    sigma = segment_of_block(I, B, S)
    J0 = sigma * S // B
    o = prefix_offset(sigma, S)

    def rows_of(J):
        if J >= J0:
            return block_range(J, B, N)
        return np.asarray(pi[g, o + J * B:o + (J + 1) * B], dtype=np.int64)
    return rows_of, J0


def _two_pass_row(qperm, g, I, B, S, N):
    """(query positions, list) of row I: natural block I and own blocks J0 .. I without a query
    permutation; with one, the positions qperm[g][I*B ...] and every block of the own segment (a
    permuted block may hold any of the segment's positions; the causal mask is per token).  The
    history blocks 0 .. J0-1 follow in both cases."""
    sigma = segment_of_block(I, B, S)
    J0 = sigma * S // B
    if qperm is None:
        return block_range(I, B, N), list(range(J0, I + 1)) + list(range(J0))
    Jend = min(-(-min((sigma + 1) * S, N) // B), num_blocks(N, B)) - 1
    qi = np.asarray(qperm[g, I * B:min((I + 1) * B, N)], dtype=np.int64)
    return qi, list(range(J0, Jend + 1)) + list(range(J0))


def s2o_prefix_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, pi: np.ndarray, block_size: int,
                         segment_size: int, gain_tau: float, scale: Optional[float] = None,
                         rows: Optional[Iterable[Tuple[int, int]]] = None, qperm: Optional[np.ndarray] = None):
    """S2O's two passes with the marginal-gain stop, history read through the prefix ranking.

    S2O, Kernel Implementation: pass 1 runs the dense causal window of the query block's own
    segment; pass 2 continues over the historical prefix in the permuted order of
    prefix_kv_ranking, cut into blocks of B keys (block J = entries J*B .. J*B+B-1 of the
    segment's order, so J = 0 holds the highest-scoring keys); S2O, Early-Stopping Rule: after
    each history block, the row stops as in s2o_attention (every query's share of that block in
    its denominator below gain_tau; that block stays processed).  The output is exact softmax
    attention over the processed keys.

    qperm (query_permutation): query block I holds positions qperm[g][I*B ...]; pass 1 then spans
    the whole own segment under the per-token causal mask, and every output row lands at its
    natural position (PBS-Attn §1: permuting queries permutes the output; the inverse permutation
    restores it).

    Returns (out [Hq][N][d], lse [Hq][N], processed {(h, I): [J in processing order]}), where
    J >= J0 names a natural block of the own segment and J < J0 a prefix-order block.
    """
    Hq, N, d = q.shape
    G = Hq // k.shape[0]
    B, S = block_size, segment_size
    NB = num_blocks(N, B)
    c = default_scale(d) if scale is None else scale
    todo = [(h, I) for h in range(Hq) for I in range(NB)] if rows is None else list(rows)
    out = np.full((Hq, N, d), np.nan)
    lse = np.full((Hq, N), np.nan)
    processed: Dict[Tuple[int, int], List[int]] = {}
    for h, I in todo:
        g = h // G
        rows_of, J0 = _prefix_rows_of(pi, g, I, B, S, N)
        qi, lst = _two_pass_row(qperm, g, I, B, S, N)
        dl, ell = _s2o_row_gains(q, k, None, h, g, I, lst, B, S, N, c, rows_of=rows_of, qi=qi)
        done: List[int] = []
        for p, J in enumerate(lst):
            done.append(J)
            if J < J0 and np.all(dl[p] < gain_tau * ell[p]):
                break
        processed[(h, I)] = done
        keys = np.concatenate([rows_of(J) for J in done])
        _attend(q, k, v, h, g, qi, keys, c, out, lse)
    return out, lse, processed


def two_pass_attention_on(q: np.ndarray, k: np.ndarray, v: np.ndarray, pi: np.ndarray,
                          entries: Dict[Tuple[int, int], Sequence[int]], block_size: int, segment_size: int,
                          scale: Optional[float] = None, qperm: Optional[np.ndarray] = None):
    """Softmax attention of each listed row (h, I) over the keys of the given two-pass entries
    (J >= J0: natural block J; J < J0: block J of the segment's prefix order), causal per query;
    the output of s2o_prefix_attention for a given processed set.  Returns (out, lse), NaN on rows
    not listed."""
    Hq, N, d = q.shape
    G = Hq // k.shape[0]
    B, S = block_size, segment_size
    c = default_scale(d) if scale is None else scale
    out = np.full((Hq, N, d), np.nan)
    lse = np.full((Hq, N), np.nan)
    for (h, I), lst in entries.items():
        rows_of, _ = _prefix_rows_of(pi, h // G, I, B, S, N)
        qi, _ = _two_pass_row(qperm, h // G, I, B, S, N)
        keys = np.concatenate([rows_of(J) for J in lst]) if len(lst) else np.zeros(0, dtype=np.int64)
        _attend(q, k, v, h, h // G, qi, keys, c, out, lse)
    return out, lse


def s2o_prefix_gain_ratios(q: np.ndarray, k: np.ndarray, pi: np.ndarray, block_size: int, segment_size: int,
                           scale: Optional[float] = None, rows: Optional[Iterable[Tuple[int, int]]] = None,
                           qperm: Optional[np.ndarray] = None) -> Dict[Tuple[int, int], np.ndarray]:
    """s2o_gain_ratios for the lists of s2o_prefix_attention: max_i dl_i / l_i at every position of
    the whole list (pass 1, then prefix blocks 0 .. J0-1), NaN on the own segment."""
    Hq, N, d = q.shape
    G = Hq // k.shape[0]
    B, S = block_size, segment_size
    NB = num_blocks(N, B)
    c = default_scale(d) if scale is None else scale
    todo = [(h, I) for h in range(Hq) for I in range(NB)] if rows is None else list(rows)
    res: Dict[Tuple[int, int], np.ndarray] = {}
    for h, I in todo:
        g = h // G
        rows_of, J0 = _prefix_rows_of(pi, g, I, B, S, N)
        qi, lst = _two_pass_row(qperm, g, I, B, S, N)
        dl, ell = _s2o_row_gains(q, k, None, h, g, I, lst, B, S, N, c, rows_of=rows_of, qi=qi)
        r = (dl / ell).max(axis=1)
        r[[J >= J0 for J in lst]] = np.nan
        res[(h, I)] = r
    return res


def _lists_to_mask(lists: Dict[Tuple[int, int], Sequence[int]], Hq: int, NB: int):
    count = np.zeros((Hq, NB), dtype=np.int64)
    idx = np.full((Hq, NB * (NB + 1) // 2), -1, dtype=np.int64)
    for (h, I), lst in lists.items():
        srt = sorted(lst)
        o = tri_offset(I)
        count[h, I] = len(srt)
        idx[h, o:o + len(srt)] = srt
    return count, idx


# ----------------------------------------------------------------------------- stage 3: attention

def block_sparse_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, perm: Optional[np.ndarray],
                           count: Optional[np.ndarray], idx: Optional[np.ndarray], block_size: int,
                           segment_size: Optional[int], scale: Optional[float] = None,
                           theta: Optional[np.ndarray] = None,
                           rows: Optional[Iterable[Tuple[int, int]]] = None,
                           return_weights: bool = False):
    """Causal block-sparse attention over the selected (permuted) key blocks.

    Sparser Block-Sparse Attention via Token Permutation, Problem Statement: blocks outside the
    mask are skipped; S2O §1: selected tiles are gathered by index; S2O §3: the result is the
    online-softmax state (m, l, acc) over the visited blocks, i.e. exact softmax attention over
    their union.  For query i of block I of head h the keys are
        K_hi = { j in key_rows_of_block(J, I) : J in sel(h, I), j <= i }.
    count/idx None means every J <= I.

    Early stop (Block Sparse Flash Attention, Approach): with theta [Hq][NB], a selected J != I
    whose exact tile max  max_{i in I, j in rows(J), j <= i} c q_i.k_j  is below theta[h, I] is
    dropped before the softmax (no V load, no PV, no change to m or l).

    rows: optional iterable of (h, I) to evaluate (others stay NaN).
    A query left with no key (possible only when the diagonal block is not selected and the gate
    drops every other tile) gets out = 0 and lse = -inf.
    Returns (out [Hq][N][d], lse [Hq][N], kept {(h, I): [J ...]}, weights or None).
    weights (only with return_weights) maps (h, i) -> (key positions, probabilities).
    """
    Hq, N, d = q.shape
    Hkv = k.shape[0]
    G = Hq // Hkv
    B, S = block_size, segment_size
    NB = num_blocks(N, B)
    c = default_scale(d) if scale is None else scale
    out = np.full((Hq, N, d), np.nan)
    lse = np.full((Hq, N), np.nan)
    kept: Dict[Tuple[int, int], List[int]] = {}
    weights = {} if return_weights else None
    todo = [(h, I) for h in range(Hq) for I in range(NB)] if rows is None else list(rows)
    for h, I in todo:
        g = h // G
        perm_g = None if perm is None else perm[g]
        qi = block_range(I, B, N)
        if count is None:
            sel = list(range(I + 1))
        else:
            o = tri_offset(I)
            sel = [int(J) for J in idx[h, o:o + int(count[h, I])]]
        keep_lists = []
        kept_J = []
        for J in sel:
            kj = key_rows_of_block(J, I, perm_g, B, S, N)
            if theta is not None and J != I:
                st = c * (q[h, qi] @ k[g, kj].T)
                st = np.where(kj[None, :] <= qi[:, None], st, -np.inf)
                if st.max() < theta[h, I]:
                    continue
            keep_lists.append(kj)
            kept_J.append(J)
        kept[(h, I)] = kept_J
        keys = np.concatenate(keep_lists) if keep_lists else np.zeros(0, dtype=np.int64)
        _attend(q, k, v, h, g, qi, keys, c, out, lse, weights)
    return out, lse, kept, weights


def _attend(q, k, v, h, g, qi, keys, c, out, lse, weights=None):
    """Softmax attention of the queries qi of head h over the key positions `keys`, each query
    seeing only keys j <= i; writes out[h, qi] and lse[h, qi].  A query with no key gets out = 0
    and lse = -inf."""
    s = c * (q[h, qi] @ k[g, keys].T)                          # [rows of I][keys]
    s = np.where(keys[None, :] <= qi[:, None], s, -np.inf)
    for r, i in enumerate(qi):
        ok = keys <= i
        if not ok.any():
            out[h, i] = 0.0
            lse[h, i] = -np.inf
            if weights is not None:
                weights[(h, int(i))] = (keys[:0], np.zeros(0))
            continue
        m = s[r].max()
        e = np.exp(s[r] - m)
        l = e.sum()
        out[h, i] = (e @ v[g, keys]) / l
        lse[h, i] = m + np.log(l)
        if weights is not None:
            weights[(h, int(i))] = (keys, e / l)


def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: Optional[float] = None,
                    causal: bool = True, allowed: Optional[np.ndarray] = None):
    """Direct softmax(c Q K^T + mask) V per head (GQA: query head h reads KV head h // G).

    allowed: optional [N][N] boolean matrix of (i, j) pairs that may attend (combined with the
    causal rule when causal is True).  Returns (out [Hq][N][d], lse [Hq][N]).
    """
    Hq, N, d = q.shape
    Hkv = k.shape[0]
    G = Hq // Hkv
    c = default_scale(d) if scale is None else scale
    ok = np.ones((N, N), dtype=bool)
    if causal:
        ok &= np.tri(N, dtype=bool)
    if allowed is not None:
        ok &= allowed
    out = np.empty((Hq, N, d))
    lse = np.empty((Hq, N))
    for h in range(Hq):
        g = h // G
        s = np.where(ok, c * (q[h] @ k[g].T), -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        l = e.sum(axis=1, keepdims=True)
        out[h] = (e / l) @ v[g]
        lse[h] = (m + np.log(l))[:, 0]
    return out, lse


# ----------------------------------------------------------------------------- early-stop support

def tile_max(q: np.ndarray, k: np.ndarray, block_size: int, scale: Optional[float] = None,
             rows: Optional[Iterable[Tuple[int, int]]] = None) -> np.ndarray:
    """Exact per-tile max of the scaled causal logits, natural order, packed lower triangle.

    Block Sparse Flash Attention, Approach: the gate looks at the exact QK^T scores of a tile.
    Entry (h, I, J), J <= I, is max over i in block I, j in block J, j <= i of c q_i.k_j.
    Returns [Hq][NB(NB+1)/2] (rows not requested stay NaN).
    """
    Hq, N, d = q.shape
    Hkv = k.shape[0]
    G = Hq // Hkv
    B = block_size
    NB = num_blocks(N, B)
    c = default_scale(d) if scale is None else scale
    out = np.full((Hq, NB * (NB + 1) // 2), np.nan)
    todo = [(h, I) for h in range(Hq) for I in range(NB)] if rows is None else list(rows)
    for h, I in todo:
        g = h // G
        qi = block_range(I, B, N)
        for J in range(I + 1):
            kj = block_range(J, B, N)
            st = c * (q[h, qi] @ k[g, kj].T)
            st = np.where(kj[None, :] <= qi[:, None], st, -np.inf)
            out[h, tri_offset(I) + J] = st.max()
    return out


def calibrate_thresholds(tmax: np.ndarray, num_blocks_: int, keep: int) -> np.ndarray:
    """Per (head, query block) threshold that keeps the `keep` largest tile maxima of the row.

    Block Sparse Flash Attention, Approach: thresholds are calibrated offline so that roughly the
    top-k blocks per query survive.  theta[h, I] is the keep-th largest tile max over J <= I, and
    -inf when the row has no more than `keep` tiles.
    """
    Hq = tmax.shape[0]
    theta = np.full((Hq, num_blocks_), -np.inf)
    for h in range(Hq):
        for I in range(num_blocks_):
            if I + 1 > keep:
                row = tmax[h, tri_offset(I):tri_offset(I) + I + 1]
                theta[h, I] = np.sort(row)[::-1][keep - 1]
    return theta


def kept_bitmap(kept: Dict[Tuple[int, int], Sequence[int]], num_q_heads: int, nb: int) -> np.ndarray:
    """Bitmap [Hq][ceil(NB(NB+1)/2 / 32)] uint32 with bit (tri_offset(I) + J) set for each kept tile."""
    ntri = nb * (nb + 1) // 2
    words = -(-ntri // 32)
    bm = np.zeros((num_q_heads, words), dtype=np.uint32)
    for (h, I), lst in kept.items():
        for J in lst:
            t = tri_offset(I) + J
            bm[h, t // 32] |= np.uint32(1) << np.uint32(t % 32)
    return bm
