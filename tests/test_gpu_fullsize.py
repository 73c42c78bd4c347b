"""GPU parity at the benchmarked sizes, on outputs the oracle can compute row by row.

The GPU path runs exactly as bench.py launches it (same workloads, same calls); the oracle then
checks the whole permutation, every (32K) or sampled (128K) mask row, and a seeded sample of
attention rows (query head, query block), including the last and first blocks.
"""
import sys

import numpy as np
import pytest

import oracle
from parity import (F32_U, bitmap_to_kept, bitmap_to_kept_square, compare_gate, compare_importance, compare_lse,
                    compare_mask, compare_out,
                    compare_perm, compare_prefix_rank, compare_ranked, compare_s2o_stops, compare_sample_mask,
                    gate_error_bound, imp_rtol, kept_to_mask, two_pass_lists)
from workloads import WORKLOADS, bf16_bits_to_f32, generate_for

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_blocks_amd as pbsa
    return pbsa


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _load(w, seed=None):
    x = generate_for(w, seed=seed)
    dev = {n: torch.from_numpy(x[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("q", "k", "v")}
    host = {n: bf16_bits_to_f32(x[n]).astype(np.float64) for n in ("q", "k", "v")}
    return dev, host


def _sample_rows(Hq, NB, n, seed):
    rng = np.random.default_rng(seed)
    rows = {(0, NB - 1), (Hq - 1, NB - 1), (Hq // 2, 0), (1, NB // 2)}
    while len(rows) < n:
        rows.add((int(rng.integers(Hq)), int(rng.integers(NB))))
    return sorted(rows)


def _rows_slice(out, rows, B, N):
    """Copy of `out` restricted to the sampled rows (others NaN) for compare_out."""
    sel = np.full(out.shape, np.nan)
    for h, I in rows:
        a, b = I * B, min((I + 1) * B, N)
        sel[h, a:b] = out[h, a:b]
    return sel


def test_fullsize_32k_pipeline():
    pbsa = _need_gpu()
    w = WORKLOADS["llama8b_32k"]
    _log(f"[fullsize] {w.name}")
    dev, host = _load(w)
    q, k, v = host["q"], host["k"], host["v"]
    B, S, NB, Hq, N = w.block_size, w.segment_size, w.num_blocks, w.num_q_heads, w.seq_len
    perm_t, imp_t = pbsa.build_segment_permutation(dev["q"], dev["k"], B, S, return_importance=True)
    count_t, idx_t, prob_t = pbsa.estimate_block_mask(dev["q"], dev["k"], perm_t, B, S, w.mass_tau, w.force_diag,
                                                      w.force_first, return_prob=True)
    out_t, lse_t = pbsa.block_sparse_attn_prefill(dev["q"], dev["k"], dev["v"], perm_t, count_t, idx_t, B, S)
    torch.cuda.synchronize()
    imp_o = oracle.key_importance(q, k, B)
    compare_importance(imp_t.cpu().numpy(), imp_o, imp_rtol(q, k))
    perm_g = perm_t.cpu().numpy()
    ties = compare_perm(perm_g, oracle.segment_permutation(imp_o, S), imp_o, S)
    _log(f"[fullsize] permutation ok ({ties} recorded ties)")
    count_o, idx_o, prob_o = oracle.block_mask(q, k, perm_g, B, S, w.mass_tau, w.force_diag, w.force_first)
    cg, ig = count_t.cpu().numpy(), idx_t.cpu().numpy()
    ties = compare_mask(cg, ig, count_o, idx_o, prob_o, w.mass_tau)
    _log(f"[fullsize] mask ok ({ties} tie rows), density {cg.sum() / (Hq * NB * (NB + 1) / 2):.3f}")
    rows = _sample_rows(Hq, NB, 12, 7)
    out_o, lse_o, _, _ = oracle.block_sparse_attention(q, k, v, perm_g, cg, ig, B, S, rows=rows)
    mx, mean = compare_out(_rows_slice(out_t.cpu().numpy(), rows, B, N), out_o)
    compare_lse(lse_t.cpu().numpy(), lse_o)
    _log(f"[fullsize] attention rows {rows}: max abs {mx:.2e} mean abs {mean:.2e}")
    # dense causal mode on sampled rows
    out_d = pbsa.block_sparse_attn_prefill(dev["q"], dev["k"], dev["v"], block_size=B, return_lse=False)
    torch.cuda.synchronize()
    drows = _sample_rows(Hq, NB, 6, 8)
    ref, _, _, _ = oracle.block_sparse_attention(q, k, v, None, None, None, B, S, rows=drows)
    compare_out(_rows_slice(out_d.cpu().numpy(), drows, B, N), ref, "dense 32K")


def test_fullsize_128k_sampled():
    pbsa = _need_gpu()
    w = WORKLOADS["llama8b_128k"]
    _log(f"[fullsize] {w.name}")
    dev, host = _load(w)
    q, k, v = host["q"], host["k"], host["v"]
    B, S, NB, Hq, N = w.block_size, w.segment_size, w.num_blocks, w.num_q_heads, w.seq_len
    perm_t, imp_t = pbsa.build_segment_permutation(dev["q"], dev["k"], B, S, return_importance=True)
    count_t, idx_t, prob_t = pbsa.estimate_block_mask(dev["q"], dev["k"], perm_t, B, S, w.mass_tau, return_prob=True)
    out_t, lse_t = pbsa.block_sparse_attn_prefill(dev["q"], dev["k"], dev["v"], perm_t, count_t, idx_t, B, S)
    torch.cuda.synchronize()
    imp_o = oracle.key_importance(q, k, B)
    compare_importance(imp_t.cpu().numpy(), imp_o, imp_rtol(q, k))
    perm_g = perm_t.cpu().numpy()
    compare_perm(perm_g, oracle.segment_permutation(imp_o, S), imp_o, S)
    _log("[fullsize] 128K permutation ok")
    # mask rows of two query heads, in full
    cg, ig, pg = count_t.cpu().numpy(), idx_t.cpu().numpy(), prob_t.cpu().numpy()
    for h in (0, Hq - 1):
        sub = slice(h, h + 1)
        g = h // (Hq // w.num_kv_heads)
        co, io, po = oracle.block_mask(q[sub], k[g:g + 1], perm_g[g:g + 1], B, S, w.mass_tau)
        compare_mask(cg[sub], ig[sub], co, io, po, w.mass_tau)
    _log("[fullsize] 128K mask rows of heads 0 and last ok")
    rows = _sample_rows(Hq, NB, 8, 9)
    out_o, lse_o, _, _ = oracle.block_sparse_attention(q, k, v, perm_g, cg, ig, B, S, rows=rows)
    mx, mean = compare_out(_rows_slice(out_t.cpu().numpy(), rows, B, N), out_o)
    compare_lse(lse_t.cpu().numpy(), lse_o)
    _log(f"[fullsize] 128K attention rows {rows}: max abs {mx:.2e} mean abs {mean:.2e}")


def test_fullsize_64k_sweep_sampled():
    """The 64K density-sweep workload (S = 4096) at both ends of its mass targets, permutation on and
    off, launched as the sweep launches it: the whole permutation, the mask rows of two heads in
    full, and sampled attention rows."""
    pbsa = _need_gpu()
    w = WORKLOADS["llama8b_64k_sweep"]
    _log(f"[fullsize] {w.name}")
    dev, host = _load(w)
    q, k, v = host["q"], host["k"], host["v"]
    B, S, NB, Hq, N = w.block_size, w.segment_size, w.num_blocks, w.num_q_heads, w.seq_len
    G = Hq // w.num_kv_heads
    perm_t, imp_t = pbsa.build_segment_permutation(dev["q"], dev["k"], B, S, return_importance=True)
    torch.cuda.synchronize()
    imp_o = oracle.key_importance(q, k, B)
    compare_importance(imp_t.cpu().numpy(), imp_o, imp_rtol(q, k))
    perm_g = perm_t.cpu().numpy()
    compare_perm(perm_g, oracle.segment_permutation(imp_o, S), imp_o, S)
    _log("[fullsize] 64K permutation ok")
    for tau in (w.taus[0], w.taus[-1]):
        for use_perm in (True, False):
            pp_t, pp_g = (perm_t, perm_g) if use_perm else (None, None)
            count_t, idx_t, prob_t = pbsa.estimate_block_mask(dev["q"], dev["k"], pp_t, B, S, tau, return_prob=True)
            out_t, lse_t = pbsa.block_sparse_attn_prefill(dev["q"], dev["k"], dev["v"], pp_t, count_t, idx_t, B, S)
            torch.cuda.synchronize()
            cg, ig = count_t.cpu().numpy(), idx_t.cpu().numpy()
            for h in (0, Hq - 1):
                g = h // G
                co, io, po = oracle.block_mask(q[h:h + 1], k[g:g + 1], None if pp_g is None else pp_g[g:g + 1], B, S,
                                               tau)
                compare_mask(cg[h:h + 1], ig[h:h + 1], co, io, po, tau)
            rows = _sample_rows(Hq, NB, 5, 17 + int(use_perm))
            out_o, lse_o, _, _ = oracle.block_sparse_attention(q, k, v, pp_g, cg, ig, B, S, rows=rows)
            mx, mean = compare_out(_rows_slice(out_t.cpu().numpy(), rows, B, N), out_o)
            compare_lse(lse_t.cpu().numpy(), lse_o)
            _log(f"[fullsize] 64K tau {tau} permutation {use_perm}: density "
                 f"{cg.sum() / (Hq * NB * (NB + 1) / 2):.3f}, rows {rows} max abs {mx:.2e} mean abs {mean:.2e}")


def test_max_blocks_sampled():
    """The largest sequence the library accepts: 2048 key blocks (N = 262144 at B = 128) with the
    largest segment (8192), on two query heads of one KV head: the whole permutation, every mask
    row, and sampled attention rows including the last block (the longest list) and the dense
    kernel on them."""
    pbsa = _need_gpu()
    from workloads import generate
    N, Hq, Hkv, d, B, S, tau = 262144, 2, 1, 64, 128, 8192, 0.9
    NB = N // B
    _log(f"[fullsize] max blocks: N={N} B={B} S={S} NB={NB}")
    x = generate(N, Hq, Hkv, d, 16, 512, 21)
    dev = {n: torch.from_numpy(x[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("q", "k", "v")}
    q, k, v = (bf16_bits_to_f32(x[n]).astype(np.float64) for n in ("q", "k", "v"))
    perm_t, imp_t = pbsa.build_segment_permutation(dev["q"], dev["k"], B, S, return_importance=True)
    count_t, idx_t, prob_t = pbsa.estimate_block_mask(dev["q"], dev["k"], perm_t, B, S, tau, return_prob=True)
    out_t, lse_t = pbsa.block_sparse_attn_prefill(dev["q"], dev["k"], dev["v"], perm_t, count_t, idx_t, B, S)
    dense_t, dense_lse_t = pbsa.block_sparse_attn_prefill(dev["q"], dev["k"], dev["v"], block_size=B)
    torch.cuda.synchronize()
    imp_o = oracle.key_importance(q, k, B)
    compare_importance(imp_t.cpu().numpy(), imp_o, imp_rtol(q, k))
    perm_g = perm_t.cpu().numpy()
    compare_perm(perm_g, oracle.segment_permutation(imp_o, S), imp_o, S)
    cg, ig = count_t.cpu().numpy(), idx_t.cpu().numpy()
    co, io, po = oracle.block_mask(q, k, perm_g, B, S, tau)
    compare_mask(cg, ig, co, io, po, tau)
    _log(f"[fullsize] max blocks: permutation and every mask row ok (density {cg.sum() / (Hq * NB * (NB + 1) / 2):.3f})")
    rows = [(0, NB - 1), (1, NB - 1), (0, 0), (1, NB // 2), (0, 1365)]
    out_o, lse_o, _, _ = oracle.block_sparse_attention(q, k, v, perm_g, cg, ig, B, S, rows=rows)
    mx, mean = compare_out(_rows_slice(out_t.cpu().numpy(), rows, B, N), out_o)
    compare_lse(lse_t.cpu().numpy(), lse_o)
    full = {(h, I): list(range(I + 1)) for h, I in rows}
    fc = np.zeros((Hq, NB), dtype=np.int64)
    fi = np.full((Hq, NB * (NB + 1) // 2), -1, dtype=np.int64)
    for (h, I), lst in full.items():
        fc[h, I] = len(lst)
        fi[h, oracle.tri_offset(I):oracle.tri_offset(I) + len(lst)] = lst
    dense_o, dense_lse_o, _, _ = oracle.block_sparse_attention(q, k, v, None, fc, fi, B, S, rows=rows)
    dmx, dmean = compare_out(_rows_slice(dense_t.cpu().numpy(), rows, B, N), dense_o, "dense")
    compare_lse(dense_lse_t.cpu().numpy(), dense_lse_o)
    _log(f"[fullsize] max blocks rows {rows}: sparse max abs {mx:.2e} mean {mean:.2e}; dense max abs {dmx:.2e}")


def test_fullsize_64k_early_stop_sampled():
    pbsa = _need_gpu()
    w = WORKLOADS["llama8b_64k_earlystop"]
    _log(f"[fullsize] {w.name}")
    dev, host = _load(w)
    cal, _ = _load(w, seed=w.calib_seed)
    B, NB, Hq, N = w.block_size, w.num_blocks, w.num_q_heads, w.seq_len
    tm_cal = pbsa.tile_max(cal["q"], cal["k"], B).cpu().numpy()
    del cal
    theta = oracle.calibrate_thresholds(tm_cal.astype(np.float64), NB, w.calib_keep).astype(np.float32)
    theta_t = torch.from_numpy(theta).cuda()
    out_t, lse_t, kept_t = pbsa.block_sparse_attn_prefill(dev["q"], dev["k"], dev["v"], block_size=B,
                                                          early_stop_theta=theta_t, return_kept=True)
    tm_g = pbsa.tile_max(dev["q"], dev["k"], B).cpu().numpy()
    torch.cuda.synchronize()
    kept = bitmap_to_kept(kept_t.cpu().numpy(), NB)
    # the gate equals the fp32 decision on the kernel's own tile maxima, for every row
    for (h, I), lst in kept.items():
        o = oracle.tri_offset(I)
        want = [J for J in range(I + 1) if J == I or tm_g[h, o + J] >= theta[h, I]]
        assert lst == want, (h, I)
    # sampled rows: fp64 tile maxima, and outputs on the realised kept set
    q, k, v = host["q"], host["k"], host["v"]
    rows = _sample_rows(Hq, NB, 6, 10)
    tm_o = oracle.tile_max(q, k, B, rows=rows)
    bound = gate_error_bound(q, k, None, B, None, rows)
    exact = {}
    for h, I in rows:  # GPU tile maxima within the fp32 bound, decisions against the fp64 oracle
        o = oracle.tri_offset(I)
        m = tm_o[h, o:o + I + 1]
        err = np.abs(tm_g[h, o:o + I + 1] - m)
        assert (err <= bound[(h, I)] + 4 * F32_U * np.abs(m)).all(), (h, I, err.max())
        exact[(h, I)] = m
    n, band = compare_gate(kept, {r: list(range(r[1] + 1)) for r in rows}, exact, bound, theta)
    _log(f"[fullsize] 64K early stop: {n} sampled gate decisions, {band} inside the fp32 bound")
    assert band <= max(2, n // 200), (n, band)
    kc, ki = kept_to_mask(kept, Hq, NB)
    out_o, lse_o, _, _ = oracle.block_sparse_attention(q, k, v, None, kc, ki, B, None, rows=rows)
    mx, mean = compare_out(_rows_slice(out_t.cpu().numpy(), rows, B, N), out_o)
    frac = sum(len(v) for v in kept.values()) / (Hq * NB * (NB + 1) / 2)
    _log(f"[fullsize] 64K early stop: kept fraction {frac:.3f}, rows {rows}: max abs {mx:.2e} mean {mean:.2e}")


def test_fullsize_32k_marginal_gain_sampled():
    """Marginal-gain early stop at 32K: every ranked row, and the stop and outputs of sampled rows."""
    pbsa = _need_gpu()
    w = WORKLOADS["llama8b_32k"]
    gain_tau = 0.01
    _log(f"[fullsize] {w.name} marginal-gain stop, gain_tau {gain_tau}")
    dev, host = _load(w)
    q, k, v = host["q"], host["k"], host["v"]
    B, S, NB, Hq, N = w.block_size, w.segment_size, w.num_blocks, w.num_q_heads, w.seq_len
    perm_t = pbsa.build_segment_permutation(dev["q"], dev["k"], B, S)
    count_t, idx_t = pbsa.estimate_block_mask(dev["q"], dev["k"], perm_t, B, S, w.mass_tau, ranked=True)
    out_t, lse_t, kept_t = pbsa.s2o_attn_prefill(dev["q"], dev["k"], dev["v"], perm_t, count_t, idx_t, B, S,
                                                 gain_tau, return_kept=True)
    torch.cuda.synchronize()
    perm_g, cg, ig = perm_t.cpu().numpy(), count_t.cpu().numpy(), idx_t.cpu().numpy()
    count_o, idx_o, _ = oracle.ranked_blocks(q, k, perm_g, B, S)
    ties = compare_ranked(cg, ig, count_o, idx_o, oracle.pooled_block_logits(q, k, perm_g, B, S))
    _log(f"[fullsize] ranked order ok ({ties} recorded ties)")
    kept = bitmap_to_kept(kept_t.cpu().numpy(), NB)
    rows = _sample_rows(Hq, NB, 12, 11)
    ratios = oracle.s2o_gain_ratios(q, k, perm_g, cg, ig, B, S, rows=rows)
    _, near = compare_s2o_stops(kept, cg, ig, ratios, gain_tau)
    kc, ki = kept_to_mask({r: kept[r] for r in rows}, Hq, NB)
    out_o, lse_o, _, _ = oracle.block_sparse_attention(q, k, v, perm_g, kc, ki, B, S, rows=rows)
    mx, mean = compare_out(_rows_slice(out_t.cpu().numpy(), rows, B, N), out_o, "s2o 32K")
    compare_lse(lse_t.cpu().numpy(), lse_o)
    frac = sum(len(x) for x in kept.values()) / (Hq * NB * (NB + 1) / 2)
    _log(f"[fullsize] 32K marginal-gain stop: processed {frac:.3f}, sampled rows {rows} ({near} in band): "
         f"max abs {mx:.2e} mean {mean:.2e}")


def test_fullsize_32k_two_pass_sampled():
    """S2O two-pass attention at 32K: the whole historical ranking, and the stop and outputs of
    sampled rows."""
    pbsa = _need_gpu()
    w = WORKLOADS["llama8b_32k"]
    gain_tau = 0.01
    _log(f"[fullsize] {w.name} two-pass, gain_tau {gain_tau}")
    dev, host = _load(w)
    q, k, v = host["q"], host["k"], host["v"]
    B, S, NB, Hq, N = w.block_size, w.segment_size, w.num_blocks, w.num_q_heads, w.seq_len
    rank_t = pbsa.build_prefix_kv_ranking(dev["q"], dev["k"], B, S)
    out_t, lse_t, kept_t = pbsa.s2o_prefix_attn_prefill(dev["q"], dev["k"], dev["v"], rank_t, B, S, gain_tau,
                                                        return_kept=True)
    torch.cuda.synchronize()
    pi_g = rank_t.cpu().numpy().astype(np.int64)
    pi_o, score_o = oracle.prefix_kv_ranking(q, k, S)
    ties = compare_prefix_rank(pi_g, pi_o, score_o, S)
    _log(f"[fullsize] historical ranking ok ({ties} recorded ties)")
    kept = bitmap_to_kept(kept_t.cpu().numpy(), NB)
    rows = _sample_rows(Hq, NB, 12, 12)
    cg, ig = two_pass_lists(Hq, N, B, S)
    ratios = oracle.s2o_prefix_gain_ratios(q, k, pi_g, B, S, rows=rows)
    _, near = compare_s2o_stops(kept, cg, ig, ratios, gain_tau)
    out_o, lse_o = oracle.two_pass_attention_on(q, k, v, pi_g, {r: kept[r] for r in rows}, B, S)
    mx, mean = compare_out(_rows_slice(out_t.cpu().numpy(), rows, B, N), out_o, "two-pass 32K")
    compare_lse(lse_t.cpu().numpy(), lse_o)
    frac = sum(len(x) for x in kept.values()) / (Hq * NB * (NB + 1) / 2)
    _log(f"[fullsize] 32K two-pass: processed {frac:.3f}, sampled rows {rows} ({near} in band): "
         f"max abs {mx:.2e} mean {mean:.2e}")


def test_fullsize_32k_query_permuted_two_pass_sampled():
    """Query permutation at 32K: the whole query order, and the stop and outputs of sampled rows."""
    pbsa = _need_gpu()
    w = WORKLOADS["llama8b_32k"]
    gain_tau = 0.01
    _log(f"[fullsize] {w.name} query-permuted two-pass, gain_tau {gain_tau}")
    dev, host = _load(w)
    q, k, v = host["q"], host["k"], host["v"]
    B, S, NB, Hq, N = w.block_size, w.segment_size, w.num_blocks, w.num_q_heads, w.seq_len
    qperm_t = pbsa.build_query_permutation(dev["q"], dev["k"], B, S)
    rank_t = pbsa.build_prefix_kv_ranking(dev["q"], dev["k"], B, S)
    out_t, lse_t, kept_t = pbsa.s2o_prefix_attn_prefill(dev["q"], dev["k"], dev["v"], rank_t, B, S, gain_tau,
                                                        qperm=qperm_t, return_kept=True)
    torch.cuda.synchronize()
    qp_g = qperm_t.cpu().numpy().astype(np.int64)
    ties = compare_perm(qp_g, oracle.query_permutation(q, k, S), oracle.query_guide_scores(q, k), S)
    _log(f"[fullsize] query order ok ({ties} recorded ties)")
    pi_g = rank_t.cpu().numpy().astype(np.int64)
    kept = bitmap_to_kept_square(kept_t.cpu().numpy(), NB)
    rows = _sample_rows(Hq, NB, 10, 13)
    cg, ig = two_pass_lists(Hq, N, B, S, permuted_queries=True)
    ratios = oracle.s2o_prefix_gain_ratios(q, k, pi_g, B, S, rows=rows, qperm=qp_g)
    _, near = compare_s2o_stops(kept, cg, ig, ratios, gain_tau, row_stride=NB)
    out_o, lse_o = oracle.two_pass_attention_on(q, k, v, pi_g, {r: kept[r] for r in rows}, B, S, qperm=qp_g)
    ok = ~np.isnan(out_o)
    mx, mean = compare_out(np.where(ok, out_t.cpu().numpy(), np.nan), out_o, "qperm two-pass 32K")
    compare_lse(lse_t.cpu().numpy(), lse_o)
    _log(f"[fullsize] 32K query-permuted two-pass: sampled rows {rows} ({near} in band): max abs {mx:.2e} mean {mean:.2e}")


def test_max_segments_two_pass_sampled():
    """The historical ranking at its limit of 256 segments (N = 16384, S = B = 64): the whole
    ranking and the whole query order, then the stop and outputs of sampled rows, without and with
    the query permutation."""
    pbsa = _need_gpu()
    from workloads import generate
    N, Hq, Hkv, d, B, S, gain_tau = 16384, 2, 1, 64, 64, 64, 0.02
    NB = N // B
    _log(f"[fullsize] max segments: N={N} B={B} S={S} segments={N // S}")
    x = generate(N, Hq, Hkv, d, 0, 64, 58)
    dev = {n: torch.from_numpy(x[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("q", "k", "v")}
    q, k, v = (bf16_bits_to_f32(x[n]).astype(np.float64) for n in ("q", "k", "v"))
    rank_t = pbsa.build_prefix_kv_ranking(dev["q"], dev["k"], B, S)
    qperm_t = pbsa.build_query_permutation(dev["q"], dev["k"], B, S)
    torch.cuda.synchronize()
    pi_g = rank_t.cpu().numpy().astype(np.int64)
    pi_o, score_o = oracle.prefix_kv_ranking(q, k, S)
    ties = compare_prefix_rank(pi_g, pi_o, score_o, S)
    qp_g = qperm_t.cpu().numpy().astype(np.int64)
    qties = compare_perm(qp_g, oracle.query_permutation(q, k, S), oracle.query_guide_scores(q, k), S)
    _log(f"[fullsize] max segments: ranking ({ties} ties) and query order ({qties} ties) ok")
    rows = _sample_rows(Hq, NB, 8, 58)
    for permuted in (False, True):
        out_t, lse_t, kept_t = pbsa.s2o_prefix_attn_prefill(dev["q"], dev["k"], dev["v"], rank_t, B, S, gain_tau,
                                                            qperm=qperm_t if permuted else None, return_kept=True)
        torch.cuda.synchronize()
        qp = qp_g if permuted else None
        kept = (bitmap_to_kept_square if permuted else bitmap_to_kept)(kept_t.cpu().numpy(), NB)
        cg, ig = two_pass_lists(Hq, N, B, S, permuted_queries=permuted)
        ratios = oracle.s2o_prefix_gain_ratios(q, k, pi_g, B, S, rows=rows, qperm=qp)
        _, near = compare_s2o_stops(kept, cg, ig, ratios, gain_tau, **({"row_stride": NB} if permuted else {}))
        out_o, lse_o = oracle.two_pass_attention_on(q, k, v, pi_g, {r: kept[r] for r in rows}, B, S, qperm=qp)
        ok = ~np.isnan(out_o)
        mx, mean = compare_out(np.where(ok, out_t.cpu().numpy(), np.nan), out_o, "two-pass, 256 segments")
        compare_lse(lse_t.cpu().numpy(), lse_o)
        _log(f"[fullsize] max segments, query permutation {permuted}: rows {rows} ({near} in band) "
             f"max abs {mx:.2e} mean {mean:.2e}")


def test_fullsize_32k_sample_attention_mask():
    """SampleAttention's mask at 32K (8 trunks of 16 sampled rows per query head): masses, kept
    patterns and every mask row against the oracle, and sampled attention rows on the mask."""
    pbsa = _need_gpu()
    w = WORKLOADS["llama8b_32k"]
    tau, nt, rpt = 0.9, 8, 16
    _log(f"[fullsize] {w.name} SampleAttention mask, tau {tau}, trunks {nt}x{rpt}")
    dev, host = _load(w)
    q, k, v = host["q"], host["k"], host["v"]
    B, NB, Hq, N = w.block_size, w.num_blocks, w.num_q_heads, w.seq_len
    count_t, idx_t, col_t, sl_t = pbsa.sample_attention_mask(dev["q"], dev["k"], B, tau, nt, rpt, return_masses=True)
    out_t, lse_t = pbsa.block_sparse_attn_prefill(dev["q"], dev["k"], dev["v"], None, count_t, idx_t, B, 0)
    torch.cuda.synchronize()
    cg, ig = count_t.cpu().numpy(), idx_t.cpu().numpy()
    col_o, sl_o = oracle.sampled_masses(q, k, nt, rpt)
    ties = compare_sample_mask(cg, ig, col_t.cpu().numpy(), sl_t.cpu().numpy(), col_o, sl_o, tau, B, True, False,
                               imp_rtol(q, k))
    rows = _sample_rows(Hq, NB, 8, 14)
    out_o, lse_o, _, _ = oracle.block_sparse_attention(q, k, v, None, cg, ig, B, None, rows=rows)
    mx, mean = compare_out(_rows_slice(out_t.cpu().numpy(), rows, B, N), out_o, "sample mask 32K")
    compare_lse(lse_t.cpu().numpy(), lse_o)
    _log(f"[fullsize] 32K SampleAttention: {ties} tie heads, density {cg.sum() / (Hq * NB * (NB + 1) / 2):.3f}, "
         f"rows {rows}: max abs {mx:.2e} mean {mean:.2e}")
