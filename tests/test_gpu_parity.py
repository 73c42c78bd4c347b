"""GPU parity: every stage of the HIP path against the fp64 oracle on the same seeded inputs.

Stage-wise: each stage gets the same upstream input on both sides (the GPU's own upstream output,
checked first), so a recorded tie in one stage cannot cascade.  Tie rules: tests/parity.py.
"""
import math
import sys

import numpy as np
import pytest

import oracle
from parity import (F32_U, bitmap_to_kept, bitmap_to_kept_square, compare_gate, compare_importance, compare_lse,
                    compare_mask, compare_out,
                    compare_perm, compare_prefix_rank, compare_ranked, compare_s2o_stops, compare_sample_mask,
                    gate_error_bound, imp_rtol, kept_to_mask, two_pass_lists)
from workloads import bf16_bits_to_f32, bf16_round_bits, generate

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_blocks_amd as pbsa  # noqa: F401 (raises if the library is missing)
    return pbsa


# (name, N, Hq, Hkv, d, B, S, stripes, band, tau, seed)
CASES = [
    ("single_head_1k", 1024, 1, 1, 64, 64, 256, 8, 0, 0.9, 1001),
    ("gqa_ragged_2125", 2125, 4, 2, 128, 128, 512, 16, 256, 0.9, 7),
    ("b64_d128_ragged_1500", 1500, 2, 1, 128, 64, 256, 8, 128, 0.8, 8),
    ("b128_d64_ragged_1000", 1000, 4, 1, 64, 128, 256, 8, 128, 0.95, 9),
    ("shorter_than_a_block_100", 100, 2, 2, 128, 128, 128, 2, 0, 0.9, 10),
    ("b64_d64_pairs_ragged_777", 777, 4, 2, 64, 64, 128, 8, 64, 0.9, 11),
    ("single_token_1", 1, 2, 1, 64, 64, 64, 0, 0, 0.9, 12),
    ("single_token_b128_d128_gqa", 1, 4, 2, 128, 128, 128, 0, 0, 0.5, 13),
]


def _inputs(N, Hq, Hkv, d, stripes, band, seed):
    x = generate(N, Hq, Hkv, d, stripes, band, seed)
    dev = {n: torch.from_numpy(x[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("q", "k", "v")}
    host = {n: bf16_bits_to_f32(x[n]).astype(np.float64) for n in ("q", "k", "v")}
    return dev, host


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_pipeline_stagewise(case):
    pbsa = _need_gpu()
    name, N, Hq, Hkv, d, B, S, stripes, band, tau, seed = case
    _log(f"[parity] {name}: N={N} Hq={Hq} Hkv={Hkv} d={d} B={B} S={S}")
    dev, host = _inputs(N, Hq, Hkv, d, stripes, band, seed)
    q, k, v = host["q"], host["k"], host["v"]
    NB = oracle.num_blocks(N, B)

    # stage 1
    perm_t, imp_t = pbsa.build_segment_permutation(dev["q"], dev["k"], B, S, return_importance=True)
    torch.cuda.synchronize()
    imp_g, perm_g = imp_t.cpu().numpy(), perm_t.cpu().numpy()
    imp_o = oracle.key_importance(q, k, B)
    compare_importance(imp_g, imp_o, imp_rtol(q, k))
    compare_perm(perm_g, oracle.segment_permutation(imp_o, S), imp_o, S)

    # stage 2, on the GPU's permutation
    for use_perm in (True, False):
        count_t, idx_t, prob_t = pbsa.estimate_block_mask(dev["q"], dev["k"], perm_t if use_perm else None, B, S,
                                                          tau, return_prob=True)
        torch.cuda.synchronize()
        count_o, idx_o, prob_o = oracle.block_mask(q, k, perm_g if use_perm else None, B, S, tau)
        pg = prob_t.cpu().numpy()
        for I in range(NB):
            o = oracle.tri_offset(I)
            np.testing.assert_allclose(pg[:, o:o + I + 1], prob_o[:, o:o + I + 1], rtol=1e-11, atol=1e-300)
        compare_mask(count_t.cpu().numpy(), idx_t.cpu().numpy(), count_o, idx_o, prob_o, tau)

    # stage 3, on the GPU's permutation and mask
    count_t, idx_t = pbsa.estimate_block_mask(dev["q"], dev["k"], perm_t, B, S, tau)
    out_t, lse_t, kept_t, err_t = pbsa.block_sparse_attn_prefill(dev["q"], dev["k"], dev["v"], perm_t, count_t, idx_t,
                                                                 B, S, return_kept=True, return_error=True)
    torch.cuda.synchronize()
    assert int(err_t.item()) == 0
    cg, ig = count_t.cpu().numpy(), idx_t.cpu().numpy()
    out_o, lse_o, kept_o, _ = oracle.block_sparse_attention(q, k, v, perm_g, cg, ig, B, S)
    mx, mean = compare_out(out_t.cpu().numpy(), out_o)
    compare_lse(lse_t.cpu().numpy(), lse_o)
    assert bitmap_to_kept(kept_t.cpu().numpy(), NB) == kept_o
    _log(f"[parity] {name}: attention max abs {mx:.2e} mean abs {mean:.2e}")


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_dense_causal_mode(case):
    pbsa = _need_gpu()
    name, N, Hq, Hkv, d, B, S, stripes, band, tau, seed = case
    dev, host = _inputs(N, Hq, Hkv, d, stripes, band, seed + 100)
    out_t, lse_t = pbsa.block_sparse_attn_prefill(dev["q"], dev["k"], dev["v"], block_size=B)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.dense_attention(host["q"], host["k"], host["v"])
    compare_out(out_t.cpu().numpy(), ref, "dense")
    compare_lse(lse_t.cpu().numpy(), ref_lse)


def test_full_mask_with_permutation_equals_dense():
    """tau = 1 keeps every block; reading past segments through perm must not change the result."""
    pbsa = _need_gpu()
    N, Hq, Hkv, d, B, S = 1536, 4, 2, 128, 128, 512
    dev, host = _inputs(N, Hq, Hkv, d, 12, 256, 21)
    perm = pbsa.build_segment_permutation(dev["q"], dev["k"], B, S)
    count, idx = pbsa.estimate_block_mask(dev["q"], dev["k"], perm, B, S, 1.0)
    out = pbsa.block_sparse_attn_prefill(dev["q"], dev["k"], dev["v"], perm, count, idx, B, S, return_lse=False)
    torch.cuda.synchronize()
    assert (count.cpu().numpy() == np.arange(1, oracle.num_blocks(N, B) + 1)[None, :]).all()
    ref, _ = oracle.dense_attention(host["q"], host["k"], host["v"])
    compare_out(out.cpu().numpy(), ref, "full mask")


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (3, 1)])
def test_mask_without_permutation(Hq, Hkv):
    """Permutation off (perm = NULL) with a segment size set: every key block is read in natural order."""
    pbsa = _need_gpu()
    N, d, B, S = 1700, 128, 128, 512
    dev, host = _inputs(N, Hq, Hkv, d, 12, 256, 71)
    count, idx = pbsa.estimate_block_mask(dev["q"], dev["k"], None, B, S, 0.8)
    out, lse = pbsa.block_sparse_attn_prefill(dev["q"], dev["k"], dev["v"], None, count, idx, B, S)
    torch.cuda.synchronize()
    cg, ig = count.cpu().numpy(), idx.cpu().numpy()
    co, io, po = oracle.block_mask(host["q"], host["k"], None, B, S, 0.8)
    compare_mask(cg, ig, co, io, po, 0.8)
    out_o, lse_o, _, _ = oracle.block_sparse_attention(host["q"], host["k"], host["v"], None, cg, ig, B, S)
    compare_out(out.cpu().numpy(), out_o, "mask without permutation")
    compare_lse(lse.cpu().numpy(), lse_o)


@pytest.mark.parametrize("groups", [1, 3])
def test_mask_with_exact_ties(groups):
    """Key rows equal inside each block and across block groups, so the pooled logits of a row take
    one value (groups = 1) or three (block 0 alone, the even and the odd blocks): the cut falls
    inside runs of exactly equal p.  Equal p are taken smallest J first, and tau = 0.61803 leaves
    every cut at least 0.0026 of mass from tau, so the lists must equal the oracle's exactly."""
    pbsa = _need_gpu()
    N, Hq, Hkv, d, B, S, tau = 2048, 2, 1, 128, 128, 512, 0.61803
    x = generate(N, Hq, Hkv, d, 0, 0, 81)
    rng = np.random.default_rng(82)
    rows = [bf16_round_bits(rng.standard_normal(d).astype(np.float32)) for _ in range(3)]
    kbits = x["k"].copy()
    for J in range(N // B):
        grp = 0 if groups == 1 else (2 if J == 0 else J % 2)
        kbits[:, J * B:(J + 1) * B, :] = rows[grp]
    qd = torch.from_numpy(x["q"].view(np.int16)).view(torch.bfloat16).cuda()
    kd = torch.from_numpy(kbits.view(np.int16)).view(torch.bfloat16).cuda()
    qh = bf16_bits_to_f32(x["q"]).astype(np.float64)
    kh = bf16_bits_to_f32(kbits).astype(np.float64)
    _log(f"[exact ties] groups={groups} N={N} Hq={Hq} tau={tau}")
    count, idx, prob = pbsa.estimate_block_mask(qd, kd, None, B, S, tau, return_prob=True)
    torch.cuda.synchronize()
    cg, ig, pg = count.cpu().numpy(), idx.cpu().numpy(), prob.cpu().numpy()
    co, io, po = oracle.block_mask(qh, kh, None, B, S, tau)
    NB = N // B
    tied = sum(I + 1 - len(np.unique(pg[h, oracle.tri_offset(I):oracle.tri_offset(I) + I + 1]))
               for h in range(Hq) for I in range(NB))
    _log(f"[exact ties] {tied} probabilities equal to another of their row on the GPU")
    assert tied > 0  # the selection really meets exact ties
    assert compare_mask(cg, ig, co, io, po, tau) == 0
    for h in range(Hq):
        for I in range(NB):
            o = oracle.tri_offset(I)
            assert cg[h, I] == co[h, I], (h, I)
            assert np.array_equal(ig[h, o:o + cg[h, I]], io[h, o:o + co[h, I]]), (h, I)


# query heads paired per workgroup (even G) and not, every supported (d, B), one ragged N
@pytest.mark.parametrize("Hq,Hkv,d,B,N", [(4, 2, 128, 128, 2048), (3, 1, 128, 128, 2048), (4, 2, 64, 64, 1900),
                                          (2, 1, 128, 64, 2048), (4, 2, 64, 128, 2048)])
def test_early_stop_gate(Hq, Hkv, d, B, N):
    pbsa = _need_gpu()
    keep = 6
    dev, host = _inputs(N, Hq, Hkv, d, 16, 256, 31)
    cal, _ = _inputs(N, Hq, Hkv, d, 16, 256, 32)
    NB = oracle.num_blocks(N, B)
    q, k, v = host["q"], host["k"], host["v"]

    # tile max of the calibration draw and of the evaluation draw
    tm_cal = pbsa.tile_max(cal["q"], cal["k"], B).cpu().numpy()
    tm_o = oracle.tile_max(q, k, B)
    tm_g = pbsa.tile_max(dev["q"], dev["k"], B).cpu().numpy()
    all_rows = [(h, I) for h in range(Hq) for I in range(NB)]
    bound = gate_error_bound(q, k, None, B, None, all_rows)
    for h, I in all_rows:  # every GPU tile max within the fp32 bound of the exact one
        o = oracle.tri_offset(I)
        m = tm_o[h, o:o + I + 1]
        err = np.abs(tm_g[h, o:o + I + 1] - m)
        assert (err <= bound[(h, I)] + 4 * F32_U * np.abs(m)).all(), (h, I, err.max(), bound[(h, I)].min())
    theta = oracle.calibrate_thresholds(tm_cal.astype(np.float64), NB, keep).astype(np.float32)
    theta_t = torch.from_numpy(theta).cuda()
    # the library's own calibration picks the same values from the same tile maxima
    theta_lib = pbsa.calibrate_thresholds(torch.from_numpy(tm_cal).cuda(), cal["q"], cal["k"], B, keep)
    assert np.array_equal(theta_lib.cpu().numpy(), theta)

    for mode in ("dense", "masked"):
        if mode == "dense":
            count_t = idx_t = None
            cnt_np = idx_np = None
        else:
            count_t, idx_t = pbsa.estimate_block_mask(dev["q"], dev["k"], None, B, 512, 0.95)
            cnt_np, idx_np = count_t.cpu().numpy(), idx_t.cpu().numpy()
        out_t, lse_t, kept_t = pbsa.block_sparse_attn_prefill(dev["q"], dev["k"], dev["v"], None, count_t, idx_t, B, 512,
                                                              early_stop_theta=theta_t, return_kept=True)
        torch.cuda.synchronize()
        kept_g = bitmap_to_kept(kept_t.cpu().numpy(), NB)
        sel = {}
        for h in range(Hq):
            for I in range(NB):
                o = oracle.tri_offset(I)
                sel[(h, I)] = list(range(I + 1)) if cnt_np is None else [int(x) for x in idx_np[h, o:o + cnt_np[h, I]]]
                # the gate equals the fp32 decision on the kernel's own tile maxima
                want = [J for J in sel[(h, I)] if J == I or np.float32(tm_g[h, o + J]) >= theta[h, I]]
                assert kept_g[(h, I)] == want, (h, I)
        # and the fp64 oracle's decision wherever it is clear of the fp32 error bound
        exact = {(h, I): tm_o[h, oracle.tri_offset(I):oracle.tri_offset(I) + I + 1] for h, I in all_rows}
        n, band = compare_gate(kept_g, sel, exact, bound, theta)
        print(f"[early stop {mode}] {n} gate decisions, {band} inside the fp32 bound", flush=True)
        assert band <= max(2, n // 200), (n, band)
        # outputs equal block-sparse attention on the realised kept set
        kc, ki = kept_to_mask(kept_g, Hq, NB)
        out_o, lse_o, _, _ = oracle.block_sparse_attention(q, k, v, None, kc, ki, B, 512)
        compare_out(out_t.cpu().numpy(), out_o, f"early stop ({mode})")
        compare_lse(lse_t.cpu().numpy(), lse_o)


def test_threshold_limits():
    pbsa = _need_gpu()
    N, Hq, Hkv, d, B = 1000, 2, 1, 128, 128
    dev, host = _inputs(N, Hq, Hkv, d, 8, 128, 41)
    NB = oracle.num_blocks(N, B)
    ref = pbsa.block_sparse_attn_prefill(dev["q"], dev["k"], dev["v"], block_size=B, return_lse=False)
    lo = torch.full((Hq, NB), -math.inf, device="cuda")
    out_lo = pbsa.block_sparse_attn_prefill(dev["q"], dev["k"], dev["v"], block_size=B, early_stop_theta=lo,
                                            return_lse=False)
    hi = torch.full((Hq, NB), math.inf, device="cuda")
    out_hi = pbsa.block_sparse_attn_prefill(dev["q"], dev["k"], dev["v"], block_size=B, early_stop_theta=hi,
                                            return_lse=False)
    torch.cuda.synchronize()
    # theta = -inf keeps every tile: dense causal attention
    dense, _ = oracle.dense_attention(host["q"], host["k"], host["v"])
    compare_out(out_lo.cpu().numpy(), dense, "theta=-inf")
    assert (out_lo - ref).abs().max().item() <= 2e-2
    blk = np.arange(N) // B
    diag_only, _ = oracle.dense_attention(host["q"], host["k"], host["v"], allowed=blk[:, None] == blk[None, :])
    compare_out(out_hi.cpu().numpy(), diag_only, "theta=+inf")


def _tile_max_fp64(q, k, perm, B, S, h, I, J, G):
    """c * max of q_i . k_j over i in block I, j in the rows block J stands for when read by I, j <= i."""
    N, d = q.shape[1], q.shape[2]
    qi = np.arange(I * B, min((I + 1) * B, N))
    kj = oracle.key_rows_of_block(J, I, None if perm is None else perm[h // G], B, S, N)
    st = (q[h, qi] @ k[h // G, kj].T) / math.sqrt(d)
    return np.where(kj[None, :] <= qi[:, None], st, -np.inf).max()


def test_early_stop_with_permutation():
    """The gate on a permuted sparse mask: tile maxima over the gathered (permuted) rows."""
    pbsa = _need_gpu()
    N, Hq, Hkv, d, B, S = 1664, 4, 2, 128, 128, 512
    dev, host = _inputs(N, Hq, Hkv, d, 12, 256, 61)
    q, k, v = host["q"], host["k"], host["v"]
    NB, G = oracle.num_blocks(N, B), Hq // Hkv
    perm_t = pbsa.build_segment_permutation(dev["q"], dev["k"], B, S)
    count_t, idx_t = pbsa.estimate_block_mask(dev["q"], dev["k"], perm_t, B, S, 0.97)
    perm, cnt, idx = perm_t.cpu().numpy(), count_t.cpu().numpy(), idx_t.cpu().numpy()
    # thresholds halfway between the two middle fp64 tile maxima of each row (so no tile max sits on
    # a threshold by construction), and about half the off-diagonal tiles go
    theta = np.full((Hq, NB), -np.inf, dtype=np.float32)
    tmax = {}
    for h in range(Hq):
        for I in range(NB):
            o = oracle.tri_offset(I)
            sel = [int(J) for J in idx[h, o:o + cnt[h, I]]]
            tmax[(h, I)] = {J: _tile_max_fp64(q, k, perm, B, S, h, I, J, G) for J in sel}
            off = sorted(m for J, m in tmax[(h, I)].items() if J != I)
            if len(off) >= 2:
                theta[h, I] = np.float32(0.5 * (off[len(off) // 2 - 1] + off[len(off) // 2]))
            elif off:
                theta[h, I] = np.float32(off[0] + 1.0)
    out_t, lse_t, kept_t = pbsa.block_sparse_attn_prefill(dev["q"], dev["k"], dev["v"], perm_t, count_t, idx_t, B, S,
                                                          early_stop_theta=torch.from_numpy(theta).cuda(),
                                                          return_kept=True)
    torch.cuda.synchronize()
    kept = bitmap_to_kept(kept_t.cpu().numpy(), NB)
    rows = list(tmax)
    full_bound = gate_error_bound(q, k, perm, B, S, rows)
    # the calibration statistic read through the same permutation: every tile within the fp32 bound
    # of the fp64 value, and the gate's decisions equal the ones these fp32 maxima give
    tm_p = pbsa.tile_max(dev["q"], dev["k"], B, perm=perm_t, segment_size=S).cpu().numpy()
    for h, I in rows:
        o = oracle.tri_offset(I)
        for J in range(I + 1):
            m = _tile_max_fp64(q, k, perm, B, S, h, I, J, G)
            assert abs(tm_p[h, o + J] - m) <= full_bound[(h, I)][J] + 4 * F32_U * abs(m), (h, I, J)
        want = [J for J in sorted(tmax[(h, I)]) if J == I or tm_p[h, o + J] >= theta[h, I]]
        assert kept[(h, I)] == want, (h, I)
    sel = {r: sorted(tm) for r, tm in tmax.items()}
    exact = {r: np.array([tm.get(J, np.nan) for J in range(r[1] + 1)]) for r, tm in tmax.items()}
    n, band = compare_gate(kept, sel, exact, full_bound, theta)
    print(f"[early stop with permutation] {n} gate decisions, {band} inside the fp32 bound", flush=True)
    assert band <= max(2, n // 200), (n, band)
    dropped = sum(len(sel[r]) - len(kept[r]) for r in rows)
    assert dropped > 0
    kc, ki = kept_to_mask(kept, Hq, NB)
    out_o, lse_o, _, _ = oracle.block_sparse_attention(q, k, v, perm, kc, ki, B, S)
    compare_out(out_t.cpu().numpy(), out_o, "early stop with permutation")
    compare_lse(lse_t.cpu().numpy(), lse_o)


@pytest.mark.parametrize("Hq,Hkv,d,B,N,mode", [(4, 2, 128, 128, 2125, "mask"), (3, 1, 128, 128, 1500, "mask"),
                                               (4, 2, 64, 64, 1900, "dense"), (4, 2, 128, 128, 2048, "gate")])
def test_bf16_output(Hq, Hkv, d, B, N, mode):
    """pbsa_block_sparse_attn_prefill_bf16out: every output element is the fp32 result rounded to the
    nearest bf16 (ties to even), bit for bit, on the paired and one-head mask paths, the dense path
    and the early-stop path; the lse is the same; and the bf16 output stays within the attention
    tolerances of the oracle."""
    pbsa = _need_gpu()
    S = 512
    _log(f"[bf16 out] {mode}: N={N} Hq={Hq} Hkv={Hkv} d={d} B={B}")
    dev, host = _inputs(N, Hq, Hkv, d, 16, 256, 91)
    q, k, v = dev["q"], dev["k"], dev["v"]
    perm = count = idx = theta = None
    if mode == "mask":
        perm = pbsa.build_segment_permutation(q, k, B, S)
        count, idx = pbsa.estimate_block_mask(q, k, perm, B, S, 0.9)
    elif mode == "gate":
        theta = pbsa.calibrate_thresholds(pbsa.tile_max(q, k, B), q, k, B, 6)
    out32, lse32 = pbsa.block_sparse_attn_prefill(q, k, v, perm, count, idx, B, S, early_stop_theta=theta)
    out16, lse16 = pbsa.block_sparse_attn_prefill(q, k, v, perm, count, idx, B, S, early_stop_theta=theta,
                                                  out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert out16.dtype == torch.bfloat16
    got = out16.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, bf16_round_bits(out32.cpu().numpy()))
    assert torch.equal(lse16, lse32)
    if mode != "gate":  # the early-stop path's fp32 output is checked against the oracle elsewhere
        cg = count.cpu().numpy() if count is not None else None
        ig = idx.cpu().numpy() if idx is not None else None
        pg = perm.cpu().numpy() if perm is not None else None
        out_o, _, _, _ = oracle.block_sparse_attention(host["q"], host["k"], host["v"], pg, cg, ig, B, S)
        compare_out(bf16_bits_to_f32(got).astype(np.float64), out_o, f"bf16 output ({mode})")


def test_deterministic():
    pbsa = _need_gpu()
    N, Hq, Hkv, d, B, S = 2048, 4, 2, 128, 128, 512
    dev, _ = _inputs(N, Hq, Hkv, d, 16, 256, 51)
    res = []
    for _ in range(2):
        perm, imp = pbsa.build_segment_permutation(dev["q"], dev["k"], B, S, return_importance=True)
        count, idx, prob = pbsa.estimate_block_mask(dev["q"], dev["k"], perm, B, S, 0.9, return_prob=True)
        out, lse = pbsa.block_sparse_attn_prefill(dev["q"], dev["k"], dev["v"], perm, count, idx, B, S)
        torch.cuda.synchronize()
        # only the first count entries of each idx / prob row are defined
        valid = torch.zeros_like(idx, dtype=torch.bool)
        cnt = count.cpu().numpy()
        for h in range(Hq):
            for I in range(cnt.shape[1]):
                o = oracle.tri_offset(I)
                valid[h, o:o + int(cnt[h, I])] = True
        pvalid = torch.zeros_like(prob, dtype=torch.bool)
        for I in range(cnt.shape[1]):
            pvalid[:, oracle.tri_offset(I):oracle.tri_offset(I) + I + 1] = True
        res.append([perm.clone(), imp.clone(), count.clone(), idx[valid].clone(), prob[pvalid].clone(),
                    out.clone(), lse.clone()])
    for a, b in zip(*res):
        assert torch.equal(a, b)


def test_bad_indices_are_flagged_not_read():
    """Out-of-range mask entries and permutation entries are skipped by the kernel's own bounds
    checks and reported through the device error word."""
    pbsa = _need_gpu()
    N, Hq, Hkv, d, B, S = 1024, 2, 1, 128, 128, 256
    dev, host = _inputs(N, Hq, Hkv, d, 8, 0, 61)
    NB = oracle.num_blocks(N, B)
    count = torch.full((Hq, NB), 1, dtype=torch.int32, device="cuda")
    idx = torch.zeros((Hq, NB * (NB + 1) // 2), dtype=torch.int32, device="cuda")
    for I in range(NB):
        idx[:, oracle.tri_offset(I)] = I
    idx[0, oracle.tri_offset(5)] = 7          # J > I
    count[1, 3] = 2
    idx[1, oracle.tri_offset(3) + 1] = -4     # negative J
    out, err = pbsa.block_sparse_attn_prefill(dev["q"], dev["k"], dev["v"], None, count, idx, B, S,
                                              return_lse=False, return_error=True)
    torch.cuda.synchronize()
    assert int(err.item()) & 1
    # a permutation entry outside [0, N): rows of segments >= 1 read block 0 through it
    perm = torch.arange(N, dtype=torch.int32, device="cuda").repeat(Hkv, 1)
    perm[0, 10] = N + 5
    count2 = torch.full((Hq, NB), 2, dtype=torch.int32, device="cuda")
    count2[:, 0] = 1
    idx2 = torch.zeros((Hq, NB * (NB + 1) // 2), dtype=torch.int32, device="cuda")
    for I in range(1, NB):
        idx2[:, oracle.tri_offset(I) + 1] = I
    out, err = pbsa.block_sparse_attn_prefill(dev["q"], dev["k"], dev["v"], perm, count2, idx2, B, S,
                                              return_lse=False, return_error=True)
    torch.cuda.synchronize()
    assert int(err.item()) & 2
    assert torch.isfinite(out).all()


def test_strided_layout_matches_contiguous():
    """[N][H][d] (token-major) tensors passed through strides give the same result."""
    pbsa = _need_gpu()
    N, Hq, Hkv, d, B, S = 1024, 4, 2, 128, 128, 256
    dev, _ = _inputs(N, Hq, Hkv, d, 8, 128, 71)
    qs = dev["q"].transpose(0, 1).contiguous().transpose(0, 1)
    ks = dev["k"].transpose(0, 1).contiguous().transpose(0, 1)
    vs = dev["v"].transpose(0, 1).contiguous().transpose(0, 1)
    assert qs.stride(1) == Hq * d
    perm = pbsa.build_segment_permutation(dev["q"], dev["k"], B, S)
    perm_s = pbsa.build_segment_permutation(qs, ks, B, S)
    c, i = pbsa.estimate_block_mask(dev["q"], dev["k"], perm, B, S, 0.9)
    cs, is_ = pbsa.estimate_block_mask(qs, ks, perm_s, B, S, 0.9)
    o = pbsa.block_sparse_attn_prefill(dev["q"], dev["k"], dev["v"], perm, c, i, B, S, return_lse=False)
    os_ = pbsa.block_sparse_attn_prefill(qs, ks, vs, perm_s, cs, is_, B, S, return_lse=False)
    # outputs written through strides too (token-major views), fp32 and bf16
    ov = torch.empty((N, Hq, d), dtype=torch.float32, device="cuda").transpose(0, 1)
    ob = torch.empty((N, Hq, d), dtype=torch.bfloat16, device="cuda").transpose(0, 1)
    pbsa.block_sparse_attn_prefill(qs, ks, vs, perm_s, cs, is_, B, S, out=ov, return_lse=False)
    pbsa.block_sparse_attn_prefill(qs, ks, vs, perm_s, cs, is_, B, S, out=ob, return_lse=False)
    torch.cuda.synchronize()
    assert torch.equal(perm, perm_s) and torch.equal(c, cs)
    assert torch.equal(o, os_)
    assert torch.equal(ov, o)
    bits = ob.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, bf16_round_bits(o.cpu().numpy()))


@pytest.mark.parametrize("N,B,keep", [(4096, 128, 5), (2100, 64, 1), (1024, 64, 16), (8192, 128, 64)])
def test_calibrate_thresholds_exact(N, B, keep):
    """keep-th largest tile max per row, with negative values, heavy ties and ragged NB: the kernel
    selects one of the row's values, so it must equal the oracle's selection exactly."""
    pbsa = _need_gpu()
    Hq, Hkv, d = 3, 1, 64
    NB = oracle.num_blocks(N, B)
    rng = np.random.default_rng(N + keep)
    tm = rng.standard_normal((Hq, NB * (NB + 1) // 2)).astype(np.float32) * 3.0
    tm[0] = np.round(tm[0])              # many equal values
    tm[1, ::7] = -0.0                    # signed zeros among negatives and positives
    tm[1, 3::11] = 0.0
    q = torch.zeros((Hq, N, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((Hkv, N, d), dtype=torch.bfloat16, device="cuda")
    got = pbsa.calibrate_thresholds(torch.from_numpy(tm).cuda(), q, k, B, keep).cpu().numpy()
    want = oracle.calibrate_thresholds(tm.astype(np.float64), NB, keep).astype(np.float32)
    assert np.array_equal(np.isneginf(got), np.isneginf(want))
    fin = np.isfinite(want)
    assert np.array_equal(got[fin], want[fin])


# marginal-gain early stop: (name, N, Hq, Hkv, d, B, S, stripes, band, gain_tau, seed); without
# stripes the stop falls in the middle of most lists, with them right after the first history block
S2O_CASES = [
    ("flat_b64_d128_gqa_2048", 2048, 4, 2, 128, 64, 256, 0, 0, 0.05, 31),
    ("band_b128_d64_ragged_4000", 4000, 4, 1, 64, 128, 512, 0, 256, 0.02, 32),
    ("stripes_b128_d128_ragged_3000", 3000, 2, 1, 128, 128, 512, 4, 256, 0.05, 33),
    ("flat_b64_d64_ragged_1100", 1100, 2, 2, 64, 64, 128, 0, 64, 0.1, 34),
    ("flat_b128_d128_threshold_one_2048", 2048, 2, 1, 128, 128, 256, 0, 128, 1.0, 35),
]


@pytest.mark.parametrize("case", S2O_CASES, ids=[c[0] for c in S2O_CASES])
def test_marginal_gain_stagewise(case):
    pbsa = _need_gpu()
    name, N, Hq, Hkv, d, B, S, stripes, band, gain_tau, seed = case
    _log(f"[parity] s2o {name}: N={N} Hq={Hq} Hkv={Hkv} d={d} B={B} S={S} gain_tau={gain_tau}")
    dev, host = _inputs(N, Hq, Hkv, d, stripes, band, seed)
    q, k, v = host["q"], host["k"], host["v"]
    NB = oracle.num_blocks(N, B)
    perm_t = pbsa.build_segment_permutation(dev["q"], dev["k"], B, S)
    torch.cuda.synchronize()
    perm_g = perm_t.cpu().numpy()

    # ranked order, on the GPU's permutation
    count_t, idx_t = pbsa.estimate_block_mask(dev["q"], dev["k"], perm_t, B, S, 0.9, ranked=True)
    torch.cuda.synchronize()
    cg, ig = count_t.cpu().numpy(), idx_t.cpu().numpy()
    count_o, idx_o, _ = oracle.ranked_blocks(q, k, perm_g, B, S)
    ties = compare_ranked(cg, ig, count_o, idx_o, oracle.pooled_block_logits(q, k, perm_g, B, S))

    # the stop, on the GPU's ranked lists
    out_t, lse_t, kept_t, err_t = pbsa.s2o_attn_prefill(dev["q"], dev["k"], dev["v"], perm_t, count_t, idx_t, B, S,
                                                        gain_tau, return_kept=True, return_error=True)
    torch.cuda.synchronize()
    assert int(err_t.item()) == 0
    kept = bitmap_to_kept(kept_t.cpu().numpy(), NB)
    ratios = oracle.s2o_gain_ratios(q, k, perm_g, cg, ig, B, S)
    rows, near = compare_s2o_stops(kept, cg, ig, ratios, gain_tau)
    frac = sum(len(x) for x in kept.values()) / float(Hq * NB * (NB + 1) // 2)

    # softmax attention over what was processed
    kc, ki = kept_to_mask(kept, Hq, NB)
    out_o, lse_o, _, _ = oracle.block_sparse_attention(q, k, v, perm_g, kc, ki, B, S)
    mx, mean = compare_out(out_t.cpu().numpy(), out_o, "s2o")
    compare_lse(lse_t.cpu().numpy(), lse_o)
    _log(f"[parity] s2o {name}: rank ties {ties}, rows {rows}, decided in band {near}, processed {frac:.3f}, "
         f"max abs {mx:.2e} mean abs {mean:.2e}")


@pytest.mark.parametrize("d,B,N", [(128, 128, 2048), (64, 64, 1500)])
def test_marginal_gain_zero_threshold_is_dense(d, B, N):
    """gain_tau = 0 never stops: every J <= I is processed and the result is dense causal attention."""
    pbsa = _need_gpu()
    Hq, Hkv, S = 4, 2, 4 * B
    dev, host = _inputs(N, Hq, Hkv, d, 8, 2 * B, 41)
    NB = oracle.num_blocks(N, B)
    perm = pbsa.build_segment_permutation(dev["q"], dev["k"], B, S)
    count, idx = pbsa.estimate_block_mask(dev["q"], dev["k"], perm, B, S, 0.9, ranked=True)
    out, lse, kept = pbsa.s2o_attn_prefill(dev["q"], dev["k"], dev["v"], perm, count, idx, B, S, 0.0,
                                           return_kept=True)
    torch.cuda.synchronize()
    assert all(lst == list(range(I + 1)) for (h, I), lst in bitmap_to_kept(kept.cpu().numpy(), NB).items())
    ref, ref_lse = oracle.dense_attention(host["q"], host["k"], host["v"])
    compare_out(out.cpu().numpy(), ref, "s2o gain_tau 0")
    compare_lse(lse.cpu().numpy(), ref_lse)


def test_marginal_gain_is_deterministic_and_skips_bad_entries():
    pbsa = _need_gpu()
    N, Hq, Hkv, d, B, S = 2048, 2, 1, 128, 128, 512
    dev, _ = _inputs(N, Hq, Hkv, d, 0, 256, 42)
    NB = oracle.num_blocks(N, B)
    perm = pbsa.build_segment_permutation(dev["q"], dev["k"], B, S)
    count, idx = pbsa.estimate_block_mask(dev["q"], dev["k"], perm, B, S, 0.9, ranked=True)
    a = pbsa.s2o_attn_prefill(dev["q"], dev["k"], dev["v"], perm, count, idx, B, S, 0.03, return_kept=True)
    b = pbsa.s2o_attn_prefill(dev["q"], dev["k"], dev["v"], perm, count, idx, B, S, 0.03, return_kept=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    # an entry past I and a count past I + 1 are flagged and not read
    idx2, count2 = idx.clone(), count.clone()
    idx2[0, oracle.tri_offset(9) + 1] = 12
    count2[1, 2] = 7
    out, err = pbsa.s2o_attn_prefill(dev["q"], dev["k"], dev["v"], perm, count2, idx2, B, S, 0.03,
                                     return_lse=False, return_error=True)
    torch.cuda.synchronize()
    assert int(err.item()) & 1 and int(err.item()) & 4
    assert torch.isfinite(out).all()
    assert NB == 16


# S2O two-pass attention over the historical ranking: (name, N, Hq, Hkv, d, B, S, stripes, band,
# gain_tau, seed).  S = 128 and 192 exercise radix tiles shorter than a workgroup and a segment that
# is not a power of two; 8192 with S = 4096 the widest tiles.
TWO_PASS_CASES = [
    ("flat_b64_d128_gqa_2048", 2048, 4, 2, 128, 64, 256, 0, 0, 0.05, 51),
    ("band_b128_d64_ragged_4000", 4000, 4, 1, 64, 128, 512, 0, 256, 0.02, 52),
    ("stripes_b128_d128_ragged_3000", 3000, 2, 1, 128, 128, 512, 4, 256, 0.05, 53),
    ("flat_b64_d64_s128_ragged_1100", 1100, 2, 2, 64, 64, 128, 0, 64, 0.1, 54),
    ("s192_b64_d128_1536", 1536, 2, 1, 128, 64, 192, 0, 64, 0.05, 55),
    ("s4096_b128_d128_8192", 8192, 2, 1, 128, 128, 4096, 8, 512, 0.01, 56),
    ("one_segment_b128_700", 700, 2, 1, 128, 128, 1024, 0, 0, 0.05, 57),
]


@pytest.mark.parametrize("case", TWO_PASS_CASES, ids=[c[0] for c in TWO_PASS_CASES])
def test_two_pass_stagewise(case):
    pbsa = _need_gpu()
    name, N, Hq, Hkv, d, B, S, stripes, band, gain_tau, seed = case
    _log(f"[parity] two-pass {name}: N={N} Hq={Hq} Hkv={Hkv} d={d} B={B} S={S} gain_tau={gain_tau}")
    dev, host = _inputs(N, Hq, Hkv, d, stripes, band, seed)
    q, k, v = host["q"], host["k"], host["v"]
    NB = oracle.num_blocks(N, B)

    rank_t = pbsa.build_prefix_kv_ranking(dev["q"], dev["k"], B, S)
    torch.cuda.synchronize()
    pi_g = rank_t.cpu().numpy().astype(np.int64)
    pi_o, score_o = oracle.prefix_kv_ranking(q, k, S)
    ties = compare_prefix_rank(pi_g, pi_o, score_o, S)

    out_t, lse_t, kept_t, err_t = pbsa.s2o_prefix_attn_prefill(dev["q"], dev["k"], dev["v"], rank_t, B, S, gain_tau,
                                                               return_kept=True, return_error=True)
    torch.cuda.synchronize()
    assert int(err_t.item()) == 0
    kept = bitmap_to_kept(kept_t.cpu().numpy(), NB)
    cg, ig = two_pass_lists(Hq, N, B, S)
    ratios = oracle.s2o_prefix_gain_ratios(q, k, pi_g, B, S)
    rows, near = compare_s2o_stops(kept, cg, ig, ratios, gain_tau)
    out_o, lse_o = oracle.two_pass_attention_on(q, k, v, pi_g, kept, B, S)
    mx, mean = compare_out(out_t.cpu().numpy(), out_o, "two-pass")
    compare_lse(lse_t.cpu().numpy(), lse_o)
    frac = sum(len(x) for x in kept.values()) / float(Hq * NB * (NB + 1) // 2)
    _log(f"[parity] two-pass {name}: rank ties {ties}, rows {rows}, decided in band {near}, processed {frac:.3f}, "
         f"max abs {mx:.2e} mean abs {mean:.2e}")


@pytest.mark.parametrize("d,B,N,S", [(128, 128, 2048, 512), (64, 64, 1500, 256)])
def test_two_pass_zero_threshold_is_dense(d, B, N, S):
    pbsa = _need_gpu()
    Hq, Hkv = 4, 2
    dev, host = _inputs(N, Hq, Hkv, d, 8, 2 * B, 58)
    NB = oracle.num_blocks(N, B)
    rank = pbsa.build_prefix_kv_ranking(dev["q"], dev["k"], B, S)
    out, lse, kept = pbsa.s2o_prefix_attn_prefill(dev["q"], dev["k"], dev["v"], rank, B, S, 0.0, return_kept=True)
    torch.cuda.synchronize()
    assert all(lst == list(range(I + 1)) for (h, I), lst in bitmap_to_kept(kept.cpu().numpy(), NB).items())
    ref, ref_lse = oracle.dense_attention(host["q"], host["k"], host["v"])
    compare_out(out.cpu().numpy(), ref, "two-pass gain_tau 0")
    compare_lse(lse.cpu().numpy(), ref_lse)


def test_two_pass_is_deterministic_and_bounds_the_ranking():
    pbsa = _need_gpu()
    N, Hq, Hkv, d, B, S = 2048, 2, 1, 128, 128, 512
    dev, _ = _inputs(N, Hq, Hkv, d, 0, 256, 59)
    r1 = pbsa.build_prefix_kv_ranking(dev["q"], dev["k"], B, S)
    r2 = pbsa.build_prefix_kv_ranking(dev["q"], dev["k"], B, S)
    a = pbsa.s2o_prefix_attn_prefill(dev["q"], dev["k"], dev["v"], r1, B, S, 0.03, return_kept=True)
    b = pbsa.s2o_prefix_attn_prefill(dev["q"], dev["k"], dev["v"], r1, B, S, 0.03, return_kept=True)
    torch.cuda.synchronize()
    assert torch.equal(r1, r2)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    # an entry of segment 2's order that is not in its prefix (a key of segment 2 itself) is skipped
    bad = r1.clone()
    bad[0, oracle.prefix_offset(2, S) + 3] = 2 * S + 10
    out, err = pbsa.s2o_prefix_attn_prefill(dev["q"], dev["k"], dev["v"], bad, B, S, 0.0, return_lse=False,
                                            return_error=True)
    torch.cuda.synchronize()
    assert int(err.item()) & 2
    assert torch.isfinite(out).all()


# S2O query permutation in the two-pass path: (name, N, Hq, Hkv, d, B, S, stripes, band, gain_tau, seed)
QPERM_CASES = [
    ("flat_b64_d128_gqa_2048", 2048, 4, 2, 128, 64, 256, 0, 0, 0.05, 61),
    ("band_b128_d64_ragged_4000", 4000, 4, 1, 64, 128, 512, 0, 256, 0.02, 62),
    ("stripes_b128_d128_ragged_3000", 3000, 2, 1, 128, 128, 512, 4, 256, 0.05, 63),
    ("s192_b64_d64_ragged_1500", 1500, 2, 2, 64, 64, 192, 0, 64, 0.1, 64),
]


@pytest.mark.parametrize("case", QPERM_CASES, ids=[c[0] for c in QPERM_CASES])
def test_query_permuted_two_pass_stagewise(case):
    pbsa = _need_gpu()
    name, N, Hq, Hkv, d, B, S, stripes, band, gain_tau, seed = case
    _log(f"[parity] qperm {name}: N={N} Hq={Hq} Hkv={Hkv} d={d} B={B} S={S} gain_tau={gain_tau}")
    dev, host = _inputs(N, Hq, Hkv, d, stripes, band, seed)
    q, k, v = host["q"], host["k"], host["v"]
    NB = oracle.num_blocks(N, B)
    qperm_t = pbsa.build_query_permutation(dev["q"], dev["k"], B, S)
    rank_t = pbsa.build_prefix_kv_ranking(dev["q"], dev["k"], B, S)
    torch.cuda.synchronize()
    qp_g = qperm_t.cpu().numpy().astype(np.int64)
    qties = compare_perm(qp_g, oracle.query_permutation(q, k, S), oracle.query_guide_scores(q, k), S)
    pi_g = rank_t.cpu().numpy().astype(np.int64)
    out_t, lse_t, kept_t, err_t = pbsa.s2o_prefix_attn_prefill(dev["q"], dev["k"], dev["v"], rank_t, B, S, gain_tau,
                                                               qperm=qperm_t, return_kept=True, return_error=True)
    torch.cuda.synchronize()
    assert int(err_t.item()) == 0
    kept = bitmap_to_kept_square(kept_t.cpu().numpy(), NB)
    cg, ig = two_pass_lists(Hq, N, B, S, permuted_queries=True)
    ratios = oracle.s2o_prefix_gain_ratios(q, k, pi_g, B, S, qperm=qp_g)
    rows, near = compare_s2o_stops(kept, cg, ig, ratios, gain_tau, row_stride=NB)
    out_o, lse_o = oracle.two_pass_attention_on(q, k, v, pi_g, kept, B, S, qperm=qp_g)
    assert not np.isnan(out_o).any()
    mx, mean = compare_out(out_t.cpu().numpy(), out_o, "qperm two-pass")
    compare_lse(lse_t.cpu().numpy(), lse_o)
    _log(f"[parity] qperm {name}: query-order ties {qties}, rows {rows}, decided in band {near}, "
         f"max abs {mx:.2e} mean abs {mean:.2e}")


def test_query_permuted_two_pass_zero_threshold_is_dense_and_flags_bad_entries():
    pbsa = _need_gpu()
    N, Hq, Hkv, d, B, S = 1800, 4, 2, 128, 128, 512
    dev, host = _inputs(N, Hq, Hkv, d, 8, 256, 65)
    qperm = pbsa.build_query_permutation(dev["q"], dev["k"], B, S)
    rank = pbsa.build_prefix_kv_ranking(dev["q"], dev["k"], B, S)
    out, lse = pbsa.s2o_prefix_attn_prefill(dev["q"], dev["k"], dev["v"], rank, B, S, 0.0, qperm=qperm)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.dense_attention(host["q"], host["k"], host["v"])
    compare_out(out.cpu().numpy(), ref, "qperm gain_tau 0")
    compare_lse(lse.cpu().numpy(), ref_lse)
    # a query-order entry outside its segment is flagged and that query skipped
    bad = qperm.clone()
    bad[0, 700] = 100                           # segment 1 slot pointing into segment 0
    out2, err = pbsa.s2o_prefix_attn_prefill(dev["q"], dev["k"], dev["v"], rank, B, S, 0.0, qperm=bad,
                                             return_lse=False, return_error=True)
    torch.cuda.synchronize()
    assert int(err.item()) & 8
    assert torch.isfinite(out2[:, :100]).all()


# SampleAttention mask: (name, N, Hq, Hkv, d, B, stripes, band, cia_tau, n_trunks, rows_per_trunk, seed)
SAMPLE_CASES = [
    ("gqa_b128_d128_2048", 2048, 4, 2, 128, 128, 16, 256, 0.9, 4, 16, 71),
    ("ragged_b64_d64_1500", 1500, 2, 1, 64, 64, 8, 128, 0.6, 3, 8, 72),
    ("flat_b128_d64_ragged_3000", 3000, 4, 4, 64, 128, 0, 256, 0.95, 8, 4, 73),
    ("one_trunk_b64_d128_777", 777, 2, 2, 128, 64, 8, 64, 0.8, 1, 32, 74),
]


@pytest.mark.parametrize("case", SAMPLE_CASES, ids=[c[0] for c in SAMPLE_CASES])
def test_sample_attention_mask_and_attention(case):
    pbsa = _need_gpu()
    name, N, Hq, Hkv, d, B, stripes, band, tau, nt, rpt, seed = case
    _log(f"[parity] sample {name}: N={N} Hq={Hq} Hkv={Hkv} d={d} B={B} tau={tau} trunks={nt}x{rpt}")
    dev, host = _inputs(N, Hq, Hkv, d, stripes, band, seed)
    q, k, v = host["q"], host["k"], host["v"]
    count_t, idx_t, col_t, sl_t = pbsa.sample_attention_mask(dev["q"], dev["k"], B, tau, nt, rpt, return_masses=True)
    torch.cuda.synchronize()
    cg, ig = count_t.cpu().numpy(), idx_t.cpu().numpy()
    _, _, _, _, col_o, sl_o = oracle.sample_attention_mask(q, k, B, tau, nt, rpt)
    ties = compare_sample_mask(cg, ig, col_t.cpu().numpy(), sl_t.cpu().numpy(), col_o, sl_o, tau, B, True, False,
                               imp_rtol(q, k))
    out_t, lse_t = pbsa.block_sparse_attn_prefill(dev["q"], dev["k"], dev["v"], None, count_t, idx_t, B, 0)
    torch.cuda.synchronize()
    out_o, lse_o, _, _ = oracle.block_sparse_attention(q, k, v, None, cg, ig, B, None)
    mx, mean = compare_out(out_t.cpu().numpy(), out_o, "sample mask attention")
    compare_lse(lse_t.cpu().numpy(), lse_o)
    NB = oracle.num_blocks(N, B)
    _log(f"[parity] sample {name}: ties {ties}, density {cg.sum() / (Hq * NB * (NB + 1) / 2):.3f}, "
         f"max abs {mx:.2e} mean abs {mean:.2e}")


def test_sample_attention_mask_with_exact_ties():
    """Every key row equal: each sampled row weights its visible keys uniformly, so the column and
    slash masses are piecewise constant (exactly equal between consecutive sampled rows) and the
    cut falls inside runs of equal masses.  The kernel's kept patterns must be the oracle's cut of
    the GPU's own masses exactly (equal masses taken in index order)."""
    pbsa = _need_gpu()
    N, Hq, Hkv, d, B, tau, nt, rpt = 2048, 2, 1, 128, 128, 0.61803, 4, 8
    x = generate(N, Hq, Hkv, d, 0, 0, 83)
    row = bf16_round_bits(np.random.default_rng(84).standard_normal(d).astype(np.float32))
    kbits = x["k"].copy()
    kbits[:, :, :] = row
    qd = torch.from_numpy(x["q"].view(np.int16)).view(torch.bfloat16).cuda()
    kd = torch.from_numpy(kbits.view(np.int16)).view(torch.bfloat16).cuda()
    qh = bf16_bits_to_f32(x["q"]).astype(np.float64)
    kh = bf16_bits_to_f32(kbits).astype(np.float64)
    _log(f"[exact ties] sample mask N={N} Hq={Hq} tau={tau} trunks={nt}x{rpt}")
    count_t, idx_t, col_t, sl_t = pbsa.sample_attention_mask(qd, kd, B, tau, nt, rpt, return_masses=True)
    torch.cuda.synchronize()
    col_g, sl_g = col_t.cpu().numpy(), sl_t.cpu().numpy()
    tied = sum(N - len(np.unique(m[h])) for m in (col_g, sl_g) for h in range(Hq))
    _log(f"[exact ties] {tied} masses equal to another of their head and family on the GPU")
    assert tied > 0
    _, _, _, _, col_o, sl_o = oracle.sample_attention_mask(qh, kh, B, tau, nt, rpt)
    compare_sample_mask(count_t.cpu().numpy(), idx_t.cpu().numpy(), col_g, sl_g, col_o, sl_o, tau, B, True, False,
                        imp_rtol(qh, kh))


def test_sample_attention_full_target_is_dense():
    pbsa = _need_gpu()
    N, Hq, Hkv, d, B = 1024, 2, 1, 128, 128
    dev, host = _inputs(N, Hq, Hkv, d, 8, 128, 75)
    count, idx = pbsa.sample_attention_mask(dev["q"], dev["k"], B, 1.0, 4, 8, force_diag=False)
    torch.cuda.synchronize()
    assert (count.cpu().numpy() == np.arange(1, N // B + 1)[None, :]).all()


def test_estimators_are_deterministic():
    """The historical ranking, the query permutation and SampleAttention's mask give identical results
    on repeated calls (every sum runs in a fixed order)."""
    pbsa = _need_gpu()
    N, Hq, Hkv, d, B, S = 2048, 4, 2, 128, 128, 512
    dev, _ = _inputs(N, Hq, Hkv, d, 8, 256, 81)
    res = []
    for _ in range(2):
        r = pbsa.build_prefix_kv_ranking(dev["q"], dev["k"], B, S)
        qp = pbsa.build_query_permutation(dev["q"], dev["k"], B, S)
        c, i, col, sl = pbsa.sample_attention_mask(dev["q"], dev["k"], B, 0.8, 4, 16, return_masses=True)
        torch.cuda.synchronize()
        valid = torch.zeros_like(i, dtype=torch.bool)
        cnt = c.cpu().numpy()
        for h in range(Hq):
            for I in range(cnt.shape[1]):
                o = oracle.tri_offset(I)
                valid[h, o:o + int(cnt[h, I])] = True
        res.append([r.clone(), qp.clone(), c.clone(), i[valid].clone(), col.clone(), sl.clone()])
    for a, b in zip(*res):
        assert torch.equal(a, b)
