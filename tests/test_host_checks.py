"""Host-side checks that need no GPU: the binding's argument validation, and the fp32 error bound
that the early-stop parity tests use (checked against an fp32 evaluation of the same scores)."""
import math

import numpy as np
import pytest

import oracle
from parity import F32_U, compare_gate, fp32_sum_gamma, gate_error_bound

torch = pytest.importorskip("torch")


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def _qkv(N=256, Hq=4, Hkv=2, d=64):
    rng = np.random.default_rng(5)
    return (_bf16(rng.standard_normal((Hq, N, d))), _bf16(rng.standard_normal((Hkv, N, d))),
            _bf16(rng.standard_normal((Hkv, N, d))))


def test_attention_argument_checks():
    from block_sparse_attention_blocks_amd import _check_attn_args, num_blocks
    q, k, v = _qkv()
    Hq, N, d = q.shape
    B = 64
    NB = num_blocks(N, B)
    ok = dict(perm=torch.zeros((2, N), dtype=torch.int32), block_count=torch.zeros((Hq, NB), dtype=torch.int32),
              block_idx=torch.zeros((Hq, NB * (NB + 1) // 2), dtype=torch.int32),
              theta=torch.zeros((Hq, NB), dtype=torch.float32), out=torch.zeros((Hq, N, d), dtype=torch.float32),
              lse=torch.zeros((Hq, N), dtype=torch.float32))

    def run(**over):
        a = dict(ok)
        a.update(over)
        _check_attn_args(q, k, v, a["perm"], a["block_count"], a["block_idx"], B, a["theta"], a["out"], a["lse"],
                         require_gpu=False)

    run()  # the well-formed set passes
    run(perm=None, block_count=None, block_idx=None, theta=None, out=None, lse=None)
    bad = {
        "perm": torch.zeros((2, N), dtype=torch.int64),                    # int64 (argsort's default)
        "block_count": torch.zeros((Hq, NB), dtype=torch.int64),
        "block_idx": torch.zeros((Hq, NB * (NB + 1) // 2 - 1), dtype=torch.int32),  # undersized
        "theta": torch.zeros((Hq, NB), dtype=torch.float64),
        "out": torch.zeros((Hq, N - 1, d), dtype=torch.float32),          # undersized output
        "lse": torch.zeros((Hq, N), dtype=torch.float32)[:, ::1].t().contiguous().t(),  # not contiguous
    }
    for name, t in bad.items():
        with pytest.raises(ValueError):
            run(**{name: t})
    with pytest.raises(ValueError):  # count without idx
        run(block_idx=None)
    with pytest.raises(ValueError):  # out with a strided last dimension
        run(out=torch.zeros((Hq, N, 2 * d), dtype=torch.float32)[:, :, ::2])
    # k and v must match q in tokens and head_dim, and v must match k
    with pytest.raises(ValueError):
        _check_attn_args(q, k[:, :-8], v[:, :-8], None, None, None, B, require_gpu=False)
    with pytest.raises(ValueError):
        _check_attn_args(q, k, v[:, :, :32].contiguous(), None, None, None, B, require_gpu=False)
    with pytest.raises(ValueError):
        _check_attn_args(q[:3], k, v, None, None, None, B, require_gpu=False)  # 3 heads over 2 KV heads
    with pytest.raises(ValueError):  # not bf16
        _check_attn_args(q.float(), k, v, None, None, None, B, require_gpu=False)
    with pytest.raises(ValueError):  # CPU tensors are refused by the public path
        _check_attn_args(q, k, v, None, None, None, B)


def test_gamma_is_the_fp32_summation_bound():
    assert fp32_sum_gamma(1) == pytest.approx(F32_U)
    assert fp32_sum_gamma(128) == pytest.approx(128 * 2.0 ** -24, rel=1e-5)


def _fp32_tile_max(q, k, perm, B, S, h, I, G):
    """The gate's statistic evaluated the way a GPU does in the worst case this test can build: each
    dot product summed left to right in fp32 from exact products, the max taken, then one fp32
    multiply by the fp32-rounded scale."""
    N, d = q.shape[1], q.shape[2]
    c32 = np.float32(1.0 / math.sqrt(d))
    qi = oracle.block_range(I, B, N)
    res = []
    for J in range(I + 1):
        kj = oracle.key_rows_of_block(J, I, None if perm is None else perm[h // G], B, S, N)
        prods = (q[h, qi][:, None, :] * k[h // G, kj][None, :, :]).astype(np.float32)  # exact: bf16 x bf16
        acc = np.zeros(prods.shape[:2], dtype=np.float32)
        for t in range(d):
            acc = (acc + prods[:, :, t]).astype(np.float32)
        acc = np.where(kj[None, :] <= qi[:, None], acc, np.float32(-np.inf))
        res.append(float(np.float32(acc.max()) * c32))
    return np.array(res)


@pytest.mark.parametrize("use_perm", [False, True])
def test_gate_bound_covers_fp32_scores(make_inputs, use_perm):
    N, Hq, Hkv, d, B, S = 320, 2, 1, 128, 64, 128
    q, k, _ = make_inputs(N, Hq, Hkv, d, n_stripes=6, band=128, seed=17)
    perm = None
    if use_perm:
        perm = oracle.segment_permutation(oracle.key_importance(q, k, B), S)
    NB, G = oracle.num_blocks(N, B), Hq // Hkv
    rows = [(h, I) for h in range(Hq) for I in range(NB)]
    bound = gate_error_bound(q, k, perm, B, S, rows)
    worst = 0.0
    for h, I in rows:
        exact = np.array([(q[h, oracle.block_range(I, B, N)] @ k[h // G, oracle.key_rows_of_block(
            J, I, None if perm is None else perm[h // G], B, S, N)].T /
            math.sqrt(d))[np.where(oracle.key_rows_of_block(J, I, None if perm is None else perm[h // G], B, S, N)[
                None, :] <= oracle.block_range(I, B, N)[:, None])].max() for J in range(I + 1)])
        got = _fp32_tile_max(q, k, perm, B, S, h, I, G)
        lim = bound[(h, I)] + 4 * F32_U * np.abs(exact)
        assert (np.abs(got - exact) <= lim).all(), (h, I)
        worst = max(worst, float((np.abs(got - exact) / lim).max()))
    assert worst < 1.0


def test_compare_gate_catches_a_wrong_decision():
    bound = {(0, 3): np.full(4, 1e-5)}
    sel = {(0, 3): [0, 1, 2, 3]}
    exact = {(0, 3): np.array([1.0, 0.5, 0.20000001, 9.0])}
    theta = np.array([[0.0, 0.0, 0.0, 0.2]])
    # 0 and 1 clear of theta (kept), 2 inside the band (either way), 3 the diagonal
    assert compare_gate({(0, 3): [0, 1, 3]}, sel, exact, bound, theta) == (3, 1)
    assert compare_gate({(0, 3): [0, 1, 2, 3]}, sel, exact, bound, theta) == (3, 1)
    with pytest.raises(AssertionError):  # a tile clear of theta dropped
        compare_gate({(0, 3): [0, 3]}, sel, exact, bound, theta)
    with pytest.raises(AssertionError):  # the diagonal dropped
        compare_gate({(0, 3): [0, 1]}, sel, exact, bound, theta)


def test_importance_bound_covers_fp32_exponentials(make_inputs):
    """The importance pass keeps exp(s - chunk max) rounded to fp32 between its launches: evaluate
    the mean that way (64-key chunks, as the kernel does) and check it against the oracle within
    IMP_RTOL, and that the rounding is actually visible (the bound is not vacuous)."""
    from parity import IMP_ATOL, IMP_RTOL, compare_importance
    N, Hq, Hkv, d, B = 700, 4, 2, 64, 64
    q, k, _ = make_inputs(N, Hq, Hkv, d, n_stripes=6, band=64, seed=21)
    G, c = Hq // Hkv, 1.0 / math.sqrt(d)
    rows = np.arange(N - B, N)
    ok = np.arange(N)[None, :] <= rows[:, None]
    sim = np.zeros((Hkv, N))
    for g in range(Hkv):
        for h in range(g * G, (g + 1) * G):
            s = np.where(ok, c * (q[h, rows] @ k[g].T), -np.inf)
            lse = np.log(np.exp(s - s.max(1, keepdims=True)).sum(1)) + s.max(1)
            for c0 in range(0, N, 64):
                blk = s[:, c0:c0 + 64]
                m = blk.max(1, keepdims=True)
                mm = np.where(np.isfinite(m), m, 0.0)
                e32 = np.exp(blk - mm).astype(np.float32).astype(np.float64)
                w = np.where(np.isfinite(m), np.exp(m - lse[:, None]), 0.0)
                sim[g, c0:c0 + 64] += (e32 * w).sum(0)
        sim[g] /= G * len(rows)
    imp_o = oracle.key_importance(q, k, B)
    worst = compare_importance(sim, imp_o)
    assert 1e-9 < worst <= IMP_RTOL
    # an error just outside the bound is caught
    planted = imp_o.copy()
    j = int(np.argmax(imp_o[0]))
    planted[0, j] *= 1 + 2 * IMP_RTOL
    with pytest.raises(AssertionError):
        compare_importance(planted, imp_o)
    assert IMP_ATOL < 1e-40
