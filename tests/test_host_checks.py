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
    imp_rtol, and that the rounding is actually visible (the bound is not vacuous)."""
    from parity import IMP_ATOL, compare_importance, imp_rtol
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
    rtol = imp_rtol(q, k)
    assert 2.0 ** -24 < rtol < 2.0 ** -24 * 1.1  # the logit term is small beside the storage rounding
    worst = compare_importance(sim, imp_o, rtol)
    assert 1e-9 < worst <= rtol
    # an error just outside the bound is caught
    planted = imp_o.copy()
    j = int(np.argmax(imp_o[0]))
    planted[0, j] *= 1 + 2 * rtol
    with pytest.raises(AssertionError):
        compare_importance(planted, imp_o, rtol)
    assert IMP_ATOL < 1e-40


def _bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest even), returned in fp64."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def _fixed_digits(row: np.ndarray, E: int | None = None):
    """The 42-bit fixed-point form of a bf16 row and its six digits, written from the description
    of the importance logits: x = M 2^(e' - 134), V = trunc(M 2^(e' - E + 34)), +-V in two's
    complement = D_0 2^35 + sum_a D_a 2^(35 - 7a), E the row's largest e' or a larger exponent
    shared with other rows (a key chunk's).  Returns (E, digits [d][6])."""
    f, ex = np.frexp(np.abs(row))
    e = np.where(row == 0, 0, np.maximum(ex + 126, 0))
    ep = np.maximum(e, 1)
    M = np.abs(row) / np.ldexp(1.0, ep - 134)
    assert np.all(M == np.round(M)) and np.all(M <= 255)  # the row really is bf16
    E = int(ep.max()) if E is None else E
    assert E >= ep.max()
    digs = []
    for m, p, x in zip(M.astype(np.int64), ep, row):
        sh = 34 - (E - int(p))
        v = (int(m) << sh) if sh >= 0 else (int(m) >> -sh)
        v = -v if x < 0 else v
        dg = [v >> 35] + [(v >> (35 - 7 * a)) & 127 for a in range(1, 6)]
        assert -128 <= dg[0] <= 127 and sum(x_ << (35 - 7 * a) for a, x_ in enumerate(dg)) == v
        digs.append(dg)
    return E, np.array(digs, dtype=np.int64)


def test_importance_logit_digits_within_bound():
    """The importance logits are exact integer sums of digit products (levels a + b <= 5) scaled by
    2^(Eq + Ek - 301): model that on the CPU with exact integers and check every logit against the
    correctly rounded c q.k within the bound the parity tests use (parity.imp_logit_error), on rows
    with narrow and very wide exponent spreads, zeros, subnormals and large values; the level sums
    stay inside int32 as the kernel needs.  Planted slips (a dropped level, a wrong digit weight)
    break the bound."""
    import math
    from parity import imp_logit_error
    rng = np.random.default_rng(7)

    def model(qr, kr, c, drop_level=None, shift=7, ek=None):
        Eq, Dq = _fixed_digits(qr)
        Ek, Dk = _fixed_digits(kr, ek)
        A = [sum(int(Dq[:, a] @ Dk[:, L - a]) for a in range(L + 1)) if L != drop_level else 0 for L in range(6)]
        assert all(abs(x) < 2 ** 31 for x in A)
        c01, c23, c45 = A[0] * 2 ** shift + A[1], A[2] * 2 ** shift + A[3], A[4] * 2 ** shift + A[5]
        assert all(abs(x) < 2 ** 31 for x in (c01, c23, c45))
        t = (float(c01) * 16384.0 + float(c23)) * 16384.0 + float(c45)
        return t * math.ldexp(c, Eq - 150) * math.ldexp(1.0, Ek - 151)

    worst, caught5 = 0.0, 0
    for trial in range(160):
        d = (64, 128)[trial % 2]
        q, k = rng.standard_normal(d), rng.standard_normal(d)
        kind = trial % 5
        if kind == 1:  # exponents spread over 2^-60 .. 2^10: truncated elements on both sides
            q *= np.exp2(rng.integers(-60, 10, d))
            k *= np.exp2(rng.integers(-60, 10, d))
        elif kind == 2:  # zeros, bf16 subnormals, a large leading element
            q[rng.integers(0, d, 8)] = 0.0
            k[:4] = 3e-39
            q[0] = 1e20
        elif kind == 3:
            q, k = q * 40, k * 0.01
        elif kind == 4:  # every element at the row's top exponent
            q, k = np.sign(q) * (1 + np.abs(q) % 1), np.sign(k) * (1 + np.abs(k) % 1)
        q, k = _bf16_round(q), _bf16_round(k)
        c = 1.0 / math.sqrt(d)
        exact = c * math.fsum(q * k)
        bound = imp_logit_error(q[None, None], k[None, None], c) + 4 * 2.0 ** -53 * abs(exact)
        err = abs(model(q, k, c) - exact)
        assert err <= bound, (trial, err, bound)
        # the key row inside a chunk whose largest exponent is up to 2^12 above its own: the bound
        # over a key set holding that larger row still covers it
        ek = _fixed_digits(k)[0] + int(rng.integers(1, 13))
        big = np.zeros((2, d))
        big[0], big[1, 0] = k, np.ldexp(1.0, ek - 127)
        bound_c = imp_logit_error(q[None, None], big[None], c) + 4 * 2.0 ** -53 * abs(exact)
        assert abs(model(q, k, c, ek=ek) - exact) <= bound_c, (trial, ek)
        worst = max(worst, err / bound)
        if kind == 0:
            assert abs(model(q, k, c, drop_level=1) - exact) > bound  # a dropped level is caught
            assert abs(model(q, k, c, shift=6) - exact) > bound       # a wrong digit weight is caught
        elif kind == 1:  # the low levels matter once elements sit far below the row's largest
            caught5 += abs(model(q, k, c, drop_level=5) - exact) > bound
    assert worst > 1e-3  # the bound is not vacuous: the truncation shows in some rows
    assert caught5 >= 16  # of the 32 wide-spread pairs
