"""Parity on randomly drawn shapes: the checks of test_gpu_parity.py over cases generated from a
fixed seed, so the shapes vary widely (d, B, segment length, GQA ratio, ragged N, stripe and band
structure, thresholds) while every run draws the same cases.  Each case goes through the same tie
rules and bounds as the hand-picked ones (tests/parity.py)."""
import numpy as np
import pytest

import test_gpu_parity as P

pytestmark = pytest.mark.gpu


def _cases(seed=2026, n=32):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        d = int(rng.choice([64, 128]))
        B = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 3]))
        G = int(rng.choice([1, 2, 3, 4]))
        N = int(rng.integers(B + 1, 2600))
        S = B * int(rng.integers(1, 9))
        stripes = int(rng.choice([0, 4, 16]))
        band = int(rng.choice([0, 64, 256]))
        seed_c = int(rng.integers(1, 1 << 30))
        kind = ("stagewise", "two_pass", "marginal_gain", "query_permuted", "sample", "gate")[c % 6]
        if kind == "stagewise":
            args = (f"r{c}", N, Hkv * G, Hkv, d, B, S, stripes, band, float(rng.uniform(0.5, 0.99)), seed_c)
        elif kind in ("two_pass", "marginal_gain", "query_permuted"):
            args = (f"r{c}", N, Hkv * G, Hkv, d, B, S, stripes, band, float(rng.choice([0.0, 0.005, 0.02, 0.1])),
                    seed_c)
        elif kind == "sample":
            nt = int(rng.integers(1, 9))
            rpt = int(rng.integers(1, 33))
            while (nt - 1) * -(-N // nt) + rpt > N:  # every trunk must hold rpt positions
                nt = max(1, nt - 1)
            args = (f"r{c}", N, Hkv * G, Hkv, d, B, stripes, band, float(rng.uniform(0.5, 0.99)), nt, rpt, seed_c)
        else:
            args = (Hkv * G, Hkv, d, B, N)
        out.append((kind, args))
    return out


CASES = _cases()


@pytest.mark.parametrize("kind,args", CASES, ids=[f"{k}-{i}" for i, (k, _) in enumerate(CASES)])
def test_random_shape(kind, args):
    if kind == "stagewise":
        P.test_pipeline_stagewise(args)
    elif kind == "two_pass":
        P.test_two_pass_stagewise(args)
    elif kind == "marginal_gain":
        P.test_marginal_gain_stagewise(args)
    elif kind == "query_permuted":
        P.test_query_permuted_two_pass_stagewise(args)
    elif kind == "sample":
        P.test_sample_attention_mask_and_attention(args)
    else:
        P.test_early_stop_gate(*args)
