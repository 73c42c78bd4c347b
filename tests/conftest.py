import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


def small_inputs(N, Hq, Hkv, d, n_stripes=0, band=0, seed=0):
    """bf16-rounded stripe inputs of a small shape, widened to fp64 for the oracle."""
    from workloads import bf16_bits_to_f32, generate
    x = generate(N, Hq, Hkv, d, n_stripes, band, seed)
    return tuple(bf16_bits_to_f32(x[n]).astype(np.float64) for n in ("q", "k", "v"))


@pytest.fixture
def make_inputs():
    return small_inputs
