"""Seeded stripe-structured attention inputs (input synthesis only).

The pages measure on real models and long-context suites; neither weights nor datasets are
available, so these synthetic tensors stand in for them.  They keep the layer shape of
Llama-3.1-8B attention (32 query heads, 8 KV heads, head dim 128) and plant the structure the
pages describe as typical of long-context attention maps: vertical "stripe" keys that attract
attention from many queries (S2O, "The Stripe Discovery"; PBS-Attn, "Problem Statement"
on scattered heavy hitters) and a local band near the diagonal.

Draw order for one ``generate`` call (NumPy ``Generator(PCG64(seed))``, fp32):
  1. Q [Hq][N][d], K [Hkv][N][d], V [Hkv][N][d] from N(0, 1);
  2. one direction u_g per KV head from N(0, I_d), normalised;
  3. stripe positions per KV head, ``rng.choice(N, n_stripes, replace=False)``;
  4. band chunk directions r_{g,c} (chunk = band_width / 2 tokens) from N(0, I_d), normalised.
Then q_{h,t} += sqrt(d) * u_{g(h)}; k_{g,t} += 4 * sqrt(d) * u_g for every stripe t; and, when
the band is on, k_{g,t} += a * r_{g,c(t)} and q_{h,t} += a * (r_{g,c(t)} + r_{g,c(t)-1}) with
a^2 = sqrt(d) * ln 2, so that a query's logit against a key 0..band_width-1 tokens back gains
ln 2 (attention weight x2).  Finally every value is rounded to bf16 (round to nearest even).
g(h) = h // (Hq / Hkv).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = bits + np.uint32(0x7FFF) + lsb
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to the fp32 values they encode (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class Workload:
    """One named input shape plus the method settings it is measured with."""

    name: str
    seq_len: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    segment_size: Optional[int]      # None: no key permutation
    n_stripes: int                   # planted stripe keys per KV head
    band_width: int                  # 0: no local band
    mass_tau: float                  # cumulative pooled-mass target of the block mask
    force_diag: bool = True
    force_first: bool = True
    seed: int = 0
    calib_seed: Optional[int] = None  # early-stop threshold calibration draw
    calib_keep: int = 0               # tiles kept per query block by the calibrated thresholds
    taus: Tuple[float, ...] = field(default_factory=tuple)

    @property
    def num_blocks(self) -> int:
        return -(-self.seq_len // self.block_size)

    @property
    def dense_causal_flop(self) -> float:
        """2 * N^2 * d * Hq: the FLOP of causal attention counted as a dense product would (QK^T + PV over the lower triangle)."""
        return 2.0 * self.seq_len * self.seq_len * self.head_dim * self.num_q_heads


WORKLOADS = {
    # Single head, seq 1024, d 64, block 64, segment 256; fp32 N(0,1) rounded to bf16; 8 stripes.
    "single_head_1k": Workload("single_head_1k", 1024, 1, 1, 64, 64, 256, 8, 0, 0.9, seed=1001),
    # Llama-3.1-8B-shaped layer at 32K: 32q/8kv, d 128, block 128, segment 2048, 64 stripes/head, band 512.
    "llama8b_32k": Workload("llama8b_32k", 32768, 32, 8, 128, 128, 2048, 64, 512, 0.9, seed=1002),
    # Same layer at 128K, 0.02% stripe keys (26 per head), segment 4096.
    "llama8b_128k": Workload("llama8b_128k", 131072, 32, 8, 128, 128, 4096, 26, 512, 0.9, seed=1003),
    # Density sweep at 64K: mass target in {0.8, 0.9, 0.95, 0.99}, permutation on and off.
    "llama8b_64k_sweep": Workload("llama8b_64k_sweep", 65536, 32, 8, 128, 128, 4096, 64, 512, 0.9,
                                  seed=1004, taus=(0.8, 0.9, 0.95, 0.99)),
    # Tile-max early stop at 64K: dense causal tiles, thresholds calibrated on a second draw
    # to keep the top 64 KV blocks per query block; only the diagonal is forced.
    "llama8b_64k_earlystop": Workload("llama8b_64k_earlystop", 65536, 32, 8, 128, 128, None, 64, 512, 1.0,
                                      force_diag=True, force_first=False, seed=1005,
                                      calib_seed=2005, calib_keep=64),
}


def generate(seq_len: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
             n_stripes: int, band_width: int, seed: int):
    """Draw one stripe-structured input; return bf16 bit patterns and the planted positions.

    Returns a dict with ``q`` [Hq][N][d], ``k`` and ``v`` [Hkv][N][d] as uint16 bf16 bits,
    and ``stripes`` [Hkv][n_stripes] (sorted positions of the planted keys).
    """
    N, Hq, Hkv, d = seq_len, num_q_heads, num_kv_heads, head_dim
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError("num_q_heads must be a positive multiple of num_kv_heads")
    G = Hq // Hkv
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((Hq, N, d), dtype=np.float32)
    k = rng.standard_normal((Hkv, N, d), dtype=np.float32)
    v = rng.standard_normal((Hkv, N, d), dtype=np.float32)
    u = rng.standard_normal((Hkv, d))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    n_s = min(n_stripes, N)
    stripes = np.stack([np.sort(rng.choice(N, n_s, replace=False)) for _ in range(Hkv)]) \
        if n_s > 0 else np.zeros((Hkv, 0), np.int64)
    chunk = band_width // 2 if band_width > 0 else 0
    if chunk > 0:
        n_chunks = -(-N // chunk)
        r = rng.standard_normal((Hkv, n_chunks, d))
        r /= np.linalg.norm(r, axis=2, keepdims=True)

    sd = math.sqrt(d)
    for g in range(Hkv):
        shift = (sd * u[g]).astype(np.float32)
        for h in range(g * G, (g + 1) * G):
            q[h] += shift
        if n_s:
            k[g, stripes[g]] += (4.0 * sd * u[g]).astype(np.float32)
        if chunk > 0:
            a = math.sqrt(sd * math.log(2.0))
            c_of_t = np.arange(N) // chunk
            rk = (a * r[g]).astype(np.float32)                      # [n_chunks][d]
            k[g] += rk[c_of_t]
            prev = np.concatenate([np.zeros((1, d), np.float32), rk[:-1]], axis=0)
            qband = rk[c_of_t] + prev[c_of_t]
            for h in range(g * G, (g + 1) * G):
                q[h] += qband
    out = {
        "q": bf16_round_bits(q),
        "k": bf16_round_bits(k),
        "v": bf16_round_bits(v),
        "stripes": stripes,
    }
    return out


def generate_for(w: Workload, seed: Optional[int] = None, seq_len: Optional[int] = None):
    """``generate`` with a workload's shape and recipe (optionally another seed or length)."""
    return generate(seq_len or w.seq_len, w.num_q_heads, w.num_kv_heads, w.head_dim,
                    w.n_stripes, w.band_width, w.seed if seed is None else seed)
