"""Schedule independence of the persistent attention kernel.

Each query row (h, I) is computed by one workgroup, tile by tile in the row's list order, so the
output must not depend on which workgroup takes a row, in which order rows are taken, or how many
workgroups there are.  These tests run the mask path and the dense path under several launch
options of pbsa_block_sparse_attn_prefill_ex (default order, rows taken from the back of the
deques, a grid capped to a handful of workgroups, both) and require out, lse and the kept-tile
bitmap to be bitwise equal; the first schedule is also checked against the oracle.
"""
import sys

import numpy as np
import pytest

import oracle
from parity import compare_lse, compare_out
from workloads import bf16_bits_to_f32, generate

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# (name, N, Hq, Hkv, d, B, S, stripes, band, tau, seed): head pairs per workgroup (even G) and
# one head per workgroup (odd G, three deques), ragged tails
CASES = [
    ("pairs_gqa_4000", 4000, 8, 2, 128, 128, 1024, 16, 256, 0.9, 31),
    ("single_heads_3kv_1500", 1500, 3, 3, 64, 64, 256, 8, 128, 0.85, 32),
]

SCHEDULES = [
    ("default", 0, False),
    ("claim_back", 0, True),
    ("grid_1", 1, False),
    ("grid_7_claim_back", 7, True),
    ("grid_3", 3, False),
]


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("path", ["mask", "dense"])
def test_outputs_do_not_depend_on_the_schedule(case, path):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_blocks_amd as pbsa
    name, N, Hq, Hkv, d, B, S, stripes, band, tau, seed = case
    _log(f"[schedule] {name} {path}: N={N} Hq={Hq} Hkv={Hkv} d={d} B={B} S={S}")
    x = generate(N, Hq, Hkv, d, stripes, band, seed)
    dev = {n: torch.from_numpy(x[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("q", "k", "v")}
    perm = count = idx = None
    if path == "mask":
        perm = pbsa.build_segment_permutation(dev["q"], dev["k"], B, S)
        count, idx = pbsa.estimate_block_mask(dev["q"], dev["k"], perm, B, S, tau)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    results = {}
    for sname, max_wg, back in SCHEDULES:
        for rep in range(2):  # the same schedule twice: run-to-run
            _log(f"[schedule]   {sname} rep {rep}")
            out, lse, kept, err = pbsa.block_sparse_attn_prefill(
                dev["q"], dev["k"], dev["v"], perm, count, idx, B, S, return_kept=True, return_error=True,
                workspace=ws, max_workgroups=max_wg, claim_back=back)
            torch.cuda.synchronize()
            assert int(err.item()) == 0
            got = (out.cpu().numpy().view(np.uint32), lse.cpu().numpy().view(np.uint32), kept.cpu().numpy())
            if not results:
                results["ref"] = got
                ref_name = sname
            else:
                for what, a, b in zip(("out", "lse", "kept"), got, results["ref"]):
                    nd = int((a != b).sum())
                    assert nd == 0, f"{sname} rep {rep}: {nd} {what} words differ from {ref_name}"
    # the first schedule against the oracle (the others equal it bitwise)
    host = {n: bf16_bits_to_f32(x[n]).astype(np.float64) for n in ("q", "k", "v")}
    if path == "mask":
        out_o, lse_o, _, _ = oracle.block_sparse_attention(host["q"], host["k"], host["v"], perm.cpu().numpy(),
                                                           count.cpu().numpy(), idx.cpu().numpy(), B, S)
    else:
        out_o, lse_o = oracle.dense_attention(host["q"], host["k"], host["v"])
    out_g = results["ref"][0].view(np.float32).astype(np.float64)
    lse_g = results["ref"][1].view(np.float32).astype(np.float64)
    compare_out(out_g, out_o)
    compare_lse(lse_g, lse_o)
