"""The attention entry point without a workspace (pbsa_block_sparse_attn_prefill_noalloc), called
through the C ABI, against pbsa_block_sparse_attn_prefill on the same inputs: two calls in a row,
the second on a smaller input, each bit for bit equal to the workspace entry point (they run the
same kernels) and within the tolerances of the oracle."""
import ctypes

import numpy as np
import pytest

import oracle
from parity import compare_lse, compare_out
from workloads import bf16_bits_to_f32, generate

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _case(N, Hq, Hkv, d, B, S, seed, tau):
    import block_sparse_attention_blocks_amd as pbsa
    from block_sparse_attention_blocks_amd import _lib
    x = generate(N, Hq, Hkv, d, 8, 256, seed)
    dev = {n: torch.from_numpy(x[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("q", "k", "v")}
    host = {n: bf16_bits_to_f32(x[n]).astype(np.float64) for n in ("q", "k", "v")}
    q, k, v = dev["q"], dev["k"], dev["v"]
    perm = pbsa.build_segment_permutation(q, k, B, S)
    count, idx = pbsa.estimate_block_mask(q, k, perm, B, S, tau)
    shape = pbsa.make_shape(q, k, B, S)
    outs = []
    lib = _lib.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    for noalloc in (False, True):
        out = torch.full((Hq, N, d), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((Hq, N), float("nan"), dtype=torch.float32, device="cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        if noalloc:
            st = lib.pbsa_block_sparse_attn_prefill_noalloc(ctypes.byref(shape), p(q), p(k), p(v), p(perm), p(count),
                                                            p(idx), None, p(out), p(lse), None, p(err), stream)
        else:
            ws = torch.empty(pbsa.workspace_size(shape, pbsa.PBSA_OP_ATTENTION) + 256, dtype=torch.uint8,
                             device="cuda")
            wsa = ws[(-ws.data_ptr()) % 256:]
            st = lib.pbsa_block_sparse_attn_prefill(ctypes.byref(shape), p(q), p(k), p(v), p(perm), p(count), p(idx),
                                                    None, p(out), p(lse), None, p(err), p(wsa), wsa.numel(), stream)
        assert st == 0, st
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        outs.append((out.cpu().numpy(), lse.cpu().numpy()))
    (o_ws, l_ws), (o_na, l_na) = outs
    assert np.array_equal(o_ws.view(np.int32), o_na.view(np.int32)), "out differs from the workspace entry point"
    assert np.array_equal(l_ws.view(np.int32), l_na.view(np.int32)), "lse differs from the workspace entry point"
    out_o, lse_o, _, _ = oracle.block_sparse_attention(host["q"], host["k"], host["v"], perm.cpu().numpy(),
                                                       count.cpu().numpy(), idx.cpu().numpy(), B, S)
    compare_out(o_na, out_o, f"no-alloc N={N}")
    compare_lse(l_na, lse_o)


def test_noalloc_attention_matches_workspace_entry_point():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("[no-alloc] N=2048 Hq=8 Hkv=2 d=128 B=128 S=512", flush=True)
    _case(2048, 8, 2, 128, 128, 512, 71, 0.9)
    print("[no-alloc] second call, smaller: N=700 Hq=4 Hkv=4 d=64 B=64 S=256", flush=True)
    _case(700, 4, 4, 64, 64, 256, 72, 0.95)
