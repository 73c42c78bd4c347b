"""Host-side checks of the C ABI: exported symbols and argument validation (no GPU work).

Every call here is rejected (or is an N = 0 no-op) before the library touches the GPU.
"""
import ctypes
import os
import re

import pytest

from block_sparse_attention_blocks_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pbsa.h")

FAKE = ctypes.c_void_p(0x10000)  # 16-byte aligned, never dereferenced: every call below fails validation


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pbsa_[a-z_]+)\s*\(", text)))


def shape(N=1024, Hq=4, Hkv=2, d=128, B=128, S=512, scale=0.0):
    s = _lib.PbsaShape()
    s.seq_len, s.num_q_heads, s.num_kv_heads, s.head_dim = N, Hq, Hkv, d
    s.block_size, s.segment_size, s.softmax_scale = B, S, scale
    return s


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) >= {"pbsa_build_segment_permutation", "pbsa_estimate_block_mask",
                          "pbsa_block_sparse_attn_prefill", "pbsa_tile_max", "pbsa_calibrate_thresholds",
                          "pbsa_workspace_size", "pbsa_status_string", "pbsa_version"}
    lib = _lib.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert lib.pbsa_version() >= 100


def test_status_strings():
    for st in range(5):
        assert _lib.status_string(st)
    assert _lib.status_string(99) == "unknown status"


def test_shape_struct_layout_matches_header():
    # 6 int32 + float (28 bytes) padded to 32, then 6 int64
    assert ctypes.sizeof(_lib.PbsaShape) == 32 + 6 * 8
    assert _lib.PbsaShape.q_stride_head.offset == 32


def ws_size(s, op):
    return _lib.lib().pbsa_workspace_size(ctypes.byref(s), op)


def test_workspace_sizes_monotone_in_n():
    for op in (_lib.PBSA_OP_PERMUTATION, _lib.PBSA_OP_MASK, _lib.PBSA_OP_ATTENTION):
        prev = 0
        for N in (0, 1, 127, 128, 129, 1000, 4096, 32768, 131072):
            n = ws_size(shape(N=N), op)
            assert n != _lib.SIZE_MAX
            assert n >= prev
            prev = n
    assert ws_size(shape(), 7) == _lib.SIZE_MAX


@pytest.mark.parametrize("kw,expect", [
    (dict(d=96), _lib.PBSA_ERR_UNSUPPORTED),
    (dict(B=32), _lib.PBSA_ERR_UNSUPPORTED),
    (dict(S=16384), _lib.PBSA_ERR_UNSUPPORTED),
    (dict(N=128 * 2049), _lib.PBSA_ERR_UNSUPPORTED),
    (dict(S=192), _lib.PBSA_ERR_INVALID_ARG),        # not a multiple of B
    (dict(Hq=6, Hkv=4), _lib.PBSA_ERR_INVALID_ARG),  # Hq % Hkv
    (dict(N=-1), _lib.PBSA_ERR_INVALID_ARG),
    (dict(Hkv=0), _lib.PBSA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), _lib.PBSA_ERR_INVALID_ARG),
])
def test_shape_validation(kw, expect):
    s = shape(**kw)
    l = _lib.lib()
    assert ws_size(s, 0) == _lib.SIZE_MAX
    assert l.pbsa_build_segment_permutation(ctypes.byref(s), FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None) == expect
    assert l.pbsa_estimate_block_mask(ctypes.byref(s), FAKE, FAKE, None, 0.9, 3, FAKE, FAKE, None, FAKE,
                                      1 << 40, None) == expect
    assert l.pbsa_block_sparse_attn_prefill(ctypes.byref(s), FAKE, FAKE, FAKE, None, None, None, None, FAKE,
                                            None, None, None, None, 0, None) == expect
    assert l.pbsa_tile_max(ctypes.byref(s), FAKE, FAKE, None, FAKE, None) == expect


def test_null_shape_and_pointers():
    l = _lib.lib()
    E = _lib.PBSA_ERR_INVALID_ARG
    assert l.pbsa_build_segment_permutation(None, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None) == E
    s = shape()
    assert l.pbsa_build_segment_permutation(ctypes.byref(s), None, FAKE, FAKE, None, FAKE, 1 << 40, None) == E
    assert l.pbsa_build_segment_permutation(ctypes.byref(s), FAKE, FAKE, None, None, FAKE, 1 << 40, None) == E
    assert l.pbsa_estimate_block_mask(ctypes.byref(s), FAKE, FAKE, None, 0.9, 3, None, FAKE, None, FAKE,
                                      1 << 40, None) == E
    assert l.pbsa_block_sparse_attn_prefill(ctypes.byref(s), FAKE, FAKE, None, None, None, None, None, FAKE,
                                            None, None, None, None, 0, None) == E
    # count without idx
    assert l.pbsa_block_sparse_attn_prefill(ctypes.byref(s), FAKE, FAKE, FAKE, None, FAKE, None, None, FAKE,
                                            None, None, None, None, 0, None) == E
    # misaligned tensor
    bad = ctypes.c_void_p(0x10002)
    assert l.pbsa_block_sparse_attn_prefill(ctypes.byref(s), bad, FAKE, FAKE, None, None, None, None, FAKE,
                                            None, None, None, None, 0, None) == E
    assert l.pbsa_tile_max(ctypes.byref(s), FAKE, FAKE, None, None, None) == E
    assert l.pbsa_calibrate_thresholds(ctypes.byref(s), None, 64, FAKE, None) == E
    assert l.pbsa_calibrate_thresholds(ctypes.byref(s), FAKE, 64, None, None) == E
    assert l.pbsa_calibrate_thresholds(ctypes.byref(s), FAKE, 0, FAKE, None) == E


def test_permutation_needs_segments_and_mask_needs_valid_tau_and_flags():
    l = _lib.lib()
    E = _lib.PBSA_ERR_INVALID_ARG
    s0 = shape(S=0)
    assert l.pbsa_build_segment_permutation(ctypes.byref(s0), FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None) == E
    assert l.pbsa_estimate_block_mask(ctypes.byref(s0), FAKE, FAKE, FAKE, 0.9, 3, FAKE, FAKE, None, FAKE,
                                      1 << 40, None) == E
    s = shape()
    for tau in (0.0, -0.5, 1.0000001, float("nan")):
        assert l.pbsa_estimate_block_mask(ctypes.byref(s), FAKE, FAKE, None, tau, 3, FAKE, FAKE, None, FAKE,
                                          1 << 40, None) == E
    assert l.pbsa_estimate_block_mask(ctypes.byref(s), FAKE, FAKE, None, 0.9, 8, FAKE, FAKE, None, FAKE,
                                      1 << 40, None) == E
    # the ranked order (flag 4) needs segments
    assert l.pbsa_estimate_block_mask(ctypes.byref(s0), FAKE, FAKE, None, 0.9, _lib.PBSA_MASK_RANKED, FAKE, FAKE,
                                      None, FAKE, 1 << 40, None) == E
    # and writes no probabilities
    assert l.pbsa_estimate_block_mask(ctypes.byref(s), FAKE, FAKE, FAKE, 0.9, _lib.PBSA_MASK_RANKED, FAKE, FAKE,
                                      FAKE, FAKE, 1 << 40, None) == E


def test_marginal_gain_entry_validates_before_launch():
    l = _lib.lib()
    E = _lib.PBSA_ERR_INVALID_ARG
    s = shape()
    ws = ctypes.c_void_p(0x10000)
    args = lambda sh, cnt, idx, tau: (ctypes.byref(sh), FAKE, FAKE, FAKE, None, cnt, idx, tau, FAKE, None, None,
                                      None, ws, 1 << 20, None)
    assert l.pbsa_s2o_attn_prefill(*args(s, None, FAKE, 0.01)) == E        # no mask
    assert l.pbsa_s2o_attn_prefill(*args(s, FAKE, None, 0.01)) == E
    assert l.pbsa_s2o_attn_prefill(*args(s, FAKE, FAKE, -0.5)) == E        # threshold < 0
    assert l.pbsa_s2o_attn_prefill(*args(s, FAKE, FAKE, float("nan"))) == E
    assert l.pbsa_s2o_attn_prefill(*args(s, FAKE, FAKE, float("inf"))) == E
    assert l.pbsa_s2o_attn_prefill(*args(shape(S=0), FAKE, FAKE, 0.01)) == E  # needs segments
    assert l.pbsa_s2o_attn_prefill(ctypes.byref(s), FAKE, FAKE, FAKE, None, FAKE, FAKE, 0.01, FAKE, None, None,
                                   None, None, 0, None) == _lib.PBSA_ERR_WORKSPACE
    s0 = shape(N=0)
    assert l.pbsa_s2o_attn_prefill(*args(s0, FAKE, FAKE, 0.01)) == 0


def test_workspace_checks():
    l = _lib.lib()
    W = _lib.PBSA_ERR_WORKSPACE
    s = shape()
    need = ws_size(s, _lib.PBSA_OP_PERMUTATION)
    assert need > 0
    assert l.pbsa_build_segment_permutation(ctypes.byref(s), FAKE, FAKE, FAKE, None, None, need, None) == W
    assert l.pbsa_build_segment_permutation(ctypes.byref(s), FAKE, FAKE, FAKE, None, FAKE, need - 1, None) == W
    assert l.pbsa_build_segment_permutation(ctypes.byref(s), FAKE, FAKE, FAKE, None,
                                            ctypes.c_void_p(0x10010), need, None) == W  # not 256-aligned
    # attention: the work deques
    needa = ws_size(s, _lib.PBSA_OP_ATTENTION)
    assert needa > 0
    assert l.pbsa_block_sparse_attn_prefill(ctypes.byref(s), FAKE, FAKE, FAKE, None, None, None, None, FAKE,
                                            None, None, None, None, 0, None) == W
    assert l.pbsa_block_sparse_attn_prefill(ctypes.byref(s), FAKE, FAKE, FAKE, None, None, None, None, FAKE,
                                            None, None, None, FAKE, needa - 1, None) == W
    assert l.pbsa_block_sparse_attn_prefill(ctypes.byref(s), FAKE, FAKE, FAKE, None, None, None, None, FAKE,
                                            None, None, None, ctypes.c_void_p(0x10010), needa, None) == W
    needm = ws_size(s, _lib.PBSA_OP_MASK)
    assert l.pbsa_estimate_block_mask(ctypes.byref(s), FAKE, FAKE, None, 0.9, 3, FAKE, FAKE, None, FAKE,
                                      needm - 8, None) == W


def test_stride_validation():
    l = _lib.lib()
    s = shape()
    s.q_stride_head, s.q_stride_token = 1024 * 128, 100  # token stride < d
    assert l.pbsa_tile_max(ctypes.byref(s), FAKE, FAKE, None, FAKE, None) == _lib.PBSA_ERR_INVALID_ARG
    s.q_stride_token = 132  # not a multiple of 8
    assert l.pbsa_tile_max(ctypes.byref(s), FAKE, FAKE, None, FAKE, None) == _lib.PBSA_ERR_INVALID_ARG


def test_empty_sequence_is_a_no_op():
    l = _lib.lib()
    s = shape(N=0)
    assert l.pbsa_build_segment_permutation(ctypes.byref(s), FAKE, FAKE, FAKE, None, FAKE, 1 << 20, None) == 0
    assert l.pbsa_estimate_block_mask(ctypes.byref(s), FAKE, FAKE, None, 0.9, 3, FAKE, FAKE, None, FAKE,
                                      1 << 20, None) == 0
    assert l.pbsa_block_sparse_attn_prefill(ctypes.byref(s), FAKE, FAKE, FAKE, None, None, None, None, FAKE,
                                            None, None, None, None, 0, None) == 0
    assert l.pbsa_tile_max(ctypes.byref(s), FAKE, FAKE, None, FAKE, None) == 0
    assert l.pbsa_calibrate_thresholds(ctypes.byref(s), FAKE, 4, FAKE, None) == 0


def test_prefix_rank_length_and_workspace():
    l = _lib.lib()
    assert l.pbsa_prefix_rank_length(ctypes.byref(shape(N=1024, S=512))) == 512          # 2 segments
    assert l.pbsa_prefix_rank_length(ctypes.byref(shape(N=2000, S=512))) == 512 * 4 * 3 // 2
    assert l.pbsa_prefix_rank_length(ctypes.byref(shape(N=512, S=512))) == 0             # one segment
    assert l.pbsa_prefix_rank_length(ctypes.byref(shape(N=0))) == 0
    assert l.pbsa_prefix_rank_length(ctypes.byref(shape(S=0))) == -1                     # segments off
    assert l.pbsa_prefix_rank_length(ctypes.byref(shape(N=64 * 300, B=64, S=64))) == -1  # > 256 segments
    assert ws_size(shape(S=0), _lib.PBSA_OP_PREFIX_RANK) == _lib.SIZE_MAX
    prev = 0
    for n in (512, 1024, 2048, 4096, 8192):
        w = ws_size(shape(N=n, S=512), _lib.PBSA_OP_PREFIX_RANK)
        assert w != _lib.SIZE_MAX and w >= prev
        prev = w


def test_prefix_ranking_and_two_pass_entry_validate_before_launch():
    l = _lib.lib()
    E, W, U = _lib.PBSA_ERR_INVALID_ARG, _lib.PBSA_ERR_WORKSPACE, _lib.PBSA_ERR_UNSUPPORTED
    s = shape(N=2048, S=512)
    ws = ctypes.c_void_p(0x10000)
    big = 1 << 40
    rank = l.pbsa_build_prefix_kv_ranking
    assert rank(ctypes.byref(shape(S=0)), FAKE, FAKE, FAKE, ws, big, None) == E
    assert rank(ctypes.byref(s), None, FAKE, FAKE, ws, big, None) == E
    assert rank(ctypes.byref(s), FAKE, FAKE, None, ws, big, None) == E          # output missing
    assert rank(ctypes.byref(s), FAKE, FAKE, FAKE, None, 0, None) == W          # workspace missing
    assert rank(ctypes.byref(shape(N=64 * 300, B=64, S=64)), FAKE, FAKE, FAKE, ws, big, None) == U
    assert rank(ctypes.byref(shape(N=0)), FAKE, FAKE, None, None, 0, None) == 0       # nothing to rank
    assert rank(ctypes.byref(shape(N=400, S=512)), FAKE, FAKE, None, None, 0, None) == 0
    att = l.pbsa_s2o_prefix_attn_prefill
    args = lambda sh, kvr, tau, w=ws: (ctypes.byref(sh), FAKE, FAKE, FAKE, kvr, None, tau, FAKE, None, None, None,
                                       w, big if w else 0, None)
    assert att(*args(s, FAKE, -1.0)) == E
    assert att(*args(s, FAKE, float("nan"))) == E
    assert att(*args(s, FAKE, float("inf"))) == E
    assert att(*args(shape(S=0), FAKE, 0.01)) == E
    assert att(*args(s, None, 0.01)) == E                                       # ranking missing
    assert att(*args(s, FAKE, 0.01, None)) == W
    assert att(*args(shape(N=64 * 300, B=64, S=64), FAKE, 0.01)) == U
    assert att(*args(shape(N=0), None, 0.01)) == 0


def test_query_permutation_entry_validates_before_launch():
    l = _lib.lib()
    E, W = _lib.PBSA_ERR_INVALID_ARG, _lib.PBSA_ERR_WORKSPACE
    s = shape(N=2048, S=512)
    ws = ctypes.c_void_p(0x10000)
    big = 1 << 40
    qp = l.pbsa_build_query_permutation
    assert ws_size(shape(S=0), _lib.PBSA_OP_QUERY_PERM) == _lib.SIZE_MAX
    assert ws_size(shape(N=0), _lib.PBSA_OP_QUERY_PERM) == 0
    assert ws_size(s, _lib.PBSA_OP_QUERY_PERM) >= 8 * 2 * 2048      # fp64 scores at least
    assert qp(ctypes.byref(shape(S=0)), FAKE, FAKE, FAKE, ws, big, None) == E
    assert qp(ctypes.byref(s), FAKE, FAKE, None, ws, big, None) == E
    assert qp(ctypes.byref(s), None, FAKE, FAKE, ws, big, None) == E
    assert qp(ctypes.byref(s), FAKE, FAKE, FAKE, None, 0, None) == W
    assert qp(ctypes.byref(shape(N=0)), FAKE, FAKE, FAKE, None, 0, None) == 0


def test_sample_attention_entry_validates_before_launch():
    l = _lib.lib()
    E, W = _lib.PBSA_ERR_INVALID_ARG, _lib.PBSA_ERR_WORKSPACE
    s = shape(N=1000, S=0)
    ws = ctypes.c_void_p(0x10000)
    big = 1 << 40
    size = l.pbsa_sample_mask_workspace_size
    assert size(ctypes.byref(s), 4, 8) not in (0, _lib.SIZE_MAX)
    assert size(ctypes.byref(s), 0, 8) == _lib.SIZE_MAX
    assert size(ctypes.byref(s), 4, 0) == _lib.SIZE_MAX
    assert size(ctypes.byref(s), 3, 334) == _lib.SIZE_MAX      # chunks of 334: the last holds 332
    assert size(ctypes.byref(s), 3, 332) != _lib.SIZE_MAX
    assert size(ctypes.byref(shape(N=0)), 4, 8) == 0
    m = l.pbsa_sample_attention_mask
    args = lambda sh, tau, nt, rpt, fl=1, w=ws: (ctypes.byref(sh), FAKE, FAKE, tau, nt, rpt, fl, FAKE, FAKE, None, None,
                                                 w, big if w else 0, None)
    assert m(*args(s, 0.0, 4, 8)) == E
    assert m(*args(s, 1.5, 4, 8)) == E
    assert m(*args(s, float("nan"), 4, 8)) == E
    assert m(*args(s, 0.9, 0, 8)) == E
    assert m(*args(s, 0.9, 3, 334)) == E
    assert m(*args(s, 0.9, 4, 8, fl=4)) == E                   # ranked flag not accepted here
    assert m(*args(s, 0.9, 4, 8, w=None)) == W
    assert m(*args(shape(N=0), 0.9, 4, 8, w=None)) == 0
    assert m(ctypes.byref(s), FAKE, FAKE, 0.9, 4, 8, 1, None, FAKE, None, None, ws, big, None) == E


def test_noalloc_attention_validates_before_touching_the_device():
    l = _lib.lib()
    E = _lib.PBSA_ERR_INVALID_ARG
    s = shape()
    f = l.pbsa_block_sparse_attn_prefill_noalloc
    assert f(None, FAKE, FAKE, FAKE, None, None, None, None, FAKE, None, None, None, None) == E
    assert f(ctypes.byref(s), FAKE, FAKE, None, None, None, None, None, FAKE, None, None, None, None) == E
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, None, FAKE, None, None, FAKE, None, None, None, None) == E
    bad = ctypes.c_void_p(0x10002)
    assert f(ctypes.byref(s), bad, FAKE, FAKE, None, None, None, None, FAKE, None, None, None, None) == E
    s0 = shape(N=0)
    assert f(ctypes.byref(s0), FAKE, FAKE, FAKE, None, None, None, None, FAKE, None, None, None, None) == 0
    s.head_dim = 96
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, None, None, None, None, FAKE, None, None, None,
             None) == _lib.PBSA_ERR_UNSUPPORTED


def test_launch_options_entry_validates_before_launch():
    l = _lib.lib()
    E = _lib.PBSA_ERR_INVALID_ARG
    s = shape()
    f = l.pbsa_block_sparse_attn_prefill_ex
    ws = ctypes.c_void_p(0x100000)
    assert ctypes.sizeof(_lib.PbsaLaunchOptions) == 8
    for bad in (_lib.PbsaLaunchOptions(-1, 0), _lib.PbsaLaunchOptions(0, 2), _lib.PbsaLaunchOptions(4, 0x80000000)):
        assert f(ctypes.byref(s), FAKE, FAKE, FAKE, None, None, None, None, FAKE, None, None, None, ws, 256,
                 ctypes.byref(bad), None) == E
    ok = _lib.PbsaLaunchOptions(16, _lib.PBSA_LAUNCH_CLAIM_BACK)
    # the other arguments are checked as in pbsa_block_sparse_attn_prefill
    assert f(ctypes.byref(s), FAKE, FAKE, None, None, None, None, None, FAKE, None, None, None, ws, 256,
             ctypes.byref(ok), None) == E
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, None, None, None, None, FAKE, None, None, None, ws, 8,
             ctypes.byref(ok), None) == _lib.PBSA_ERR_WORKSPACE
    s0 = shape(N=0)
    assert f(ctypes.byref(s0), FAKE, FAKE, FAKE, None, None, None, None, FAKE, None, None, None, None, 0,
             None, None) == 0
    assert f(ctypes.byref(s0), FAKE, FAKE, FAKE, None, None, None, None, FAKE, None, None, None, None, 0,
             ctypes.byref(ok), None) == 0


def test_bf16_output_entry_validates_before_launch():
    """pbsa_block_sparse_attn_prefill_bf16out checks its arguments as pbsa_block_sparse_attn_prefill
    does (the output pointer included), before any launch."""
    l = _lib.lib()
    E = _lib.PBSA_ERR_INVALID_ARG
    s = shape()
    f = l.pbsa_block_sparse_attn_prefill_bf16out
    ws = ctypes.c_void_p(0x100000)
    assert f(None, FAKE, FAKE, FAKE, None, None, None, None, FAKE, None, None, None, ws, 256, None) == E
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, None, None, None, None, None, None, None, None, ws, 256, None) == E
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, None, FAKE, None, None, FAKE, None, None, None, ws, 256, None) == E
    bad = ctypes.c_void_p(0x10002)  # misaligned output
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, None, None, None, None, bad, None, None, None, ws, 256, None) == E
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, None, None, None, None, FAKE, None, None, None, ws, 8,
             None) == _lib.PBSA_ERR_WORKSPACE
    s0 = shape(N=0)
    assert f(ctypes.byref(s0), FAKE, FAKE, FAKE, None, None, None, None, FAKE, None, None, None, None, 0, None) == 0
    s.head_dim = 96
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, None, None, None, None, FAKE, None, None, None, ws, 256,
             None) == _lib.PBSA_ERR_UNSUPPORTED


def test_stride_extents_are_bounded_without_overflow():
    l = _lib.lib()
    U = _lib.PBSA_ERR_UNSUPPORTED
    big8 = (1 << 63) - 8
    for sh, st in ((big8, big8), (big8, 128), (1 << 62, 128), (1024 * 128, big8), (1024 * 128, 1 << 21),
                   (1 << 47, 128)):
        for which in ("q", "kv"):
            s = shape()
            setattr(s, f"{which}_stride_head", sh)
            setattr(s, f"{which}_stride_token", st)
            assert l.pbsa_tile_max(ctypes.byref(s), FAKE, FAKE, None, FAKE, None) == U, (which, sh, st)
