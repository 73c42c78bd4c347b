"""Permuted block-sparse attention prefill for MI355X (gfx950): thin torch binding of libpbsa.

Each function marshals torch device tensors into the C ABI of ``include/pbsa.h`` and enqueues the
work on torch's current HIP stream.  Every step of the computation runs in the library's HIP
kernels; torch only provides device memory and the stream.  Layouts: q [Hq][N][d], k and v
[Hkv][N][d] bf16 with a contiguous last dimension (any head/token strides that are multiples of
8 elements); out fp32 [Hq][N][d].
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import (PBSA_FORCE_DIAG, PBSA_FORCE_FIRST, PBSA_MASK_RANKED, PBSA_OP_ATTENTION, PBSA_OP_MASK,  # noqa: F401
                   PBSA_OP_PERMUTATION, PBSA_OP_PREFIX_RANK, PBSA_OP_QUERY_PERM, PbsaError, PbsaShape)

__all__ = [
    "build_segment_permutation",
    "estimate_block_mask",
    "block_sparse_attn_prefill",
    "tile_max",
    "calibrate_thresholds",
    "s2o_attn_prefill",
    "build_prefix_kv_ranking",
    "prefix_rank_length",
    "s2o_prefix_attn_prefill",
    "build_query_permutation",
    "sample_attention_mask",
    "sample_mask_workspace_size",
    "workspace_size",
    "make_shape",
    "num_blocks",
    "PbsaError",
]


def num_blocks(seq_len: int, block_size: int) -> int:
    return -(-seq_len // block_size)


def _check_tensor(name: str, t: Optional[torch.Tensor], dtype, shape, device, contiguous: bool = True) -> None:
    """t is None, or a tensor of this dtype and exact shape on `device` (None: any), contiguous if asked."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device} (got {t.device})")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_qkv(q: torch.Tensor, k: torch.Tensor, v: Optional[torch.Tensor], block_size: int,
               require_gpu: bool = True) -> None:
    """q [Hq][N][d], k and v [Hkv][N][d] bf16 on one device, Hq a multiple of Hkv, v with k's strides."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t is None:
            continue
        if not isinstance(t, torch.Tensor) or (require_gpu and t.device.type != "cuda"):
            raise ValueError(f"{name} must be a GPU tensor (the library has no CPU path)")
        if t.dtype != torch.bfloat16 or t.dim() != 3 or t.stride(2) != 1:
            raise ValueError(f"{name} must be bf16 [heads][tokens][d] with a contiguous last dimension")
        if t.device != q.device:
            raise ValueError(f"{name} must be on the device of q")
    if k.shape[1:] != q.shape[1:]:
        raise ValueError(f"k must match q in tokens and head_dim (q {tuple(q.shape)}, k {tuple(k.shape)})")
    if k.shape[0] < 1 or q.shape[0] % k.shape[0]:
        raise ValueError("the number of query heads must be a multiple of the number of KV heads")
    if v is not None and (v.shape != k.shape or v.stride() != k.stride()):
        raise ValueError("k and v must share shape and strides")
    if not isinstance(block_size, int) or block_size <= 0:
        raise ValueError("block_size must be a positive int")


def _check_attn_args(q, k, v, perm, block_count, block_idx, block_size, theta=None, out=None, lse=None,
                     require_gpu: bool = True, out_dtype=torch.float32) -> None:
    """Argument check of the attention entry points: int32 perm [Hkv][N], int32 block_count [Hq][NB]
    and block_idx [Hq][NB(NB+1)/2] (both or neither), fp32 theta [Hq][NB], out [Hq][N][d] of
    out_dtype with a contiguous last dimension, fp32 lse [Hq][N], all contiguous and on q's device."""
    _check_qkv(q, k, v, block_size, require_gpu)
    Hq, N, d = q.shape
    Hkv = k.shape[0]
    NB = num_blocks(N, block_size)
    dev = q.device
    _check_tensor("perm", perm, torch.int32, (Hkv, N), dev)
    if (block_count is None) != (block_idx is None):
        raise ValueError("block_count and block_idx are given together or not at all")
    _check_tensor("block_count", block_count, torch.int32, (Hq, NB), dev)
    _check_tensor("block_idx", block_idx, torch.int32, (Hq, NB * (NB + 1) // 2), dev)
    _check_tensor("early_stop_theta", theta, torch.float32, (Hq, NB), dev)
    if out is not None:
        _check_tensor("out", out, out_dtype, (Hq, N, d), dev, contiguous=False)
        if out.stride(2) != 1:
            raise ValueError("out must have a contiguous last dimension")
    _check_tensor("lse", lse, torch.float32, (Hq, N), dev)


def make_shape(q: torch.Tensor, k: torch.Tensor, block_size: int, segment_size: int,
               scale: Optional[float] = None, out: Optional[torch.Tensor] = None) -> PbsaShape:
    """pbsa_shape for q [Hq][N][d] and k (and v) [Hkv][N][d] with their strides."""
    s = PbsaShape()
    s.seq_len = q.shape[1]
    s.num_q_heads = q.shape[0]
    s.num_kv_heads = k.shape[0]
    s.head_dim = q.shape[2]
    s.block_size = block_size
    s.segment_size = segment_size or 0
    s.softmax_scale = float(scale) if scale else 0.0
    s.q_stride_head, s.q_stride_token = q.stride(0), q.stride(1)
    s.kv_stride_head, s.kv_stride_token = k.stride(0), k.stride(1)
    if out is not None:
        s.o_stride_head, s.o_stride_token = out.stride(0), out.stride(1)
    else:
        s.o_stride_head, s.o_stride_token = q.shape[1] * q.shape[2], q.shape[2]
    return s


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def workspace_size(shape: PbsaShape, op: int) -> int:
    n = _lib.lib().pbsa_workspace_size(ctypes.byref(shape), op)
    if n == _lib.SIZE_MAX:
        raise PbsaError(_lib.PBSA_ERR_INVALID_ARG, "pbsa_workspace_size")
    return n


def _workspace(shape: PbsaShape, op: int, device, ws: Optional[torch.Tensor]) -> Tuple[Optional[torch.Tensor], int]:
    need = workspace_size(shape, op)
    if need == 0:
        return None, 0
    if ws is None or ws.numel() * ws.element_size() < need:
        ws = torch.empty(need + 256, dtype=torch.uint8, device=device)
    # 256-byte alignment of the start (torch allocations are, but views need not be)
    off = (-ws.data_ptr()) % 256
    ws = ws[off:]
    return ws, ws.numel()


def build_segment_permutation(q: torch.Tensor, k: torch.Tensor, block_size: int, segment_size: int,
                              scale: Optional[float] = None, return_importance: bool = False,
                              perm: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Stage 1: int32 index list perm [Hkv][N] (and fp64 importance [Hkv][N] if asked)."""
    _check_qkv(q, k, None, block_size)
    _check_tensor("perm", perm, torch.int32, (k.shape[0], k.shape[1]), q.device)
    shape = make_shape(q, k, block_size, segment_size, scale)
    Hkv, N = k.shape[0], k.shape[1]
    if perm is None:
        perm = torch.empty((Hkv, N), dtype=torch.int32, device=q.device)
    imp = torch.empty((Hkv, N), dtype=torch.float64, device=q.device) if return_importance else None
    ws, nbytes = _workspace(shape, PBSA_OP_PERMUTATION, q.device, workspace)
    st = _lib.lib().pbsa_build_segment_permutation(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(perm), _ptr(imp),
                                                   _ptr(ws), nbytes, _stream())
    _lib.check(st, "pbsa_build_segment_permutation")
    return (perm, imp) if return_importance else perm


def estimate_block_mask(q: torch.Tensor, k: torch.Tensor, perm: Optional[torch.Tensor], block_size: int,
                        segment_size: int, mass_tau: float, force_diag: bool = True, force_first: bool = True,
                        scale: Optional[float] = None, return_prob: bool = False,
                        out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
                        workspace: Optional[torch.Tensor] = None, ranked: bool = False):
    """Stage 2: (block_count int32 [Hq][NB], block_idx int32 [Hq][NB(NB+1)/2][, prob fp64]).

    ranked: list every J <= I in the order of the marginal-gain early stop instead of applying the
    mass cut (mass_tau and the force flags are then not used, and no probabilities are written)."""
    _check_qkv(q, k, None, block_size)
    _check_tensor("perm", perm, torch.int32, (k.shape[0], k.shape[1]), q.device)
    shape = make_shape(q, k, block_size, segment_size, scale)
    Hq, N = q.shape[0], q.shape[1]
    NB = num_blocks(N, block_size)
    if out is None:
        count = torch.empty((Hq, NB), dtype=torch.int32, device=q.device)
        idx = torch.empty((Hq, NB * (NB + 1) // 2), dtype=torch.int32, device=q.device)
    else:
        count, idx = out
        _check_tensor("block_count", count, torch.int32, (Hq, NB), q.device)
        _check_tensor("block_idx", idx, torch.int32, (Hq, NB * (NB + 1) // 2), q.device)
    prob = torch.empty((Hq, NB * (NB + 1) // 2), dtype=torch.float64, device=q.device) if return_prob else None
    flags = (PBSA_FORCE_DIAG if force_diag else 0) | (PBSA_FORCE_FIRST if force_first else 0)
    if ranked:
        if return_prob:
            raise ValueError("the ranked order writes no probabilities")
        flags |= PBSA_MASK_RANKED
    ws, nbytes = _workspace(shape, PBSA_OP_MASK, q.device, workspace)
    st = _lib.lib().pbsa_estimate_block_mask(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(perm), float(mass_tau),
                                             flags, _ptr(count), _ptr(idx), _ptr(prob), _ptr(ws), nbytes, _stream())
    _lib.check(st, "pbsa_estimate_block_mask")
    return (count, idx, prob) if return_prob else (count, idx)


def block_sparse_attn_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                              perm: Optional[torch.Tensor] = None, block_count: Optional[torch.Tensor] = None,
                              block_idx: Optional[torch.Tensor] = None, block_size: int = 128,
                              segment_size: int = 0, early_stop_theta: Optional[torch.Tensor] = None,
                              scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                              lse: Optional[torch.Tensor] = None, return_lse: bool = True,
                              return_kept: bool = False, return_error: bool = False,
                              workspace: Optional[torch.Tensor] = None, no_alloc: bool = False,
                              max_workgroups: int = 0, claim_back: bool = False,
                              out_dtype: Optional[torch.dtype] = None):
    """Stage 3: out fp32 [Hq][N][d] (+ lse fp32 [Hq][N], kept-tile bitmap, device error word).
    out_dtype torch.bfloat16 (or a bf16 out): pbsa_block_sparse_attn_prefill_bf16out, the fp32
    result rounded to bf16 as it is stored (not with no_alloc or launch options).
    workspace: optional preallocated device buffer of at least workspace_size(shape, PBSA_OP_ATTENTION)
    bytes (the work deques); one is allocated per call otherwise.  no_alloc: call
    pbsa_block_sparse_attn_prefill_noalloc instead, whose work deques live in the library (no
    workspace); pass out, and lse or return_lse=False, so that this call allocates nothing either.
    max_workgroups / claim_back: launch options of pbsa_block_sparse_attn_prefill_ex (a cap on the
    persistent grid, and the order workgroups take rows in); results do not depend on them."""
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.float32
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be torch.float32 or torch.bfloat16")
    bf16_out = out_dtype == torch.bfloat16
    _check_attn_args(q, k, v, perm, block_count, block_idx, block_size, early_stop_theta, out, lse,
                     out_dtype=out_dtype)
    if int(max_workgroups) < 0:
        raise ValueError("max_workgroups must be >= 0")
    if no_alloc and (max_workgroups or claim_back):
        raise ValueError("launch options are not available with no_alloc")
    if bf16_out and (no_alloc or max_workgroups or claim_back):
        raise ValueError("the bf16 output is not available with no_alloc or launch options")
    Hq, N, d = q.shape
    if out is None:
        out = torch.empty((Hq, N, d), dtype=out_dtype, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((Hq, N), dtype=torch.float32, device=q.device)
    NB = num_blocks(N, block_size)
    kept = None
    if return_kept:
        words = -(-(NB * (NB + 1) // 2) // 32)
        kept = torch.zeros((Hq, words), dtype=torch.int32, device=q.device)
    err = torch.zeros(1, dtype=torch.int32, device=q.device) if return_error else None
    shape = make_shape(q, k, block_size, segment_size, scale, out=out)
    if no_alloc:
        st = _lib.lib().pbsa_block_sparse_attn_prefill_noalloc(
            ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(perm), _ptr(block_count), _ptr(block_idx),
            _ptr(early_stop_theta), _ptr(out), _ptr(lse), _ptr(kept), _ptr(err), _stream())
        _lib.check(st, "pbsa_block_sparse_attn_prefill_noalloc")
    elif bf16_out:
        ws, nbytes = _workspace(shape, PBSA_OP_ATTENTION, q.device, workspace)
        st = _lib.lib().pbsa_block_sparse_attn_prefill_bf16out(
            ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(perm), _ptr(block_count), _ptr(block_idx),
            _ptr(early_stop_theta), _ptr(out), _ptr(lse), _ptr(kept), _ptr(err), _ptr(ws), nbytes, _stream())
        _lib.check(st, "pbsa_block_sparse_attn_prefill_bf16out")
    elif max_workgroups or claim_back:
        ws, nbytes = _workspace(shape, PBSA_OP_ATTENTION, q.device, workspace)
        opt = _lib.PbsaLaunchOptions(int(max_workgroups), _lib.PBSA_LAUNCH_CLAIM_BACK if claim_back else 0)
        st = _lib.lib().pbsa_block_sparse_attn_prefill_ex(
            ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(perm), _ptr(block_count), _ptr(block_idx),
            _ptr(early_stop_theta), _ptr(out), _ptr(lse), _ptr(kept), _ptr(err), _ptr(ws), nbytes,
            ctypes.byref(opt), _stream())
        _lib.check(st, "pbsa_block_sparse_attn_prefill_ex")
    else:
        ws, nbytes = _workspace(shape, PBSA_OP_ATTENTION, q.device, workspace)
        st = _lib.lib().pbsa_block_sparse_attn_prefill(
            ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(perm), _ptr(block_count), _ptr(block_idx),
            _ptr(early_stop_theta), _ptr(out), _ptr(lse), _ptr(kept), _ptr(err), _ptr(ws), nbytes, _stream())
        _lib.check(st, "pbsa_block_sparse_attn_prefill")
    res = [out]
    if return_lse:
        res.append(lse)
    if return_kept:
        res.append(kept)
    if return_error:
        res.append(err)
    return res[0] if len(res) == 1 else tuple(res)


def s2o_attn_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, perm: Optional[torch.Tensor],
                     block_count: torch.Tensor, block_idx: torch.Tensor, block_size: int, segment_size: int,
                     gain_tau: float, scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None, return_lse: bool = True, return_kept: bool = False,
                     return_error: bool = False, workspace: Optional[torch.Tensor] = None):
    """Attention with the marginal-gain early stop over a ranked list (estimate_block_mask with
    ranked=True): out fp32 [Hq][N][d] (+ lse, processed-block bitmap, device error word)."""
    if block_count is None or block_idx is None:
        raise ValueError("the marginal-gain stop needs the ranked lists block_count and block_idx")
    _check_attn_args(q, k, v, perm, block_count, block_idx, block_size, None, out, lse)
    Hq, N, d = q.shape
    if out is None:
        out = torch.empty((Hq, N, d), dtype=torch.float32, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((Hq, N), dtype=torch.float32, device=q.device)
    NB = num_blocks(N, block_size)
    kept = None
    if return_kept:
        words = -(-(NB * (NB + 1) // 2) // 32)
        kept = torch.zeros((Hq, words), dtype=torch.int32, device=q.device)
    err = torch.zeros(1, dtype=torch.int32, device=q.device) if return_error else None
    shape = make_shape(q, k, block_size, segment_size, scale, out=out)
    ws, nbytes = _workspace(shape, PBSA_OP_ATTENTION, q.device, workspace)
    st = _lib.lib().pbsa_s2o_attn_prefill(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(perm), _ptr(block_count), _ptr(block_idx),
        float(gain_tau), _ptr(out), _ptr(lse), _ptr(kept), _ptr(err), _ptr(ws), nbytes, _stream())
    _lib.check(st, "pbsa_s2o_attn_prefill")
    res = [out]
    if return_lse:
        res.append(lse)
    if return_kept:
        res.append(kept)
    if return_error:
        res.append(err)
    return res[0] if len(res) == 1 else tuple(res)


def prefix_rank_length(q: torch.Tensor, k: torch.Tensor, block_size: int, segment_size: int) -> int:
    """Entries per KV head of the historical ranking (S * nseg * (nseg - 1) / 2)."""
    n = _lib.lib().pbsa_prefix_rank_length(ctypes.byref(make_shape(q, k, block_size, segment_size)))
    if n < 0:
        raise PbsaError(_lib.PBSA_ERR_UNSUPPORTED, "pbsa_prefix_rank_length")
    return n


def build_prefix_kv_ranking(q: torch.Tensor, k: torch.Tensor, block_size: int, segment_size: int,
                            out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """S2O historical ranking: int32 [Hkv][prefix_rank_length] holding, for every segment sigma >= 1
    at offset S*sigma*(sigma-1)/2, the keys before the segment by descending score against the
    segment's mean query."""
    _check_qkv(q, k, None, block_size)
    shape = make_shape(q, k, block_size, segment_size)
    L = prefix_rank_length(q, k, block_size, segment_size)
    if out is None:
        out = torch.empty((k.shape[0], L), dtype=torch.int32, device=q.device)
    elif out.dtype != torch.int32 or out.shape != (k.shape[0], L) or not out.is_contiguous():
        raise ValueError("out must be a contiguous int32 [Hkv][prefix_rank_length] tensor")
    ws, nbytes = _workspace(shape, PBSA_OP_PREFIX_RANK, q.device, workspace)
    st = _lib.lib().pbsa_build_prefix_kv_ranking(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(out) if L else None,
                                                 _ptr(ws), nbytes, _stream())
    _lib.check(st, "pbsa_build_prefix_kv_ranking")
    return out


def build_query_permutation(q: torch.Tensor, k: torch.Tensor, block_size: int, segment_size: int,
                            out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """S2O query permutation: int32 [Hkv][N], each segment's positions by descending score against the
    KV head's mean key (averaged over its query heads), ties by position."""
    _check_qkv(q, k, None, block_size)
    shape = make_shape(q, k, block_size, segment_size)
    if out is None:
        out = torch.empty((k.shape[0], q.shape[1]), dtype=torch.int32, device=q.device)
    elif out.dtype != torch.int32 or out.shape != (k.shape[0], q.shape[1]) or not out.is_contiguous():
        raise ValueError("out must be a contiguous int32 [Hkv][N] tensor")
    ws, nbytes = _workspace(shape, PBSA_OP_QUERY_PERM, q.device, workspace)
    st = _lib.lib().pbsa_build_query_permutation(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(out), _ptr(ws), nbytes,
                                                 _stream())
    _lib.check(st, "pbsa_build_query_permutation")
    return out


def s2o_prefix_attn_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kv_rank: torch.Tensor,
                            block_size: int, segment_size: int, gain_tau: float, scale: Optional[float] = None,
                            out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                            return_lse: bool = True, return_kept: bool = False, return_error: bool = False,
                            workspace: Optional[torch.Tensor] = None, qperm: Optional[torch.Tensor] = None):
    """S2O two-pass attention with the marginal-gain stop over the historical ranking of
    build_prefix_kv_ranking: out fp32 [Hq][N][d] (+ lse, processed-entry bitmap, device error word).
    qperm (build_query_permutation) permutes the queries inside segments; rows still come back at
    their natural positions, and the kept bitmap then has NB bits per (h, I) row."""
    _check_attn_args(q, k, v, None, None, None, block_size, None, out, lse)
    Hq, N, d = q.shape
    L = prefix_rank_length(q, k, block_size, segment_size)
    if kv_rank.dtype != torch.int32 or kv_rank.shape != (k.shape[0], L) or not kv_rank.is_contiguous():
        raise ValueError("kv_rank must be the contiguous int32 [Hkv][prefix_rank_length] ranking")
    if out is None:
        out = torch.empty((Hq, N, d), dtype=torch.float32, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((Hq, N), dtype=torch.float32, device=q.device)
    if qperm is not None and (qperm.dtype != torch.int32 or qperm.shape != (k.shape[0], N)
                              or not qperm.is_contiguous()):
        raise ValueError("qperm must be the contiguous int32 [Hkv][N] query permutation")
    NB = num_blocks(N, block_size)
    kept = None
    if return_kept:
        bits = NB * NB if qperm is not None else NB * (NB + 1) // 2
        kept = torch.zeros((Hq, -(-bits // 32)), dtype=torch.int32, device=q.device)
    err = torch.zeros(1, dtype=torch.int32, device=q.device) if return_error else None
    shape = make_shape(q, k, block_size, segment_size, scale, out=out)
    ws, nbytes = _workspace(shape, PBSA_OP_ATTENTION, q.device, workspace)
    st = _lib.lib().pbsa_s2o_prefix_attn_prefill(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(kv_rank) if L else None, _ptr(qperm), float(gain_tau),
        _ptr(out), _ptr(lse), _ptr(kept), _ptr(err), _ptr(ws), nbytes, _stream())
    _lib.check(st, "pbsa_s2o_prefix_attn_prefill")
    res = [out]
    if return_lse:
        res.append(lse)
    if return_kept:
        res.append(kept)
    if return_error:
        res.append(err)
    return res[0] if len(res) == 1 else tuple(res)


def sample_mask_workspace_size(q: torch.Tensor, k: torch.Tensor, block_size: int, n_trunks: int,
                               rows_per_trunk: int) -> int:
    """Workspace bytes of sample_attention_mask for this shape and sampling."""
    shape = make_shape(q, k, block_size, 0)
    need = _lib.lib().pbsa_sample_mask_workspace_size(ctypes.byref(shape), int(n_trunks), int(rows_per_trunk))
    if need == _lib.SIZE_MAX:
        raise PbsaError(_lib.PBSA_ERR_INVALID_ARG, "pbsa_sample_mask_workspace_size")
    return need


def sample_attention_mask(q: torch.Tensor, k: torch.Tensor, block_size: int, cia_tau: float, n_trunks: int,
                          rows_per_trunk: int, force_diag: bool = True, force_first: bool = False,
                          scale: Optional[float] = None, return_masses: bool = False,
                          out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
                          workspace: Optional[torch.Tensor] = None):
    """SampleAttention's block mask: (block_count int32 [Hq][NB], block_idx int32 [Hq][NB(NB+1)/2]
    [, col fp64 [Hq][N], slash fp64 [Hq][N]]), for block_sparse_attn_prefill with perm = None."""
    _check_qkv(q, k, None, block_size)
    shape = make_shape(q, k, block_size, 0, scale)
    Hq, N = q.shape[0], q.shape[1]
    NB = num_blocks(N, block_size)
    if out is None:
        count = torch.empty((Hq, NB), dtype=torch.int32, device=q.device)
        idx = torch.empty((Hq, NB * (NB + 1) // 2), dtype=torch.int32, device=q.device)
    else:
        count, idx = out
    col = torch.empty((Hq, N), dtype=torch.float64, device=q.device) if return_masses else None
    slash = torch.empty((Hq, N), dtype=torch.float64, device=q.device) if return_masses else None
    need = sample_mask_workspace_size(q, k, block_size, n_trunks, rows_per_trunk)
    ws, nbytes = None, 0
    if need:
        ws = workspace
        if ws is None or ws.numel() * ws.element_size() < need + 256:
            ws = torch.empty(need + 256, dtype=torch.uint8, device=q.device)
        ws = ws[(-ws.data_ptr()) % 256:]
        nbytes = ws.numel()
    flags = (PBSA_FORCE_DIAG if force_diag else 0) | (PBSA_FORCE_FIRST if force_first else 0)
    st = _lib.lib().pbsa_sample_attention_mask(ctypes.byref(shape), _ptr(q), _ptr(k), float(cia_tau), int(n_trunks),
                                               int(rows_per_trunk), flags, _ptr(count), _ptr(idx), _ptr(col),
                                               _ptr(slash), _ptr(ws), nbytes, _stream())
    _lib.check(st, "pbsa_sample_attention_mask")
    return (count, idx, col, slash) if return_masses else (count, idx)


def tile_max(q: torch.Tensor, k: torch.Tensor, block_size: int, scale: Optional[float] = None,
             perm: Optional[torch.Tensor] = None, segment_size: int = 0) -> torch.Tensor:
    """Calibration helper: fp32 [Hq][NB(NB+1)/2] per-tile max of the scaled causal logits, as the
    early-stop gate computes it.  perm (with segment_size): tiles of earlier segments are read
    through the permutation, as the gate reads them on a permuted mask."""
    _check_qkv(q, k, None, block_size)
    _check_tensor("perm", perm, torch.int32, (k.shape[0], k.shape[1]), q.device)
    shape = make_shape(q, k, block_size, segment_size if perm is not None else 0, scale)
    NB = num_blocks(q.shape[1], block_size)
    tm = torch.empty((q.shape[0], NB * (NB + 1) // 2), dtype=torch.float32, device=q.device)
    st = _lib.lib().pbsa_tile_max(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(perm), _ptr(tm), _stream())
    _lib.check(st, "pbsa_tile_max")
    return tm


def calibrate_thresholds(tile_max_: torch.Tensor, q: torch.Tensor, k: torch.Tensor, block_size: int,
                         keep: int) -> torch.Tensor:
    """Early-stop thresholds fp32 [Hq][NB] from calibration tile maxima (as from tile_max on q, k):
    the keep-th largest tile max of each query block's row, -inf for rows of at most keep tiles."""
    _check_qkv(q, k, None, block_size)
    shape = make_shape(q, k, block_size, 0)
    NB = num_blocks(q.shape[1], block_size)
    if tile_max_.dtype != torch.float32 or tile_max_.shape != (q.shape[0], NB * (NB + 1) // 2) \
            or not tile_max_.is_contiguous():
        raise ValueError("tile_max must be contiguous fp32 [Hq][NB(NB+1)/2]")
    theta = torch.empty((q.shape[0], NB), dtype=torch.float32, device=q.device)
    st = _lib.lib().pbsa_calibrate_thresholds(ctypes.byref(shape), _ptr(tile_max_), int(keep), _ptr(theta),
                                             _stream())
    _lib.check(st, "pbsa_calibrate_thresholds")
    return theta


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
