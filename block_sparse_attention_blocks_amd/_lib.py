"""ctypes view of libpbsa.so: the pbsa_shape struct, status codes and raw entry points.

Loading fails loudly when the library has not been built; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpbsa.so")

PBSA_OK = 0
PBSA_ERR_INVALID_ARG = 1
PBSA_ERR_UNSUPPORTED = 2
PBSA_ERR_WORKSPACE = 3
PBSA_ERR_HIP = 4

PBSA_OP_PERMUTATION = 0
PBSA_OP_MASK = 1
PBSA_OP_ATTENTION = 2
PBSA_OP_PREFIX_RANK = 3
PBSA_OP_QUERY_PERM = 4

PBSA_FORCE_DIAG = 1
PBSA_FORCE_FIRST = 2
PBSA_MASK_RANKED = 4

SIZE_MAX = ctypes.c_size_t(-1).value


class PbsaShape(ctypes.Structure):
    _fields_ = [
        ("seq_len", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("segment_size", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("q_stride_head", ctypes.c_int64),
        ("q_stride_token", ctypes.c_int64),
        ("kv_stride_head", ctypes.c_int64),
        ("kv_stride_token", ctypes.c_int64),
        ("o_stride_head", ctypes.c_int64),
        ("o_stride_token", ctypes.c_int64),
    ]


PBSA_LAUNCH_CLAIM_BACK = 1


class PbsaLaunchOptions(ctypes.Structure):
    _fields_ = [
        ("max_workgroups", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
    ]


class PbsaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


_lib = None

_P = ctypes.c_void_p
_SIG = {
    "pbsa_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(PbsaShape), ctypes.c_int]),
    "pbsa_build_segment_permutation": (ctypes.c_int, [ctypes.POINTER(PbsaShape), _P, _P, _P, _P, _P,
                                                      ctypes.c_size_t, _P]),
    "pbsa_estimate_block_mask": (ctypes.c_int, [ctypes.POINTER(PbsaShape), _P, _P, _P, ctypes.c_double,
                                                ctypes.c_uint32, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "pbsa_block_sparse_attn_prefill": (ctypes.c_int, [ctypes.POINTER(PbsaShape), _P, _P, _P, _P, _P, _P, _P,
                                                      _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "pbsa_block_sparse_attn_prefill_bf16out": (ctypes.c_int, [ctypes.POINTER(PbsaShape), _P, _P, _P, _P, _P, _P,
                                                              _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "pbsa_block_sparse_attn_prefill_ex": (ctypes.c_int, [ctypes.POINTER(PbsaShape), _P, _P, _P, _P, _P, _P, _P,
                                                         _P, _P, _P, _P, _P, ctypes.c_size_t,
                                                         ctypes.POINTER(PbsaLaunchOptions), _P]),
    "pbsa_block_sparse_attn_prefill_noalloc": (ctypes.c_int, [ctypes.POINTER(PbsaShape), _P, _P, _P, _P, _P, _P,
                                                              _P, _P, _P, _P, _P, _P]),
    "pbsa_s2o_attn_prefill": (ctypes.c_int, [ctypes.POINTER(PbsaShape), _P, _P, _P, _P, _P, _P, ctypes.c_float,
                                             _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "pbsa_build_prefix_kv_ranking": (ctypes.c_int, [ctypes.POINTER(PbsaShape), _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "pbsa_prefix_rank_length": (ctypes.c_int64, [ctypes.POINTER(PbsaShape)]),
    "pbsa_s2o_prefix_attn_prefill": (ctypes.c_int, [ctypes.POINTER(PbsaShape), _P, _P, _P, _P, _P, ctypes.c_float,
                                                    _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "pbsa_build_query_permutation": (ctypes.c_int, [ctypes.POINTER(PbsaShape), _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "pbsa_sample_attention_mask": (ctypes.c_int, [ctypes.POINTER(PbsaShape), _P, _P, ctypes.c_double, ctypes.c_int32,
                                                  ctypes.c_int32, ctypes.c_uint32, _P, _P, _P, _P, _P,
                                                  ctypes.c_size_t, _P]),
    "pbsa_sample_mask_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(PbsaShape), ctypes.c_int32, ctypes.c_int32]),
    "pbsa_tile_max": (ctypes.c_int, [ctypes.POINTER(PbsaShape), _P, _P, _P, _P, _P]),
    "pbsa_calibrate_thresholds": (ctypes.c_int, [ctypes.POINTER(PbsaShape), _P, ctypes.c_int32, _P, _P]),
    "pbsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pbsa_version": (ctypes.c_int32, []),
}


def lib() -> ctypes.CDLL:
    """The loaded library; raises if libpbsa.so is missing (build it with build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} not found: the HIP library has not been built "
                              "(run __graft_entry__.build() or block_sparse_attention_blocks_amd/build.py)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIG.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def status_string(status: int) -> str:
    return lib().pbsa_status_string(status).decode()


def check(status: int, what: str) -> None:
    if status != PBSA_OK:
        raise PbsaError(status, what)
