"""ctypes mirror of include/prism.h and the loader of libprism.so.

Argument marshalling only: every step of the estimator and the attention runs
in the library's HIP kernels. The library must be built first
(``python -m block_sparse_attention_band_amd.build``); loading fails loudly
otherwise.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libprism.so")

PRISM_ABI_VERSION = 7

# prism_status_t
(OK, ERR_NULL, ERR_DTYPE, ERR_SHAPE, ERR_STRIDE, ERR_ALIGN, ERR_CONFIG, ERR_WORKSPACE, ERR_UNSUPPORTED, ERR_LAUNCH,
 ERR_SCRATCH) = range(11)
STATUS_NAMES = ["PRISM_OK", "PRISM_ERR_NULL", "PRISM_ERR_DTYPE", "PRISM_ERR_SHAPE", "PRISM_ERR_STRIDE",
                "PRISM_ERR_ALIGN", "PRISM_ERR_CONFIG", "PRISM_ERR_WORKSPACE", "PRISM_ERR_UNSUPPORTED",
                "PRISM_ERR_LAUNCH", "PRISM_ERR_SCRATCH"]
NOALLOC_SCRATCH_BYTES = 40 << 20
BF16, FP32 = 0, 1
ROPE_INTERLEAVED, ROPE_HALF = 0, 1
TAU_FULLSPEC, TAU_NONE, TAU_UNIT, TAU_PERVEC = 0, 1, 2, 3
MASK_U8, MASK_BITS = 0, 1
MERGE_UNION, MERGE_INTERSECT, MERGE_MIX = 0, 1, 2
BANDS_STATIC, BANDS_ADAPTIVE = 0, 1
EST_KEEP_LOGITS = 1
EST_SINGLE_LAUNCH = 2
SINGLE_MAX_WGS = 4096  # barrier words in the workspace's barrier section


class PrismTensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("batch", ctypes.c_int64), ("seq", ctypes.c_int64), ("heads", ctypes.c_int64), ("head_dim", ctypes.c_int64),
        ("stride_b", ctypes.c_int64), ("stride_s", ctypes.c_int64), ("stride_h", ctypes.c_int64),
    ]


class PrismMask(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p), ("batch", ctypes.c_int64), ("heads", ctypes.c_int64),
        ("nq_blocks", ctypes.c_int64), ("nk_blocks", ctypes.c_int64),
        ("block_size", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("format", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


class PrismCfg(ctypes.Structure):
    _fields_ = [
        ("block_size", ctypes.c_int32), ("d_high", ctypes.c_int32), ("d_low", ctypes.c_int32), ("p", ctypes.c_float),
        ("causal", ctypes.c_int32), ("rope_layout", ctypes.c_int32), ("tau_mode", ctypes.c_int32),
        ("flags", ctypes.c_int32), ("merge", ctypes.c_int32), ("band_mode", ctypes.c_int32),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


class PrismWorkspaceLayout(ctypes.Structure):
    _fields_ = [
        ("qbar_offset", ctypes.c_size_t), ("kbar_offset", ctypes.c_size_t), ("qsq_offset", ctypes.c_size_t),
        ("ksq_offset", ctypes.c_size_t), ("tau_offset", ctypes.c_size_t), ("logits_offset", ctypes.c_size_t),
        ("logits_plane", ctypes.c_int64), ("spectrum_offset", ctypes.c_size_t), ("split_offset", ctypes.c_size_t),
        ("total_bytes", ctypes.c_size_t),
        ("nb", ctypes.c_int64), ("seg_lo", ctypes.c_int32), ("seg_hi", ctypes.c_int32),
        ("overlap", ctypes.c_int32), ("reserved", ctypes.c_int32), ("barrier_offset", ctypes.c_size_t),
    ]


# every function include/prism.h declares: (name, restype, argtypes)
SIGNATURES = [
    ("prism_abi_version", ctypes.c_int, []),
    ("prism_status_str", ctypes.c_char_p, [ctypes.c_int]),
    ("prism_estimate_workspace_bytes", ctypes.c_size_t,
     [ctypes.POINTER(PrismTensor), ctypes.POINTER(PrismTensor), ctypes.POINTER(PrismCfg)]),
    ("prism_estimate_workspace_layout", ctypes.c_int,
     [ctypes.POINTER(PrismTensor), ctypes.POINTER(PrismTensor), ctypes.POINTER(PrismCfg),
      ctypes.POINTER(PrismWorkspaceLayout)]),
    ("prism_estimate", ctypes.c_int,
     [ctypes.POINTER(PrismTensor), ctypes.POINTER(PrismTensor), ctypes.POINTER(PrismCfg),
      ctypes.POINTER(PrismMask), ctypes.c_void_p]),
    ("prism_estimate_noalloc", ctypes.c_int,
     [ctypes.POINTER(PrismTensor), ctypes.POINTER(PrismTensor), ctypes.POINTER(PrismCfg),
      ctypes.POINTER(PrismMask), ctypes.c_void_p]),
    ("prism_block_sparse_attn", ctypes.c_int,
     [ctypes.POINTER(PrismTensor), ctypes.POINTER(PrismTensor), ctypes.POINTER(PrismTensor),
      ctypes.POINTER(PrismMask), ctypes.POINTER(PrismTensor), ctypes.c_void_p]),
]

_lib = None


def lib() -> ctypes.CDLL:
    """Load libprism.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m block_sparse_attention_band_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        if handle.prism_abi_version() != PRISM_ABI_VERSION:
            raise RuntimeError("libprism ABI version mismatch")
        _lib = handle
    return _lib


class PrismError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__(f"{where}: {name} ({lib().prism_status_str(status).decode()})")


def check(status: int, where: str) -> None:
    if status != OK:
        raise PrismError(status, where)
