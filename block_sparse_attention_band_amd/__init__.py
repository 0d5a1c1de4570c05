"""Prism on MI355X: the spectral-aware block-importance estimator and the
causal block-sparse attention prefill, as HIP kernels behind the C ABI of
libprism.so (include/prism.h).

This module only marshals arguments: it turns torch tensors (device memory on
the current HIP stream) into the ABI's plain descriptors and calls the
library. Every step of the path runs in the library's kernels; there is no
fallback. Tensors are [batch, seq, heads, 128] with the last dim contiguous
(any batch/seq/head strides), bf16 or fp32. Block masks are either uint8
[batch, heads, nb, nb] (one byte per block) or bit-packed int32
[batch, heads, nb, ceil(nb / 32)] (bit j % 32 of word j / 32 = key block j).
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

from . import _abi
from ._abi import PrismCfg, PrismError, PrismMask, PrismTensor, PrismWorkspaceLayout, lib

__all__ = ["EstimatorConfig", "estimate", "estimate_noalloc", "block_sparse_attn", "workspace_bytes",
           "workspace_layout", "PrismError", "lib"]

_ROPE = {"interleaved": _abi.ROPE_INTERLEAVED, "half": _abi.ROPE_HALF}
_TAU = {"fullspec": _abi.TAU_FULLSPEC, "none": _abi.TAU_NONE, "unit": _abi.TAU_UNIT,
        "pervec": _abi.TAU_PERVEC}
_MERGE = {"union": _abi.MERGE_UNION, "intersect": _abi.MERGE_INTERSECT, "mix": _abi.MERGE_MIX}
_BANDS = {"static": _abi.BANDS_STATIC, "adaptive": _abi.BANDS_ADAPTIVE}


@dataclass(frozen=True)
class EstimatorConfig:
    """Prism's estimator settings (defaults: B=128, d_high=64, d_low=96, p=0.95)."""

    block_size: int = 128
    d_high: int = 64
    d_low: int = 96
    p: float = 0.95
    causal: bool = True
    rope_layout: str = "interleaved"
    tau_mode: str = "fullspec"
    keep_logits: bool = False  # also store the band logits in the workspace (inspection)
    merge: str = "union"       # "union" (the pages' step 7), "intersect" or "mix"
    band_mode: str = "static"  # "static" (the pages' split) or "adaptive" (per head)
    single_launch: bool = False  # the whole estimator as one persistent kernel (grid barrier)


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return _abi.BF16
    if t.dtype == torch.float32:
        return _abi.FP32
    return 99  # rejected by the library with PRISM_ERR_DTYPE


def tensor_desc(t) -> PrismTensor:
    """Descriptor of a [batch, seq, heads, head_dim] tensor (no copy)."""
    if t.dim() != 4:
        raise ValueError("expected a [batch, seq, heads, head_dim] tensor")
    if t.stride(3) != 1:
        raise ValueError("the head_dim stride must be 1")
    b, n, h, d = t.shape
    sb, ss, sh, _ = t.stride()
    return PrismTensor(t.data_ptr(), _dtype_code(t), 0, b, n, h, d, sb, ss, sh)


def mask_desc(m, block_size: int, causal: bool) -> PrismMask:
    """Descriptor of a block mask: uint8 [b, H, nb, nb], or int32 [b, H, nb, ceil(nb/32)] bit-packed."""
    torch = _torch()
    if m.dim() != 4 or not m.is_contiguous() or m.dtype not in (torch.uint8, torch.int32):
        raise ValueError("mask must be a contiguous uint8 [batch, heads, nb, nb] or int32 "
                         "[batch, heads, nb, ceil(nb/32)] tensor")
    b, h, nq, w = m.shape
    if m.dtype == torch.uint8:
        return PrismMask(m.data_ptr(), b, h, nq, w, block_size, int(bool(causal)), _abi.MASK_U8, 0)
    if w != (nq + 31) // 32:
        raise ValueError("a bit-packed mask row holds ceil(nb / 32) int32 words")
    return PrismMask(m.data_ptr(), b, h, nq, nq, block_size, int(bool(causal)), _abi.MASK_BITS, 0)


def _cfg(cfg: EstimatorConfig, workspace=None) -> PrismCfg:
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return PrismCfg(cfg.block_size, cfg.d_high, cfg.d_low, cfg.p, int(bool(cfg.causal)), _ROPE[cfg.rope_layout],
                    _TAU[cfg.tau_mode],
                    (_abi.EST_KEEP_LOGITS if cfg.keep_logits else 0) | (_abi.EST_SINGLE_LAUNCH if cfg.single_launch else 0),
                    _MERGE[cfg.merge],
                    _BANDS[cfg.band_mode], ws_ptr, ws_bytes)


def _stream(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def workspace_layout(q, k, cfg: EstimatorConfig = EstimatorConfig()) -> PrismWorkspaceLayout:
    out = PrismWorkspaceLayout()
    qd, kd, c = tensor_desc(q), tensor_desc(k), _cfg(cfg)
    _abi.check(lib().prism_estimate_workspace_layout(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(c),
                                                     ctypes.byref(out)), "prism_estimate_workspace_layout")
    return out


def workspace_bytes(q, k, cfg: EstimatorConfig = EstimatorConfig()) -> int:
    return workspace_layout(q, k, cfg).total_bytes


def new_workspace(q, k, cfg: EstimatorConfig = EstimatorConfig()):
    """A device workspace of the size prism_estimate needs (torch allocation)."""
    torch = _torch()
    n = workspace_bytes(q, k, cfg)
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def estimate(q, k, cfg: EstimatorConfig = EstimatorConfig(), *, workspace=None, mask_out=None, bits: bool = False):
    """Prism's block mask M for post-RoPE q, k: uint8 [batch, Hq, nb, nb] (1 = compute), or with
    bits=True (or an int32 mask_out) bit-packed int32 [batch, Hq, nb, ceil(nb / 32)]."""
    torch = _torch()
    L = workspace_layout(q, k, cfg)
    if workspace is None:
        workspace = torch.empty(L.total_bytes, dtype=torch.uint8, device=q.device)
    if mask_out is None:
        if bits:
            mask_out = torch.empty((q.shape[0], q.shape[2], L.nb, (L.nb + 31) // 32), dtype=torch.int32,
                                   device=q.device)
        else:
            mask_out = torch.empty((q.shape[0], q.shape[2], L.nb, L.nb), dtype=torch.uint8, device=q.device)
    qd, kd, c = tensor_desc(q), tensor_desc(k), _cfg(cfg, workspace)
    md = mask_desc(mask_out, cfg.block_size, cfg.causal)
    _abi.check(lib().prism_estimate(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(c), ctypes.byref(md),
                                    ctypes.c_void_p(_stream(q))), "prism_estimate")
    return mask_out


def estimate_noalloc(q, k, cfg: EstimatorConfig = EstimatorConfig(), *, mask_out=None, bits: bool = False):
    """prism_estimate_noalloc: the same mask as estimate(), with the library's own device
    scratch as the workspace (no workspace argument; nothing allocated by the library).
    A mask_out given by the caller makes the call allocation-free end to end."""
    torch = _torch()
    if mask_out is None:
        nb = (q.shape[1] + cfg.block_size - 1) // cfg.block_size
        shape = (q.shape[0], q.shape[2], nb, (nb + 31) // 32 if bits else nb)
        mask_out = torch.empty(shape, dtype=torch.int32 if bits else torch.uint8, device=q.device)
    qd, kd, c = tensor_desc(q), tensor_desc(k), _cfg(cfg)
    md = mask_desc(mask_out, cfg.block_size, cfg.causal)
    _abi.check(lib().prism_estimate_noalloc(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(c), ctypes.byref(md),
                                            ctypes.c_void_p(_stream(q))), "prism_estimate_noalloc")
    return mask_out


def block_sparse_attn(q, k, v, mask, *, causal: bool = True, block_size: int = 128, out=None):
    """Attention of q over the key blocks mask selects: out [batch, seq, Hq, 128]."""
    torch = _torch()
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    qd, kd, vd, od = tensor_desc(q), tensor_desc(k), tensor_desc(v), tensor_desc(out)
    md = mask_desc(mask, block_size, causal)
    _abi.check(lib().prism_block_sparse_attn(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(vd), ctypes.byref(md),
                                             ctypes.byref(od), ctypes.c_void_p(_stream(q))), "prism_block_sparse_attn")
    return out
