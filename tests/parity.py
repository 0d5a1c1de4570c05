"""Helpers shared by the GPU parity tests: moving synthetic inputs to the
device, running the oracle head by head, and comparing masks and outputs.

Mask rule: the GPU mask must equal the oracle's except at blocks whose
inclusion is decided within rounding:
  * cum-mass ties: in either branch, the oracle's cumulative mass before the
    block (exclusive) or through it (inclusive), in the oracle's sorted order,
    lies within 1e-4 of p;
  * score ties: in either branch, the block's oracle logit is within 1e-4 of
    the logit of that row's boundary block (the last one the oracle keeps),
    so fp32 rounding can swap the two across the boundary.
Both classes are counted and reported; every other mismatch fails.
"""
from __future__ import annotations

import numpy as np

import oracle.prism_oracle as po
from synth import to_f64

MASS_TOL = 1e-4
LOGIT_TOL = 1e-4


def to_device(x: np.ndarray, dtype: str, layout: str = "bshd"):
    """uint16 bf16 bits or float32 [b, N, H, d] -> torch CUDA tensor; 'bhsd'
    stores it head-major and returns the [b, N, H, d] strided view."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x))
    if layout == "bhsd":
        return t.permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3)
    return t.cuda()


def oracle_estimate_heads(q, k, dtype, *, block, d_high, d_low, p, causal, rope_layout="interleaved",
                          tau_mode="fullspec", heads=None):
    """Per-head oracle results {(b, h): dict} widening one head at a time."""
    b, N, Hq, _ = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    heads = range(Hq) if heads is None else heads
    out = {}
    kbars = {}
    for bb in range(b):
        for h in heads:
            g = h // G
            if (bb, g) not in kbars:
                kbars[(bb, g)] = po.mean_pool(to_f64(k[bb, :, g, :], dtype), block)
            out[(bb, h)] = po.estimate_head(to_f64(q[bb, :, h, :], dtype), None, block=block, d_high=d_high,
                                            d_low=d_low, p=p, causal=causal, rope_layout=rope_layout,
                                            tau_mode=tau_mode, kbar=kbars[(bb, g)])
    return out


def _branch_excuses(S, L, sel_oracle, i, J, p):
    """For one row i and branch: per admissible block, (mass-tie, score-tie) flags."""
    s = S[i, J]
    order = np.argsort(-s, kind="stable")
    cum = np.cumsum(s[order])
    excl = np.concatenate([[0.0], cum[:-1]])
    rank = np.empty_like(order)
    rank[order] = np.arange(len(order))
    mass_tie = (np.abs(excl[rank] - p) <= MASS_TOL) | (np.abs(cum[rank] - p) <= MASS_TOL)
    kept = np.flatnonzero(sel_oracle[i, J])
    if kept.size == 0 or p >= 1.0:
        score_tie = np.zeros(len(J), bool)
    else:
        last = kept[np.argmax(rank[kept])]  # the oracle's last kept block in sorted order
        lv = L[i, J]
        score_tie = np.abs(lv - lv[last]) <= LOGIT_TOL * max(1.0, abs(lv[last]))
    return mass_tie, score_tie


def compare_masks(gpu_mask: np.ndarray, oracle: dict, p: float, causal: bool) -> dict:
    """Classify every differing block of gpu_mask [b, H, nb, nb] against the oracle."""
    stats = {"blocks": 0, "mismatch": 0, "mass_tie": 0, "score_tie": 0, "unexcused": 0, "where": []}
    for (bb, h), r in oracle.items():
        g = gpu_mask[bb, h]
        o = r["mask"]
        nb = o.shape[0]
        stats["blocks"] += int(np.tril(np.ones((nb, nb))).sum()) if causal else nb * nb
        diff = np.argwhere(g != o)
        for i in np.unique(diff[:, 0]) if diff.size else []:
            J = po.admissible(int(i), nb, causal)
            cols = diff[diff[:, 0] == i, 1]
            flags = [_branch_excuses(r[f"S_{z}"], r[f"L_{z}"], r[f"m_{z}"], int(i), J, p) for z in ("high", "low")]
            for j in cols:
                stats["mismatch"] += 1
                if j >= len(J):  # outside the admissible range: never excusable
                    stats["unexcused"] += 1
                    stats["where"].append((bb, h, int(i), int(j)))
                    continue
                if any(f[0][j] for f in flags):
                    stats["mass_tie"] += 1
                elif any(f[1][j] for f in flags):
                    stats["score_tie"] += 1
                else:
                    stats["unexcused"] += 1
                    stats["where"].append((bb, h, int(i), int(j)))
    return stats


def gpu_to_np_mask(m) -> np.ndarray:
    return m.cpu().numpy()


def bf16_tensor_to_f64(t) -> np.ndarray:
    import torch
    return t.float().cpu().numpy().astype(np.float64) if t.dtype == torch.bfloat16 else t.cpu().numpy().astype(np.float64)


def logit_row(i, nb, causal):
    """start (floats) of row i of a logit plane: packed lower triangle with
    rows padded to 4 floats when causal, rows of round_up(nb, 4) otherwise"""
    if not causal:
        return i * ((nb + 3) // 4 * 4)
    q, r = i // 4, i % 4
    return 8 * q * (q + 1) + 4 * r * (q + 1)


def pack_bits(m: np.ndarray) -> np.ndarray:
    """uint8 block mask [..., nb] -> the bit-packed form [..., ceil(nb / 32)]
    int32 (bit j % 32 of word j / 32 set when block j is nonzero)."""
    nb = m.shape[-1]
    W = -(-nb // 32)
    pad = np.zeros(m.shape[:-1] + (W * 32,), np.uint64)
    pad[..., :nb] = m != 0
    words = (pad.reshape(m.shape[:-1] + (W, 32)) << np.arange(32, dtype=np.uint64)).sum(-1)
    return words.astype(np.uint32).view(np.int32)


def unpack_bits(w: np.ndarray, nb: int) -> np.ndarray:
    """Inverse of pack_bits: [..., W] int32 -> uint8 [..., nb]."""
    u = w.view(np.uint32).astype(np.uint64)
    bits = (u[..., None] >> np.arange(32, dtype=np.uint64)) & np.uint64(1)
    return bits.reshape(w.shape[:-1] + (w.shape[-1] * 32,))[..., :nb].astype(np.uint8)
