"""Helpers shared by the GPU parity tests: moving synthetic inputs to the
device, running the oracle head by head, and comparing masks and outputs.

Mask rule: the GPU mask must equal the oracle's except at blocks whose
inclusion is decided within rounding. Two classes, each counted:
  * mass ties (the pass criterion's own class): in a branch, the oracle's
    cumulative mass before the block (exclusive) or through it (inclusive),
    in the oracle's sorted order, lies within MASS_TOL = 1e-4 of p;
  * key ties: in a branch, the oracle logits of the block and of its partner
    across that row's boundary (the first block the oracle drops, for a
    block it keeps; the last block it keeps, for one it drops) differ by at
    most 2 * LOGIT_TOL_REL * max(1, max_j |L_ij|) + KEY_ULP in log2 units.
    LOGIT_TOL_REL is the per-row bound on the GPU's fp32 band logits that the
    stage tests assert against the oracle's (so no pair further apart than
    twice it can change order), and KEY_ULP is one rounding of the fp32 key
    exp2(L - max), under which two logits closer than that can get equal
    keys, which the kernels order by block index.
A block the oracle keeps and the GPU drops needs an excuse in every branch
the oracle keeps it in; a block the oracle drops and the GPU keeps, in one
branch. Every other mismatch fails.
"""
from __future__ import annotations

import numpy as np

import oracle.prism_oracle as po
from synth import to_f64

MASS_TOL = 1e-4
# per-row bound on |GPU logit - oracle logit| (log2 units) relative to
# max(1, max_j |L_ij|); measured at full size: 4.2e-7 to 4.9e-7
LOGIT_TOL_REL = 4e-6
KEY_ULP = 2.0 ** -22  # one rounding of an fp32 key in [2^-k, 1], as a log2 difference (with margin)
LOG2E = 1.4426950408889634


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
                          tau_mode="fullspec", heads=None, merge="union", band_mode="static"):
    """Per-head oracle results {(b, h): dict} widening one head at a time
    (adaptive bands need every query head's spectrum, so they widen all)."""
    b, N, Hq, _ = q.shape
    Hkv = k.shape[2]
    if band_mode == "adaptive":
        r = po.estimate(to_f64(q, dtype), to_f64(k, dtype), block=block, d_high=d_high, d_low=d_low, p=p,
                        causal=causal, rope_layout=rope_layout, tau_mode=tau_mode, heads=heads, keep=True,
                        merge=merge, band_mode=band_mode)
        return r["per_head"]
    heads = range(Hq) if heads is None else heads
    out = {}
    kbars = {}
    for bb in range(b):
        for h in heads:
            g = po.kv_head(h, Hq, Hkv)
            if (bb, g) not in kbars:
                kbars[(bb, g)] = po.mean_pool(to_f64(k[bb, :, g, :], dtype), block)
            out[(bb, h)] = po.estimate_head(to_f64(q[bb, :, h, :], dtype), None, block=block, d_high=d_high,
                                            d_low=d_low, p=p, causal=causal, rope_layout=rope_layout,
                                            tau_mode=tau_mode, kbar=kbars[(bb, g)], merge=merge)
    return out


def key_tie_window(row_logits):
    """score/key-tie window (log2 units) of one row from its oracle logits (natural units)"""
    fin = row_logits[np.isfinite(row_logits)]
    lmax = float(np.abs(fin).max()) * LOG2E if fin.size else 0.0
    return 2.0 * LOGIT_TOL_REL * max(1.0, lmax) + KEY_ULP


def _branch_excuses(S, L, sel_oracle, i, J, p):
    """For one row i and branch: per admissible block, (mass-tie flag,
    key-tie flag, oracle gap to the boundary partner in log2 units)."""
    s = S[i, J]
    order = np.argsort(-s, kind="stable")
    cum = np.cumsum(s[order])
    excl = np.concatenate([[0.0], cum[:-1]])
    rank = np.empty_like(order)
    rank[order] = np.arange(len(order))
    mass_tie = (np.abs(excl[rank] - p) <= MASS_TOL) | (np.abs(cum[rank] - p) <= MASS_TOL)
    n = len(J)
    gap = np.full(n, np.inf)
    kept = sel_oracle[i, J].astype(bool)
    if 0 < kept.sum() < n and p < 1.0:
        lv = L[i, J]
        last = order[int(kept.sum()) - 1]   # the oracle keeps a prefix of its order
        first = order[int(kept.sum())]
        gap = np.where(kept, lv - lv[first], lv[last] - lv) * LOG2E
    key_tie = gap <= key_tie_window(L[i, J])
    return mass_tie, key_tie, gap


def decisions(r: dict, merge: str) -> list:
    """The Top-P decisions a head's mask is made of: the two branches (union,
    intersection) or the one on the equal-weight mixture; each as
    (name, S, L, kept) with L the natural-log scores."""
    if merge == "mix":
        S = 0.5 * (r["S_high"] + r["S_low"])
        with np.errstate(divide="ignore"):
            L = np.where(S > 0, np.log(np.where(S > 0, S, 1.0)), -np.inf)
        return [("mix", S, L, r["mask"])]
    return [("high", r["S_high"], r["L_high"], r["m_high"]), ("low", r["S_low"], r["L_low"], r["m_low"])]


def compare_masks(gpu_mask: np.ndarray, oracle: dict, p: float, causal: bool, merge: str = "union") -> dict:
    """Classify every differing block of gpu_mask [b, H, nb, nb] against the
    oracle (rule in the module docstring). Returns counts and, for the key
    ties, the largest oracle gap (log2 units) and its ratio to the window.
    Which decisions must be excused follows the merge: a union block the
    oracle keeps needs an excuse in every branch that keeps it, one it drops
    in some branch; an intersection block the oracle keeps needs one in some
    branch, one it drops in every branch that drops it; a mixture block in
    the one decision."""
    stats = {"blocks": 0, "mismatch": 0, "mass_tie": 0, "score_tie": 0, "unexcused": 0, "where": [],
             "max_key_gap": 0.0, "max_key_gap_over_window": 0.0}
    for (bb, h), r in oracle.items():
        g = gpu_mask[bb, h]
        o = r["mask"]
        nb = o.shape[0]
        stats["blocks"] += nb * (nb + 1) // 2 if causal else nb * nb
        diff = np.argwhere(g != o)
        dec = decisions(r, merge)
        for i in np.unique(diff[:, 0]) if diff.size else []:
            J = po.admissible(int(i), nb, causal)
            cols = diff[diff[:, 0] == i, 1]
            br = {name: _branch_excuses(S, L, m, int(i), J, p) for name, S, L, m in dec}
            win = {name: key_tie_window(L[i, J]) for name, S, L, m in dec}
            for j in cols:
                stats["mismatch"] += 1
                if j >= len(J):  # outside the admissible range: never excusable
                    stats["unexcused"] += 1
                    stats["where"].append((bb, h, int(i), int(j)))
                    continue
                kept_by = [name for name, S, L, m in dec if m[i, j]]
                dropped_by = [name for name, S, L, m in dec if not m[i, j]]
                if merge == "mix":
                    need, ok = ["mix"], all
                elif merge == "intersect":
                    need, ok = (list(br), any) if o[i, j] else (dropped_by, all)
                else:
                    need, ok = (kept_by, all) if o[i, j] else (list(br), any)
                if ok(br[z][0][j] for z in need):
                    stats["mass_tie"] += 1
                elif ok(br[z][0][j] or br[z][1][j] for z in need):
                    stats["score_tie"] += 1
                    for z in need:
                        if br[z][1][j] and not br[z][0][j]:
                            stats["max_key_gap"] = max(stats["max_key_gap"], float(br[z][2][j]))
                            stats["max_key_gap_over_window"] = max(stats["max_key_gap_over_window"],
                                                                    float(br[z][2][j]) / win[z])
                else:
                    stats["unexcused"] += 1
                    stats["where"].append((bb, h, int(i), int(j)))
    return stats


def logit_errors(gpu_logits: np.ndarray, oracle_logits: np.ndarray) -> tuple[float, float]:
    """GPU band logits (log2 units, -inf where not admissible) against the
    oracle's (natural units): (largest absolute error, largest per-row error
    relative to max(1, max_j |L_ij|)), both in log2 units."""
    ol = oracle_logits * LOG2E
    adm = np.isfinite(ol)
    assert np.array_equal(adm, np.isfinite(gpu_logits))
    err = np.where(adm, np.abs(gpu_logits - np.where(adm, ol, 0.0)), 0.0)
    scale = np.maximum(1.0, np.where(adm, np.abs(ol), 0.0).max(axis=1))
    return float(err.max()), float((err.max(axis=1) / scale).max())


def record_parity(name: str, stats: dict, extra: dict | None = None) -> None:
    """Append one configuration's mask comparison counts to the JSON-lines
    file named by the PRISM_PARITY_LOG environment variable (if set)."""
    import json
    import os
    path = os.environ.get("PRISM_PARITY_LOG")
    if not path:
        return
    rec = {"case": name, **{k: v for k, v in stats.items() if k != "where"}, **(extra or {})}
    with open(path, "a") as f:
        f.write(json.dumps(rec) + "\n")


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
