"""Block recall of Prism's estimator against plain mean pooling on the
Qwen3-8B-shaped workload with planted slash and vertical structure.

    python tests/recall_planted.py [--seq 16384] [--heads 4]

Ground truth is the dense causal attention itself (CPU, float64): for each
query block i and key block j, A[i, j] = mean over the block's queries of the
softmax mass on the keys of block j. For a block mask M the script reports
  density        selected fraction of the causal blocks,
  mass recall    sum(A * M) / sum(A), averaged over heads,
  planted recall fraction of the planted blocks that are selected: the
                 diagonal and the block before it (slash: keys carry the
                 query of 1-4 tokens later) and every key block holding a
                 token n = 0 mod 4096 (vertical),
for Prism (d_high=64, d_low=96, RMS-energy temperature), Prism without the
temperature, and plain mean pooling (one full band, no temperature) at the
same p and at the p that matches Prism's density. With --equal-recall it also
runs the two rejected temperature readings (unit-energy, per-vector RMS) and
reports, for every estimator, the density it needs to reach the mass recall
Prism has at the pages' p. --split-sweep does the same over a sweep of band
splits (d_high, d_low) with the adopted temperature. The estimators are the CPU
oracle's; the GPU path produces the same masks up to counted ties (it takes
any even band widths).
"""
from __future__ import annotations

import argparse
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle.prism_oracle as po  # noqa: E402
from synth import WORKLOADS, make_qkv, to_f64  # noqa: E402


def block_attention_mass(q64, k64, block):
    """A[h, i, j] for q [N, Hq, d], k [N, Hkv, d] (GQA), causal, float64."""
    N, Hq, d = q64.shape
    G = Hq // k64.shape[1]
    nb = -(-N // block)
    A = np.zeros((Hq, nb, nb))
    for h in range(Hq):
        kh = k64[:, h // G]
        for i in range(nb):
            t0, t1 = i * block, min((i + 1) * block, N)
            lg = q64[t0:t1, h] @ kh[:t1].T / np.sqrt(d)
            lg = np.where(np.arange(t1)[None, :] <= np.arange(t0, t1)[:, None], lg, -np.inf)
            pr = np.exp(lg - lg.max(1, keepdims=True))
            pr /= pr.sum(1, keepdims=True)
            for j in range(i + 1):
                A[h, i, j] = pr[:, j * block: min((j + 1) * block, t1)].sum(1).mean()
    return A


def planted_blocks(seq, block):
    nb = -(-seq // block)
    P = np.zeros((nb, nb), bool)
    for i in range(nb):
        P[i, i] = True
        if i:
            P[i, i - 1] = True
        for n in range(0, seq, 4096):
            if n // block <= i:
                P[i, n // block] = True
    return P


def masks(q64, k64, block, p, **kw):
    Hq = q64.shape[1]
    G = Hq // k64.shape[1]
    nb = -(-q64.shape[0] // block)
    M = np.zeros((Hq, nb, nb), bool)
    for h in range(Hq):
        M[h] = po.estimate_head(q64[:, h], k64[:, h // G], block=block, p=p, causal=True, **kw)["mask"].astype(bool)
    return M


def metrics(M, A, P):
    nb = M.shape[-1]
    tri = np.tril(np.ones((nb, nb), bool))
    density = M.sum() / (M.shape[0] * tri.sum())
    mass = float(((A * M).sum((1, 2)) / A.sum((1, 2))).mean())
    planted = (M & P[None]).sum() / (M.shape[0] * P.sum())
    return float(density), mass, float(planted)


PRISM = dict(d_high=64, d_low=96, tau_mode="fullspec")
PRISM_NO_TAU = dict(d_high=64, d_low=96, tau_mode="none")
PRISM_UNIT = dict(d_high=64, d_low=96, tau_mode="unit")
PRISM_PERVEC = dict(d_high=64, d_low=96, tau_mode="pervec")
PLAIN = dict(d_high=128, d_low=128, tau_mode="none")
ESTIMATORS = {"prism": PRISM, "prism_no_tau": PRISM_NO_TAU, "prism_unit_tau": PRISM_UNIT,
              "prism_pervec_tau": PRISM_PERVEC, "plain": PLAIN}


def p_for(target, metric_ix, q64, k64, A, P, block, kw, lo=0.3, hi=0.99999, iters=16):
    """Smallest p (bisection) at which metric `metric_ix` (0 density, 1 mass
    recall) of the estimator reaches `target`; returns (p, metrics)."""
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if metrics(masks(q64, k64, block, mid, **kw), A, P)[metric_ix] < target:
            lo = mid
        else:
            hi = mid
    return hi, metrics(masks(q64, k64, block, hi, **kw), A, P)


def run(seq=16384, heads=4, verbose=True, equal_recall=False):
    w = WORKLOADS["qwen3_8b_64k"].scaled(seq=seq, hq=heads, hkv=1)
    q, k, _ = make_qkv(w, with_v=False)
    q64, k64 = to_f64(q, "bf16")[0], to_f64(k, "bf16")[0]
    A = block_attention_mass(q64, k64, w.block)
    P = planted_blocks(w.seq, w.block)
    rows = {}
    rows["prism"] = (w.p,) + metrics(masks(q64, k64, w.block, w.p, **PRISM), A, P)
    rows["prism_no_tau"] = (w.p,) + metrics(masks(q64, k64, w.block, w.p, **PRISM_NO_TAU), A, P)
    rows["plain_same_p"] = (w.p,) + metrics(masks(q64, k64, w.block, w.p, **PLAIN), A, P)
    pm, m = p_for(rows["prism"][1], 0, q64, k64, A, P, w.block, PLAIN, lo=0.5, hi=0.9999, iters=14)
    rows["plain_density_matched"] = (pm,) + m
    recall = {}
    if equal_recall:
        # the temperature readings side by side: density each needs to reach
        # the mass recall Prism (adopted reading) has at the pages' p
        rows["prism_unit_tau"] = (w.p,) + metrics(masks(q64, k64, w.block, w.p, **PRISM_UNIT), A, P)
        rows["prism_pervec_tau"] = (w.p,) + metrics(masks(q64, k64, w.block, w.p, **PRISM_PERVEC), A, P)
        target = rows["prism"][2]
        for name, kw in ESTIMATORS.items():
            recall[name] = (target,) + p_for(target, 1, q64, k64, A, P, w.block, kw)
    if verbose:
        print(f"qwen3-shaped planted workload: seq={seq} heads={heads} (1 KV head), B=128")
        print(f"{'estimator':24s} {'p':>7s} {'density':>8s} {'mass recall':>12s} {'planted recall':>15s}")
        for name, (p, d, m, pr) in rows.items():
            print(f"{name:24s} {p:7.4f} {d:8.4f} {m:12.5f} {pr:15.4f}")
        if recall:
            print(f"at equal mass recall {next(iter(recall.values()))[0]:.5f}:")
            for name, (t, p, (d, m, pr)) in recall.items():
                print(f"{name:24s} {p:7.4f} {d:8.4f} {m:12.5f} {pr:15.4f}")
    return rows, A, P, recall


def split_sweep(seq=16384, heads=4, splits=((32, 96), (48, 96), (64, 96), (80, 96), (96, 96), (64, 64),
                                          (64, 80), (64, 112), (64, 128), (32, 112), (96, 64)), verbose=True):
    """Band-split ablation: for each (d_high, d_low), the density Prism needs
    to reach the mass recall the pages' split (64, 96) has at the pages' p."""
    w = WORKLOADS["qwen3_8b_64k"].scaled(seq=seq, hq=heads, hkv=1)
    q, k, _ = make_qkv(w, with_v=False)
    q64, k64 = to_f64(q, "bf16")[0], to_f64(k, "bf16")[0]
    A = block_attention_mass(q64, k64, w.block)
    P = planted_blocks(w.seq, w.block)
    target = metrics(masks(q64, k64, w.block, w.p, **PRISM), A, P)[1]
    out = {}
    for dh, dl in splits:
        kw = dict(d_high=dh, d_low=dl, tau_mode="fullspec")
        out[(dh, dl)] = p_for(target, 1, q64, k64, A, P, w.block, kw)
        if verbose:
            p, (d, m, pr) = out[(dh, dl)]
            print(f"d_high={dh:3d} d_low={dl:3d}  p={p:.4f} density={d:.4f} mass={m:.5f} planted={pr:.4f}", flush=True)
    return target, out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--seq", type=int, default=16384)
    ap.add_argument("--heads", type=int, default=4)
    ap.add_argument("--equal-recall", action="store_true",
                    help="also compare the temperature readings at equal mass recall")
    ap.add_argument("--split-sweep", action="store_true",
                    help="density at equal mass recall over a sweep of band splits")
    a = ap.parse_args()
    if a.split_sweep:
        split_sweep(a.seq, a.heads)
    else:
        run(a.seq, a.heads, equal_recall=a.equal_recall)
