"""Pins of the CPU oracle to facts fixed by the Prism pages and by mathematics.

Each check is written as a function that returns an error measure, so the
planted-mistake tests at the bottom can show that a plausible slip in the
oracle (swapped bands, a dropped scale, a strict inequality, a missing causal
mask) makes a pin fail.
"""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle.prism_oracle as po
from synth import WORKLOADS, apply_rope, rope_tables

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                key, val = line.split()
                vals[key] = float(val)
    return vals


def dirichlet(B, theta):
    """|mean_{m<B} exp(i m theta)| = |sin(B theta/2) / (B sin(theta/2))|, signed."""
    return np.sin(B * theta / 2) / (B * np.sin(theta / 2))


def freqs(d, base):
    return base ** (-2.0 * np.arange(d // 2) / d)


# --------------------------------------------------------------- golden values
def test_hyperparameters_match_pages():
    g = read_golden("prism_hyperparameters.txt")
    for name, w in WORKLOADS.items():
        assert w.block == g["block_size"] and w.d_high == g["d_high"] and w.d_low == g["d_low"], name
        assert w.p == (g["p_qwen"] if name.startswith("qwen") else g["p_llama"]), name


# ------------------------------------------- pin 1: pooling under RoPE (closed form)
def pooling_decay_error(base, B=128, d=128, block_index=3):
    """Pool RoPE-rotated unit pairs over one block and compare the pooled pair
    with the closed form: amplitude D_B(theta_j), phase at the block centre.
    Returns (max err vs Dirichlet form, max err of |pooled| vs |sinc|)."""
    N = (block_index + 1) * B
    cos, sin = rope_tables(N, d, base)
    x = np.zeros((N, d))
    x[:, 0::2] = 1.0  # every pair starts as the unit vector (1, 0)
    xr = apply_rope(x, cos, sin, "interleaved")
    pooled = po.mean_pool(xr, B)[block_index]
    th = freqs(d, base)
    centre = block_index * B + (B - 1) / 2.0
    amp = dirichlet(B, th)
    expect = np.empty(d)
    expect[0::2] = amp * np.cos(centre * th)
    expect[1::2] = amp * np.sin(centre * th)
    err_exact = np.abs(pooled - expect).max()
    lam = np.hypot(pooled[0::2], pooled[1::2])
    # the pages' closed form: lambda_j(B) ~ sinc(B theta_j / 2 pi) (normalised sinc)
    err_sinc = np.abs(lam - np.abs(np.sinc(B * th / (2 * np.pi)))).max()
    return err_exact, err_sinc


@pytest.mark.parametrize("base", [1e4, 5e5, 1e6])
def test_pooling_is_lowpass_sinc(base):
    """Prism review, novelty paragraph: mean pooling under RoPE attenuates pair j
    by lambda_j(B) ~ sinc(B theta_j / 2 pi)."""
    e_exact, e_sinc = pooling_decay_error(base)
    assert e_exact < 1e-12
    assert e_sinc < 1e-3


def test_pooling_dead_zone():
    """gist.science Technical Summary 1: the fastest-rotating pairs collapse to
    near zero after pooling, the slowest pass through."""
    th = freqs(128, 5e5)
    lam = np.abs(dirichlet(128, th))
    assert lam[:8].max() < 0.05 and lam[-4:].min() > 0.99


# --------------------------------- pin 2: RMS and temperature (closed form)
def tau_closed_form_error(rope_layout, d_high, d_low, base=5e5, B=64, nb=5, seed=0):
    """Q = K = RoPE(x) for a constant pre-rotation x over full blocks: each pair's
    pooled energy is D_B(theta_j)^2 |x_j|^2 in every block, so
    tau_z = [sum_{j in F_z} D^2 |x_j|^2 / |D_z|] / [sum_j D^2 |x_j|^2 / d]."""
    d = 128
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(d)
    N = nb * B
    cos, sin = rope_tables(N, d, base)
    xr = apply_rope(np.tile(x, (N, 1)), cos, sin, rope_layout)
    r = po.estimate_head(xr, xr, block=B, d_high=d_high, d_low=d_low, p=0.9, rope_layout=rope_layout)
    D2 = dirichlet(B, freqs(d, base)) ** 2
    if rope_layout == "interleaved":
        e = x[0::2] ** 2 + x[1::2] ** 2
    else:
        e = x[: d // 2] ** 2 + x[d // 2:] ** 2
    pair = D2 * e
    F_hi = np.arange(0, d_high // 2)
    F_lo = np.arange(d // 2 - d_low // 2, d // 2)
    full = pair.sum() / d
    t_hi = (pair[F_hi].sum() / (2 * len(F_hi))) / full
    t_lo = (pair[F_lo].sum() / (2 * len(F_lo))) / full
    r_hi = math.sqrt(pair[F_hi].sum() / (2 * len(F_hi)))
    rel = lambda a, b: abs(a - b) / abs(b)
    return max(rel(r["tau"][0], t_hi), rel(r["tau"][1], t_lo), rel(r["rms_q"][0], r_hi),
               rel(r["rms_k"][2], math.sqrt(full)))


@pytest.mark.parametrize("rope_layout", ["interleaved", "half"])
@pytest.mark.parametrize("d_high,d_low", [(64, 96), (32, 112), (48, 48), (128, 128)])
def test_tau_closed_form(rope_layout, d_high, d_low):
    assert tau_closed_form_error(rope_layout, d_high, d_low) < 1e-12


def test_tau_unit_closed_form_and_pervec_equals_fullspec_on_constant_blocks():
    """The rejected readings on the same construction: 'unit' gives
    tau_z = R(Qbar,D_z) R(Kbar,D_z) = sum_{j in F_z} D^2 |x_j|^2 / |D_z|; every
    pooled block is the same vector, so the per-vector RMS equals the head's
    and 'pervec' logits equal the adopted reading's."""
    d, B, nb, base = 128, 64, 5, 5e5
    x = np.random.default_rng(0).standard_normal(d)
    cos, sin = rope_tables(nb * B, d, base)
    xr = apply_rope(np.tile(x, (nb * B, 1)), cos, sin, "interleaved")
    kw = dict(block=B, d_high=64, d_low=96, p=0.9)
    u = po.estimate_head(xr, xr, tau_mode="unit", **kw)
    f = po.estimate_head(xr, xr, **kw)
    v = po.estimate_head(xr, xr, tau_mode="pervec", **kw)
    pair = dirichlet(B, freqs(d, base)) ** 2 * (x[0::2] ** 2 + x[1::2] ** 2)
    assert abs(u["tau"][0] - pair[:32].sum() / 64) < 1e-12 * u["tau"][0]
    assert abs(u["tau"][1] - pair[16:].sum() / 96) < 1e-12 * u["tau"][1]
    assert v["tau"] == (1.0, 1.0)
    for key in ("L_high", "L_low"):
        fin = np.isfinite(f[key])
        assert np.array_equal(fin, np.isfinite(v[key]))
        assert np.abs(v[key][fin] - f[key][fin]).max() <= 1e-12 * np.abs(f[key][fin]).max()


def test_tau_unit_logits_invariant_to_scaling_q_and_k():
    """Unit-energy normalisation divides out the scale of Q and K."""
    rng = np.random.default_rng(5)
    q, k = rng.standard_normal((700, 128)), rng.standard_normal((700, 128))
    a = po.estimate_head(q, k, block=128, d_high=64, d_low=96, p=0.95, tau_mode="unit")
    b = po.estimate_head(3.7 * q, 0.2 * k, block=128, d_high=64, d_low=96, p=0.95, tau_mode="unit")
    fin = np.isfinite(a["L_high"])
    for key in ("L_high", "L_low"):
        assert np.allclose(a[key][fin], b[key][fin], rtol=1e-12, atol=0)
    assert np.array_equal(a["mask"], b["mask"])


def test_tau_pervec_is_band_rescaled_to_own_full_rms():
    """Per-vector reading by another route: rescale each pooled vector's band
    to the RMS of its own full spectrum, then take the plain band dot
    product / sqrt(d_z)."""
    rng = np.random.default_rng(6)
    q = rng.standard_normal((900, 128)) * np.linspace(0.2, 2.0, 128)
    k = rng.standard_normal((900, 128)) * np.linspace(2.0, 0.3, 128)
    r = po.estimate_head(q, k, block=128, d_high=64, d_low=96, p=0.95, tau_mode="pervec", causal=False)
    qb, kb = r["qbar"], r["kbar"]
    for key, dims in (("L_high", np.arange(64)), ("L_low", np.arange(32, 128))):
        qz = qb[:, dims] * (np.linalg.norm(qb, axis=1) / math.sqrt(128) /
                            (np.linalg.norm(qb[:, dims], axis=1) / math.sqrt(len(dims))))[:, None]
        kz = kb[:, dims] * (np.linalg.norm(kb, axis=1) / math.sqrt(128) /
                            (np.linalg.norm(kb[:, dims], axis=1) / math.sqrt(len(dims))))[:, None]
        want = qz @ kz.T / math.sqrt(len(dims))
        assert np.abs(r[key] - want).max() <= 1e-12 * np.abs(want).max()


@pytest.mark.parametrize("mode", ["unit", "pervec"])
def test_rejected_readings_reduce_to_plain_pooling_with_equal_bands(mode, monkeypatch):
    """With D_z = D_full the per-vector factors are 1; 'unit' rescales both
    branches alike, so both branches still select the same blocks."""
    rng = np.random.default_rng(7)
    q, k = rng.standard_normal((300, 128)), rng.standard_normal((300, 128))
    base = po.estimate_head(q, k, block=32, d_high=128, d_low=128, p=0.8, tau_mode="none")
    r = po.estimate_head(q, k, block=32, d_high=128, d_low=128, p=0.8, tau_mode=mode)
    assert np.array_equal(r["m_high"], r["m_low"])
    if mode == "pervec":
        fin = np.isfinite(base["L_high"])
        assert np.allclose(r["L_high"][fin], base["L_high"][fin], rtol=1e-12, atol=0)
        assert np.array_equal(r["mask"], base["mask"])


def test_tau_attenuated_high_band_is_amplified():
    """gist.science 2B: the high branch's pooled logits are attenuated, and the
    calibration restores them (tau_high < 1 divides the logits up)."""
    w = WORKLOADS["llama3_8b_32k"].scaled(seq=4096, hq=1, hkv=1)
    from synth import make_qkv, to_f64
    q, k, _ = make_qkv(w, with_v=False)
    r = po.estimate_head(to_f64(q, w.dtype)[0, :, 0], to_f64(k, w.dtype)[0, :, 0], block=128,
                         d_high=64, d_low=96, p=0.95)
    assert r["tau"][0] < 1.0 < r["tau"][1]


def test_tau_scale_invariant():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((700, 128))
    k = rng.standard_normal((700, 128))
    a = po.estimate_head(q, k, block=128, d_high=64, d_low=96, p=0.95)
    b = po.estimate_head(3.7 * q, 0.2 * k, block=128, d_high=64, d_low=96, p=0.95)
    assert np.allclose(a["tau"], b["tau"], rtol=1e-12, atol=0)


def test_tau_degenerate_is_one():
    q = np.zeros((256, 128))
    k = np.ones((256, 128))
    r = po.estimate_head(q, k, block=128, d_high=64, d_low=96, p=0.95)
    assert r["tau"] == (1.0, 1.0) and r["degenerate"] == 2


# --------------- special case: equal bands = plain mean-pooled block attention
def brute_topp(s, p):
    """Minimal-cardinality subset with mass >= p, by enumeration; returns (k, best mass set)."""
    n = len(s)
    for kk in range(1, n + 1):
        best, best_set = -1.0, None
        for c in itertools.combinations(range(n), kk):
            m = s[list(c)].sum()
            if m > best:
                best, best_set = m, set(c)
        if best >= p:
            return kk, best_set
    return n, set(range(n))


def plain_pooled_error(causal, seed=2, B=16, N=139, d=128, p=0.8):
    """d_high = d_low = d: tau = 1 and both branches equal plain pooled attention
    softmax(Qbar Kbar^T / sqrt(d)) with Top-P, checked with scipy's softmax and
    brute-force subset enumeration. Returns the number of violations."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((N, d)) + 0.3 * rng.standard_normal(d)
    k = rng.standard_normal((N, d)) + 0.3 * rng.standard_normal(d)
    r = po.estimate_head(q, k, block=B, d_high=d, d_low=d, p=p, causal=causal)
    bad = 0
    bad += r["tau"] != (1.0, 1.0)
    nb = -(-N // B)
    qb = np.stack([q[i * B:(i + 1) * B].sum(0) / len(q[i * B:(i + 1) * B]) for i in range(nb)])
    kb = np.stack([k[i * B:(i + 1) * B].sum(0) / len(k[i * B:(i + 1) * B]) for i in range(nb)])
    logits = np.einsum("id,jd->ij", qb, kb) / math.sqrt(d)
    for i in range(nb):
        J = list(range(i + 1)) if causal else list(range(nb))
        s = scipy.special.softmax(logits[i, J])
        bad += np.abs(r["S_high"][i, J] - s).max() > 1e-12
        kk, best = brute_topp(s, p)
        sel = set(np.flatnonzero(r["m_high"][i, J]).tolist())
        bad += sel != best or len(sel) != kk
        bad += not np.array_equal(r["m_high"][i], r["m_low"][i])
        bad += not np.array_equal(r["mask"][i], r["m_high"][i])
    return bad


@pytest.mark.parametrize("causal", [True, False])
def test_equal_bands_reduce_to_plain_pooling(causal):
    assert plain_pooled_error(causal) == 0


# ------------------------------------------------------------- softmax rows
def test_softmax_rows():
    rng = np.random.default_rng(3)
    qb, kb = rng.standard_normal((12, 128)), rng.standard_normal((12, 128))
    hi, _, _ = po.band_dims(128, 64, 96)
    L, S = po.band_scores(qb, kb, hi, 0.7, causal=True)
    for i in range(12):
        assert abs(S[i, : i + 1].sum() - 1) < 1e-14
        assert np.all(S[i, i + 1:] == 0) and np.all(np.isneginf(L[i, i + 1:]))
        assert np.abs(S[i, : i + 1] - scipy.special.softmax(L[i, : i + 1])).max() < 1e-15


# ------------------------------------------------------- pin 3: Top-P invariants
def topp_violations(trials=300, seed=4):
    rng = np.random.default_rng(seed)
    bad = 0
    for _ in range(trials):
        n = int(rng.integers(1, 11))
        s = scipy.special.softmax(rng.standard_normal(n) * rng.uniform(0.1, 4))
        p = float(rng.uniform(0.05, 0.999))
        sel = po.top_p(s, p)
        mass = s[sel].sum()
        kk, best = brute_topp(s, p)
        bad += sel.sum() != kk
        bad += mass < p and sel.sum() != n
        bad += set(np.flatnonzero(sel).tolist()) != best
        if (~sel).any():
            bad += s[sel].min() < s[~sel].max()
        if sel.sum() > 1:
            bad += mass - s[sel].min() >= p  # minimal: dropping the smallest falls short
    return bad


def test_top_p_bruteforce_and_invariants():
    assert topp_violations() == 0


def hand_topp_violations():
    bad = 0
    bad += not po.top_p(np.array([0.2, 0.3, 0.5]), 1.0).all()
    bad += po.top_p(np.array([0.0, 1.0, 0.0]), 0.95).tolist() != [False, True, False]
    for n, p in [(7, 0.95), (16, 0.95), (30, 0.95), (10, 0.93)]:
        bad += po.top_p(np.full(n, 1.0 / n), p).sum() != math.ceil(p * n)
    # equal scores: the lower block index goes first
    bad += po.top_p(np.array([0.25, 0.25, 0.25, 0.25]), 0.5).tolist() != [True, True, False, False]
    bad += po.top_p(np.array([0.1, 0.3, 0.3, 0.3]), 0.55).tolist() != [False, True, True, False]
    return bad


def test_top_p_hand_cases():
    assert hand_topp_violations() == 0


# ------------------------------------------------- pin 4: union and causality
def small_estimate(seed=5, N=1000, B=64, causal=True):
    rng = np.random.default_rng(seed)
    s = rng.standard_normal(128)
    cos, sin = rope_tables(N, 128, 1e4)
    q = apply_rope(0.7 * s + 0.7 * rng.standard_normal((N, 128)), cos, sin, "interleaved")
    k = apply_rope(0.7 * s + 0.7 * rng.standard_normal((N, 128)), cos, sin, "interleaved")
    return po.estimate_head(q, k, block=B, d_high=64, d_low=96, p=0.9, causal=causal)


def test_union_semantics():
    r = small_estimate()
    M, Mh, Ml = r["mask"].astype(bool), r["m_high"].astype(bool), r["m_low"].astype(bool)
    assert (M >= Mh).all() and (M >= Ml).all() and (M <= (Mh | Ml)).all()
    assert np.array_equal(po.union(r["m_low"], r["m_high"]), r["mask"])
    assert (Mh != Ml).any()  # the two branches really differ on this input
    assert M.sum(axis=1).min() >= 1  # Top-P keeps at least the argmax


def test_mask_causal_upper_triangle_zero():
    r = small_estimate()
    assert not np.triu(r["mask"], 1).any()
    r = small_estimate(causal=False)
    assert np.triu(r["mask"], 1).any()


def test_attention_causal_perturbation():
    rng = np.random.default_rng(6)
    N, B, d = 300, 64, 128
    q, k, v = (rng.standard_normal((1, N, 1, d)) for _ in range(3))
    nb = -(-N // B)
    mask = np.tril(np.ones((1, 1, nb, nb), np.uint8))
    o1 = po.block_sparse_attention(q, k, v, mask, block=B)
    t0 = 150
    k2, v2 = k.copy(), v.copy()
    k2[:, t0 + 1:] = rng.standard_normal(k2[:, t0 + 1:].shape)
    v2[:, t0 + 1:] = rng.standard_normal(v2[:, t0 + 1:].shape)
    o2 = po.block_sparse_attention(q, k2, v2, mask, block=B)
    assert np.array_equal(o1[:, : t0 + 1], o2[:, : t0 + 1])
    assert not np.array_equal(o1[:, t0 + 1:], o2[:, t0 + 1:])


# ----------------------------------------- pin 5: all blocks = dense attention
def sdpa(q, k, v, causal, attn_mask=None):
    """torch reference in float64 on the CPU: q [b,N,H,d], k/v [b,N,Hkv,d]."""
    G = q.shape[2] // k.shape[2]
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=attn_mask, is_causal=causal)
    return o.permute(0, 2, 1, 3).numpy()


def dense_error(causal, N=333, B=64, Hq=4, Hkv=2, seed=7):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((2, N, Hq, 128))
    k = rng.standard_normal((2, N, Hkv, 128))
    v = rng.standard_normal((2, N, Hkv, 128))
    nb = -(-N // B)
    mask = np.ones((2, Hq, nb, nb), np.uint8)
    o = po.block_sparse_attention(q, k, v, mask, block=B, causal=causal)
    return np.abs(o - sdpa(q, k, v, causal)).max()


@pytest.mark.parametrize("causal", [True, False])
def test_all_blocks_equals_dense(causal):
    assert dense_error(causal) < 1e-12


def test_diagonal_mask_is_block_local():
    rng = np.random.default_rng(8)
    N, B = 300, 64
    q, k, v = (rng.standard_normal((1, N, 1, 128)) for _ in range(3))
    nb = -(-N // B)
    mask = np.eye(nb, dtype=np.uint8)[None, None]
    o = po.block_sparse_attention(q, k, v, mask, block=B, causal=True)
    t = np.arange(N)
    allowed = (t[None, :] // B == t[:, None] // B) & (t[None, :] <= t[:, None])
    ref = sdpa(q, k, v, False, attn_mask=torch.from_numpy(allowed))
    assert np.abs(o - ref).max() < 1e-12


def test_empty_row_outputs_zero():
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((1, 256, 1, 128)) for _ in range(3))
    mask = np.array([[[[1, 0], [0, 0]]]], np.uint8)
    o = po.block_sparse_attention(q, k, v, mask, block=128)
    assert np.all(o[0, 128:] == 0) and np.abs(o[0, :128]).sum() > 0


# ------------------------------------------- grouped-query head mapping
def gqa_estimate_error(Hq=6, Hkv=2, N=1000, seed=12):
    """The estimator on a GQA input against the same heads run as plain
    multi-head attention on K repeated G times along the head axis with
    torch.repeat_interleave (the grouping torch's attention uses). Returns the
    number of differing mask entries plus the largest temperature difference."""
    w = WORKLOADS["llama3_8b_32k"].scaled(seq=N, hq=Hq, hkv=Hkv)
    from synth import make_qkv, to_f64
    q, k, _ = make_qkv(w, with_v=False)
    q64, k64 = to_f64(q, "bf16"), to_f64(k, "bf16")
    G = Hq // Hkv
    k_rep = torch.from_numpy(k64).repeat_interleave(G, dim=2).numpy()
    kw = dict(block=128, d_high=64, d_low=96, p=0.9, causal=True)
    a = po.estimate(q64, k64, **kw)
    b = po.estimate(q64, k_rep, **kw)
    return int((a["mask"] != b["mask"]).sum()) + float(np.abs(a["tau"] - b["tau"]).max())


def gqa_attention_error(Hq=6, Hkv=2, N=300, B=64, seed=13):
    """All-blocks attention on GQA input against torch's own grouped-query
    attention (scaled_dot_product_attention with enable_gqa), fp64 on the CPU."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, N, Hq, 128))
    k = rng.standard_normal((1, N, Hkv, 128))
    v = rng.standard_normal((1, N, Hkv, 128))
    nb = -(-N // B)
    mask = np.ones((1, Hq, nb, nb), np.uint8)
    o = po.block_sparse_attention(q, k, v, mask, block=B, causal=True)
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, enable_gqa=True)
    return float(np.abs(o - ref.permute(0, 2, 1, 3).numpy()).max())


def test_gqa_mapping_estimate_matches_repeated_kv():
    assert gqa_estimate_error() == 0
    assert gqa_estimate_error(Hq=8, Hkv=2) == 0


def test_gqa_mapping_attention_matches_torch_gqa():
    assert gqa_attention_error() < 1e-12
    assert gqa_attention_error(Hq=8, Hkv=4) < 1e-12


# ------------------------------------------- merge variants (weaknesses paragraph)
def merge_case(merge, d_high=64, d_low=96, p=0.9, seed=31):
    w = WORKLOADS["llama3_8b_32k"].scaled(seq=2600, hq=2, hkv=1, seed=seed)
    from synth import make_qkv, to_f64
    q, k, _ = make_qkv(w, with_v=False)
    return po.estimate(to_f64(q, "bf16"), to_f64(k, "bf16"), block=128, d_high=d_high, d_low=d_low, p=p,
                       merge=merge, keep=True)


def intersect_error():
    """intersection = blocks both branches keep: a subset of each branch and
    of the union, and equal to them when the bands coincide"""
    r = merge_case("intersect")
    bad = 0
    for key, rr in r["per_head"].items():
        m = rr["mask"].astype(bool)
        bad += int((m & ~rr["m_high"].astype(bool)).sum() + (m & ~rr["m_low"].astype(bool)).sum())
        bad += int((rr["m_high"].astype(bool) & rr["m_low"].astype(bool) & ~m).sum())
    same = merge_case("intersect", d_high=128, d_low=128)
    for rr in same["per_head"].values():
        bad += int((rr["mask"] != rr["m_high"]).sum())
    return bad


def mix_bruteforce_error(trials=200, seed=5):
    """weighted merge on random tiny rows: the kept set is the minimum-size
    subset of the mixture (S_high + S_low) / 2 whose mass reaches p (found
    by enumeration); the kept mass reaches p"""
    rng = np.random.default_rng(seed)
    bad = 0
    for _ in range(trials):
        n = int(rng.integers(1, 10))
        sh, sl = rng.dirichlet(np.ones(n) * 0.7), rng.dirichlet(np.ones(n) * 0.7)
        p = float(rng.uniform(0.3, 0.99))
        # square non-causal score matrices (every row the same distribution); row 0 is checked
        sel = po.mix_mask(np.tile(sh, (n, 1)), np.tile(sl, (n, 1)), p, causal=False)[0].astype(bool)
        mixv = 0.5 * (sh + sl)
        best = None
        for size in range(1, n + 1):
            for sub in itertools.combinations(range(n), size):
                if mixv[list(sub)].sum() >= p:
                    best = size
                    break
            if best:
                break
        bad += int(sel.sum() != best) + int(mixv[sel].sum() < p - 1e-12)
    return bad


def test_intersect_semantics():
    assert intersect_error() == 0


def test_mix_is_top_p_of_the_equal_weight_mixture():
    assert mix_bruteforce_error() == 0
    # identical branches: the mixture is the branch itself
    same = merge_case("mix", d_high=128, d_low=128)
    for rr in same["per_head"].values():
        assert np.array_equal(rr["mask"], rr["m_high"])


# ------------------------------------------- per-head adaptive band split
def spectral_heads(profiles, layout="interleaved", base=5e5, B=128, nb=6):
    """Query heads whose pre-rotation vector is one constant x_h per head
    (|x_h pair j|^2 = profiles[h][j]) and one KV head with x = 1 in every
    pair, over nb full blocks; returns q, k [1, N, H, d] post-RoPE."""
    d = 128
    N = nb * B
    cos, sin = rope_tables(N, d, base)
    H = len(profiles)
    q = np.zeros((1, N, H, d))
    for h, prof in enumerate(profiles):
        x = np.zeros(d)
        amp = np.sqrt(np.asarray(prof, float))
        if layout == "interleaved":
            x[0::2] = amp
        else:
            x[: d // 2] = amp
        q[0, :, h, :] = apply_rope(np.tile(x, (N, 1)), cos, sin, layout)
    xk = np.zeros(d)
    if layout == "interleaved":
        xk[0::2] = 1.0
    else:
        xk[: d // 2] = 1.0
    k = apply_rope(np.tile(xk, (N, 1)), cos, sin, layout)[None, :, None, :]
    return q, k


def closed_form_split(profiles, base=5e5, B=128, d_high=64, d_low=96):
    """The split rule evaluated on the closed-form pooled spectra: pair j of a
    constant vector pooled over a full block keeps D_B(theta_j)^2 of its
    energy (Dirichlet kernel), so P_j = D^2 |x_j|^2 * D^2 * 1."""
    th = freqs(128, base)
    D2 = dirichlet(B, th) ** 2
    spectra = np.stack([D2 * np.asarray(prof, float) * D2 for prof in profiles])
    mean = spectra.mean(axis=0)
    share = mean[: d_high // 2].sum() / mean.sum()
    o = (d_high + d_low - 128) // 2
    out = []
    for P in spectra:
        c = np.cumsum(P) / P.sum()
        jh = next(j for j in range(max(8, o), 64 - 8 + 1, 8) if c[j - 1] >= share * (1 - 1e-9))
        out.append((2 * jh, 128 - 2 * (jh - o)))
    return out


def adaptive_split_error(layout="interleaved"):
    """oracle splits vs the closed form on heads whose energy sits in slow,
    fast, transition and all pairs (the cases differ by at least 8 pairs)"""
    j = np.arange(64)
    profiles = [np.ones(64), (j >= 40).astype(float), ((j >= 12) & (j < 36)).astype(float) + 0.01,
                np.exp(-j / 10.0)]
    q, k = spectral_heads(profiles, layout)
    r = po.estimate(q, k, block=128, d_high=64, d_low=96, p=0.9, band_mode="adaptive", rope_layout=layout)
    got = [tuple(x) for x in r["bands"][0].tolist()]
    want = closed_form_split(profiles)
    return got, want


@pytest.mark.parametrize("layout", ["interleaved", "half"])
def test_adaptive_split_closed_form(layout):
    got, want = adaptive_split_error(layout)
    assert got == want
    assert len(set(want)) >= 3  # the heads really get different splits
    assert all(dh + dl == 160 for dh, dl in want)


def test_adaptive_split_identical_heads_keep_static():
    """every head with the same spectrum (here the same input) gets the static
    split back, whatever the spectrum; scaling all queries changes nothing"""
    j = np.arange(64)
    for prof in (np.ones(64), np.exp(-j / 7.0), (j % 3 == 0).astype(float) + 0.1):
        q, k = spectral_heads([prof, prof, prof])
        for scale in (1.0, 37.0):
            r = po.estimate(q * scale, k, block=128, d_high=64, d_low=96, p=0.9, band_mode="adaptive")
            assert r["bands"][0].tolist() == [[64, 96]] * 3


# --------------------------------------------- planted mistakes must be caught
def test_planted_swapped_bands_caught(monkeypatch):
    good = po.band_dims

    def swapped(d, dh, dl, layout="interleaved"):
        hi, lo, full = good(d, dh, dl, layout)
        return lo, hi, full

    monkeypatch.setattr(po, "band_dims", swapped)
    assert tau_closed_form_error("interleaved", 64, 96) > 1e-3


def test_planted_rms_without_sqrt_caught(monkeypatch):
    monkeypatch.setattr(po, "band_rms", lambda xb, dims: float(np.mean(xb[:, dims] ** 2)))
    assert tau_closed_form_error("interleaved", 64, 96) > 1e-3


def test_planted_inverted_tau_caught(monkeypatch):
    good = po.temperature

    def inverted(*a, **kw):
        t, deg = good(*a, **kw)
        return 1.0 / t, deg

    monkeypatch.setattr(po, "temperature", inverted)
    assert tau_closed_form_error("interleaved", 64, 96) > 1e-3


def test_planted_half_layout_bands_caught(monkeypatch):
    good = po.band_dims
    # slicing the first d_high physical dims of a rotate-half tensor (the rejected reading)
    monkeypatch.setattr(po, "band_dims", lambda d, dh, dl, layout="interleaved": good(d, dh, dl, "interleaved"))
    assert tau_closed_form_error("half", 64, 96) > 1e-3


def test_planted_missing_sqrt_d_caught(monkeypatch):
    good = po.band_scores

    def no_sqrt(qbar, kbar, dims, tau, causal, fq=None, fk=None):
        return good(qbar, kbar, dims, tau / math.sqrt(len(dims)), causal, fq, fk)

    monkeypatch.setattr(po, "band_scores", no_sqrt)
    assert plain_pooled_error(True) > 0


def test_planted_strict_top_p_caught(monkeypatch):
    def strict(scores, p):
        n = len(scores)
        order = np.argsort(-scores, kind="stable")
        cum = np.cumsum(scores[order])
        reach = np.flatnonzero(cum > p)
        kk = reach[0] + 1 if reach.size else n
        sel = np.zeros(n, bool)
        sel[order[:kk]] = True
        return sel

    monkeypatch.setattr(po, "top_p", strict)
    assert hand_topp_violations() > 0


def test_planted_missing_causal_mask_caught(monkeypatch):
    good = po.attention_block_row
    monkeypatch.setattr(po, "attention_block_row",
                        lambda q, k, v, row, i, block, causal: good(q, k, v, row, i, block=block, causal=False))
    assert dense_error(True) > 1e-3


def test_planted_wrong_pool_divisor_caught(monkeypatch):
    def pool_by_B(x, block):
        N, d = x.shape
        nb = -(-N // block)
        out = np.zeros((nb, d))
        for i in range(nb):
            out[i] = x[i * block: (i + 1) * block].sum(0) / block
        return out

    monkeypatch.setattr(po, "mean_pool", pool_by_B)
    # a ragged last block (139 = 8*16 + 11) exposes the wrong divisor
    assert plain_pooled_error(True) > 0


def test_planted_interleaved_gqa_mapping_caught(monkeypatch):
    # query head h reading KV head h % Hkv instead of h // G
    monkeypatch.setattr(po, "kv_head", lambda h, hq, hkv: h % hkv)
    assert gqa_estimate_error() > 0
    assert gqa_attention_error() > 1e-3


def test_planted_union_for_intersection_caught(monkeypatch):
    monkeypatch.setattr(po, "intersect", po.union)
    assert intersect_error() > 0


def test_planted_mix_without_halving_caught(monkeypatch):
    # the mixture's two distributions added without the 1/2 weights: mass 2, p then reached too early
    monkeypatch.setattr(po, "mix_mask", lambda sh, sl, p, causal: po.top_p_mask(sh + sl, p, causal))
    assert mix_bruteforce_error() > 0


def test_planted_split_from_the_slow_end_caught(monkeypatch):
    # spectra read slowest pair first
    orig = po.pair_energy
    monkeypatch.setattr(po, "pair_energy", lambda xbar, layout="interleaved": orig(xbar, layout)[::-1])
    got, want = adaptive_split_error()
    assert got != want
