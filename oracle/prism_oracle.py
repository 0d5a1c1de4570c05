"""Plain float64 CPU oracle for Prism's spectral-aware block-importance
estimator and for the block-sparse causal attention that consumes its mask.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module. It shares no code with the HIP path
(it imports nothing from it), and the HIP path never calls it.

Sources (web pages about "Prism: Spectral-Aware Block-Sparse Attention",
arXiv 2602.08426):
  * Prism review, paper.rainbus.top -- the pipeline paragraph lists the seven
    steps (1) spectral slicing ... (7) mask union; the novelty paragraph gives
    the pooling decay lambda_j(B) ~ sinc(B*theta_j/2pi) and says the
    calibration is RMS-energy based with no hyperparameters; the
    reproducibility paragraph gives B=128, d_high=64, d_low=96, p=0.95/0.93.
  * gist.science explainer, Technical Summary section 2 (dual-band estimation;
    RMS of the pooled representations gives tau_high, tau_low) and section 1
    (block-sparse attention computes only the selected blocks).
  * Abstract (insight.artgrammer.co.kr / newx.sg / fugumt.com): block-sparse
    attention for long-context pre-filling, estimation from purely block-level
    operations.

Every function works in float64 on values widened exactly from the bytes the
GPU reads. Readings taken where the pages are silent:
  * bands are RoPE frequency bands: 'interleaved' layout -> the literal
    first d_high / last d_low dims; 'half' layout -> the same frequency pairs;
  * RMS is taken over all pooled blocks of a head, per tensor and per band;
  * tau_z = R(Qbar,D_z) R(Kbar,D_z) / (R(Qbar,D_full) R(Kbar,D_full))
    (the formula is named but not printed) -- parity unpinned against the
    pages; tau = 1 if any R is 0. Two rejected readings are kept for
    comparison: 'unit' (tau_z = R(Qbar,D_z) R(Kbar,D_z), unit-energy
    normalisation) and 'pervec' (the RMS taken per pooled vector, which scales
    each block's band to the energy density of its own full spectrum);
  * causal softmax over key blocks j <= i; Top-P keeps the smallest set of
    highest scores whose mass reaches p (inclusive), ties by lower index;
  * attention scale 1/sqrt(d); a query with no admissible key outputs 0;
  * a partial last block averages the tokens it holds.
The pages list two weaknesses without giving the remedy (Prism review,
weaknesses paragraph): the static band split and the union's over-selection.
The variants built for comparison, each a reading:
  * adaptive split: each head's high band ends at the smallest multiple of 8
    RoPE pairs at which the head's share of pooled spectral energy (the
    per-pair energy of Qbar times that of Kbar, fastest pair first) reaches
    the share the static high band holds in the mean spectrum of all query
    heads; the low band keeps the static overlap (so d_high + d_low is
    unchanged), and a layer whose heads share one spectrum gets the static
    split back;
  * merges: intersection (M_high AND M_low), and a weighted merge, one Top-P
    on the equal-weight mixture (S_high + S_low) / 2 of the two branches'
    block distributions.
"""
from __future__ import annotations

import numpy as np

ROPE_LAYOUTS = ("interleaved", "half")
TAU_MODES = ("fullspec", "none", "unit", "pervec")
MERGES = ("union", "intersect", "mix")
BAND_MODES = ("static", "adaptive")


# ---------------------------------------------------------------- step (1)
def band_dims(d: int, d_high: int, d_low: int, rope_layout: str = "interleaved"):
    """Index sets of the high band, the low band and the full spectrum.

    Prism review (paper.rainbus.top), pipeline step (1): Q and K are cut into
    a high band (the first d_high dims) and a low band (the last d_low dims).
    gist.science Technical Summary 2A: the high branch isolates the dims that
    carry fine relative position, the low branch the semantic dims.
    With interleaved RoPE (pair j = dims 2j, 2j+1, frequency falling with j)
    these are literally dims [0, d_high) and [d - d_low, d). With the
    rotate-half layout (pair j = dims j, j + d/2) the same frequency pairs are
    {j, j+d/2 : j < d_high/2} and {j, j+d/2 : j >= d/2 - d_low/2}.
    """
    if rope_layout == "interleaved":
        hi = np.arange(0, d_high)
        lo = np.arange(d - d_low, d)
    elif rope_layout == "half":
        h = d // 2
        hp = np.arange(0, d_high // 2)
        lp = np.arange(h - d_low // 2, h)
        hi = np.sort(np.concatenate([hp, hp + h]))
        lo = np.sort(np.concatenate([lp, lp + h]))
    else:
        raise ValueError(rope_layout)
    return hi, lo, np.arange(d)


# ---------------------------------------------------------------- step (2)
def mean_pool(x: np.ndarray, block: int) -> np.ndarray:
    """Mean over each block of `block` tokens: x [N, d] -> [ceil(N/B), d].

    Prism review, pipeline step (2): each band is mean-pooled over blocks of
    size B independently. Pooling all d dims once and taking the bands as
    index subsets afterwards gives the same numbers. Block i holds tokens
    [iB, min((i+1)B, N)); a partial last block averages the tokens it holds.
    """
    N, d = x.shape
    nb = -(-N // block)
    out = np.empty((nb, d), dtype=np.float64)
    for i in range(nb):
        out[i] = x[i * block: min((i + 1) * block, N)].mean(axis=0)
    return out


# ---------------------------------------------------------------- step (3)
def band_rms(xbar: np.ndarray, dims: np.ndarray) -> float:
    """RMS energy of a pooled band: sqrt(mean over blocks i, dims c in D of xbar[i,c]^2).

    Prism review, pipeline step (3): the RMS of each pooled band measures its
    spectral energy density. gist.science Technical Summary 2B: the RMS of the
    pooled representations.
    """
    return float(np.sqrt(np.mean(xbar[:, dims] ** 2)))


# ---------------------------------------------------------------- step (4)
def temperature(qbar: np.ndarray, kbar: np.ndarray, dims_z: np.ndarray, dims_full: np.ndarray,
                mode: str = "fullspec") -> tuple[float, bool]:
    """Branch temperature tau_z and whether the degenerate fallback was used.

    Prism review, pipeline step (4): a per-branch temperature tau_z aligns the
    branch's logit magnitude with the full spectrum; novelty paragraph: it is
    RMS-energy based and has no hyperparameters; gist.science 2B: computed
    from the RMS of the pooled representations. The formula itself is not
    printed; the reading used here is the band's pooled energy relative to the
    full spectrum's, for query and key:
        tau_z = R(Qbar, D_z) R(Kbar, D_z) / (R(Qbar, D_full) R(Kbar, D_full)).
    mode 'none' gives tau = 1 (plain pooled scores per band). Rejected
    readings kept for comparison: 'unit', tau_z = R(Qbar, D_z) R(Kbar, D_z)
    (unit-energy normalisation with no full-spectrum reference), and
    'pervec', where the RMS is taken per pooled vector (pervec_factors) and
    the head-level tau is 1.
    """
    if mode in ("none", "pervec"):
        return 1.0, False
    if mode not in ("fullspec", "unit"):
        raise ValueError(mode)
    rq_z, rk_z = band_rms(qbar, dims_z), band_rms(kbar, dims_z)
    rq_f, rk_f = band_rms(qbar, dims_full), band_rms(kbar, dims_full)
    if min(rq_z, rk_z, rq_f, rk_f) == 0.0:
        return 1.0, True
    if mode == "unit":
        return rq_z * rk_z, False
    return (rq_z * rk_z) / (rq_f * rk_f), False


def pervec_factors(xbar: np.ndarray, dims_z: np.ndarray, dims_full: np.ndarray) -> np.ndarray:
    """Per-vector reading of the RMS calibration (Prism review, pipeline steps
    (3)-(4), taken per pooled vector instead of per head): block i's band
    z is scaled by R(xbar_i, D_full) / R(xbar_i, D_z), i.e. to the energy
    density of its own full spectrum; 1 where R(xbar_i, D_z) is 0.
    """
    rz = np.sqrt(np.mean(xbar[:, dims_z] ** 2, axis=1))
    rf = np.sqrt(np.mean(xbar[:, dims_full] ** 2, axis=1))
    out = np.ones(xbar.shape[0])
    nz = rz > 0
    out[nz] = rf[nz] / rz[nz]
    return out


# ---------------------------------------------------------------- step (5)
def admissible(i: int, nb: int, causal: bool) -> np.ndarray:
    """Key blocks a query block may score: j <= i under causal prefill."""
    return np.arange(i + 1) if causal else np.arange(nb)


def band_scores(qbar: np.ndarray, kbar: np.ndarray, dims_z: np.ndarray, tau: float,
                causal: bool, fq: np.ndarray | None = None, fk: np.ndarray | None = None
                ) -> tuple[np.ndarray, np.ndarray]:
    """Logits L and block softmax S of one branch.

    Prism review, pipeline step (5):
        S_z = softmax(Qbar_z Kbar_z^T / (tau_z sqrt(d_z))),
    the softmax of row i taken over the admissible key blocks J(i) (j <= i when
    causal). Entries outside J(i): L = -inf, S = 0. fq, fk (per-vector
    reading only) scale row i by fq[i] and column j by fk[j].
    """
    nb = qbar.shape[0]
    L = (qbar[:, dims_z] @ kbar[:, dims_z].T) / (tau * np.sqrt(len(dims_z)))
    if fq is not None:
        L = L * fq[:, None] * fk[None, :]
    S = np.zeros_like(L)
    Lm = np.full_like(L, -np.inf)
    for i in range(nb):
        J = admissible(i, nb, causal)
        row = L[i, J]
        e = np.exp(row - row.max())
        S[i, J] = e / e.sum()
        Lm[i, J] = row
    return Lm, S


# ---------------------------------------------------------------- step (6)
def top_p(scores: np.ndarray, p: float) -> np.ndarray:
    """Top-P over one row's admissible scores; returns a boolean selection.

    Prism review, pipeline step (6): each branch keeps, per query block, the
    blocks chosen by Top-P. Read as: sort descending (equal scores by lower
    block index first), keep the shortest prefix whose cumulative mass is
    >= p (all of them if the mass never reaches p, and all if p >= 1).
    """
    n = scores.shape[0]
    sel = np.zeros(n, dtype=bool)
    if n == 0:
        return sel
    if p >= 1.0:
        sel[:] = True
        return sel
    order = np.argsort(-scores, kind="stable")
    cum = np.cumsum(scores[order])
    reach = np.flatnonzero(cum >= p)
    k = reach[0] + 1 if reach.size else n
    sel[order[:k]] = True
    return sel


def top_p_mask(S: np.ndarray, p: float, causal: bool) -> np.ndarray:
    """Apply top_p to every row of a branch's score matrix over J(i)."""
    nb = S.shape[0]
    M = np.zeros(S.shape, dtype=np.uint8)
    for i in range(nb):
        J = admissible(i, nb, causal)
        M[i, J[top_p(S[i, J], p)]] = 1
    return M


# ---------------------------------------------------------------- step (7)
def union(m_high: np.ndarray, m_low: np.ndarray) -> np.ndarray:
    """Prism review, pipeline step (7): the final block mask is M_high OR M_low."""
    return (m_high.astype(bool) | m_low.astype(bool)).astype(np.uint8)


def intersect(m_high: np.ndarray, m_low: np.ndarray) -> np.ndarray:
    """Merge variant (Prism review, weaknesses paragraph: the union may
    over-select): a block is kept only when both branches keep it."""
    return (m_high.astype(bool) & m_low.astype(bool)).astype(np.uint8)


def mix_mask(S_high: np.ndarray, S_low: np.ndarray, p: float, causal: bool) -> np.ndarray:
    """Weighted-merge variant (same paragraph): one Top-P, at the same p, on
    the equal-weight mixture of the two branches' block distributions."""
    return top_p_mask(0.5 * (S_high + S_low), p, causal)


def merge_masks(r: dict, p: float, causal: bool, merge: str = "union") -> np.ndarray:
    """The final block mask of one head from its branch results r."""
    if merge == "union":
        return union(r["m_high"], r["m_low"])
    if merge == "intersect":
        return intersect(r["m_high"], r["m_low"])
    if merge == "mix":
        return mix_mask(r["S_high"], r["S_low"], p, causal)
    raise ValueError(merge)


# ------------------------------------------- per-head adaptive band split
def pair_energy(xbar: np.ndarray, rope_layout: str = "interleaved") -> np.ndarray:
    """Pooled energy of each RoPE pair, averaged over the blocks: [d/2], the
    fastest pair first (pair j = dims 2j, 2j+1 interleaved, j and j + d/2
    rotate-half)."""
    d = xbar.shape[1]
    if rope_layout == "interleaved":
        a, b = xbar[:, 0::2], xbar[:, 1::2]
    else:
        a, b = xbar[:, : d // 2], xbar[:, d // 2:]
    return np.mean(a ** 2 + b ** 2, axis=0)


SPLIT_STEP = 8          # pairs: adaptive band edges move in steps of 16 dims
SPLIT_SHARE_RTOL = 1e-9  # an energy share equal to the reference within rounding counts as reaching it


def adaptive_split(spectra: np.ndarray, d: int, d_high: int, d_low: int) -> list[tuple[int, int]]:
    """Per-head (d_high, d_low) from the heads' pair spectra [H, d/2]
    (P_j = pooled energy of pair j of Qbar times that of Kbar).

    The reference share is the fraction of the mean spectrum (over the H
    heads) that the static high band's d_high/2 pairs hold. Head h's high
    band is [0, j_h) with j_h the smallest multiple of SPLIT_STEP pairs whose
    cumulative share of the head's own spectrum reaches the reference (within
    SPLIT_SHARE_RTOL), limited so both bands keep at least SPLIT_STEP pairs;
    its low band is [j_h - o, d/2) with o = (d_high + d_low - d) / 2 the
    static overlap in pairs (negative: a gap). A head whose spectrum is zero
    keeps the static split. Needs d_high, d_low multiples of 2 * SPLIT_STEP.
    """
    npairs = d // 2
    if d_high % (2 * SPLIT_STEP) or d_low % (2 * SPLIT_STEP):
        raise ValueError("adaptive split needs band widths in multiples of 16 dims")
    o = (d_high + d_low - d) // 2
    j0 = d_high // 2
    mean = spectra.mean(axis=0)
    cm = np.cumsum(mean)
    share = cm[j0 - 1] / cm[-1] if cm[-1] > 0 else 0.0
    lo_j = max(SPLIT_STEP, o)
    hi_j = min(npairs - SPLIT_STEP, npairs + o - SPLIT_STEP)
    out = []
    for P in spectra:
        c = np.cumsum(P)
        if c[-1] <= 0 or cm[-1] <= 0:
            out.append((d_high, d_low))
            continue
        jh = hi_j
        for j in range(lo_j, hi_j + 1, SPLIT_STEP):
            if c[j - 1] / c[-1] >= share * (1.0 - SPLIT_SHARE_RTOL):
                jh = j
                break
        out.append((2 * jh, d - 2 * (jh - o)))
    return out


# ------------------------------------------------------- grouped-query heads
def kv_head(h: int, hq: int, hkv: int) -> int:
    """KV head read by query head h under grouped-query attention: the Hq query
    heads split into Hkv contiguous groups of G = Hq / Hkv, group g sharing KV
    head g (h // G). This is the convention of torch's scaled_dot_product_attention
    with enable_gqa and of repeat_interleave(K, G) along the head axis."""
    if hq % hkv:
        raise ValueError("Hq % Hkv != 0")
    return h // (hq // hkv)


# ------------------------------------------------------- steps (1)-(7) together
def estimate_head(qh: np.ndarray, kg: np.ndarray, *, block: int, d_high: int, d_low: int, p: float,
                  causal: bool = True, rope_layout: str = "interleaved", tau_mode: str = "fullspec",
                  kbar: np.ndarray | None = None, merge: str = "union", qbar: np.ndarray | None = None) -> dict:
    """The estimator for one query head: qh [N, d], kg [N, d] (its KV head);
    qbar / kbar may be passed already pooled."""
    d = (qh if qh is not None else qbar).shape[1]
    hi, lo, full = band_dims(d, d_high, d_low, rope_layout)
    if qbar is None:
        qbar = mean_pool(qh, block)
    if kbar is None:
        kbar = mean_pool(kg, block)
    tau_h, deg_h = temperature(qbar, kbar, hi, full, tau_mode)
    tau_l, deg_l = temperature(qbar, kbar, lo, full, tau_mode)
    fh = fl = (None, None)
    if tau_mode == "pervec":
        fh = (pervec_factors(qbar, hi, full), pervec_factors(kbar, hi, full))
        fl = (pervec_factors(qbar, lo, full), pervec_factors(kbar, lo, full))
    L_h, S_h = band_scores(qbar, kbar, hi, tau_h, causal, *fh)
    L_l, S_l = band_scores(qbar, kbar, lo, tau_l, causal, *fl)
    m_h = top_p_mask(S_h, p, causal)
    m_l = top_p_mask(S_l, p, causal)
    r = {"m_high": m_h, "m_low": m_l, "S_high": S_h, "S_low": S_l}
    return {
        "qbar": qbar, "kbar": kbar,
        "rms_q": (band_rms(qbar, hi), band_rms(qbar, lo), band_rms(qbar, full)),
        "rms_k": (band_rms(kbar, hi), band_rms(kbar, lo), band_rms(kbar, full)),
        "tau": (tau_h, tau_l), "degenerate": int(deg_h) + int(deg_l),
        "L_high": L_h, "L_low": L_l, "S_high": S_h, "S_low": S_l,
        "m_high": m_h, "m_low": m_l, "mask": merge_masks(r, p, causal, merge),
        "bands": (d_high, d_low),
    }


def estimate(q: np.ndarray, k: np.ndarray, *, block: int, d_high: int, d_low: int, p: float,
             causal: bool = True, rope_layout: str = "interleaved", tau_mode: str = "fullspec",
             heads=None, keep=False, merge: str = "union", band_mode: str = "static") -> dict:
    """Estimator over q [b, N, Hq, d], k [b, N, Hkv, d] (float64, BSHD).

    Query head h reads KV head kv_head(h, Hq, Hkv) (grouped-query attention).
    band_mode 'adaptive' chooses each head's bands with adaptive_split from
    the spectra of all Hq query heads of the batch entry (whatever `heads`
    selects for the output). Returns mask [b, Hq, nb, nb] (uint8), tau
    [b, Hq, 2], bands [b, Hq, 2] (d_high, d_low per head) and, with
    keep=True, the per-head intermediate dicts.
    """
    b, N, Hq, d = q.shape
    Hkv = k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq % Hkv != 0")
    nb = -(-N // block)
    heads = range(Hq) if heads is None else heads
    mask = np.zeros((b, Hq, nb, nb), dtype=np.uint8)
    tau = np.zeros((b, Hq, 2))
    bands = np.zeros((b, Hq, 2), dtype=np.int64)
    per = {}
    for bb in range(b):
        kbars = {g: mean_pool(k[bb, :, g, :], block) for g in range(Hkv)}
        qbars = {}
        split = None
        if band_mode == "adaptive":
            qbars = {h: mean_pool(q[bb, :, h, :], block) for h in range(Hq)}
            ek = {g: pair_energy(kbars[g], rope_layout) for g in kbars}
            spectra = np.stack([pair_energy(qbars[h], rope_layout) * ek[kv_head(h, Hq, Hkv)] for h in range(Hq)])
            split = adaptive_split(spectra, d, d_high, d_low)
        elif band_mode != "static":
            raise ValueError(band_mode)
        for h in heads:
            g = kv_head(h, Hq, Hkv)
            dh, dl = split[h] if split is not None else (d_high, d_low)
            r = estimate_head(q[bb, :, h, :] if h not in qbars else None, None, block=block, d_high=dh, d_low=dl,
                              p=p, causal=causal, rope_layout=rope_layout, tau_mode=tau_mode, kbar=kbars[g],
                              merge=merge, qbar=qbars.get(h))
            mask[bb, h] = r["mask"]
            tau[bb, h] = r["tau"]
            bands[bb, h] = (dh, dl)
            if keep:
                per[(bb, h)] = r
    return {"mask": mask, "tau": tau, "bands": bands, "per_head": per}


# ------------------------------------------------------ block-sparse attention
def attention_block_row(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask_row: np.ndarray, i: int, *,
                        block: int, causal: bool) -> np.ndarray:
    """Output rows of query block i for one head: q,k,v [N, d] -> [n_i, d].

    Block-sparse prefill (abstract; gist.science Technical Summary section 1):
    query t of block i attends to the keys s of the selected key blocks
    (mask_row[s // B] == 1) with s <= t when causal, by a softmax of
    q_t . k_s / sqrt(d); a query with no admissible key outputs 0.
    """
    N, d = q.shape
    t0, t1 = i * block, min((i + 1) * block, N)
    sel = np.flatnonzero(mask_row)
    if sel.size == 0:
        return np.zeros((t1 - t0, v.shape[1]))
    keys = np.concatenate([np.arange(j * block, min((j + 1) * block, N)) for j in sel])
    logits = (q[t0:t1] @ k[keys].T) / np.sqrt(d)
    if causal:
        logits = np.where(keys[None, :] <= np.arange(t0, t1)[:, None], logits, -np.inf)
    # row-wise softmax over the admissible keys (exp(-inf) = 0), then the
    # probability-weighted sum of the values; rows with no admissible key stay 0
    has = np.isfinite(logits).any(axis=1)
    rmax = np.where(has, logits.max(axis=1), 0.0)
    w = np.exp(logits - rmax[:, None])
    w[~has] = 0.0
    w[has] /= w[has].sum(axis=1, keepdims=True)
    return w @ v[keys]


def block_sparse_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray, *, block: int,
                           causal: bool = True, rows=None) -> np.ndarray:
    """O [b, N, Hq, dv] for q [b, N, Hq, d], k/v [b, N, Hkv, d], mask [b, Hq, nb, nb].

    rows: optional iterable of (b, h, i) query blocks to compute; the others
    stay NaN (so a sampled comparison can only read what was computed).
    """
    b, N, Hq, d = q.shape
    Hkv = k.shape[2]
    nb = -(-N // block)
    out = np.full((b, N, Hq, v.shape[3]), np.nan)
    if rows is None:
        rows = [(bb, h, i) for bb in range(b) for h in range(Hq) for i in range(nb)]
    for bb, h, i in rows:
        g = kv_head(h, Hq, Hkv)
        out[bb, i * block: min((i + 1) * block, N), h, :] = attention_block_row(
            q[bb, :, h, :], k[bb, :, g, :], v[bb, :, g, :], mask[bb, h, i], i, block=block, causal=causal)
    return out

