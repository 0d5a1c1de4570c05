"""The GPU tests' mask rule (tests/parity.py) on hand-built rows: which
differences it excuses as mass ties or key ties, and which it fails."""
import numpy as np
import pytest

import oracle.prism_oracle as po
from tests.parity import KEY_ULP, LOG2E, LOGIT_TOL_REL, compare_masks, key_tie_window


def oracle_dict(L_high, L_low, p, merge="union"):
    """one head's oracle results for given band logits (natural units), causal"""
    nb = L_high.shape[0]
    r = {}
    for z, L in (("high", L_high), ("low", L_low)):
        Lm = np.full((nb, nb), -np.inf)
        S = np.zeros((nb, nb))
        for i in range(nb):
            J = po.admissible(i, nb, True)
            Lm[i, J] = L[i, J]
            e = np.exp(L[i, J] - L[i, J].max())
            S[i, J] = e / e.sum()
        r[f"L_{z}"], r[f"S_{z}"] = Lm, S
        r[f"m_{z}"] = po.top_p_mask(S, p, True)
    r["mask"] = po.merge_masks(r, p, True, merge)
    return {(0, 0): r}


def row_case(delta, p=None, low_peaked=True, merge="union"):
    """8 key blocks; the high branch's last row has logits whose ranks 3 and 4
    differ by delta; p keeps ranks 0..3 there unless given"""
    nb = 8
    rng = np.random.default_rng(3)
    Lh = rng.standard_normal((nb, nb))
    Lh[7] = [2.0, 1.5, 1.0, 0.5, 0.5 - delta, 0.1, 0.0, -1.0]
    Ll = rng.standard_normal((nb, nb))
    if low_peaked:
        Ll[7] = [12.0, 0, 0, 0, 0, 0, 0, 0]
    if p is None:
        e = np.exp(Lh[7] - 2.0)
        cum = np.cumsum(e / e.sum())
        p = float((cum[2] + cum[3]) / 2)
    return oracle_dict(Lh, Ll, p, merge), p


def swapped(orc, pairs):
    g = orc[(0, 0)]["mask"].copy()[None, None]
    for (i, a, b) in pairs:
        g[0, 0, i, a], g[0, 0, i, b] = g[0, 0, i, b], g[0, 0, i, a]
    return g


def test_identical_masks_pass():
    orc, p = row_case(1e-9)
    st = compare_masks(orc[(0, 0)]["mask"][None, None], orc, p, True)
    assert st["mismatch"] == 0 and st["blocks"] == 36


def test_swap_within_key_window_is_a_key_tie():
    orc, p = row_case(1e-8)
    assert orc[(0, 0)]["mask"][7, 3] == 1 and orc[(0, 0)]["mask"][7, 4] == 0
    st = compare_masks(swapped(orc, [(7, 3, 4)]), orc, p, True)
    assert (st["mismatch"], st["score_tie"], st["unexcused"], st["mass_tie"]) == (2, 2, 0, 0)
    assert 0 < st["max_key_gap_over_window"] < 1


def test_swap_beyond_key_window_fails():
    # the window for this row: 2 * LOGIT_TOL_REL * max(1, 2 log2 e) + KEY_ULP, about 1.2e-5 in log2 units
    w = key_tie_window(np.array([2.0, 0.0]))
    assert w == pytest.approx(2 * LOGIT_TOL_REL * 2 * LOG2E + KEY_ULP)
    orc, p = row_case(2 * w / LOG2E)
    st = compare_masks(swapped(orc, [(7, 3, 4)]), orc, p, True)
    assert st["unexcused"] == 2 and st["score_tie"] == 0
    assert sorted(st["where"]) == [(0, 0, 7, 3), (0, 0, 7, 4)]


def test_flip_far_from_the_boundary_fails():
    orc, p = row_case(1e-8)
    g = orc[(0, 0)]["mask"].copy()[None, None]
    g[0, 0, 7, 1] = 0  # rank 1 of the high branch, far above the boundary
    st = compare_masks(g, orc, p, True)
    assert st["unexcused"] == 1


def test_cumulative_mass_within_1e4_of_p_is_a_mass_tie():
    orc, p0 = row_case(0.3)
    e = np.exp(orc[(0, 0)]["L_high"][7] - 2.0)
    cum = np.cumsum(np.sort(e / e.sum())[::-1])
    p = float(cum[3] - 5e-5)  # the inclusive mass of rank 3 sits 5e-5 above p
    orc, _ = row_case(0.3, p=p)
    g = orc[(0, 0)]["mask"].copy()[None, None]
    assert g[0, 0, 7, 3] == 1
    g[0, 0, 7, 3] = 0
    st = compare_masks(g, orc, p, True)
    assert (st["mass_tie"], st["unexcused"]) == (1, 0)


def test_union_needs_an_excuse_in_every_branch_that_keeps_the_block():
    # block 3 kept by the high branch only within a key tie; when the low
    # branch also keeps it (flat low row), dropping it is excused there by
    # nothing, so the difference fails
    orc, p = row_case(1e-8, low_peaked=False)
    r = orc[(0, 0)]
    if not r["m_low"][7, 3]:
        pytest.skip("the low branch of this seeded row does not keep block 3")
    g = r["mask"].copy()[None, None]
    g[0, 0, 7, 3] = 0
    st = compare_masks(g, orc, p, True)
    assert st["unexcused"] == 1


def test_above_diagonal_never_excused():
    orc, p = row_case(1e-8)
    g = orc[(0, 0)]["mask"].copy()[None, None]
    g[0, 0, 2, 5] = 1
    st = compare_masks(g, orc, p, True)
    assert st["unexcused"] == 1 and st["where"] == [(0, 0, 2, 5)]


def test_intersection_rule():
    """intersection: the high branch's rank 3/4 swap within the key window
    (the low branch keeps both blocks) is excused on both blocks; outside
    the window it fails"""
    for delta, excused in ((1e-8, True), (1e-3, False)):
        orc, p = row_case(delta, low_peaked=False, merge="intersect")
        r = orc[(0, 0)]
        if not (r["m_low"][7, 3] and r["m_low"][7, 4]):
            pytest.skip("the low branch of this seeded row does not keep blocks 3 and 4")
        assert r["mask"][7, 3] == 1 and r["mask"][7, 4] == 0
        g = r["mask"].copy()[None, None]
        g[0, 0, 7, 3], g[0, 0, 7, 4] = 0, 1
        st = compare_masks(g, orc, p, True, merge="intersect")
        assert st["mismatch"] == 2
        assert (st["unexcused"] == 0) == excused, st


def test_mixture_rule():
    """mixture: one decision on (S_high + S_low) / 2; a swap of its boundary
    pair within the key window is a key tie, a flip far above it fails"""
    nb = 8
    Lh = np.zeros((nb, nb))
    Ll = np.zeros((nb, nb))
    Lh[7] = [3.0, 2.0, 1.0, 0.0, 0.0, -1.0, -2.0, -3.0]
    Ll[7] = [3.0, 2.0, 1.0, 0.0, -1e-8, -1.0, -2.0, -3.0]  # mixture ranks 3 and 4 nearly tie
    S = 0.5 * (np.exp(Lh[7]) / np.exp(Lh[7]).sum() + np.exp(Ll[7]) / np.exp(Ll[7]).sum())
    cum = np.cumsum(np.sort(S)[::-1])
    p = float((cum[2] + cum[3]) / 2)
    orc = oracle_dict(Lh, Ll, p, merge="mix")
    r = orc[(0, 0)]
    assert r["mask"][7, :4].all() and not r["mask"][7, 4:].any()
    g = r["mask"].copy()[None, None]
    g[0, 0, 7, 3], g[0, 0, 7, 4] = 0, 1
    st = compare_masks(g, orc, p, True, merge="mix")
    assert (st["mismatch"], st["score_tie"], st["unexcused"]) == (2, 2, 0)
    g = r["mask"].copy()[None, None]
    g[0, 0, 7, 0] = 0
    assert compare_masks(g, orc, p, True, merge="mix")["unexcused"] == 1
