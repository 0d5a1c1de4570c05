"""RoPE variants the Prism pages say the method carries over to (gist.science,
Results, generalization: YaRN and M-RoPE, Qwen3-VL): the generator's angles
pinned to the variants' published definitions, and the pooling attenuation
(the band semantics the estimator relies on) pinned to closed forms under
each variant, through the oracle's own pooling and temperature.
"""
import math

import numpy as np
import pytest

import oracle.prism_oracle as po
from synth import WORKLOADS, Rope, apply_rope, rope_axes, rope_freqs, rope_positions, rope_tables


def dirichlet(n, theta):
    """mean_{m<n} exp(i m theta) has modulus |sin(n theta/2) / (n sin(theta/2))|;
    returned signed (the phase is that of the middle position)."""
    theta = np.asarray(theta, dtype=np.float64)
    out = np.ones_like(theta)
    nz = np.abs(np.sin(theta / 2)) > 0
    out[nz] = np.sin(n * theta[nz] / 2) / (n * np.sin(theta[nz] / 2))
    return out


YARN = Rope("yarn", factor=4.0, orig_ctx=32768)


# ---------------------------------------------------------------- YaRN angles
def test_yarn_frequencies_follow_ntk_by_parts():
    """theta'_j = theta_j where the pair turns more than beta_fast times over
    L0, theta_j / s where it turns fewer than beta_slow times, and the linear
    blend in between (YaRN, NTK-by-parts)."""
    d, base = 128, 1e6
    f0 = rope_freqs(d, base)
    f1 = rope_freqs(d, base, YARN)
    turns = YARN.orig_ctx * f0 / (2 * np.pi)
    fast, slow = turns > YARN.beta_fast, turns < YARN.beta_slow
    assert fast.any() and slow.any() and (~fast & ~slow).any()
    assert np.array_equal(f1[fast], f0[fast])
    assert np.allclose(f1[slow], f0[slow] / YARN.factor, rtol=1e-15, atol=0)
    mid = ~fast & ~slow
    g = (turns[mid] - 1.0) / 31.0
    assert np.allclose(f1[mid], g * f0[mid] + (1 - g) * f0[mid] / 4.0, rtol=1e-15, atol=0)
    assert np.all(np.diff(f1) < 0) and np.all(f1 <= f0)


def test_yarn_keeps_the_pooling_dead_zone():
    """Every pair that block pooling (B=128) attenuates below 0.95 keeps its
    frequency under YaRN: the pairs the high band is chosen for still rotate
    as fast, so the band split means the same thing (Qwen3-8B, 32K -> 128K)."""
    f0 = rope_freqs(128, 1e6)
    f1 = rope_freqs(128, 1e6, YARN)
    lam = np.abs(dirichlet(128, f0))
    assert (lam < 0.95).sum() >= 20
    assert np.array_equal(f1[lam < 0.95], f0[lam < 0.95])


@pytest.mark.parametrize("block_index", [0, 5])
def test_yarn_pooled_pair_is_dirichlet_at_rescaled_frequency(block_index):
    """Unit pairs rotated by the YaRN tables and mean-pooled by the oracle:
    amplitude (0.1 ln s + 1) D_B(theta'_j), phase theta'_j at the block centre."""
    d, B, base = 128, 128, 1e6
    N = (block_index + 1) * B
    cos, sin = rope_tables(N, d, base, YARN)
    x = np.zeros((N, d))
    x[:, 0::2] = 1.0
    pooled = po.mean_pool(apply_rope(x, cos, sin, "interleaved"), B)[block_index]
    th = rope_freqs(d, base, YARN)
    amp = (0.1 * math.log(4.0) + 1.0) * dirichlet(B, th)
    c = block_index * B + (B - 1) / 2.0
    assert np.abs(pooled[0::2] - amp * np.cos(c * th)).max() < 1e-12
    assert np.abs(pooled[1::2] - amp * np.sin(c * th)).max() < 1e-12


# -------------------------------------------------------------- M-RoPE angles
def test_mrope_on_text_is_plain_rope():
    """With no video prefix every token has t = h = w, so M-RoPE (either axis
    assignment) gives exactly the plain rotary tables."""
    for mode in ("sectioned", "interleaved"):
        r = Rope("mrope", mrope=mode, sections=(16, 24, 24))
        c1, s1 = rope_tables(700, 128, 1e6, r)
        c0, s0 = rope_tables(700, 128, 1e6)
        assert np.array_equal(c1, c0) and np.array_equal(s1, s0)


def test_mrope_axis_assignment_and_positions():
    """Qwen2-VL sections (16, 24, 24): contiguous pair ranges. Qwen3-VL's
    interleaved form with (24, 20, 20): h on pairs 1, 4, .., 58, w on
    2, 5, .., 59, t elsewhere. Video ids are (frame, row, column); text
    after the video continues from max(nt, nh, nw)."""
    a = rope_axes(128, Rope("mrope", sections=(16, 24, 24)))
    assert np.array_equal(a, np.repeat([0, 1, 2], [16, 24, 24]))
    b = rope_axes(128, Rope("mrope", mrope="interleaved", sections=(24, 20, 20)))
    assert np.array_equal(np.nonzero(b == 1)[0], np.arange(1, 60, 3))
    assert np.array_equal(np.nonzero(b == 2)[0], np.arange(2, 60, 3))
    assert np.bincount(b).tolist() == [24, 20, 20]
    r = Rope("mrope", sections=(16, 24, 24), grid=(2, 3, 4))
    pos = rope_positions(30, r)
    assert pos[0].tolist() == [0, 0, 0] and pos[5].tolist() == [0, 1, 1] and pos[23].tolist() == [1, 2, 3]
    assert pos[24].tolist() == [4, 4, 4] and pos[29].tolist() == [9, 9, 9]
    with pytest.raises(ValueError):
        rope_axes(128, Rope("mrope", sections=(16, 24, 20)))


@pytest.mark.parametrize("mode,sections", [("sectioned", (16, 24, 24)), ("interleaved", (24, 20, 20))])
@pytest.mark.parametrize("rows_per_block", [1, 2])
def test_mrope_video_pooling_closed_form(mode, sections, rows_per_block):
    """A video whose rows are B / rows_per_block patches wide, so every block
    holds whole rows of one frame: pooled over a block, t-axis pairs are not
    attenuated at all, h-axis pairs by D_{rows}(theta_j) and w-axis pairs by
    D_{cols}(theta_j). Under M-RoPE the fast pairs of the t axis therefore
    keep their energy after pooling, unlike under plain RoPE."""
    d, B, base = 128, 128, 5e6
    cols = B // rows_per_block
    r = Rope("mrope", mrope=mode, sections=sections, grid=(3, 4 * rows_per_block, cols))
    N = 3 * 4 * B
    cos, sin = rope_tables(N, d, base, r)
    x = np.zeros((N, d))
    x[:, 0::2] = 1.0
    pooled = po.mean_pool(apply_rope(x, cos, sin, "interleaved"), B)
    th = rope_freqs(d, base)
    ax = rope_axes(d, r)
    amp = np.where(ax == 0, 1.0, np.where(ax == 1, dirichlet(rows_per_block, th), dirichlet(cols, th)))
    pos = rope_positions(N, r)
    for i in (0, 5, 11):
        centre = pos[i * B: (i + 1) * B].mean(axis=0)[ax]  # mean id of each pair's axis
        got = pooled[i]
        assert np.abs(got[0::2] - amp * np.cos(centre * th)).max() < 1e-12
        assert np.abs(got[1::2] - amp * np.sin(centre * th)).max() < 1e-12
    # the fastest t-axis pair keeps unit amplitude; under plain RoPE it pools to ~0
    j = int(np.nonzero(ax == 0)[0][0])
    assert abs(np.hypot(pooled[2][2 * j], pooled[2][2 * j + 1]) - 1.0) < 1e-12
    assert abs(dirichlet(B, th[j])) < 0.05


# ---------------------------------------------- temperature under the variants
def tau_closed_form_error_variant(rope, base, d_high=64, d_low=96, B=128, nb=4, seed=1):
    """Q = K = rotated constant x: pooled pair energy is a_j^2 |x_j|^2 in every
    block (a_j the pooled amplitude of pair j), so tau_z is the band's mean
    of a_j^2 |x_j|^2 over the full spectrum's."""
    d = 128
    x = np.random.default_rng(seed).standard_normal(d)
    N = nb * B
    cos, sin = rope_tables(N, d, base, rope)
    xr = apply_rope(np.tile(x, (N, 1)), cos, sin, "interleaved")
    r = po.estimate_head(xr, xr, block=B, d_high=d_high, d_low=d_low, p=0.9)
    th = rope_freqs(d, base, rope)
    if rope.kind == "mrope":
        rows = B // rope.grid[2]
        ax = rope_axes(d, rope)
        a = np.where(ax == 0, 1.0, np.where(ax == 1, dirichlet(rows, th), dirichlet(rope.grid[2], th)))
    else:
        a = dirichlet(B, th) * (0.1 * math.log(rope.factor) + 1.0 if rope.kind == "yarn" else 1.0)
    pair = a ** 2 * (x[0::2] ** 2 + x[1::2] ** 2)
    full = pair.sum() / d
    t_hi = pair[: d_high // 2].sum() / d_high / full
    t_lo = pair[d // 2 - d_low // 2:].sum() / d_low / full
    rel = lambda u, v: abs(u - v) / abs(v)
    return max(rel(r["tau"][0], t_hi), rel(r["tau"][1], t_lo), rel(r["rms_q"][2], math.sqrt(full)))


@pytest.mark.parametrize("rope,base", [
    (YARN, 1e6),
    (Rope("mrope", mrope="interleaved", sections=(24, 20, 20), grid=(4, 2, 64)), 5e6),
    (Rope("mrope", sections=(16, 24, 24), grid=(2, 4, 128)), 1e6),
])
def test_tau_closed_form_under_variants(rope, base):
    assert tau_closed_form_error_variant(rope, base) < 1e-12


def test_variant_workloads_are_declared():
    w = WORKLOADS["qwen3_8b_yarn_128k"]
    assert w.rope.kind == "yarn" and w.seq == 4 * w.rope.orig_ctx
    v = WORKLOADS["qwen3_vl_8b_video_32k"]
    nt, nh, nw = v.rope.grid
    assert v.rope.kind == "mrope" and nt * nh * nw < v.seq  # video, then text
