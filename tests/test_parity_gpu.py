"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small cases compare every element at sizes that span several tiles and a
ragged tail; the five full-size workloads compare the whole mask and sampled
query-block rows of the attention output (each row is exact on its own).
Tolerances: masks per tests/parity.py; bf16 attention max-abs <= 2e-2 and
norm-relative <= 1e-2; fp32 attention max-abs <= 1e-4 * max|O|.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_attention_band_amd as prism  # noqa: E402
import oracle.prism_oracle as po  # noqa: E402
from synth import WORKLOADS, Rope, make_qkv, random_mask, to_f64  # noqa: E402
from tests.parity import (LOGIT_TOL_REL, compare_masks, logit_errors, logit_row, oracle_estimate_heads,  # noqa: E402
                          pack_bits, record_parity, to_device, unpack_bits)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    prism.lib()  # fails loudly when libprism.so is missing
    yield
    torch.cuda.synchronize()


def cfg_of(w, **kw):
    c = dict(block_size=w.block, d_high=w.d_high, d_low=w.d_low, p=w.p, causal=w.causal)
    c.update(kw)
    return prism.EstimatorConfig(**c)


def read_ws(ws, off, shape):
    n = int(np.prod(shape))
    return ws[off: off + 4 * n].view(torch.float32).reshape(shape).cpu().numpy().astype(np.float64)


def read_logits(ws, L, bh, z, causal):
    """one logit plane as a dense [nb, nb] array, -inf where nothing is stored"""
    nb = int(L.nb)
    plane = read_ws(ws, L.logits_offset + (2 * bh + z) * L.logits_plane * 4, (int(L.logits_plane),))
    out = np.full((nb, nb), -np.inf)
    for i in range(nb):
        n = i + 1 if causal else nb
        out[i, :n] = plane[logit_row(i, nb, causal): logit_row(i, nb, causal) + n]
    return out


def canonical(x, rope_layout):
    """physical dim order -> canonical frequency order (pair j at dims 2j, 2j+1)"""
    if rope_layout == "interleaved":
        return x
    d = x.shape[-1]
    out = np.empty_like(x)
    out[..., 0::2] = x[..., : d // 2]
    out[..., 1::2] = x[..., d // 2:]
    return out


# ------------------------------------------------------------ estimator cases
SMALL = {
    "gqa4_ragged": ("llama3_8b_32k", dict(seq=3000, hq=8, hkv=2), {}, "bshd", "interleaved"),
    "planted_qwen": ("qwen3_8b_64k", dict(seq=8192, hq=4, hkv=1), {}, "bshd", "interleaved"),
    "noncausal": ("llama3_8b_32k", dict(seq=2500, hq=4, hkv=1, causal=False), {}, "bshd", "interleaved"),
    "gqa8_bhsd": ("llama3_8b_32k", dict(seq=4096, hq=8, hkv=1), {}, "bhsd", "interleaved"),
    "mha_batch2": ("llama3_8b_32k", dict(seq=2000, hq=2, hkv=2, batch=2), {}, "bshd", "interleaved"),
    "half_rope": ("llama3_8b_32k", dict(seq=3000, hq=4, hkv=2), {}, "bshd", "half"),
    "gap_bands": ("llama3_8b_32k", dict(seq=3000, hq=2, hkv=1), dict(d_high=32, d_low=48), "bshd", "interleaved"),
    "equal_bands": ("llama3_8b_32k", dict(seq=3000, hq=2, hkv=1), dict(d_high=128, d_low=128), "bshd", "interleaved"),
    "odd_bands": ("llama3_8b_32k", dict(seq=3000, hq=2, hkv=1), dict(d_high=38, d_low=70), "bshd", "interleaved"),
    "p_half": ("llama3_8b_32k", dict(seq=3000, hq=2, hkv=1), dict(p=0.5), "bshd", "interleaved"),
    "p_one": ("llama3_8b_32k", dict(seq=3000, hq=2, hkv=1), dict(p=1.0), "bshd", "interleaved"),
    "tau_none": ("llama3_8b_32k", dict(seq=3000, hq=2, hkv=1), dict(tau_mode="none"), "bshd", "interleaved"),
    "tau_unit": ("llama3_8b_32k", dict(seq=3000, hq=4, hkv=2), dict(tau_mode="unit"), "bshd", "interleaved"),
    "tau_pervec": ("llama3_8b_32k", dict(seq=3000, hq=4, hkv=2), dict(tau_mode="pervec"), "bshd", "interleaved"),
    "tau_pervec_gap": ("llama3_8b_32k", dict(seq=3000, hq=2, hkv=1), dict(tau_mode="pervec", d_high=32, d_low=48),
                       "bshd", "interleaved"),
    "one_block": ("llama3_8b_32k", dict(seq=100, hq=2, hkv=1), {}, "bshd", "interleaved"),
    # a single token: one block holding one row
    "one_token": ("llama3_8b_32k", dict(seq=1, hq=2, hkv=1), {}, "bshd", "interleaved"),
    "one_token_fp32": ("tiny_fp32_2k", dict(seq=1, hq=1, hkv=1), {}, "bshd", "interleaved"),
    "fp32_iid": ("tiny_fp32_2k", dict(seq=1900, hq=2, hkv=1), {}, "bshd", "interleaved"),
    "nb_1100": ("llama3_8b_32k", dict(seq=1100 * 128 - 5, hq=1, hkv=1), {}, "bshd", "interleaved"),
    # the last length whose scores and selection run fused, and the first that goes through the planes
    "nb_1024_fused_edge": ("llama3_8b_32k", dict(seq=1024 * 128, hq=2, hkv=1), {}, "bshd", "interleaved"),
    "nb_1025_split_edge": ("llama3_8b_32k", dict(seq=1024 * 128 + 1, hq=2, hkv=1), {}, "bshd", "interleaved"),
    # RoPE variants (inputs only; the estimator is the same)
    "yarn": ("qwen3_8b_yarn_128k", dict(seq=5000, hq=4, hkv=1), {}, "bshd", "interleaved"),
    "mrope_video": ("qwen3_vl_8b_video_32k",
                    dict(seq=6000, hq=4, hkv=1, rope=Rope("mrope", mrope="interleaved", sections=(24, 20, 20),
                                                          grid=(2, 16, 48))), {}, "bshd", "interleaved"),
    # the merge variants and per-head adaptive bands (the weaknesses the review lists)
    "merge_intersect": ("llama3_8b_32k", dict(seq=3000, hq=4, hkv=2), dict(merge="intersect"), "bshd", "interleaved"),
    "merge_mix": ("llama3_8b_32k", dict(seq=3000, hq=4, hkv=2), dict(merge="mix"), "bshd", "interleaved"),
    "merge_mix_noncausal": ("llama3_8b_32k", dict(seq=2500, hq=2, hkv=1, causal=False), dict(merge="mix"), "bshd",
                            "interleaved"),
    "adaptive_spectral": ("llama3_8b_spectral_32k", dict(seq=5000, hq=8, hkv=4), dict(band_mode="adaptive"), "bshd",
                          "interleaved"),
    "adaptive_half_unit_mix": ("llama3_8b_spectral_32k", dict(seq=3000, hq=8, hkv=4),
                               dict(band_mode="adaptive", tau_mode="unit", merge="mix"), "bshd", "half"),
    "adaptive_gap_intersect": ("llama3_8b_spectral_32k", dict(seq=3000, hq=8, hkv=4),
                               dict(band_mode="adaptive", d_high=32, d_low=64, merge="intersect"), "bshd",
                               "interleaved"),
    "adaptive_batch2_bhsd": ("llama3_8b_spectral_32k", dict(seq=2000, hq=4, hkv=2, batch=2),
                             dict(band_mode="adaptive", tau_mode="none"), "bhsd", "interleaved"),
    "adaptive_nb_1100": ("llama3_8b_spectral_32k", dict(seq=1100 * 128 - 9, hq=4, hkv=2),
                         dict(band_mode="adaptive"), "bshd", "interleaved"),
    "intersect_nb_1100": ("llama3_8b_32k", dict(seq=1100 * 128, hq=2, hkv=1), dict(merge="intersect"), "bshd",
                          "interleaved"),
}


def run_estimator_case(name, base, over, cov, layout, rope_layout, check_stages=True):
    w = WORKLOADS[base].scaled(**over)
    say(f"[estimator] {name}: seq={w.seq} hq={w.hq} hkv={w.hkv} b={w.batch} {w.dtype} {layout} {cov}")
    q, k, _ = make_qkv(w, rope_layout=rope_layout, with_v=False)
    cfg = cfg_of(w, **{**cov, "rope_layout": rope_layout, "keep_logits": check_stages})
    qd, kd = to_device(q, w.dtype, layout), to_device(k, w.dtype, layout)
    L = prism.workspace_layout(qd, kd, cfg)
    ws = torch.full((L.total_bytes,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN-poisoned
    mask = torch.full((w.batch, w.hq, L.nb, L.nb), 7, dtype=torch.uint8, device="cuda")
    prism.estimate(qd, kd, cfg, workspace=ws, mask_out=mask)
    torch.cuda.synchronize()
    gm = mask.cpu().numpy()
    if check_stages:
        # the stored inspection copy changes nothing: same mask without it
        plain = prism.estimate(qd, kd, cfg_of(w, **{**cov, "rope_layout": rope_layout}))
        torch.cuda.synchronize()
        assert np.array_equal(plain.cpu().numpy(), gm)
    orc = oracle_estimate_heads(q, k, w.dtype, block=w.block, d_high=cfg.d_high, d_low=cfg.d_low, p=cfg.p,
                                causal=cfg.causal, rope_layout=rope_layout, tau_mode=cfg.tau_mode, merge=cfg.merge,
                                band_mode=cfg.band_mode)
    assert set(np.unique(gm)) <= {0, 1}
    if cfg.band_mode == "adaptive":
        # every head's split, as the oracle chooses it
        split = ws[L.split_offset: L.split_offset + w.batch * w.hq * 16].view(torch.int32).reshape(
            w.batch, w.hq, 4).cpu().numpy()
        got = {key: tuple(split[key[0], key[1], 2:].tolist()) for key in orc}
        want = {key: tuple(int(x) for x in r["bands"]) for key, r in orc.items()}
        say(f"    adaptive bands (d_high, d_low) per head: {[got[key] for key in sorted(got)]}")
        assert got == want
        for key, (dh, dl) in want.items():
            assert tuple(split[key[0], key[1], :2].tolist()) == (min(dh, 128 - dl), max(dh, 128 - dl))
    if cfg.causal:
        assert not np.triu(gm, 1).any()
    if check_stages:
        worst = 0.0
        qbar = read_ws(ws, L.qbar_offset, (w.batch, w.hq, L.nb, 128))
        kbar = read_ws(ws, L.kbar_offset, (w.batch, w.hkv, L.nb, 128))
        tau = read_ws(ws, L.tau_offset, (w.batch, w.hq, 8))
        for (bb, h), r in orc.items():
            scale = max(1.0, np.abs(r["qbar"]).max())
            assert np.abs(qbar[bb, h] - canonical(r["qbar"], rope_layout)).max() <= 2e-6 * scale, (bb, h)
            g = po.kv_head(h, w.hq, w.hkv)
            assert np.abs(kbar[bb, g] - canonical(r["kbar"], rope_layout)).max() <= 2e-6 * scale, (bb, h)
            assert np.allclose(tau[bb, h, :2], r["tau"], rtol=2e-5, atol=0), (tau[bb, h, :2], r["tau"])
            assert np.allclose(tau[bb, h, 2:5], r["rms_q"], rtol=2e-5, atol=0)
            assert np.allclose(tau[bb, h, 5:8], r["rms_k"], rtol=2e-5, atol=0)
            # band logits, log2 units, on the admissible entries: per row within
            # LOGIT_TOL_REL * max(1, max_j |L_ij|) (the bound the key-tie window uses)
            for z, key in enumerate(("L_high", "L_low")):
                gl = read_logits(ws, L, bb * w.hq + h, z, cfg.causal)
                err_abs, err_rel = logit_errors(gl, r[key])
                worst = max(worst, err_rel)
                assert err_rel <= LOGIT_TOL_REL, (bb, h, z, err_abs, err_rel)
        say(f"    logits: max per-row relative error {worst:.2e} (bound {LOGIT_TOL_REL:.0e})")
    st = compare_masks(gm, orc, cfg.p, cfg.causal, merge=cfg.merge)
    dens = gm.sum() / max(1, st["blocks"])
    say(f"    density={dens:.4f} blocks={st['blocks']} mismatch={st['mismatch']} mass_tie={st['mass_tie']} "
        f"score_tie={st['score_tie']} unexcused={st['unexcused']} {st['where'][:5]}")
    record_parity(f"small:{name}", st)
    assert st["unexcused"] == 0, st["where"][:20]
    return gm, st


@pytest.mark.parametrize("name", list(SMALL))
def test_estimator_small(name):
    run_estimator_case(name, *SMALL[name])


def _estimate_and_compare(name, q, k, dtype, cfg):
    qd, kd = to_device(q, dtype), to_device(k, dtype)
    mask = prism.estimate(qd, kd, cfg)
    torch.cuda.synchronize()
    gm = mask.cpu().numpy()
    orc = oracle_estimate_heads(q, k, dtype, block=128, d_high=cfg.d_high, d_low=cfg.d_low, p=cfg.p,
                                causal=cfg.causal)
    st = compare_masks(gm, orc, cfg.p, cfg.causal)
    say(f"[estimator] {name}: density={gm.sum() / st['blocks']:.4f} mismatch={st['mismatch']} "
        f"mass_tie={st['mass_tie']} score_tie={st['score_tie']} unexcused={st['unexcused']} {st['where'][:5]}")
    record_parity(f"special:{name}", st)
    assert st["unexcused"] == 0, st["where"][:20]
    return gm, orc


@pytest.mark.parametrize("p", [0.5, 0.95])
def test_estimator_uniform_rows(p):
    """Identical blocks: every score of a row ties, so Top-P keeps the
    ceil(p * n) lowest block indices (more than 64 equal entries per row)."""
    from synth import f32_to_bf16_bits
    N = 300 * 128
    x = f32_to_bf16_bits(np.ones((1, N, 2, 128), np.float32))
    kx = f32_to_bf16_bits(np.ones((1, N, 1, 128), np.float32))
    gm, _ = _estimate_and_compare(f"uniform p={p}", x, kx, "bf16", prism.EstimatorConfig(p=p))
    for i in (0, 1, 99, 299):
        assert gm[0, 0, i, : i + 1].sum() == int(np.ceil(p * (i + 1) - 1e-12))
        assert gm[0, 0, i, : int(np.ceil(p * (i + 1) - 1e-12))].all()


@pytest.mark.timeout(600)
def test_estimator_uniform_long_rows():
    """Identical blocks on rows of up to 4600 blocks: every entry of a row
    falls in one histogram bin, so rows past 4095 blocks hold more entries
    in a bin than a 12-bit count can (the widest selection keeps 14)."""
    from synth import f32_to_bf16_bits
    nb = 4600
    x = f32_to_bf16_bits(np.ones((1, nb * 128, 1, 128), np.float32))
    p = 0.95
    gm, _ = _estimate_and_compare("uniform long rows", x, x, "bf16", prism.EstimatorConfig(p=p))
    for i in (2047, 2048, 4094, 4095, 4096, nb - 1):
        keep = int(np.ceil(p * (i + 1) - 1e-12))
        assert gm[0, 0, i, : i + 1].sum() == keep, i
        assert gm[0, 0, i, :keep].all(), i


@pytest.mark.parametrize("a,p", [(1.1, 0.999), (1.3, 0.9999)])
def test_estimator_peaked_rows_deep_tail(a, p):
    """One dominant key block and p close to 1: the threshold falls far below
    the row max (about 2^-12 .. 2^-20 of it, beyond the first 64 quarter
    octaves for a = 1.3)."""
    from synth import f32_to_bf16_bits
    rng = np.random.default_rng(21)
    N = 200 * 128
    v = rng.standard_normal(128).astype(np.float32)
    q = 0.3 * rng.standard_normal((1, N, 2, 128)).astype(np.float32) + a * v
    k = 0.3 * rng.standard_normal((1, N, 1, 128)).astype(np.float32)
    k[0, :128, 0, :] += a * v  # key block 0 aligned with every query
    _estimate_and_compare(f"peaked a={a} p={p}", f32_to_bf16_bits(q), f32_to_bf16_bits(k), "bf16",
                          prism.EstimatorConfig(p=p))


def test_estimator_zero_keys_degenerate_temperature():
    """K = 0: every band RMS of K is 0, so the temperature falls back to 1
    (counted as degenerate) and every score of a row is 0 -- uniform rows."""
    from synth import f32_to_bf16_bits
    rng = np.random.default_rng(5)
    N = 40 * 128 - 9
    q = f32_to_bf16_bits(rng.standard_normal((1, N, 2, 128)).astype(np.float32))
    k = f32_to_bf16_bits(np.zeros((1, N, 1, 128), np.float32))
    gm, orc = _estimate_and_compare("zero keys", q, k, "bf16", prism.EstimatorConfig(p=0.9))
    assert all(r["degenerate"] == 2 for r in orc.values())
    for i in (0, 7, 39):
        assert gm[0, 0, i, : i + 1].sum() == int(np.ceil(0.9 * (i + 1) - 1e-12))


@pytest.mark.parametrize("scale", [16.0, 64.0])
def test_attention_large_logits(scale):
    """Queries scaled up so the softmax rows are nearly one-hot and running
    maxima jump by far more than the lazy-rescale slack, sub-tile after
    sub-tile (bf16 and fp32 paths)."""
    for base, seq in (("llama3_8b_32k", 2600), ("tiny_fp32_2k", 900)):
        w = WORKLOADS[base].scaled(seq=seq, hq=2, hkv=1)
        q, k, v = make_qkv(w)
        q64 = to_f64(q, w.dtype) * scale
        if w.dtype == "bf16":
            from synth import f32_to_bf16_bits
            q = f32_to_bf16_bits(q64.astype(np.float32))
        else:
            q = q64.astype(np.float32)
        mask = random_mask(1, w.hq, w.nb, 0.7, 23, True)
        qd, kd, vd = (to_device(x, w.dtype) for x in (q, k, v))
        out = torch.full_like(qd, float("nan"))
        prism.block_sparse_attn(qd, kd, vd, torch.from_numpy(mask).cuda(), out=out)
        torch.cuda.synchronize()
        say(f"[large logits] {base} x{scale}")
        check_attention(out.float().cpu().numpy(), oracle_attention(q, k, v, mask, w.dtype, True), w.dtype)


def test_estimator_deterministic_and_overwrites():
    w = WORKLOADS["llama3_8b_32k"].scaled(seq=5000, hq=8, hkv=2)
    q, k, _ = make_qkv(w, with_v=False)
    qd, kd = to_device(q, "bf16"), to_device(k, "bf16")
    cfg = cfg_of(w)
    outs = []
    for fill in (0x00, 0xFF):
        L = prism.workspace_layout(qd, kd, cfg)
        ws = torch.full((L.total_bytes,), fill, dtype=torch.uint8, device="cuda")
        m = torch.full((1, w.hq, L.nb, L.nb), fill, dtype=torch.uint8, device="cuda")
        prism.estimate(qd, kd, cfg, workspace=ws, mask_out=m)
        torch.cuda.synchronize()
        outs.append((m.cpu().numpy(), ws[: L.ksq_offset].cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1], outs[1][1])


# ------------------------------------------------- bit-packed masks, long rows
@pytest.mark.parametrize("name", ["gqa4_ragged", "noncausal", "one_block", "nb_1100", "p_one"])
def test_estimator_bit_mask_equals_byte_mask(name):
    """The bit-packed output holds exactly the byte mask's selection, padding
    bits 0 (same selection code, only the row store differs)."""
    base, over, cov, layout, rope_layout = SMALL[name]
    w = WORKLOADS[base].scaled(**over)
    say(f"[bits] {name}: seq={w.seq} hq={w.hq}")
    q, k, _ = make_qkv(w, rope_layout=rope_layout, with_v=False)
    cfg = cfg_of(w, **{**cov, "rope_layout": rope_layout})
    qd, kd = to_device(q, w.dtype, layout), to_device(k, w.dtype, layout)
    nb = w.nb
    m8 = prism.estimate(qd, kd, cfg)
    mb = torch.full((w.batch, w.hq, nb, (nb + 31) // 32), -1, dtype=torch.int32, device="cuda")
    prism.estimate(qd, kd, cfg, mask_out=mb)
    torch.cuda.synchronize()
    g8, gb = m8.cpu().numpy(), mb.cpu().numpy()
    assert np.array_equal(gb, pack_bits(g8))
    assert np.array_equal(unpack_bits(gb, nb), g8)


@pytest.mark.parametrize("dtype_base,over,density,causal", [
    ("llama3_8b_32k", dict(seq=2900, hq=4, hkv=1), 0.5, True),
    ("llama3_8b_32k", dict(seq=1500, hq=2, hkv=1), 0.6, False),
    ("tiny_fp32_2k", dict(seq=1500, hq=2, hkv=1), 0.5, True),
])
def test_attention_bit_mask_equals_byte_mask(dtype_base, over, density, causal):
    w = WORKLOADS[dtype_base].scaled(**over)
    say(f"[bits attention] seq={w.seq} {w.dtype} causal={causal}")
    q, k, v = make_qkv(w)
    m = random_mask(w.batch, w.hq, w.nb, density, 5, causal)
    if causal:
        m[:, :, 2, 5] = 1  # a set bit above the diagonal is ignored in both forms
    qd, kd, vd = (to_device(x, w.dtype) for x in (q, k, v))
    outs = []
    for mk in (torch.from_numpy(m).cuda(), torch.from_numpy(pack_bits(m)).cuda()):
        o = torch.full_like(qd, float("nan"))
        prism.block_sparse_attn(qd, kd, vd, mk, causal=causal, out=o)
        torch.cuda.synchronize()
        outs.append(o.cpu())
    assert torch.equal(outs[0].view(torch.int16) if w.dtype == "bf16" else outs[0].view(torch.int32),
                       outs[1].view(torch.int16) if w.dtype == "bf16" else outs[1].view(torch.int32))


LONG = {
    # rows longer than 2048 blocks take the 64- and 128-slot register selection and the chunked
    # attention block list
    "nb_4100_causal": ("llama3_8b_32k", dict(seq=4100 * 128 - 7, hq=1, hkv=1), dict()),
    "nb_2300_noncausal_p05": ("llama3_8b_32k", dict(seq=2300 * 128, hq=1, hkv=1, causal=False), dict(p=0.5)),
    "nb_2100_p_one": ("llama3_8b_32k", dict(seq=2100 * 128, hq=1, hkv=1), dict(p=1.0)),
    "nb_8192_max": ("llama3_8b_32k", dict(seq=8192 * 128, hq=1, hkv=1), dict()),  # 1,048,576 tokens, the largest
    "nb_2100_fp32": ("tiny_fp32_2k", dict(seq=2100 * 128 - 3, hq=1, hkv=1), dict()),
    "nb_2100_intersect": ("llama3_8b_32k", dict(seq=2100 * 128, hq=1, hkv=1), dict(merge="intersect")),
}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(LONG))
def test_long_rows(name):
    base, over, cov = LONG[name]
    w = WORKLOADS[base].scaled(**over)
    say(f"[long] {name}: seq={w.seq} nb={w.nb} causal={w.causal}")
    q, k, v = make_qkv(w)
    cfg = cfg_of(w, **cov)
    qd, kd, vd = (to_device(x, w.dtype) for x in (q, k, v))
    m8 = prism.estimate(qd, kd, cfg)
    mb = prism.estimate(qd, kd, cfg, bits=True)
    torch.cuda.synchronize()
    gm = m8.cpu().numpy()
    assert np.array_equal(mb.cpu().numpy(), pack_bits(gm))
    orc = oracle_estimate_heads(q, k, w.dtype, block=w.block, d_high=cfg.d_high, d_low=cfg.d_low, p=cfg.p,
                                causal=cfg.causal, merge=cfg.merge)
    st = compare_masks(gm, orc, cfg.p, cfg.causal, merge=cfg.merge)
    say(f"    density={gm.sum() / max(1, st['blocks']):.4f} mismatch={st['mismatch']} mass_tie={st['mass_tie']} "
        f"score_tie={st['score_tie']} unexcused={st['unexcused']} {st['where'][:5]}")
    record_parity(f"long:{name}", st)
    assert st["unexcused"] == 0, st["where"][:20]
    # attention over the bit mask on rows past 2048 blocks (several list passes)
    out = torch.full_like(qd, float("nan"))
    prism.block_sparse_attn(qd, kd, vd, mb, causal=cfg.causal, out=out)
    torch.cuda.synchronize()
    og = out.float().cpu().numpy()
    assert not np.isnan(og).any()
    for i in sorted({w.nb - 1, 2047, 2048, w.nb // 2 + 3}):
        t0, t1 = i * 128, min((i + 1) * 128, w.seq)
        oo = po.attention_block_row(to_f64(q[0, :, 0, :], w.dtype), to_f64(k[0, :, 0, :], w.dtype),
                                    to_f64(v[0, :, 0, :], w.dtype), gm[0, 0, i], i, block=128, causal=cfg.causal)
        check_attention(og[0, t0:t1, 0, :], oo, w.dtype)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("bits,batch,causal", [(False, 1, True), (True, 1, True), (False, 2, False)])
def test_attention_head_pairs_long(bits, batch, causal):
    """Past 3072 blocks, two query heads of a KV group share one workgroup and
    its K/V tiles: heads with different masks, one head with empty rows while
    its pair partner computes, a ragged end, rows on both sides of the
    2048-block list passes; batch 2 and the non-causal form too."""
    w = WORKLOADS["llama3_8b_32k"].scaled(seq=3100 * 128 - 50, hq=4, hkv=2, batch=batch)
    say(f"[pairs] seq={w.seq} nb={w.nb} hq={w.hq} hkv={w.hkv} batch={batch} causal={causal} bits={bits}")
    q, k, v = make_qkv(w)
    m = random_mask(batch, w.hq, w.nb, 0.6, 17, causal)
    m[:, 1, 1500] = 0   # head 1 computes nothing on this row; head 0 (its pair) does
    m[:, 2, :, 2048:] = 0  # head 2 selects nothing past the first list pass
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    md = torch.from_numpy(pack_bits(m) if bits else m).cuda()
    out = torch.full_like(qd, float("nan"))
    prism.block_sparse_attn(qd, kd, vd, md, causal=causal, out=out)
    torch.cuda.synchronize()
    og = out.float().cpu().numpy()
    assert not np.isnan(og).any()
    assert np.all(og[:, 1500 * 128: 1501 * 128, 1] == 0)
    for bb in range(batch):
        for h in range(w.hq):
            for i in (0, 1500, 2047, 2048, w.nb - 1):
                t0, t1 = i * 128, min((i + 1) * 128, w.seq)
                g = po.kv_head(h, w.hq, w.hkv)
                oo = po.attention_block_row(to_f64(q[bb, :, h, :], "bf16"), to_f64(k[bb, :, g, :], "bf16"),
                                            to_f64(v[bb, :, g, :], "bf16"), m[bb, h, i], i, block=128,
                                            causal=causal)
                check_attention(og[bb, t0:t1, h, :], oo, "bf16")


# ------------------------------------------------------------ attention cases
def oracle_attention(q, k, v, mask, dtype, causal, rows=None):
    return po.block_sparse_attention(to_f64(q, dtype), to_f64(k, dtype), to_f64(v, dtype), mask, block=128,
                                     causal=causal, rows=rows)


def check_attention(og, oo, dtype, rows_mask=None):
    og = og.astype(np.float64)
    if rows_mask is not None:
        og, oo = og[rows_mask], oo[rows_mask]
    assert np.isfinite(og).all()
    err = np.abs(og - oo)
    if dtype == "bf16":
        rel = np.linalg.norm(og - oo) / max(np.linalg.norm(oo), 1e-30)
        say(f"    max_abs={err.max():.3e} rel_norm={rel:.3e} max|O|={np.abs(oo).max():.3e}")
        assert err.max() <= 2e-2
        assert rel <= 1e-2
    else:
        say(f"    max_abs={err.max():.3e} max|O|={np.abs(oo).max():.3e}")
        assert err.max() <= 1e-4 * np.abs(oo).max()


ATTN = {
    "dense_causal": ("llama3_8b_32k", dict(seq=1000, hq=4, hkv=2), "ones", True, "bshd"),
    "random_ragged": ("llama3_8b_32k", dict(seq=2900, hq=4, hkv=1), 0.5, True, "bshd"),
    "noncausal_random": ("llama3_8b_32k", dict(seq=1500, hq=2, hkv=1), 0.6, False, "bshd"),
    "noncausal_dense": ("llama3_8b_32k", dict(seq=700, hq=2, hkv=2), "ones", False, "bshd"),
    "diagonal_only": ("llama3_8b_32k", dict(seq=2000, hq=2, hkv=1), "diag", True, "bshd"),
    "empty_rows": ("llama3_8b_32k", dict(seq=2048, hq=2, hkv=1), "empty", True, "bshd"),
    "upper_bits_ignored": ("llama3_8b_32k", dict(seq=1500, hq=2, hkv=1), "full_square", True, "bshd"),
    "bhsd_gqa8": ("llama3_8b_32k", dict(seq=1800, hq=8, hkv=1), 0.7, True, "bhsd"),
    "batch2": ("llama3_8b_32k", dict(seq=1300, hq=2, hkv=2, batch=2), 0.5, True, "bshd"),
    "xcd_groups": ("llama3_8b_32k", dict(seq=1024, hq=16, hkv=8), 0.8, True, "bshd"),
    "fp32_random": ("tiny_fp32_2k", dict(seq=1500, hq=2, hkv=1), 0.5, True, "bshd"),
    "fp32_noncausal": ("tiny_fp32_2k", dict(seq=600, hq=1, hkv=1), "ones", False, "bshd"),
    # sequence ends inside the first 64-key sub-tile of a block (the second lies wholly past it),
    # exactly at a sub-tile boundary, and one token into a new block
    "short_40": ("llama3_8b_32k", dict(seq=40, hq=2, hkv=1), "ones", True, "bshd"),
    "one_token": ("llama3_8b_32k", dict(seq=1, hq=2, hkv=1), "ones", True, "bshd"),
    "one_token_noncausal_fp32": ("tiny_fp32_2k", dict(seq=1, hq=2, hkv=1), "ones", False, "bshd"),
    "short_40_noncausal": ("llama3_8b_32k", dict(seq=40, hq=2, hkv=1), "ones", False, "bshd"),
    "sub_tile_192": ("llama3_8b_32k", dict(seq=192, hq=2, hkv=1), "ones", True, "bshd"),
    "one_token_block_257": ("llama3_8b_32k", dict(seq=257, hq=4, hkv=2), 0.7, True, "bshd"),
}


def make_mask(kind, w, causal, seed=11):
    nb = w.nb
    if kind == "ones":
        m = np.ones((w.batch, w.hq, nb, nb), np.uint8)
        return m * np.tril(np.ones((nb, nb), np.uint8)) if causal else m
    if kind == "full_square":
        return np.ones((w.batch, w.hq, nb, nb), np.uint8)  # upper blocks set but causal
    if kind == "diag":
        return np.broadcast_to(np.eye(nb, dtype=np.uint8), (w.batch, w.hq, nb, nb)).copy()
    if kind == "empty":
        m = random_mask(w.batch, w.hq, nb, 0.6, seed, causal)
        m[:, :, 3] = 0
        m[:, 1, 7] = 0
        return m
    return random_mask(w.batch, w.hq, nb, kind, seed, causal)


@pytest.mark.parametrize("name", list(ATTN))
def test_attention_small(name):
    base, over, kind, causal, layout = ATTN[name]
    w = WORKLOADS[base].scaled(**over)
    say(f"[attention] {name}: seq={w.seq} hq={w.hq} hkv={w.hkv} b={w.batch} {w.dtype} mask={kind} causal={causal}")
    q, k, v = make_qkv(w)
    mask = make_mask(kind, w, causal)
    qd, kd, vd = (to_device(x, w.dtype, layout) for x in (q, k, v))
    md = torch.from_numpy(mask).cuda()
    out = torch.full_like(qd, float("nan"))
    prism.block_sparse_attn(qd, kd, vd, md, causal=causal, out=out)
    torch.cuda.synchronize()
    og = out.float().cpu().numpy()
    oo = oracle_attention(q, k, v, mask, w.dtype, causal)
    check_attention(og, oo, w.dtype)
    if kind == "empty":
        assert np.all(og[:, 3 * 128: 4 * 128] == 0)


def test_attention_on_estimator_mask_and_deterministic():
    w = WORKLOADS["qwen3_8b_64k"].scaled(seq=6000, hq=4, hkv=1)
    q, k, v = make_qkv(w)
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    m = prism.estimate(qd, kd, cfg_of(w))
    outs = []
    for _ in range(2):
        o = torch.full_like(qd, float("nan"))
        prism.block_sparse_attn(qd, kd, vd, m, out=o)
        torch.cuda.synchronize()
        outs.append(o.view(torch.int16).cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    og = torch.from_numpy(outs[0]).view(torch.bfloat16).float().numpy()
    oo = oracle_attention(q, k, v, m.cpu().numpy(), "bf16", True)
    check_attention(og, oo, "bf16")


# ------------------------------------------------- graph capture, two streams
def test_graph_capture_replays_match_eager():
    """The library allocates nothing and never synchronises, so both calls can
    be captured into one HIP graph; every replay (with eager work and
    synchronisation in between) must give the eager bytes."""
    w = WORKLOADS["llama3_8b_32k"].scaled(seq=5000, hq=8, hkv=2)
    q, k, v = make_qkv(w)
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    cfg = cfg_of(w)
    ws = prism.new_workspace(qd, kd, cfg)
    mask = torch.empty((1, w.hq, w.nb, w.nb), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(qd)
    prism.estimate(qd, kd, cfg, workspace=ws, mask_out=mask)
    prism.block_sparse_attn(qd, kd, vd, mask, out=out)
    torch.cuda.synchronize()
    ref_m, ref_o = mask.clone(), out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            prism.estimate(qd, kd, cfg, workspace=ws, mask_out=mask)
            prism.block_sparse_attn(qd, kd, vd, mask, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(3):
        mask.fill_(9)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(mask, ref_m), r
        assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16)), r
        _ = (qd.float().sum() + 1).item()  # eager work between replays


def test_two_streams_concurrent_calls():
    """Calls are reentrant: two problems on two streams (own workspaces and
    outputs) give the same bytes as run alone."""
    ws_ = [WORKLOADS["llama3_8b_32k"].scaled(seq=4000, hq=4, hkv=1),
           WORKLOADS["qwen3_8b_64k"].scaled(seq=3000, hq=8, hkv=2)]
    data = []
    for w in ws_:
        q, k, v = make_qkv(w)
        qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
        cfg = cfg_of(w)
        m = prism.estimate(qd, kd, cfg)
        o = prism.block_sparse_attn(qd, kd, vd, m)
        torch.cuda.synchronize()
        data.append((qd, kd, vd, cfg, m.clone(), o.clone(), prism.new_workspace(qd, kd, cfg)))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for (qd, kd, vd, cfg, _, _, ws), st in zip(data, streams):
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            m = torch.empty((1, qd.shape[2], (qd.shape[1] + 127) // 128, (qd.shape[1] + 127) // 128),
                            dtype=torch.uint8, device="cuda")
            o = torch.empty_like(qd)
            for _ in range(3):
                prism.estimate(qd, kd, cfg, workspace=ws, mask_out=m)
                prism.block_sparse_attn(qd, kd, vd, m, out=o)
            outs.append((m, o))
    torch.cuda.synchronize()
    for (m, o), d in zip(outs, data):
        assert torch.equal(m, d[4])
        assert torch.equal(o.view(torch.int16), d[5].view(torch.int16))


# ------------------------------------------- K/V spans beyond 2 GiB (strided views)
@pytest.mark.timeout(600)
def test_fused_qkv_view_beyond_2gib():
    """Q, K, V as views into one fused QKV projection of a Llama-3-8B layer
    (32 + 8 + 8 heads of 128 per token: 12 KiB between token rows) at 180,000
    tokens, so the K and V views span 2.2 GB and every key row past token
    174,762 lies more than 2 GiB from the first. The views' results must be
    bit-identical to the same inputs stored contiguously, and sampled rows past
    that boundary must match the oracle."""
    w = WORKLOADS["llama3_8b_32k"].scaled(seq=180_000, hq=2, hkv=1)
    say(f"[fused qkv] seq={w.seq} nb={w.nb} row stride 12288 B")
    q, k, v = make_qkv(w)
    fused = torch.zeros((1, w.seq, 48, 128), dtype=torch.bfloat16, device="cuda")
    qc, kc, vc = (to_device(x, "bf16") for x in (q, k, v))
    qv, kv, vv = fused[:, :, 0:2], fused[:, :, 32:33], fused[:, :, 40:41]
    qv.copy_(qc)
    kv.copy_(kc)
    vv.copy_(vc)
    assert kv.stride(1) * 2 == 12288 and (w.seq - 1) * 12288 >= 1 << 31
    cfg = cfg_of(w)
    m_view = prism.estimate(qv, kv, cfg)
    m_cont = prism.estimate(qc, kc, cfg)
    o_view = torch.full_like(qc, float("nan"))
    o_cont = torch.full_like(qc, float("nan"))
    prism.block_sparse_attn(qv, kv, vv, m_view, out=o_view)
    prism.block_sparse_attn(qc, kc, vc, m_cont, out=o_cont)
    torch.cuda.synchronize()
    assert torch.equal(m_view, m_cont)
    assert torch.equal(o_view.view(torch.int16), o_cont.view(torch.int16))
    gm = m_view.cpu().numpy()
    og = o_view.float().cpu().numpy()
    for h in range(w.hq):
        g = po.kv_head(h, w.hq, w.hkv)
        qh, kh, vh = to_f64(q[0, :, h, :], "bf16"), to_f64(k[0, :, g, :], "bf16"), to_f64(v[0, :, g, :], "bf16")
        for i in (1366, 1400, w.nb - 1):
            t0, t1 = i * 128, min((i + 1) * 128, w.seq)
            oo = po.attention_block_row(qh, kh, vh, gm[0, h, i], i, block=128, causal=True)
            check_attention(og[0, t0:t1, h, :], oo, "bf16")


# ------------------------------------------------------------ full workloads
def oracle_workers(nb):
    """threads for the oracle's per-head work (numpy releases the GIL in its
    array kernels; BLAS is held to one thread per call meanwhile)"""
    import os
    n = min(16, os.cpu_count() or 1)
    return max(1, min(n, 8)) if nb > 4096 else n


def attention_errors(og, oo, dtype):
    """(max abs error, norm-relative error) of one query-block row"""
    og = og.astype(np.float64)
    assert np.isfinite(og).all()
    err = float(np.abs(og - oo).max())
    rel = float(np.linalg.norm(og - oo) / max(np.linalg.norm(oo), 1e-30))
    if dtype == "bf16":
        assert err <= 2e-2 and rel <= 1e-2, (err, rel)
    else:
        assert err <= 1e-4 * np.abs(oo).max(), err
    return err, rel


def sample_head_rows(nb, n, seed):
    """n query-block rows of one head: the first, the last and seeded others"""
    rng = np.random.default_rng(seed)
    rows = {0, nb - 1}
    while len(rows) < min(n, nb):
        rows.add(int(rng.integers(nb)))
    return sorted(rows)


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_full(name):
    """Every query head's mask against the oracle under the mask rule (and,
    up to 1024 blocks, every band logit within the tested bound); attention
    on 32 sampled query-block rows of every head (one row per head past 1024
    blocks, spread over both sides of the 2048-block list passes)."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    w = WORKLOADS[name]
    say(f"[workload] {name}: generating seq={w.seq} hq={w.hq} hkv={w.hkv} {w.dtype}")
    q, k, v = make_qkv(w)
    qd, kd, vd = (to_device(x, w.dtype) for x in (q, k, v))
    keep = w.nb <= 1024
    cfg = cfg_of(w, keep_logits=keep)
    L = prism.workspace_layout(qd, kd, cfg)
    ws = torch.empty(L.total_bytes, dtype=torch.uint8, device="cuda")
    mask = torch.full((1, w.hq, L.nb, L.nb), 9, dtype=torch.uint8, device="cuda")
    prism.estimate(qd, kd, cfg, workspace=ws, mask_out=mask)
    out = torch.full_like(qd, float("nan"))
    prism.block_sparse_attn(qd, kd, vd, mask, out=out)
    torch.cuda.synchronize()
    gm = mask.cpu().numpy()
    planes = None
    if keep:
        planes = ws[L.logits_offset: L.logits_offset + w.hq * 2 * L.logits_plane * 4].view(torch.float32)
        planes = planes.reshape(w.hq, 2, -1).cpu().numpy()
    del ws
    # outputs as stored (bf16 bits or fp32), widened row by row
    og = out.view(torch.int16).cpu().numpy().view(np.uint16) if w.dtype == "bf16" else out.cpu().numpy()
    assert not torch.isnan(out).any().item()
    del out
    nb = w.nb
    rows_idx = np.concatenate([np.arange(logit_row(i, nb, True), logit_row(i, nb, True) + i + 1) for i in range(nb)])
    tri = np.tril_indices(nb)

    def head_mask(h):
        r = oracle_estimate_heads(q, k, w.dtype, block=w.block, d_high=w.d_high, d_low=w.d_low, p=w.p,
                                  causal=True, heads=[h])
        st = compare_masks(gm, r, w.p, True)
        errs = (0.0, 0.0)
        if planes is not None:
            for z, key in enumerate(("L_high", "L_low")):
                gl = np.full((nb, nb), -np.inf)
                gl[tri] = planes[h, z][rows_idx]
                e = logit_errors(gl, r[(0, h)][key])
                errs = (max(errs[0], e[0]), max(errs[1], e[1]))
        return st, errs

    per_head = 32 if nb <= 1024 else 1
    special = [0, 2047, 2048, 4095, 4096, nb - 1]

    def head_attention(h):
        g = po.kv_head(h, w.hq, w.hkv)
        qh, kh, vh = (to_f64(x[0, :, hh, :], w.dtype) for x, hh in ((q, h), (k, g), (v, g)))
        rows = (sample_head_rows(nb, per_head, seed=w.seed * 1000 + h) if per_head > 1
                else [min(nb - 1, special[h % len(special)])])
        res = []
        for i in rows:
            t0, t1 = i * 128, min((i + 1) * 128, w.seq)
            oo = po.attention_block_row(qh, kh, vh, gm[0, h, i], i, block=128, causal=True)
            res.append(attention_errors(to_f64(og[0, t0:t1, h, :], w.dtype), oo, w.dtype))
        return res

    workers = oracle_workers(nb)
    say(f"    GPU done; oracle masks and attention rows over all {w.hq} heads ({workers} threads)")
    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        masks = list(ex.map(head_mask, range(w.hq)))
        attn = [e for r in ex.map(head_attention, range(w.hq)) for e in r]
    st = {"blocks": 0, "mismatch": 0, "mass_tie": 0, "score_tie": 0, "unexcused": 0, "where": [],
          "max_key_gap": 0.0, "max_key_gap_over_window": 0.0}
    for s_h, _ in masks:
        for key in ("blocks", "mismatch", "mass_tie", "score_tie", "unexcused"):
            st[key] += s_h[key]
        st["where"] += s_h["where"]
        st["max_key_gap"] = max(st["max_key_gap"], s_h["max_key_gap"])
        st["max_key_gap_over_window"] = max(st["max_key_gap_over_window"], s_h["max_key_gap_over_window"])
    lerr = (max(e[1][0] for e in masks), max(e[1][1] for e in masks))
    amax, arel = max(e[0] for e in attn), max(e[1] for e in attn)
    dens = gm.sum() / st["blocks"]
    say(f"    density={dens:.4f} mismatch={st['mismatch']} mass_tie={st['mass_tie']} score_tie={st['score_tie']} "
        f"(largest key-tie gap {st['max_key_gap']:.2e} = {st['max_key_gap_over_window']:.3f} of its window) "
        f"unexcused={st['unexcused']} {st['where'][:5]}")
    say(f"    logits: max abs error {lerr[0]:.2e}, per-row relative {lerr[1]:.2e} (bound {LOGIT_TOL_REL:.0e}); "
        f"attention over {len(attn)} rows: max_abs={amax:.3e} rel_norm={arel:.3e}")
    record_parity(f"full:{name}", st, {"density": float(dens), "heads_checked": w.hq,
                                       "logit_err_abs_log2": lerr[0], "logit_err_rel": lerr[1],
                                       "attn_rows": len(attn), "attn_max_abs": amax, "attn_rel_norm": arel})
    assert st["unexcused"] == 0, st["where"][:20]
    if keep:
        assert lerr[1] <= LOGIT_TOL_REL
