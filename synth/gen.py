"""Seeded synthetic inputs for the Prism estimator and block-sparse prefill.

This module builds inputs only. It holds none of the estimator's or the
attention's arithmetic (no pooling, RMS, temperature, softmax, Top-P or
attention), so both the HIP path and the CPU oracle may take their inputs
from it.

Post-RoPE Q and K are made the way a prefill layer would see them: a
pre-rotation vector per token, rotated by the standard rotary embedding
(pair j turns by angle t * theta_j at position t, theta_j = base^(-2j/d)).
The Prism pages name RoPE as the source of the high/low frequency split
(Prism review on paper.rainbus.top, novelty paragraph; gist.science
Technical Summary, section 1) but print no formula, so the RoFormer form is
used. Angles are computed in float64.

The pages also state that the method carries over to YaRN and M-RoPE
(gist.science, Results, generalization). Both are generated here from
their published definitions (class Rope): the estimator is unchanged, only
the angles differ.
  YaRN ("NTK-by-parts", Peng et al. 2023): with the original context L0,
    the scale s and r_j = L0 theta_j / (2 pi) (how many turns pair j makes
    over L0), gamma_j = clip((r_j - beta_slow) / (beta_fast - beta_slow),
    0, 1) and theta'_j = gamma_j theta_j + (1 - gamma_j) theta_j / s: fast
    pairs keep their frequency, slow pairs are interpolated. Q and K are
    both multiplied by the attention factor 0.1 ln(s) + 1.
  M-RoPE (Qwen2-VL; Qwen3-VL's interleaved variant): every token has three
    position ids (t, h, w) and pair j rotates by the id of its axis. Text
    tokens have t = h = w = their running position. A video prefix of
    nt x nh x nw patch tokens (frame-major, then row, then column) has ids
    (frame, row, column); text after it continues from max(nt, nh, nw).
    'sectioned' gives the first sections[0] pairs to t, the next
    sections[1] to h, the rest to w; 'interleaved' gives pair j to h when
    j = 1 mod 3 and j < 3 sections[1], to w when j = 2 mod 3 and
    j < 3 sections[2], and to t otherwise.

Every value is generated in float32, rotated in float64, rounded to float32
(round-to-nearest-even) and then, for bf16 workloads, to bfloat16
(round-to-nearest-even). The same bytes go to the GPU and to the oracle.

Seeds: one numpy PCG64 stream per (workload seed, tensor, head, batch), via
``np.random.default_rng([seed, tensor_id, head, batch])``.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

# tensor ids for seeding
T_QNOISE, T_KNOISE, T_V, T_SEMANTIC, T_SLASH = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Rope:
    """Which rotary embedding makes the post-RoPE inputs (see the module
    docstring for the formulas)."""

    kind: str = "default"  # "default", "yarn", "mrope"
    factor: float = 1.0  # YaRN scale s
    orig_ctx: int = 0  # YaRN original context L0
    beta_fast: float = 32.0
    beta_slow: float = 1.0
    mrope: str = "sectioned"  # or "interleaved"
    sections: tuple = ()  # pairs per axis (t, h, w), summing to d/2
    grid: tuple = (0, 0, 0)  # video prefix (frames, rows, columns) in patch tokens


@dataclass(frozen=True)
class Workload:
    """One synthetic attention-layer workload."""

    name: str
    seed: int
    batch: int
    seq: int
    hq: int
    hkv: int
    head_dim: int
    dtype: str  # "bf16" or "fp32"
    theta: float  # RoPE base
    kind: str  # "iid" (Q,K,V ~ N(0,1)), "semantic" (0.7*s + 0.7*z) or "spectral" (s band-limited per group)
    planted: bool  # slash + vertical structure planted in K
    p: float
    block: int = 128
    d_high: int = 64
    d_low: int = 96
    causal: bool = True
    rope: Rope = Rope()

    @property
    def nb(self) -> int:
        return -(-self.seq // self.block)

    def scaled(self, **kw) -> "Workload":
        """Same recipe at other sizes (the seed is kept unless given)."""
        return replace(self, **kw)


# The five workloads: Prism's hyperparameters B=128, d_high=64, d_low=96,
# p=0.95 (Llama) / 0.93 (Qwen) from the Prism review's reproducibility
# paragraph (paper.rainbus.top); model shapes are Llama-3-8B, Qwen3-8B and a
# one-GPU share of Llama-3-70B attention layers at 32K-128K tokens.
WORKLOADS = {
    "tiny_fp32_2k": Workload("tiny_fp32_2k", 1, 1, 2048, 1, 1, 128, "fp32", 1e4, "iid", False, 0.95),
    "llama3_8b_32k": Workload("llama3_8b_32k", 2, 1, 32768, 32, 8, 128, "bf16", 5e5, "semantic", False, 0.95),
    "llama3_8b_128k": Workload("llama3_8b_128k", 3, 1, 131072, 32, 8, 128, "bf16", 5e5, "semantic", False, 0.95),
    "qwen3_8b_64k": Workload("qwen3_8b_64k", 4, 1, 65536, 32, 8, 128, "bf16", 1e6, "semantic", True, 0.93),
    "llama3_70b_share_128k": Workload("llama3_70b_share_128k", 5, 1, 131072, 64, 8, 128, "bf16", 5e5, "semantic", False, 0.95),
    # the length the pages leave to future work: a Llama-3-8B-shaped layer at
    # 1,048,576 tokens (8192 blocks, the longest supported)
    "llama3_8b_1m": Workload("llama3_8b_1m", 8, 1, 1 << 20, 32, 8, 128, "bf16", 5e5, "semantic", False, 0.95),
    # RoPE variants the pages say the method carries over to: Qwen3-8B
    # extended from 32K to 128K by YaRN (factor 4), and a Qwen3-VL-8B-shaped
    # layer (interleaved M-RoPE, sections 24/20/20, base 5e6) over a video of
    # 16 frames x 32 x 48 patch tokens followed by text.
    "qwen3_8b_yarn_128k": Workload("qwen3_8b_yarn_128k", 6, 1, 131072, 32, 8, 128, "bf16", 1e6, "semantic", False,
                                   0.93, rope=Rope("yarn", factor=4.0, orig_ctx=32768)),
    # heads that differ in spectrum (the static band split's weakness): a
    # Llama-3-8B-shaped layer whose KV groups carry their semantic content in
    # different RoPE pair bands
    "llama3_8b_spectral_32k": Workload("llama3_8b_spectral_32k", 9, 1, 32768, 32, 8, 128, "bf16", 5e5, "spectral",
                                       False, 0.95),
    "qwen3_vl_8b_video_32k": Workload("qwen3_vl_8b_video_32k", 7, 1, 32768, 32, 8, 128, "bf16", 5e6, "semantic", False,
                                      0.93, rope=Rope("mrope", mrope="interleaved", sections=(24, 20, 20),
                                                      grid=(16, 32, 48))),
}


def _rng(seed: int, tensor_id: int, head: int, batch: int) -> np.random.Generator:
    return np.random.default_rng([seed, tensor_id, head, batch])


def rope_freqs(d: int, theta: float, rope: Rope = Rope()) -> np.ndarray:
    """theta_j (rad per position) of pairs j < d/2, YaRN-rescaled if asked."""
    j = np.arange(d // 2, dtype=np.float64)
    freq = theta ** (-2.0 * j / d)
    if rope.kind == "yarn":
        r = rope.orig_ctx * freq / (2.0 * np.pi)
        gamma = np.clip((r - rope.beta_slow) / (rope.beta_fast - rope.beta_slow), 0.0, 1.0)
        freq = gamma * freq + (1.0 - gamma) * freq / rope.factor
    return freq


def rope_positions(seq: int, rope: Rope = Rope()) -> np.ndarray:
    """Position ids [seq, 3] (t, h, w); equal columns unless M-RoPE."""
    n = np.arange(seq, dtype=np.int64)
    pos = np.repeat(n[:, None], 3, axis=1)
    if rope.kind == "mrope":
        nt, nh, nw = rope.grid
        nv = min(seq, nt * nh * nw)
        v = n[:nv]
        pos[:nv] = np.stack([v // (nh * nw), (v // nw) % nh, v % nw], axis=1)
        if seq > nv:
            pos[nv:] = (max(nt, nh, nw) + n[nv:] - nv)[:, None]
    return pos


def rope_axes(d: int, rope: Rope = Rope()) -> np.ndarray:
    """Axis (0 t, 1 h, 2 w) whose position id turns pair j."""
    j = np.arange(d // 2)
    if rope.kind != "mrope":
        return np.zeros(d // 2, np.int64)
    st, sh, sw = rope.sections
    if st + sh + sw != d // 2:
        raise ValueError("M-RoPE sections must sum to d/2")
    if rope.mrope == "sectioned":
        return np.where(j < st, 0, np.where(j < st + sh, 1, 2))
    if rope.mrope == "interleaved":
        return np.where((j % 3 == 1) & (j < 3 * sh), 1, np.where((j % 3 == 2) & (j < 3 * sw), 2, 0))
    raise ValueError(rope.mrope)


def rope_tables(seq: int, d: int, theta: float, rope: Rope = Rope()) -> tuple[np.ndarray, np.ndarray]:
    """cos/sin [seq, d/2] of the angle of pair j at token t, in float64 (for
    YaRN times the attention factor 0.1 ln(s) + 1)."""
    freq = rope_freqs(d, theta, rope)
    pos = rope_positions(seq, rope).astype(np.float64)
    ang = pos[:, rope_axes(d, rope)] * freq[None, :]
    amp = 0.1 * np.log(rope.factor) + 1.0 if rope.kind == "yarn" else 1.0
    return amp * np.cos(ang), amp * np.sin(ang)


def apply_rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray, layout: str) -> np.ndarray:
    """Rotate x [seq, d] (float64). 'interleaved' pairs dims (2j, 2j+1); 'half'
    pairs dims (j, j + d/2) (the rotate-half convention)."""
    d = x.shape[-1]
    if layout == "interleaved":
        a, b = x[..., 0::2], x[..., 1::2]
    elif layout == "half":
        a, b = x[..., : d // 2], x[..., d // 2:]
    else:
        raise ValueError(layout)
    ra = a * cos - b * sin
    rb = a * sin + b * cos
    out = np.empty_like(x)
    if layout == "interleaved":
        out[..., 0::2], out[..., 1::2] = ra, rb
    else:
        out[..., : d // 2], out[..., d // 2:] = ra, rb
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return f32_to_bf16_bits(x32) if dtype == "bf16" else x32


def _widen(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f32(x).astype(np.float64) if dtype == "bf16" else x.astype(np.float64)


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def spectral_window(d: int, g: int, hkv: int, rope_layout: str = "interleaved") -> np.ndarray:
    """Per-dim gain of KV group g's semantic vector in the 'spectral' recipe:
    RoPE pair j gets exp(-(j - c_g)^2 / (2 * 8^2)) with the centre c_g spread
    from pair 8 (fast) to pair 56 (slow) over the groups, scaled so the mean
    squared gain over the pairs is 1 (the same total energy as the isotropic
    recipe). Both dims of a pair get the pair's gain, in the pair layout of
    `rope_layout`."""
    j = np.arange(d // 2, dtype=np.float64)
    c = 8.0 + 48.0 * g / (hkv - 1) if hkv > 1 else d / 4.0
    a = np.exp(-((j - c) ** 2) / (2.0 * 8.0 ** 2))
    a /= np.sqrt(np.mean(a ** 2))
    out = np.empty(d)
    if rope_layout == "interleaved":
        out[0::2], out[1::2] = a, a
    else:
        out[: d // 2], out[d // 2:] = a, a
    return out


def make_qkv(w: Workload, rope_layout: str = "interleaved", with_v: bool = True):
    """Q [b, N, Hq, d], K [b, N, Hkv, d], V [b, N, Hkv, d] in BSHD order.

    bf16 workloads return uint16 bit patterns, fp32 workloads float32.
    Recipes:
      iid:      Q, K = RoPE(z), z ~ N(0,1) per token; V ~ N(0,1).
      semantic: Q_h = RoPE(0.7*s_g(h) + 0.7*z), K_g = RoPE(0.7*s_g + 0.7*z'),
                s_g ~ N(0,1)^d fixed per KV group g and shared by the group's
                query heads; V ~ N(0,1).
      spectral: as semantic, with s_g multiplied by spectral_window(g): each
                KV group's semantic content sits in its own band of RoPE
                pairs, from the fastest (group 0) to the slowest.
      planted (on top of semantic, on post-RoPE K of each KV group g):
        slash:    K_g[n] += 0.5 * mean_{h in g} Q_h[n + delta_n],
                  delta_n ~ U{1..4} per key (skipped past the end);
        vertical: K_g[n] += 1.0 * mean_{t, h in g} Q_h[t] for n % 4096 == 0.
    """
    b, N, Hq, Hkv, d = w.batch, w.seq, w.hq, w.hkv, w.head_dim
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    cos, sin = rope_tables(N, d, w.theta, w.rope)
    st = np.uint16 if w.dtype == "bf16" else np.float32
    q = np.empty((b, N, Hq, d), st)
    k = np.empty((b, N, Hkv, d), st)
    v = np.empty((b, N, Hkv, d), st) if with_v else None

    def semantic(bb, g):
        s = _rng(w.seed, T_SEMANTIC, g, bb).standard_normal(d, dtype=np.float32).astype(np.float64)
        if w.kind == "spectral":
            return s * spectral_window(d, g, Hkv, rope_layout)
        return s

    def pre(bb, tensor_id, head, g):
        z = _rng(w.seed, tensor_id, head, bb).standard_normal((N, d), dtype=np.float32).astype(np.float64)
        if w.kind in ("semantic", "spectral"):
            return 0.7 * semantic(bb, g)[None, :] + 0.7 * z
        return z

    def do_q(args):
        bb, h = args
        q[bb, :, h, :] = _store(apply_rope(pre(bb, T_QNOISE, h, h // G), cos, sin, rope_layout), w.dtype)

    def do_k(args):
        bb, g = args
        kk = apply_rope(pre(bb, T_KNOISE, g, g), cos, sin, rope_layout)
        if w.planted:
            qg = _widen(q[bb, :, g * G:(g + 1) * G, :], w.dtype).mean(axis=1)  # [N, d]
            delta = _rng(w.seed, T_SLASH, g, bb).integers(1, 5, size=N)
            src = np.arange(N) + delta
            ok = src < N
            kk[ok] += 0.5 * qg[src[ok]]
            kk[0::4096] += 1.0 * qg.mean(axis=0)[None, :]
        k[bb, :, g, :] = _store(kk, w.dtype)

    def do_v(args):
        bb, g = args
        z = _rng(w.seed, T_V, g, bb).standard_normal((N, d), dtype=np.float32)
        v[bb, :, g, :] = f32_to_bf16_bits(z) if w.dtype == "bf16" else z

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(do_q, [(bb, h) for bb in range(b) for h in range(Hq)]))
        list(ex.map(do_k, [(bb, g) for bb in range(b) for g in range(Hkv)]))
        if with_v:
            list(ex.map(do_v, [(bb, g) for bb in range(b) for g in range(Hkv)]))
    return q, k, v


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored values (bf16 bits or float32) to float64, exactly."""
    return _widen(x, dtype)


def random_mask(batch: int, heads: int, nb: int, density: float, seed: int, causal: bool = True) -> np.ndarray:
    """A seeded uint8 block mask [b, H, nb, nb] (1 = compute) for attention tests."""
    rng = np.random.default_rng([seed, 99])
    m = (rng.random((batch, heads, nb, nb)) < density).astype(np.uint8)
    if causal:
        m *= np.tril(np.ones((nb, nb), np.uint8))[None, None]
    return m


def planted_blocks(w: Workload) -> dict:
    """Block coordinates of the planted structure (for recall reports)."""
    B = w.block
    return {
        "slash_offsets": (1, 4),
        "vertical_key_blocks": sorted({n // B for n in range(0, w.seq, 4096)}),
    }


__all__ = [
    "Rope", "Workload", "WORKLOADS", "make_qkv", "rope_freqs", "rope_positions", "rope_axes", "rope_tables",
    "apply_rope", "f32_to_bf16_bits", "bf16_bits_to_f32", "to_f64", "random_mask", "planted_blocks",
]
