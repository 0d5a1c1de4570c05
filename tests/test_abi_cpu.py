"""The C ABI on the host: the library loads, exports what include/prism.h
declares, and rejects every bad argument with its status before any HIP call.

No call here reaches a kernel launch: every estimator / attention call has at
least one invalid argument, so the descriptors can carry fake (aligned,
non-null) device addresses that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

from block_sparse_attention_band_amd import _abi
from block_sparse_attention_band_amd._abi import PrismCfg, PrismMask, PrismTensor, PrismWorkspaceLayout

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "prism.h")
FAKE = 0x7F0000000000  # aligned, never dereferenced


@pytest.fixture(scope="module")
def lib():
    return _abi.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(prism_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert names == sorted(n for n, _, _ in _abi.SIGNATURES)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.prism_abi_version() == 7
    for s in range(11):
        assert lib.prism_status_str(s).decode() not in ("", "unknown status")
    assert lib.prism_status_str(42).decode() == "unknown status"


def tensor(seq=4096, heads=32, dtype=_abi.BF16, data=FAKE, head_dim=128, batch=1, layout="bshd"):
    if layout == "bshd":
        sb, ss, sh = seq * heads * head_dim, heads * head_dim, head_dim
    else:
        sb, ss, sh = heads * seq * head_dim, head_dim, seq * head_dim
    return PrismTensor(data, dtype, 0, batch, seq, heads, head_dim, sb, ss, sh)


def cfg(**kw):
    c = dict(block_size=128, d_high=64, d_low=96, p=0.95, causal=1, rope_layout=0, tau_mode=0, flags=0,
             workspace=FAKE, workspace_bytes=1 << 40)
    c.update(kw)
    return PrismCfg(**c)


def mask(seq=4096, heads=32, **kw):
    nb = -(-seq // 128)
    m = dict(data=FAKE, batch=1, heads=heads, nq_blocks=nb, nk_blocks=nb, block_size=128, causal=1, format=0,
             reserved=0)
    m.update(kw)
    return PrismMask(**m)


def est(lib, q, k, c, m):
    return lib.prism_estimate(ctypes.byref(q) if q is not None else None, ctypes.byref(k) if k is not None else None,
                              ctypes.byref(c) if c is not None else None, ctypes.byref(m) if m is not None else None,
                              None)


def attn(lib, q, k, v, m, o):
    r = lambda x: ctypes.byref(x) if x is not None else None
    return lib.prism_block_sparse_attn(r(q), r(k), r(v), r(m), r(o), None)


def test_logit_plane_rows_disjoint_and_padded():
    """the documented packed-triangle row starts: row i holds i + 1 floats,
    starts 16-byte aligned, and rows neither overlap nor leave a row short"""
    from tests.parity import logit_row
    for nb in (1, 2, 5, 8, 1023, 2048, 8192):
        prev_end = 0
        for i in range(nb):
            s = logit_row(i, nb, True)
            assert s % 4 == 0 and s >= prev_end
            prev_end = s + -(-(i + 1) // 4) * 4
        assert logit_row(nb, nb, True) == prev_end
        assert logit_row(3, nb, False) == 3 * (-(-nb // 4) * 4)


def test_workspace_layout(lib):
    q, k = tensor(seq=1000, heads=32), tensor(seq=1000, heads=8)
    L = PrismWorkspaceLayout()
    assert lib.prism_estimate_workspace_layout(ctypes.byref(q), ctypes.byref(k), ctypes.byref(cfg()), ctypes.byref(L)) == 0
    nb = 8
    assert L.nb == nb and (L.seg_lo, L.seg_hi, L.overlap) == (32, 64, 1)
    assert L.qbar_offset == 0 and L.kbar_offset >= 32 * nb * 128 * 4
    assert L.qsq_offset >= L.kbar_offset + 8 * nb * 128 * 4
    assert L.tau_offset >= L.ksq_offset + 8 * nb * 16
    assert L.total_bytes >= L.tau_offset + 32 * 32 and L.total_bytes % 256 == 0
    assert all(o % 256 == 0 for o in (L.kbar_offset, L.qsq_offset, L.ksq_offset, L.tau_offset))
    # up to 1024 blocks the logits stay on chip: no planes unless asked for
    assert L.logits_plane == 0 and L.total_bytes == L.logits_offset
    assert lib.prism_estimate_workspace_bytes(ctypes.byref(q), ctypes.byref(k), ctypes.byref(cfg())) == L.total_bytes
    keep = cfg(flags=E.EST_KEEP_LOGITS)
    lib.prism_estimate_workspace_layout(ctypes.byref(q), ctypes.byref(k), ctypes.byref(keep), ctypes.byref(L))
    # logit planes: 8 blocks, causal -> rows 0..7 packed with 4-float padding = 48 floats, plane 64
    assert L.logits_plane == 64 and L.logits_offset % 256 == 0
    assert L.logits_offset >= L.tau_offset + 32 * 32
    assert L.total_bytes >= L.logits_offset + 32 * 2 * 64 * 4
    assert lib.prism_estimate_workspace_bytes(ctypes.byref(q), ctypes.byref(k), ctypes.byref(keep)) == L.total_bytes
    lib.prism_estimate_workspace_layout(ctypes.byref(q), ctypes.byref(k), ctypes.byref(cfg(causal=0, flags=1)),
                                        ctypes.byref(L))
    assert L.logits_plane == 64  # 8 rows of 8 floats
    # unknown flag bits are rejected
    assert lib.prism_estimate_workspace_bytes(ctypes.byref(q), ctypes.byref(k), ctypes.byref(cfg(flags=4))) == 0
    # past 1024 blocks the logits always pass through the workspace
    q2, k2 = tensor(seq=1025 * 128, heads=2), tensor(seq=1025 * 128, heads=1)
    lib.prism_estimate_workspace_layout(ctypes.byref(q2), ctypes.byref(k2), ctypes.byref(cfg()), ctypes.byref(L))
    assert L.nb == 1025 and L.logits_plane > 0
    # a gap between the bands: the middle segment belongs to neither
    lib.prism_estimate_workspace_layout(ctypes.byref(q), ctypes.byref(k), ctypes.byref(cfg(d_high=32, d_low=48)),
                                        ctypes.byref(L))
    assert (L.seg_lo, L.seg_hi, L.overlap) == (32, 80, 0)
    assert lib.prism_estimate_workspace_bytes(ctypes.byref(q), ctypes.byref(k), ctypes.byref(cfg(p=1.5))) == 0
    for mode in (1, 2, 3):  # NONE, UNIT, PERVEC are valid temperature modes; 4 is not
        assert lib.prism_estimate_workspace_bytes(ctypes.byref(q), ctypes.byref(k), ctypes.byref(cfg(tau_mode=mode))) > 0
    assert lib.prism_estimate_workspace_bytes(ctypes.byref(q), ctypes.byref(k), ctypes.byref(cfg(tau_mode=4))) == 0


E = _abi


@pytest.mark.parametrize("case,expect", [
    (dict(q=None), E.ERR_NULL),
    (dict(q=tensor(data=0)), E.ERR_NULL),
    (dict(k=None), E.ERR_NULL),
    (dict(c=None), E.ERR_NULL),
    (dict(m=None), E.ERR_NULL),
    (dict(m=mask(data=0)), E.ERR_NULL),
    (dict(q=tensor(dtype=7)), E.ERR_DTYPE),
    (dict(k=tensor(heads=8, dtype=_abi.FP32)), E.ERR_DTYPE),
    (dict(q=tensor(seq=0)), E.ERR_SHAPE),
    (dict(k=tensor(heads=6)), E.ERR_SHAPE),           # 32 % 6 != 0
    (dict(k=tensor(heads=8, seq=2048)), E.ERR_SHAPE),
    (dict(m=mask(nq_blocks=31)), E.ERR_SHAPE),
    (dict(m=mask(heads=8)), E.ERR_SHAPE),
    (dict(q=PrismTensor(FAKE, 0, 0, 1, 4096, 32, 128, 0, 4096, 128)), E.ERR_STRIDE),
    (dict(q=tensor(data=FAKE + 8)), E.ERR_ALIGN),
    (dict(q=PrismTensor(FAKE, 0, 0, 1, 4096, 32, 128, 4096 * 4100, 4100, 128)), E.ERR_ALIGN),
    (dict(m=mask(data=FAKE + 4)), E.ERR_ALIGN),
    (dict(c=cfg(d_high=63)), E.ERR_CONFIG),
    (dict(c=cfg(d_high=0)), E.ERR_CONFIG),
    (dict(c=cfg(d_low=130)), E.ERR_CONFIG),
    (dict(c=cfg(p=0.0)), E.ERR_CONFIG),
    (dict(c=cfg(p=1.01)), E.ERR_CONFIG),
    (dict(c=cfg(p=float("nan"))), E.ERR_CONFIG),
    (dict(c=cfg(rope_layout=2)), E.ERR_CONFIG),
    (dict(c=cfg(tau_mode=5)), E.ERR_CONFIG),
    (dict(c=cfg(causal=2)), E.ERR_CONFIG),
    (dict(c=cfg(block_size=0)), E.ERR_CONFIG),
    (dict(c=cfg(workspace=0)), E.ERR_WORKSPACE),
    (dict(c=cfg(workspace=FAKE + 128)), E.ERR_WORKSPACE),
    (dict(c=cfg(workspace_bytes=1000)), E.ERR_WORKSPACE),
    (dict(q=tensor(head_dim=64), k=tensor(heads=8, head_dim=64)), E.ERR_UNSUPPORTED),
    (dict(c=cfg(block_size=64)), E.ERR_UNSUPPORTED),
    (dict(q=tensor(seq=8193 * 128), k=tensor(seq=8193 * 128, heads=8), m=mask(seq=8193 * 128)), E.ERR_UNSUPPORTED),
    (dict(m=mask(format=2)), E.ERR_CONFIG),
    (dict(c=cfg(merge=3)), E.ERR_CONFIG),
    (dict(c=cfg(merge=-1)), E.ERR_CONFIG),
    (dict(c=cfg(band_mode=2)), E.ERR_CONFIG),
    (dict(c=cfg(band_mode=1, d_high=56)), E.ERR_CONFIG),     # adaptive bands move in 16-dim steps
    (dict(c=cfg(band_mode=1, d_low=88)), E.ERR_CONFIG),
    (dict(c=cfg(band_mode=1, tau_mode=3)), E.ERR_CONFIG),    # per-vector temperature: static bands only
    # the mixture merge runs on the fused path (up to 1024 blocks)
    (dict(q=tensor(seq=1025 * 128), k=tensor(seq=1025 * 128, heads=8), m=mask(seq=1025 * 128),
          c=cfg(merge=2)), E.ERR_UNSUPPORTED),
    # launch limits: a second grid dimension of 65536, 2^32 work-items
    (dict(q=tensor(batch=65536, heads=1, seq=128), k=tensor(batch=65536, heads=1, seq=128),
          m=mask(seq=128, heads=1, batch=65536)), E.ERR_UNSUPPORTED),
    (dict(q=tensor(heads=4096, seq=8192 * 128), k=tensor(heads=8, seq=8192 * 128),
          m=mask(seq=8192 * 128, heads=4096)), E.ERR_UNSUPPORTED),
    (dict(m=mask(format=1, data=FAKE + 2)), E.ERR_ALIGN),
    # the single persistent launch: fused scores (up to 1024 blocks) and static bands only
    (dict(q=tensor(seq=1025 * 128), k=tensor(seq=1025 * 128, heads=8), m=mask(seq=1025 * 128),
          c=cfg(flags=E.EST_SINGLE_LAUNCH)), E.ERR_UNSUPPORTED),
    (dict(c=cfg(flags=E.EST_SINGLE_LAUNCH, band_mode=1)), E.ERR_UNSUPPORTED),
    (dict(c=cfg(flags=E.EST_SINGLE_LAUNCH | 8)), E.ERR_CONFIG),
])
def test_estimate_rejects(lib, case, expect):
    args = dict(q=tensor(), k=tensor(heads=8), c=cfg(), m=mask())
    args.update(case)
    assert est(lib, args["q"], args["k"], args["c"], args["m"]) == expect


@pytest.mark.parametrize("case,expect", [
    (dict(v=None), E.ERR_NULL),
    (dict(o=tensor(data=0)), E.ERR_NULL),
    (dict(m=None), E.ERR_NULL),
    (dict(v=tensor(heads=8, dtype=_abi.FP32)), E.ERR_DTYPE),
    (dict(o=tensor(dtype=_abi.FP32)), E.ERR_DTYPE),
    (dict(v=tensor(heads=4)), E.ERR_SHAPE),
    (dict(o=tensor(heads=8)), E.ERR_SHAPE),
    (dict(m=mask(nk_blocks=33)), E.ERR_SHAPE),
    (dict(m=mask(block_size=0)), E.ERR_SHAPE),
    (dict(o=PrismTensor(FAKE, 0, 0, 1, 4096, 32, 128, 4096 * 128, 64, 128 * 4096)), E.ERR_STRIDE),  # rows overlap
    (dict(m=mask(causal=3)), E.ERR_CONFIG),
    (dict(m=mask(block_size=64)), E.ERR_UNSUPPORTED),
    (dict(v=tensor(heads=8, data=FAKE + 2)), E.ERR_ALIGN),
    (dict(m=mask(format=7)), E.ERR_CONFIG),
    (dict(q=tensor(heads=4096, seq=8192 * 128), k=tensor(heads=8, seq=8192 * 128), v=tensor(heads=8, seq=8192 * 128),
          o=tensor(heads=4096, seq=8192 * 128), m=mask(seq=8192 * 128, heads=4096)), E.ERR_UNSUPPORTED),
    (dict(m=mask(format=1, data=FAKE + 1)), E.ERR_ALIGN),
    (dict(q=tensor(seq=8193 * 128), k=tensor(seq=8193 * 128, heads=8), v=tensor(seq=8193 * 128, heads=8),
          o=tensor(seq=8193 * 128), m=mask(seq=8193 * 128)), E.ERR_UNSUPPORTED),
])
def test_attention_rejects(lib, case, expect):
    args = dict(q=tensor(), k=tensor(heads=8), v=tensor(heads=8), m=mask(), o=tensor())
    args.update(case)
    assert attn(lib, args["q"], args["k"], args["v"], args["m"], args["o"]) == expect


def test_million_token_layout_and_bit_mask_accepted(lib):
    """8192 blocks (1,048,576 tokens) is the largest supported sequence; a
    4-byte aligned bit-packed mask passes the same validation as a byte mask
    (checked through the layout query and the rejection of a NULL workspace,
    neither of which launches)."""
    n = 8192 * 128
    q, k = tensor(seq=n), tensor(seq=n, heads=8)
    L = PrismWorkspaceLayout()
    assert lib.prism_estimate_workspace_layout(ctypes.byref(q), ctypes.byref(k), ctypes.byref(cfg()), ctypes.byref(L)) == 0
    assert L.nb == 8192 and L.logits_plane >= 8192 * 8193 // 2
    m = mask(seq=n, format=1, data=FAKE + 4)
    assert est(lib, q, k, cfg(workspace=0), m) == E.ERR_WORKSPACE  # every other check passed


def test_python_mask_descriptor_formats():
    import torch
    import block_sparse_attention_band_amd as prism
    u8 = prism.mask_desc(torch.zeros((1, 2, 40, 40), dtype=torch.uint8), 128, True)
    assert (u8.format, u8.nq_blocks, u8.nk_blocks) == (_abi.MASK_U8, 40, 40)
    bits = prism.mask_desc(torch.zeros((1, 2, 40, 2), dtype=torch.int32), 128, True)
    assert (bits.format, bits.nq_blocks, bits.nk_blocks) == (_abi.MASK_BITS, 40, 40)
    with pytest.raises(ValueError):
        prism.mask_desc(torch.zeros((1, 2, 40, 3), dtype=torch.int32), 128, True)


def test_layout_descriptors_bhsd_accepted_by_validation(lib):
    # BHSD strides pass validation (checked through the layout query, which never launches)
    q, k = tensor(layout="bhsd"), tensor(heads=8, layout="bhsd")
    L = PrismWorkspaceLayout()
    assert lib.prism_estimate_workspace_layout(ctypes.byref(q), ctypes.byref(k), ctypes.byref(cfg()), ctypes.byref(L)) == 0


def test_python_binding_raises_named_error(lib):
    err = _abi.PrismError(_abi.ERR_CONFIG, "prism_estimate")
    assert "PRISM_ERR_CONFIG" in str(err) and "configuration" in str(err)


def kv_tensor(row_bytes, seq=200_000, heads=8):
    """bf16 K/V descriptor whose token rows are row_bytes apart (e.g. a view
    into a fused QKV projection)"""
    ss = row_bytes // 2
    return PrismTensor(FAKE, _abi.BF16, 0, 1, seq, heads, 128, ss, ss, 128)  # batch 1: any batch stride


def test_attention_kv_row_stride_limit(lib):
    """K/V rows are addressed relative to each 64-key sub-tile, so the whole
    K/V span may pass 2 GiB and 4 GiB (a fused-QKV view of a Llama-3-8B layer,
    12 KiB per token, spans 2 GiB past 174,762 tokens); only a per-token
    stride above 16 MiB is refused. Accepted strides are shown by the next
    check failing instead (a mask of the wrong size), so nothing launches."""
    seq = 400_000
    nb = -(-seq // 128)
    q, o = tensor(seq=seq), tensor(seq=seq)
    bad_mask = mask(seq=seq, nk_blocks=nb + 1)
    for row_bytes in (12288, 1 << 16, 1 << 24):
        kv = kv_tensor(row_bytes, seq=seq)
        assert row_bytes * (seq - 1) >= (1 << 32)  # the span passes 4 GiB
        assert attn(lib, q, kv, kv, bad_mask, o) == E.ERR_SHAPE, row_bytes
    over = kv_tensor((1 << 24) + 16, seq=seq)
    ok = kv_tensor(12288, seq=seq)
    assert attn(lib, q, over, ok, bad_mask, o) == E.ERR_UNSUPPORTED
    assert attn(lib, q, ok, over, bad_mask, o) == E.ERR_UNSUPPORTED
    # fp32 K/V: the same byte limit
    ss = ((1 << 24) + 16) // 4
    f = PrismTensor(FAKE, _abi.FP32, 0, 1, seq, 8, 128, ss, ss, 128)
    qf, of_ = tensor(seq=seq, dtype=_abi.FP32), tensor(seq=seq, dtype=_abi.FP32)
    assert attn(lib, qf, f, f, bad_mask, of_) == E.ERR_UNSUPPORTED


def noalloc(lib, q, k, c, m):
    r = lambda x: ctypes.byref(x) if x is not None else None
    return lib.prism_estimate_noalloc(r(q), r(k), r(c), r(m), None)


@pytest.mark.parametrize("case,expect", [
    (dict(q=None), E.ERR_NULL),
    (dict(m=mask(data=0)), E.ERR_NULL),
    (dict(k=tensor(heads=6)), E.ERR_SHAPE),
    (dict(c=cfg(p=1.5)), E.ERR_CONFIG),
    (dict(m=mask(nq_blocks=31)), E.ERR_SHAPE),
    (dict(q=tensor(head_dim=64), k=tensor(heads=8, head_dim=64)), E.ERR_UNSUPPORTED),
])
def test_noalloc_rejects_like_estimate(lib, case, expect):
    """the no-allocation entry point runs the same argument checks, before any HIP call"""
    args = dict(q=tensor(), k=tensor(heads=8), c=cfg(workspace=0, workspace_bytes=0), m=mask())
    args.update(case)
    assert noalloc(lib, args["q"], args["k"], args["c"], args["m"]) == expect
    args["c"] = cfg() if args["c"] is not None and case.get("c") is None else args["c"]
    assert est(lib, args["q"], args["k"], args["c"], args["m"]) == expect


def test_noalloc_scratch_limit(lib):
    """problems whose workspace exceeds PRISM_NOALLOC_SCRATCH_BYTES are refused
    with PRISM_ERR_SCRATCH before any HIP call; the limit matches the header"""
    src = open(HEADER).read()
    assert "#define PRISM_NOALLOC_SCRATCH_BYTES (40u << 20)" in src
    limit = _abi.NOALLOC_SCRATCH_BYTES
    assert limit == 40 << 20
    # the 64-query-head, 8-KV-head layer at 131,072 tokens fits (37 MiB) ...
    q, k = tensor(seq=131072, heads=64), tensor(seq=131072, heads=8)
    need = lib.prism_estimate_workspace_bytes(ctypes.byref(q), ctypes.byref(k), ctypes.byref(cfg()))
    assert 36 << 20 < need <= limit
    # ... with 80 query heads it does not
    q2 = tensor(seq=131072, heads=80)
    need2 = lib.prism_estimate_workspace_bytes(ctypes.byref(q2), ctypes.byref(k), ctypes.byref(cfg()))
    assert need2 > limit
    assert noalloc(lib, q2, k, cfg(workspace=0), mask(seq=131072, heads=80)) == E.ERR_SCRATCH
    # past 1024 blocks the logit planes alone exceed it
    q3, k3 = tensor(seq=2048 * 128, heads=32), tensor(seq=2048 * 128, heads=8)
    assert noalloc(lib, q3, k3, cfg(workspace=0), mask(seq=2048 * 128)) == E.ERR_SCRATCH
    # the inspection copy of the logits counts too
    assert noalloc(lib, q, k, cfg(workspace=0, flags=E.EST_KEEP_LOGITS), mask(seq=131072, heads=64)) == E.ERR_SCRATCH


def test_adaptive_layout_sections(lib):
    """adaptive bands add a pooled-spectrum section (fp64, a value per RoPE pair of
    every query and KV head) and a per-head split section (4 int32) after the logits"""
    q, k = tensor(seq=1000, heads=32), tensor(seq=1000, heads=8)
    L = PrismWorkspaceLayout()
    assert lib.prism_estimate_workspace_layout(ctypes.byref(q), ctypes.byref(k), ctypes.byref(cfg()),
                                               ctypes.byref(L)) == 0
    static_total = L.total_bytes
    assert L.spectrum_offset == L.split_offset == L.total_bytes  # empty sections
    assert lib.prism_estimate_workspace_layout(ctypes.byref(q), ctypes.byref(k), ctypes.byref(cfg(band_mode=1)),
                                               ctypes.byref(L)) == 0
    assert L.spectrum_offset == static_total and L.spectrum_offset % 256 == 0
    assert L.split_offset >= L.spectrum_offset + (32 + 8) * 64 * 8 and L.split_offset % 256 == 0
    assert L.total_bytes >= L.split_offset + 32 * 16 and L.total_bytes % 256 == 0
    for merge in (1, 2):
        assert lib.prism_estimate_workspace_bytes(ctypes.byref(q), ctypes.byref(k), ctypes.byref(cfg(merge=merge))) \
            == static_total


def test_single_launch_layout_section(lib):
    """the single persistent launch adds a barrier section (4096 uint64 barrier words,
    the status word, a task counter, the go word, two words per query head) at the
    end of the workspace; nothing else moves"""
    q, k = tensor(seq=1000, heads=32), tensor(seq=1000, heads=8)
    L, L1 = PrismWorkspaceLayout(), PrismWorkspaceLayout()
    assert lib.prism_estimate_workspace_layout(ctypes.byref(q), ctypes.byref(k), ctypes.byref(cfg()),
                                               ctypes.byref(L)) == 0
    assert L.barrier_offset == L.total_bytes  # empty section
    assert lib.prism_estimate_workspace_layout(ctypes.byref(q), ctypes.byref(k),
                                               ctypes.byref(cfg(flags=E.EST_SINGLE_LAUNCH)), ctypes.byref(L1)) == 0
    for f in ("qbar_offset", "kbar_offset", "qsq_offset", "ksq_offset", "tau_offset", "logits_offset",
              "spectrum_offset", "split_offset", "barrier_offset"):
        assert getattr(L1, f) == getattr(L, f), f
    # 4096 barrier words, status and task counter (256 bytes), 16 go words 256 bytes apart,
    # 2 words per query head; rounded up to 256
    assert L1.total_bytes == L.total_bytes + (4096 * 8 + 256 + 16 * 256 + 32 * 16 + 255) // 256 * 256
    keep = cfg(flags=E.EST_SINGLE_LAUNCH | E.EST_KEEP_LOGITS)
    assert lib.prism_estimate_workspace_layout(ctypes.byref(q), ctypes.byref(k), ctypes.byref(keep),
                                               ctypes.byref(L1)) == 0
    assert L1.logits_plane == 64 and L1.barrier_offset >= L1.logits_offset + 32 * 2 * 64 * 4
