"""GPU: the estimator as one persistent launch (PRISM_EST_SINGLE_LAUNCH) against
the three-launch path, through the C ABI. Both run the same arithmetic in the
same order, so the masks and every workspace intermediate (block means,
segment energies, temperatures, logits when kept) must agree bit for bit; the
masks are also held to the oracle under the parity rule of tests/parity.py.
The barrier words start from garbage (a workspace filled with 0xFF) and from
the previous call's values (two calls in a row on one workspace); the
barrier's status word must stay 0."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_attention_band_amd as prism  # noqa: E402
from synth import WORKLOADS, make_qkv  # noqa: E402
from tests.parity import compare_masks, oracle_estimate_heads, to_device  # noqa: E402
from tests.test_parity_gpu import SMALL, cfg_of  # noqa: E402

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    prism.lib()
    yield
    torch.cuda.synchronize()


# every small case the single launch takes: static bands, at most 1024 blocks
SINGLE = [n for n, (base, over, cov, _, _) in SMALL.items()
          if cov.get("band_mode", "static") == "static"
          and (WORKLOADS[base].scaled(**over).seq + 127) // 128 <= 1024]


def sections(ws, L, with_logits):
    names = ["qbar", "kbar", "qsq", "ksq", "tau"] + (["logits"] if with_logits else [])
    ends = {"qbar": L.kbar_offset, "kbar": L.qsq_offset, "qsq": L.ksq_offset, "ksq": L.tau_offset,
            "tau": L.logits_offset, "logits": L.spectrum_offset}
    return {n: ws[getattr(L, n + "_offset"): ends[n]].cpu().numpy() for n in names}


def run_both(qd, kd, cfg, bits=False, calls=1):
    """(mask, sections, status) of the three-launch path and of the single launch"""
    out = []
    for single in (False, True):
        c = prism.EstimatorConfig(**{**cfg.__dict__, "single_launch": single})
        L = prism.workspace_layout(qd, kd, c)
        ws = torch.full((L.total_bytes,), 0xFF, dtype=torch.uint8, device="cuda")
        if single:
            st = L.barrier_offset + 4096 * 8
            ws[st: st + 4] = 0  # the library never clears the status word
        nb = int(L.nb)
        shape = (qd.shape[0], qd.shape[2], nb, (nb + 31) // 32 if bits else nb)
        m = None
        for _ in range(calls):
            m = torch.full(shape, 7, dtype=torch.int32 if bits else torch.uint8, device="cuda")
            prism.estimate(qd, kd, c, workspace=ws, mask_out=m)
        torch.cuda.synchronize()
        status = int(ws[L.barrier_offset + 4096 * 8: L.barrier_offset + 4096 * 8 + 4].view(torch.int32).item()) \
            if single else 0
        out.append((m.cpu().numpy(), sections(ws, L, cfg.keep_logits), status))
    return out


def assert_same(ref, single, name):
    (m0, s0, _), (m1, s1, status) = ref, single
    assert status == 0, f"{name}: a workgroup gave up at the barrier"
    assert np.array_equal(m0, m1), f"{name}: masks differ in {int((m0 != m1).sum())} entries"
    for k in s0:
        assert np.array_equal(s0[k], s1[k]), f"{name}: workspace section {k} differs"


@pytest.mark.parametrize("name", SINGLE)
def test_single_launch_equals_three_launches(name):
    base, over, cov, layout, rope_layout = SMALL[name]
    w = WORKLOADS[base].scaled(**over)
    say(f"[single] {name}: seq={w.seq} hq={w.hq} hkv={w.hkv} b={w.batch} {w.dtype} {layout} {cov}")
    q, k, _ = make_qkv(w, rope_layout=rope_layout, with_v=False)
    qd, kd = to_device(q, w.dtype, layout), to_device(k, w.dtype, layout)
    cfg = cfg_of(w, **{**cov, "rope_layout": rope_layout})
    ref, single = run_both(qd, kd, cfg)
    assert_same(ref, single, name)
    orc = oracle_estimate_heads(q, k, w.dtype, block=w.block, d_high=cfg.d_high, d_low=cfg.d_low, p=cfg.p,
                                causal=cfg.causal, rope_layout=rope_layout, tau_mode=cfg.tau_mode, merge=cfg.merge)
    res = compare_masks(single[0], orc, cfg.p, cfg.causal, merge=cfg.merge)
    assert res["unexcused"] == 0, (name, res)


@pytest.mark.parametrize("name,bits,keep,calls", [
    ("gqa4_ragged", True, False, 1),       # bit-packed rows
    ("gqa4_ragged", False, True, 1),       # logits kept in the workspace as well
    ("mha_batch2", False, False, 3),       # the barrier words hold the previous call's values
])
def test_single_launch_options(name, bits, keep, calls):
    base, over, cov, layout, rope_layout = SMALL[name]
    w = WORKLOADS[base].scaled(**over)
    say(f"[single options] {name}: bits={bits} keep_logits={keep} calls={calls}")
    q, k, _ = make_qkv(w, rope_layout=rope_layout, with_v=False)
    qd, kd = to_device(q, w.dtype, layout), to_device(k, w.dtype, layout)
    cfg = cfg_of(w, **{**cov, "rope_layout": rope_layout, "keep_logits": keep})
    ref, single = run_both(qd, kd, cfg, bits=bits, calls=calls)
    assert_same(ref, single, name)


@pytest.mark.parametrize("wname", ["llama3_8b_128k", "llama3_70b_share_128k", "llama3_8b_32k"])
def test_single_launch_full_size(wname):
    """the full layers: every head's mask and intermediates, bit for bit"""
    w = WORKLOADS[wname]
    say(f"[single full] {wname}: seq={w.seq} hq={w.hq} hkv={w.hkv}")
    q, k, _ = make_qkv(w, with_v=False)
    qd, kd = to_device(q, w.dtype), to_device(k, w.dtype)
    del q, k
    ref, single = run_both(qd, kd, cfg_of(w))
    assert_same(ref, single, wname)


def test_single_launch_many_heads_uncached_temperatures():
    """more query heads (batch x Hq = 576) than a workgroup keeps temperatures
    for in LDS: each strip reads its head's published words instead"""
    w = WORKLOADS["llama3_8b_32k"].scaled(seq=700, hq=64, hkv=8, batch=9)
    say(f"[single many heads] seq={w.seq} hq={w.hq} hkv={w.hkv} b={w.batch}")
    q, k, _ = make_qkv(w, with_v=False)
    qd, kd = to_device(q, w.dtype), to_device(k, w.dtype)
    ref, single = run_both(qd, kd, cfg_of(w))
    assert_same(ref, single, "many_heads")


def test_single_launch_refused_under_graph_capture():
    """a captured call would replay one barrier tag: the flag is refused on a
    capturing stream (nothing enqueued), and the default path still captures"""
    w = WORKLOADS["llama3_8b_32k"].scaled(seq=2000, hq=4, hkv=1)
    q, k, _ = make_qkv(w, with_v=False)
    qd, kd = to_device(q, w.dtype), to_device(k, w.dtype)
    cfg1 = cfg_of(w, single_launch=True)
    ws = prism.new_workspace(qd, kd, cfg1)
    mask = torch.empty((1, w.hq, w.nb, w.nb), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    err = None
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            try:
                prism.estimate(qd, kd, cfg1, workspace=ws, mask_out=mask)
            except prism.PrismError as e:
                err = e
            prism.estimate(qd, kd, cfg_of(w), workspace=ws, mask_out=mask)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert err is not None and err.status == prism._abi.ERR_UNSUPPORTED
    mask.fill_(9)
    g.replay()
    torch.cuda.synchronize()
    ref = prism.estimate(qd, kd, cfg1)  # eager single launch: the same bytes
    torch.cuda.synchronize()
    assert torch.equal(mask, ref)


def test_single_launch_two_streams_concurrent():
    """two single-launch calls in flight at once on two streams (own workspaces):
    each grid must become resident as a whole (cooperative launch), so neither
    waits on workgroups the other holds; both give the three-launch bytes and
    leave their status words at 0"""
    ws_ = [WORKLOADS["llama3_8b_32k"].scaled(seq=40000, hq=32, hkv=8),
           WORKLOADS["qwen3_8b_64k"].scaled(seq=30000, hq=32, hkv=8)]
    data = []
    for w in ws_:
        q, k, _ = make_qkv(w, with_v=False)
        qd, kd = to_device(q, w.dtype), to_device(k, w.dtype)
        ref = prism.estimate(qd, kd, cfg_of(w))
        cfg1 = cfg_of(w, single_launch=True)
        L = prism.workspace_layout(qd, kd, cfg1)
        ws = torch.zeros((L.total_bytes,), dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        data.append((qd, kd, cfg1, ref.clone(), ws, L))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for (qd, kd, cfg1, _, ws, L), st in zip(data, streams):
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            m = torch.empty_like(data[len(outs)][3])
            for _ in range(4):
                prism.estimate(qd, kd, cfg1, workspace=ws, mask_out=m)
            outs.append(m)
    torch.cuda.synchronize()
    for m, (qd, kd, cfg1, ref, ws, L) in zip(outs, data):
        status = int(ws[L.barrier_offset + 4096 * 8: L.barrier_offset + 4096 * 8 + 4].view(torch.int32).item())
        assert status == 0
        assert torch.equal(m, ref)
