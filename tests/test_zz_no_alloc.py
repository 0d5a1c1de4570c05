"""GPU: prism_estimate_noalloc (the library's own device scratch as the
workspace) through the C ABI, against prism_estimate with a caller workspace:
the same mask bytes on consecutive calls, each smaller than the one before,
so every later call runs on the scratch an earlier, larger call left behind."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_attention_band_amd as prism  # noqa: E402
from block_sparse_attention_band_amd import _abi  # noqa: E402
from synth import WORKLOADS, make_qkv  # noqa: E402
from tests.parity import to_device  # noqa: E402

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


# largest first: 37 MiB of scratch (64 query heads at 131,072 tokens), then
# 22 MB, then small ragged and fp32 problems
CASES = [
    ("llama3_70b_share_128k", dict(), {}),
    ("llama3_8b_128k", dict(), {}),
    ("llama3_8b_32k", dict(seq=3000, hq=8, hkv=2), dict(d_high=38, d_low=70)),
    ("tiny_fp32_2k", dict(seq=1900, hq=2, hkv=1), {}),
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("bits", [False, True])
def test_noalloc_matches_estimate_on_consecutive_calls(bits):
    for name, over, cov in CASES:
        w = WORKLOADS[name].scaled(**over)
        say(f"[noalloc] {name} seq={w.seq} hq={w.hq} hkv={w.hkv} {w.dtype} bits={bits} {cov}")
        q, k, _ = make_qkv(w, with_v=False)
        qd, kd = to_device(q, w.dtype), to_device(k, w.dtype)
        cfg = prism.EstimatorConfig(p=w.p, **cov)
        assert prism.workspace_bytes(qd, kd, cfg) <= _abi.NOALLOC_SCRATCH_BYTES
        ref = prism.estimate(qd, kd, cfg, bits=bits)
        got = torch.full_like(ref, -1 if bits else 0x5A)  # poisoned: every element must be written
        prism.estimate_noalloc(qd, kd, cfg, mask_out=got)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), name
        del qd, kd, ref, got


def test_noalloc_refuses_problems_beyond_its_scratch():
    w = WORKLOADS["llama3_8b_32k"].scaled(seq=1100 * 128, hq=16, hkv=2)  # 1100 blocks: logit planes needed
    q, k, _ = make_qkv(w, with_v=False)
    qd, kd = to_device(q, "bf16"), to_device(k, "bf16")
    cfg = prism.EstimatorConfig(p=w.p)
    assert prism.workspace_bytes(qd, kd, cfg) > _abi.NOALLOC_SCRATCH_BYTES
    m = torch.full((1, w.hq, w.nb, w.nb), 7, dtype=torch.uint8, device="cuda")
    with pytest.raises(prism.PrismError, match="PRISM_ERR_SCRATCH"):
        prism.estimate_noalloc(qd, kd, cfg, mask_out=m)
    torch.cuda.synchronize()
    assert bool((m == 7).all())  # nothing was enqueued
