"""GPU: the block-level ground truth of tests/recall_gpu.py against the CPU
float64 computation of tests/recall_planted.py at a small size, and the
variant comparison end to end."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def test_block_mass_matches_cpu_float64():
    from synth import WORKLOADS, make_qkv, to_f64
    from tests.recall_gpu import block_mass_gpu
    from tests.recall_planted import block_attention_mass
    w = WORKLOADS["qwen3_8b_64k"].scaled(seq=2000, hq=4, hkv=2)
    q, k, _ = make_qkv(w, with_v=False)
    dev = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    A = block_mass_gpu(dev(q), dev(k), 128, chunk_blocks=3).cpu().numpy()
    ref = block_attention_mass(to_f64(q, "bf16")[0], to_f64(k, "bf16")[0], 128)
    assert np.abs(A - ref).max() < 1e-5
    assert np.allclose(A.sum(-1), 1.0, atol=1e-5)


@pytest.mark.timeout(300)
def test_recall_variants_small(monkeypatch):
    import tests.recall_gpu as rg
    from synth import WORKLOADS
    monkeypatch.setitem(WORKLOADS, "qwen3_small", WORKLOADS["qwen3_8b_64k"].scaled(name="qwen3_small", seq=8192,
                                                                                   hq=8, hkv=2))
    res = rg.run("qwen3_small", iters=8)
    t = res["target_mass_recall"]
    for name, r in res["rows"].items():
        d, m, pl = r["at_equal_recall"]
        assert 0 < d <= 1 and m >= t - 1e-9 and 0 <= pl <= 1, name
