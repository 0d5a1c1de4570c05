"""The block-recall measurement (tests/recall_planted.py) at a small size:
its metric behaves as defined, and its comparison runs end to end."""
import numpy as np

from tests.recall_planted import block_attention_mass, masks, metrics, planted_blocks, run, split_sweep


def test_block_mass_rows_sum_to_one_and_full_mask_recalls_all():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((700, 2, 128))
    k = rng.standard_normal((700, 1, 128))
    A = block_attention_mass(q, k, 128)
    nb = A.shape[-1]
    assert np.allclose(A.sum(-1), 1.0, atol=1e-12)  # each query's softmax sums to 1
    assert not np.triu(A, 1).any()
    full = np.broadcast_to(np.tril(np.ones((nb, nb), bool)), A.shape)
    d, m, pr = metrics(full, A, planted_blocks(700, 128))
    assert d == 1.0 and abs(m - 1.0) < 1e-12 and pr == 1.0
    empty = np.zeros_like(full)
    assert metrics(empty, A, planted_blocks(700, 128))[:2] == (0.0, 0.0)


def test_recall_comparison_small():
    rows, A, P, recall = run(seq=4096, heads=2, verbose=True, equal_recall=True)
    for name, (p, d, m, pr) in rows.items():
        assert 0 < d <= 1 and 0 < m <= 1 and 0 < pr <= 1, name
    # density matching hits Prism's density within one block row's worth
    assert abs(rows["plain_density_matched"][1] - rows["prism"][1]) < 0.02
    # equal-recall search reaches the target mass recall for every reading
    for name, (target, p, (d, m, pr)) in recall.items():
        assert m >= target - 1e-9 and 0 < d <= 1, name


def test_split_sweep_small():
    target, out = split_sweep(seq=4096, heads=2, splits=((64, 96), (32, 112)), verbose=True)
    # the pages' split at its own p reaches the target at p <= the pages' p
    assert out[(64, 96)][0] <= 0.93 + 1e-9
    for (dh, dl), (p, (d, m, pr)) in out.items():
        assert m >= target - 1e-9 and 0 < d <= 1, (dh, dl)
